"""The no-allocation decode call (csa_decode_index_topk_noalloc): through
the C ABI it gives exactly what csa_decode_index_topk gives with a caller
workspace (caches, selection, scores), on two calls in a row, the second
with a smaller input, so the library's scratch is reused with stale
contents from the first; a request beyond the scratch is refused before
anything is launched."""
import numpy as np
import pytest
import torch

import long_context_sparse_11_amd as L
from oracle import csa_oracle as O
from tests.helpers import dev, host
from tests.test_gpu_parity import _fresh_case, _fresh_jobs_and_refs, i32, i64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    L.lib()


def _both(N, Tq, n_ent, seed):
    d = _fresh_case("bf16", N, Tq, n_ent, False, seed=seed)
    m, K = d["m"], 512
    out = []
    for noalloc in (False, True):
        kidx, pool = dev(d["k_idx"]), dev(d["pool"])
        jobs, _ = _fresh_jobs_and_refs(d, kidx, pool)
        fn = L.csa_decode_index_topk_noalloc if noalloc else L.csa_decode_index_topk
        idx, sc, alls = fn(dev(d["q"]), dev(d["w"]), i32(d["n_ent"]), i64(d["q_pos0"]), K, m,
                           jobs, block_pos0=i64(d["block_pos0"]), want_scores=True,
                           want_all_scores=True)
        out.append((idx, sc, alls, kidx, pool))
    torch.cuda.synchronize()
    (i0, s0, a0, k0, p0), (i1, s1, a1, k1, p1) = out
    assert torch.equal(i0, i1) and torch.equal(s0, s1)
    assert torch.equal(k0, k1) and torch.equal(p0, p1)
    # scores of each query's visible entries (later columns are unspecified)
    for b in range(d["B"]):
        for t in range(Tq):
            nv = O.visible_count(int(d["q_pos0"][b]) + t, m, int(d["n_ent"][b]))
            assert np.array_equal(host(a0)[b, t, :nv], host(a1)[b, t, :nv]), (b, t)
    return host(i1)


def test_noalloc_decode_matches_workspace_call_twice():
    big = _both(40000, 2, [40000, 39001], seed=81)     # two-level select: candidates in scratch
    small = _both(3000, 1, [3000, 2500], seed=82)      # smaller, over the first call's contents
    assert big.shape == (2, 2, 512) and small.shape == (2, 1, 512)
    assert (small >= 0).sum() == 2 * 512


def test_noalloc_rejects_requests_beyond_the_scratch():
    # 2 x 8 queries x 2^20 entries of float32 scores exceed 32 MiB: refused
    # before any argument is read or anything launched
    B, Tq, N = 2, 8, 1 << 20
    need = L.csa_index_topk_ws_bytes(B, Tq, 64, N, 512)
    assert need > 32 << 20
    st = L.lib().csa_decode_index_topk_noalloc(1, B, Tq, 64, 128, N, 512, 4, 1, None, None, 2,
                                               None, None, None, None, None, None, None, None)
    assert st == -5
    assert "scratch" in L.lib().csa_status_string(st).decode()
