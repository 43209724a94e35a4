"""GPU parity of the streaming decode state: the window ring, the window-row
write, the device-side advance of positions and entry counts, the decode
call on steps that close no block, and a whole streamed decode from an
empty cache checked against the oracle run on the full token history.

Rules as in test_gpu_parity: attention and entries row-wise (bf16 2e-2);
selections by the band rule at 1e-4, plus the exact rule against the GPU's
own scores.  Stage isolation: each step's new cache entries are checked
against the oracle's compressor first; the oracle's indexer then ranks the
keys as the GPU stored them; the streamed attention is run on the oracle's
index sets (against the oracle's own entries), and the step's own output is
checked against the oracle's attention over the rows the GPU selected.
"""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_11_amd as L
from long_context_sparse_11_amd import synth
from oracle import csa_oracle as O
from tests.helpers import TOL_BF16, TOL_F32, check_band, dev, host, rowwise_rel_err
from tests.test_gpu_parity import _fresh_case, _fresh_jobs_and_refs, i32, i64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    L.lib()


def _ring_from_linear(lin, pos0, L_win):
    """Ring copy of a linear window buffer: token pos0 + r at row (pos0 + r) % L_win."""
    ring = np.empty_like(lin)
    for b in range(lin.shape[0]):
        for r in range(lin.shape[1]):
            ring[b, (pos0[b] + r) % L_win] = lin[b, r]
    return ring


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_ring_window_equals_linear_window(dt):
    """The same rows in a ring give bit-identical attention (CSA and HCA)."""
    rng = np.random.default_rng(40)
    H, D, R = (64, 512, 64) if dt == "bf16" else (4, 64, 16)
    B, N, K, W = 2, 300, 16, 24
    L_win = 24
    t = np.array([1000, 37])                      # query positions
    win_pos0 = t - W + 1
    win_pos0[1] = 14                              # sequence 1: window starts at token 14
    T = lambda x: synth.Tensor(x.astype(np.float32), dt)
    q = T(rng.standard_normal((B, 1, H, D)))
    pool = T(rng.standard_normal((B, N, D)))
    lin = rng.standard_normal((B, L_win, D)).astype(np.float32)
    ring = _ring_from_linear(lin, win_pos0, L_win)
    sink = rng.standard_normal(H).astype(np.float32)
    idx = np.sort(rng.choice(N, size=(B, 1, K)), axis=-1).astype(np.int32)
    a, la = L.csa_sparse_attn(dev(q), dev(pool), dev(idx), dev(T(lin)), i64(win_pos0), W,
                              dev(sink), i64(t), rope_dims=R, want_lse=True)
    b_, lb = L.csa_sparse_attn(dev(q), dev(pool), dev(idx), dev(T(ring)), None, W, dev(sink),
                               i64(t), rope_dims=R, want_lse=True)
    assert torch.equal(a, b_) and torch.equal(la, lb)
    n_ent = np.array([N, 9], np.int32)
    h1, _ = L.hca_attn(dev(q), dev(pool), i32(n_ent), 4, dev(T(lin)), i64(win_pos0), W,
                       dev(sink), i64(t), rope_dims=R)
    h2, _ = L.hca_attn(dev(q), dev(pool), i32(n_ent), 4, dev(T(ring)), None, W, dev(sink),
                       i64(t), rope_dims=R)
    assert torch.equal(h1, h2)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_window_row_writes_its_ring_slot(dt):
    rng = np.random.default_rng(41)
    B, D, R, L_win = 3, (512 if dt == "bf16" else 64), 16, 24
    kv = synth.Tensor(rng.standard_normal((B, 1, D)).astype(np.float32), dt)
    gain = (1 + 0.02 * rng.standard_normal(D)).astype(np.float32)
    pos = np.array([5, 24, 1000])
    win = dev(synth.Tensor(rng.standard_normal((B, L_win, D)).astype(np.float32), dt))
    before = win.clone()
    L.csa_window_row(dev(kv), i64(pos), win, gain=dev(gain), rope_dims=R)
    ref = O.csa_compress(kv.f32, None, None, 1, gain=gain, rope_dims=R, pos0=pos)[:, 0]
    tol = TOL_BF16 if dt == "bf16" else TOL_F32
    got, old = host(win), host(before)
    for b in range(B):
        r = pos[b] % L_win
        assert rowwise_rel_err(got[b, r][None], ref[b][None]) <= tol
        keep = [i for i in range(L_win) if i != r]
        assert np.array_equal(got[b, keep], old[b, keep])


def test_decode_advance_counts():
    B, m, N_cap = 3, 4, 6
    q_pos = torch.tensor([-1, 2, 40], dtype=torch.int64, device="cuda")
    n_ent = torch.zeros(B, dtype=torch.int32, device="cuda")
    blk = torch.zeros(B, dtype=torch.int64, device="cuda")
    want_pos = np.array([-1, 2, 40])
    for _ in range(9):
        L.csa_decode_advance(q_pos, n_ent, blk, m, N_cap)
        want_pos = want_pos + 1
        t = want_pos
        assert np.array_equal(host(q_pos), t)
        assert np.array_equal(host(n_ent), np.minimum((t + 1) // m, N_cap))
        assert np.array_equal(host(blk), np.where((t + 1) % m == 0, t + 1 - m, -1))


def test_decode_call_on_a_step_that_closes_no_block():
    """block_pos0 = -1 for sequence 0: its caches stay untouched and its
    selection ranks the stored entries (all scored by the indexer)."""
    d = _fresh_case("bf16", 3000, 1, [3000, 2500], False, seed=17)
    m, K = d["m"], 512
    kidx, pool = dev(d["k_idx"]), dev(d["pool"])
    k0, p0 = kidx.clone(), pool.clone()
    jobs, _ = _fresh_jobs_and_refs(d, kidx, pool)
    blk = d["block_pos0"].copy()
    blk[0] = -1
    gidx, _, gall = L.csa_decode_index_topk(dev(d["q"]), dev(d["w"]), i32(d["n_ent"]),
                                            i64(d["q_pos0"]), K, m, jobs, block_pos0=i64(blk),
                                            want_all_scores=True)
    assert torch.equal(kidx[0], k0[0]) and torch.equal(pool[0], p0[0])
    assert not torch.equal(kidx[1], k0[1])
    # sequence 0 against the indexer alone on the untouched keys
    idx2, _, all2 = L.csa_index_topk(dev(d["q"]), dev(d["w"]), k0, i32(d["n_ent"]),
                                     i64(d["q_pos0"]), K, m, want_all_scores=True)
    nv = O.visible_count(int(d["q_pos0"][0]), m, int(d["n_ent"][0]))
    assert np.array_equal(host(gall)[0, 0, :nv], host(all2)[0, 0, :nv])
    assert np.array_equal(host(gidx)[0], host(idx2)[0])


@pytest.mark.parametrize("window_in_step", [False, True])
def test_streamed_decode_matches_the_full_history(window_in_step):
    """40 tokens streamed one decode step at a time from an empty cache (B =
    2, Flash shapes, m = 4, top-4, window 16 in a ring of 16): positions and
    counts advance on the device, each step writes its window row (its own
    call, or the decode call's third job), closes a block every m tokens
    (pool and key entries) and attends.  The caches and every step's
    selection and attention match the oracle on the whole history."""
    rng = np.random.default_rng(50)
    B, T, m, K, W = 2, 40, 4, 4, 16
    H, D, R, Hi, Di = 64, 512, 64, 64, 128
    N_cap, L_win = 16, 16
    f = lambda *s, sc=1.0: (rng.standard_normal(s) * sc).astype(np.float32)
    bf = lambda x: synth.Tensor(x, "bf16")
    kv, q, q_idx = bf(f(B, T, D)), bf(f(B, T, H, D)), bf(f(B, T, Hi, Di))
    w_idx = f(B, T, Hi, sc=0.02)
    streams = {n: bf(f(B, T, D)) for n in ("c_a", "z_a", "c_b", "z_b")}
    kstreams = {n: bf(f(B, T, Di)) for n in ("c_a", "z_a", "c_b", "z_b")}
    bias = {n: f(m, D, sc=0.02) for n in ("a", "b")}
    kbias = {n: f(m, Di, sc=0.02) for n in ("a", "b")}
    gain, wgain = 1 + f(D, sc=0.02), 1 + f(D, sc=0.02)
    sink = f(H, sc=0.02)
    scale = 1.0 / math.sqrt(D)

    # device state
    q_pos = torch.full((B,), -1, dtype=torch.int64, device="cuda")
    n_ent = torch.zeros(B, dtype=torch.int32, device="cuda")
    blk = torch.zeros(B, dtype=torch.int64, device="cuda")
    pool = torch.zeros((B, N_cap, D), dtype=torch.bfloat16, device="cuda")
    kidx = torch.zeros((B, N_cap, Di), dtype=torch.bfloat16, device="cuda")
    ring = torch.zeros((B, L_win, D), dtype=torch.bfloat16, device="cuda")
    dev_s = {n: dev(v) for n, v in streams.items()}
    dev_k = {n: dev(v) for n, v in kstreams.items()}
    cur = {n: torch.zeros((B, m, D), dtype=torch.bfloat16, device="cuda") for n in streams}
    kcur = {n: torch.zeros((B, m, Di), dtype=torch.bfloat16, device="cuda") for n in kstreams}
    prev = {n: torch.zeros((B, m, D), dtype=torch.bfloat16, device="cuda") for n in ("c_b", "z_b")}
    kprev = {n: torch.zeros((B, m, Di), dtype=torch.bfloat16, device="cuda") for n in ("c_b", "z_b")}
    jobs = [dict(c_a=kcur["c_a"], z_a=kcur["z_a"], c_b=kcur["c_b"], z_b=kcur["z_b"],
                 prev_c_b=kprev["c_b"], prev_z_b=kprev["z_b"], bias_a=dev(kbias["a"]),
                 bias_b=dev(kbias["b"]), out=kidx),
            dict(c_a=cur["c_a"], z_a=cur["z_a"], c_b=cur["c_b"], z_b=cur["z_b"],
                 prev_c_b=prev["c_b"], prev_z_b=prev["z_b"], bias_a=dev(bias["a"]),
                 bias_b=dev(bias["b"]), gain=dev(gain), rope_dims=R, out=pool)]
    kv_d, q_d, qi_d, w_d = dev(kv), dev(q), dev(q_idx), dev(w_idx)
    kv_cur = torch.zeros((B, 1, D), dtype=torch.bfloat16, device="cuda")
    if window_in_step:
        jobs.append(dict(c_a=kv_cur, gain=dev(wgain), rope_dims=R, out=ring))

    # the oracle's caches over the full history (rounded to the caches' bf16)
    pool_ref = O.csa_compress(streams["c_a"].f32, streams["z_a"].f32, bias["a"], m,
                              c_b=streams["c_b"].f32, z_b=streams["z_b"].f32, bias_b=bias["b"],
                              gain=gain, rope_dims=R, pos0=[0, 0])
    keys_ref = O.csa_compress(kstreams["c_a"].f32, kstreams["z_a"].f32, kbias["a"], m,
                              c_b=kstreams["c_b"].f32, z_b=kstreams["z_b"].f32, bias_b=kbias["b"])
    win_ref = O.csa_compress(kv.f32, None, None, 1, gain=wgain, rope_dims=R, pos0=[0, 0])
    r16 = lambda x: bf(np.asarray(x, np.float32)).f32
    pool_r, keys_r, win_r = r16(pool_ref), r16(keys_ref), r16(win_ref)

    excused = 0
    for t in range(T):
        L.csa_decode_advance(q_pos, n_ent, blk, m, N_cap)
        s = t % m
        for n in streams:
            cur[n][:, s] = dev_s[n][:, t]
            kcur[n][:, s] = dev_k[n][:, t]
        if window_in_step:
            kv_cur.copy_(kv_d[:, t:t + 1])
        else:
            L.csa_window_row(kv_d[:, t:t + 1].contiguous(), q_pos, ring, gain=dev(wgain),
                             rope_dims=R)
        idx, _, alls = L.csa_decode_index_topk(qi_d[:, t:t + 1].contiguous(),
                                               w_d[:, t:t + 1].contiguous(), n_ent, q_pos, K, m,
                                               jobs, block_pos0=blk, want_all_scores=True)
        out, _ = L.csa_sparse_attn(q_d[:, t:t + 1].contiguous(), pool, idx, ring, None, W,
                                   dev(sink), q_pos, rope_dims=R)
        nv = O.visible_count(t, m, N_cap)
        keys_g, pool_g, ring_g = host(kidx), host(pool), host(ring)
        if (t + 1) % m == 0:   # this step closed block nv - 1: its entries first
            e = nv - 1
            assert rowwise_rel_err(keys_g[:, e], keys_ref[:, e]) <= TOL_BF16, t
            assert rowwise_rel_err(pool_g[:, e], pool_ref[:, e]) <= TOL_BF16, t
        assert rowwise_rel_err(ring_g[:, t % L_win], win_ref[:, t]) <= TOL_BF16, t
        # the oracle's selection at t on the keys as stored (stage isolation)
        ridx = np.full((B, 1, K), -1, np.int64)
        for b in range(B):
            sc = O.index_scores(q_idx.f32[b, t], w_idx[b, t], keys_g[b, :nv]).astype(np.float32)
            ridx[b, 0] = O.select_topk(sc, nv, K)
            g = host(idx)[b, 0].astype(np.int64)
            excused += check_band(g, ridx[b, 0], sc, nv, K)
            assert np.array_equal(g, O.select_topk(host(alls)[b, 0, :nv], nv, K)), (t, b)
        # the attention on the oracle's index sets and the oracle's own
        # entries, and the step's output on the GPU's selection and rows
        iso, _ = L.csa_sparse_attn(q_d[:, t:t + 1].contiguous(), pool, i32(ridx), ring, None, W,
                                   dev(sink), q_pos, rope_dims=R)
        lo = max(0, t - W + 1)
        win_slots = [p % L_win for p in range(lo, t + 1)]
        for b in range(B):
            rows = np.concatenate([pool_r[b, [v for v in ridx[b, 0] if v >= 0]],
                                   win_r[b, lo:t + 1]]).reshape(-1, D)
            ro, _ = O.attend(q.f32[b, t], t, rows, sink, scale, R)
            assert rowwise_rel_err(host(iso)[b, 0], ro) <= TOL_BF16, (t, b)
            gsel = [v for v in host(idx)[b, 0] if v >= 0]
            rows_g = np.concatenate([pool_g[b, gsel], ring_g[b, win_slots]]).reshape(-1, D)
            rg, _ = O.attend(q.f32[b, t], t, rows_g, sink, scale, R)
            assert rowwise_rel_err(host(out)[b, 0], rg) <= TOL_BF16, (t, b)
        if (t + 1) % m == 0:   # the closed block's stream b becomes the overlap state
            for n in ("c_b", "z_b"):
                prev[n].copy_(cur[n])
                kprev[n].copy_(kcur[n])
    torch.cuda.synchronize()
    n = T // m
    assert rowwise_rel_err(host(pool)[:, :n], pool_ref[:, :n]) <= TOL_BF16
    assert rowwise_rel_err(host(kidx)[:, :n], keys_ref[:, :n]) <= TOL_BF16
    for p in range(T - L_win, T):
        assert rowwise_rel_err(host(ring)[:, p % L_win], win_ref[:, p]) <= TOL_BF16
    assert np.array_equal(host(q_pos), [T - 1, T - 1])
    assert np.array_equal(host(n_ent), [n, n])


def test_graph_captured_streaming_step_matches_eager():
    """One streaming step (advance, decode call with the window row as its
    third job, attention over the ring) captured in a HIP graph and replayed
    12 times, with eager work and synchronisation between the replays: every
    replay equals an eager run of the same step on an identical state,
    bitwise (positions, counts, caches, selection, output)."""
    rng = np.random.default_rng(71)
    B, m, K, W, H, D, R, Hi, Di, N_cap = 2, 4, 4, 16, 64, 512, 64, 64, 128, 16
    f = lambda *s, sc=1.0: (rng.standard_normal(s) * sc).astype(np.float32)
    bfd = lambda x: dev(synth.Tensor(x, "bf16"))

    def state():
        st = dict(q_pos=torch.full((B,), 9, dtype=torch.int64, device="cuda"),
                  n_ent=torch.zeros(B, dtype=torch.int32, device="cuda"),
                  blk=torch.zeros(B, dtype=torch.int64, device="cuda"),
                  pool=torch.zeros((B, N_cap, D), dtype=torch.bfloat16, device="cuda"),
                  kidx=torch.zeros((B, N_cap, Di), dtype=torch.bfloat16, device="cuda"),
                  ring=torch.zeros((B, W, D), dtype=torch.bfloat16, device="cuda"),
                  idx=torch.empty((B, 1, K), dtype=torch.int32, device="cuda"),
                  out=torch.empty((B, 1, H, D), dtype=torch.bfloat16, device="cuda"))
        st["ws_i"] = torch.empty(L.csa_index_topk_ws_bytes(B, 1, Hi, N_cap, K), dtype=torch.uint8,
                                 device="cuda")
        st["ws_a"] = torch.empty(max(L.csa_attn_ws_bytes(B, 1, H, D, K + W), 1),
                                 dtype=torch.uint8, device="cuda")
        return st

    s_kv = {n: bfd(f(B, m, D)) for n in ("c_a", "z_a", "c_b", "z_b", "prev_c_b", "prev_z_b")}
    s_k = {n: bfd(f(B, m, Di)) for n in ("c_a", "z_a", "c_b", "z_b", "prev_c_b", "prev_z_b")}
    kv_row, q, qi = bfd(f(B, 1, D)), bfd(f(B, 1, H, D)), bfd(f(B, 1, Hi, Di))
    wi, sink = dev(f(B, 1, Hi, sc=0.02)), dev(f(H, sc=0.02))
    gain, wgain = dev(1 + f(D, sc=0.02)), dev(1 + f(D, sc=0.02))
    bk = {n: dev(f(m, Di, sc=0.02)) for n in ("a", "b")}
    bv = {n: dev(f(m, D, sc=0.02)) for n in ("a", "b")}

    def step(st):
        L.csa_decode_advance(st["q_pos"], st["n_ent"], st["blk"], m, N_cap)
        jobs = [dict(**s_k, bias_a=bk["a"], bias_b=bk["b"], out=st["kidx"]),
                dict(**s_kv, bias_a=bv["a"], bias_b=bv["b"], gain=gain, rope_dims=R,
                     out=st["pool"]),
                dict(c_a=kv_row, gain=wgain, rope_dims=R, out=st["ring"])]
        L.csa_decode_index_topk(qi, wi, st["n_ent"], st["q_pos"], K, m, jobs,
                                block_pos0=st["blk"], ws=st["ws_i"], idx_out=st["idx"])
        L.csa_sparse_attn(q, st["pool"], st["idx"], st["ring"], None, W, sink, st["q_pos"],
                          rope_dims=R, out=st["out"], ws=st["ws_a"])

    eager, graphed = state(), state()
    step(graphed)                     # warm-up outside the capture, mirrored eagerly
    step(eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(graphed)
    keys = ("q_pos", "n_ent", "blk", "pool", "kidx", "ring", "idx", "out")
    for r in range(12):
        g.replay()
        step(eager)
        torch.cuda.synchronize()
        junk = torch.randn(1 << 16, device="cuda").sum()   # eager work between replays
        for k in keys:
            assert torch.equal(graphed[k], eager[k]), (r, k)
    assert int(host(eager["n_ent"])[0]) >= 5 and junk is not None
