"""GPU parity of the MX FP4 indexer-key calls against the CPU oracle.

The oracle quantizes (float64, the nearest E2M1 value with ties to the even
code) and dequantizes exactly; the quantizer's codes and scale bytes must
match it bit for bit on identical inputs.  Index scores are compared with a
float32 accumulation bound computed per (query, key) from the oracle's own
values: a bf16 query value times an FP4 key value is exact in float32, so
only the Di-term dot and the Hi-term weighted sum round, each term by at most
one unit of 2^-24 relative per addition.  Selections follow the band rule and
must equal the oracle's select applied to the GPU's own float32 scores.
"""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_11_amd as L
from long_context_sparse_11_amd import synth
from oracle import csa_oracle as O
from tests.helpers import TOL_BF16, check_band, dev, host, rowwise_rel_err
from tests.test_gpu_parity import _fresh_case, _fresh_jobs_and_refs, i32, i64

pytestmark = pytest.mark.gpu

MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    L.lib()


def _edge_rows(rng, D=128):
    """Rows that hit every rule: exact grid points and midpoints at several
    scales (the block maximum 6 * 2^k fixes the scale), points next to
    midpoints, saturation, all-zero and single-value blocks, block maxima at
    and just below a power of two, and normal draws over a wide range."""
    rows = []
    grid = np.array(O.E2M1_GRID)
    for k in (-90, -20, -3, 0, 1, 7, 60, 100):
        blk = np.concatenate([[6.0], MIDS, -MIDS, grid[1:], -grid[1:], [0.0, -0.0, 7.99, -5.0]])
        blk = np.resize(blk, 32)
        near = np.concatenate([[6.0], MIDS * (1 + 2.0 ** -20), MIDS * (1 - 2.0 ** -20),
                               -MIDS * (1 + 2.0 ** -20)])
        near = np.resize(near, 32)
        row = np.concatenate([blk, near, blk[::-1], rng.standard_normal(32)]) * 2.0 ** k
        rows.append(row[:D])
    rows.append(np.zeros(D))
    one = np.zeros(D)
    one[37] = -3.0
    rows.append(one)
    for k in (-5, 0, 9):
        r = rng.standard_normal(D) * 0.1
        r[3], r[40], r[70], r[100] = 2.0 ** k, -(2.0 ** k) * (1 - 2.0 ** -23), 2.0 ** k * 1.5, 4.0
        rows.append(r)
    for k in range(-30, 31, 6):
        rows.append(rng.standard_normal(D) * 2.0 ** k)
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_quantize_mxfp4_bit_exact(dt):
    rng = np.random.default_rng(21)
    x = synth.Tensor(np.concatenate([_edge_rows(rng), rng.standard_normal((200, 128))
                                     .astype(np.float32)]), dt)
    codes, scales = L.csa_quantize_mxfp4(dev(x))
    rc, rs = O.mxfp4_quantize(x.f32)
    assert np.array_equal(host(scales), rs)
    assert np.array_equal(host(codes), rc)


def test_quantize_mxfp4_ragged_rows_and_widths():
    """Row counts and widths whose pair count is not a multiple of the
    workgroup: the tail stays inside the buffers and matches."""
    rng = np.random.default_rng(22)
    for rows, D in ((1, 32), (37, 96), (5, 224), (0, 64)):
        x = (rng.standard_normal((rows, D)) * 3).astype(np.float32)
        codes, scales = L.csa_quantize_mxfp4(dev(x))
        rc, rs = O.mxfp4_quantize(x) if rows else (np.zeros((0, D // 2)), np.zeros((0, D // 32)))
        assert np.array_equal(host(codes), rc) and np.array_equal(host(scales), rs)


def _score_bound(q, w, k):
    """First-order float32 accumulation bound of each score, from the oracle's
    values: (Di + Hi + 2) * 2^-24 * sum_h |w_h| sum_c |q_hc| |k_sc|."""
    Hi, Di = q.shape
    mag = (np.abs(w)[:, None] * (np.abs(q) @ np.abs(k).T)).sum(0)
    return mag * (Di + Hi + 2) * 2.0 ** -24 + 1e-30


def _check_fp4_index(q, w, codes, scales, n_ent, q_pos0, K, m):
    """csa_index_topk_mxfp4 and csa_index_scores_mxfp4 against the oracle on
    the dequantized keys."""
    qf = q.f32
    B, Tq, Hi, Di = qf.shape
    kf = O.mxfp4_dequantize(codes, scales)
    gidx, gsc, gall = L.csa_index_topk_mxfp4(dev(q), dev(w), dev(codes), dev(scales), i32(n_ent),
                                             i64(q_pos0), K, m, want_scores=True,
                                             want_all_scores=True)
    gidx, gsc, gall = host(gidx).astype(np.int64), host(gsc), host(gall)
    alone = host(L.csa_index_scores_mxfp4(dev(q), dev(w), dev(codes), dev(scales), i32(n_ent),
                                          i64(q_pos0), m))
    ridx, rsc = O.csa_index_topk(qf, w, kf, n_ent, q_pos0, K, m)
    for b in range(B):
        for t in range(Tq):
            nv = O.visible_count(q_pos0[b] + t, m, n_ent[b])
            if nv:
                ref = O.index_scores(qf[b, t], w[b, t], kf[b, :nv])
                bound = _score_bound(qf[b, t], w[b, t], kf[b, :nv])
                err = np.abs(gall[b, t, :nv].astype(np.float64) - ref)
                assert np.all(err <= bound), (b, t, float((err / bound).max()))
                assert np.array_equal(alone[b, t, :nv], gall[b, t, :nv])
            check_band(gidx[b, t], ridx[b, t], rsc[b, t], nv, K)
            assert np.array_equal(gidx[b, t], O.select_topk(gall[b, t, :nv], nv, K)), (b, t)
            sel = gidx[b, t]
            assert np.array_equal(gsc[b, t][sel >= 0], gall[b, t][sel[sel >= 0]])


@pytest.mark.parametrize("kind,B,N,n_ent", [("csa64k_fp4", 2, 5000, [5000, 3001]),
                                            ("csa64k_fp4", 3, 700, [700, 513, 0]),
                                            ("csa1m_fp4", 2, 40000, [40000, 39999]),
                                            ("csa1m_fp4", 2, 262144, [262144, 200001])])
def test_index_mxfp4_decode(kind, B, N, n_ent):
    """Decode shapes (the streaming MFMA kernel; 40,000 entries take the
    two-level select; 2 x 262,144 entries give each wave several tiles, the
    ring of tiles in flight), heavy-tailed scales in csa1m_fp4."""
    d = synth.decode(kind, 3, B=B, N=N, skip=("pool", "q", "win"))
    n_ent = np.array(n_ent, np.int32)
    q_pos0 = 4 * n_ent.astype(np.int64) - 1
    _check_fp4_index(d["q_idx"], d["w_idx"], d["k_codes"], d["k_scales"], n_ent, q_pos0, d["K"],
                     d["m"])


def _rand_fp4(rng, B, N, Di):
    return (rng.integers(0, 256, size=(B, N, Di // 2), dtype=np.uint8),
            rng.integers(120, 131, size=(B, N, Di // 32), dtype=np.uint8))


@pytest.mark.parametrize("Tq,pos0,N", [(3, 2799, 700), (40, 2040, 700), (16, 100000, 1100)])
def test_index_mxfp4_few_and_many_queries(Tq, pos0, N):
    """Tq < 8 (decode kernel, several queries) and Tq >= 8 (the prefill
    kernel, FP4 tiles converted on their way into LDS), ragged tails."""
    rng = np.random.default_rng(Tq + N)
    q = synth.Tensor(rng.standard_normal((1, Tq, 64, 128)).astype(np.float32), "bf16")
    w = (0.02 * rng.standard_normal((1, Tq, 64))).astype(np.float32)
    codes, scales = _rand_fp4(rng, 1, N, 128)
    _check_fp4_index(q, w, codes, scales, np.array([N - 3], np.int32), np.array([pos0]), 512, 4)


def test_index_mxfp4_generic_shape():
    """A shape outside the MFMA kernels (4 heads x 32) takes the VALU path."""
    rng = np.random.default_rng(5)
    q = synth.Tensor(rng.standard_normal((2, 5, 4, 32)).astype(np.float32), "bf16")
    w = np.abs(rng.standard_normal((2, 5, 4))).astype(np.float32)
    codes, scales = _rand_fp4(rng, 2, 60, 32)
    _check_fp4_index(q, w, codes, scales, np.array([60, 41], np.int32), np.array([200, 150]),
                     16, 4)


def _near_rule(x, s):
    """Elements whose exact value sits so close to a rounding boundary (a
    midpoint of the grid, or for the block maximum a power of two) that float32
    pooling may fall on the other side: those may differ by one code."""
    Xs = np.repeat(np.exp2(s.astype(np.float64) - 127), 32)
    a = np.abs(x) / Xs
    near = np.min(np.abs(a[:, None] - MIDS[None]), axis=1) <= 1e-4 * np.maximum(a, 1)
    for blk in range(len(s)):
        amax = np.abs(x[32 * blk: 32 * blk + 32]).max()
        if amax > 0:
            f = amax / 2.0 ** math.floor(math.log2(amax))
            if min(abs(f - 1), abs(f - 2)) <= 1e-4:
                near[32 * blk: 32 * blk + 32] = True
    return near


def _gpu_fresh_key(kref, gc, gs):
    """The GPU's fresh FP4 key (codes gc, scale bytes gs) against the oracle's
    quantization of the pooled float value kref.  Where the value is clear of
    every rounding boundary the codes must agree exactly; next to a boundary
    float32 pooling may land on the other side, so the GPU's value must be a
    neighbouring grid point: within one grid step (at most twice the block
    scale) of the exact value.  Returns the dequantized GPU key, the input on
    which the later stages are checked (stage isolation: the selection is then
    held at the 1e-4 band)."""
    oc, os_ = O.mxfp4_quantize(kref)
    near = _near_rule(kref, os_)
    gq = O.mxfp4_dequantize(gc, gs)
    rq = O.mxfp4_dequantize(oc, os_)
    assert np.array_equal(gq[~near], rq[~near])
    step = 2 * np.repeat(np.exp2(np.maximum(gs, os_).astype(np.float64) - 127), 32)
    assert np.all(np.abs(gq - kref)[near] <= step[near])
    return gq


@pytest.mark.parametrize("N,Tq,n_ent,key_norm_rope", [
    (2000, 1, [2000, 1995], False), (20000, 3, [20000, 20000, 7000], True),
    (700, 1, [700, 0], False), (262144, 1, [262144, 131071], False)])
def test_decode_index_topk_mxfp4_fused(N, Tq, n_ent, key_norm_rope):
    """The decode step with FP4 indexer keys: the closing block's key is
    pooled, quantized and written to row n_entries-1 of the codes and scales
    (rest untouched); the KV entry goes to the bf16 pool as before; the
    selection ranks the FP4 keys with the fresh one."""
    d = _fresh_case("bf16", N, Tq, n_ent, key_norm_rope, seed=N + 7 * Tq)
    B, m, K, Di = d["B"], d["m"], 512, d["Di"]
    rng = np.random.default_rng(N)
    codes, scales = _rand_fp4(rng, B, N, Di)
    kc, ks, pool = dev(codes), dev(scales), dev(d["pool"])
    kc0, ks0, p0 = kc.clone(), ks.clone(), pool.clone()
    jobs, (kref, vref) = _fresh_jobs_and_refs(d, None, pool)
    gidx, gsc, gall = L.csa_decode_index_topk_mxfp4(
        dev(d["q"]), dev(d["w"]), kc, ks, i32(d["n_ent"]), i64(d["q_pos0"]), K, m, jobs,
        block_pos0=i64(d["block_pos0"]), want_scores=True, want_all_scores=True)
    gidx, gsc, gall = host(gidx).astype(np.int64), host(gsc), host(gall)
    kin_c, kin_s = codes.copy(), scales.copy()
    for b in range(B):
        r = int(d["n_ent"][b]) - 1
        keep = [i for i in range(N) if i != r]
        for got, before in ((kc, kc0), (ks, ks0), (pool, p0)):
            assert torch.equal(got[b, keep], before[b, keep]), b
        if r < 0:
            continue
        assert rowwise_rel_err(host(pool[b, r])[None], vref[b][None]) <= TOL_BF16, b
        # the GPU's stored code (checked against the oracle's quantization)
        # is the key the oracle ranks: stage isolation
        _gpu_fresh_key(kref[b], host(kc[b, r]), host(ks[b, r]))
        kin_c[b, r], kin_s[b, r] = host(kc[b, r]), host(ks[b, r])
    kf = O.mxfp4_dequantize(kin_c, kin_s)
    qf = d["q"].f32
    _, rsc = O.csa_index_topk(qf, d["w"], kf, d["n_ent"], d["q_pos0"], K, m)
    for b in range(B):
        r = int(d["n_ent"][b]) - 1
        for t in range(Tq):
            nv = O.visible_count(d["q_pos0"][b] + t, m, d["n_ent"][b])
            if nv:
                bound = _score_bound(qf[b, t], d["w"][b, t], kf[b, :nv])
                err = np.abs(gall[b, t, :nv].astype(np.float64) - rsc[b, t, :nv])
                assert np.all(err <= bound), (b, t, float((err / bound).max()))
            assert np.array_equal(gidx[b, t], O.select_topk(gall[b, t, :nv], nv, K)), (b, t)
            check_band(gidx[b, t], O.select_topk(rsc[b, t, :nv], nv, K), rsc[b, t], nv, K)
            sel = gidx[b, t]
            assert np.array_equal(gsc[b, t][sel >= 0], gall[b, t][sel[sel >= 0]])


def test_decode_mxfp4_rejects_unfused_shapes():
    """FP4 fresh keys are written only by the fused launch: a shape it does
    not cover (8 queries) is refused before anything is written."""
    d = _fresh_case("bf16", 600, 8, [600], False, seed=1)
    rng = np.random.default_rng(2)
    codes, scales = _rand_fp4(rng, 1, 600, 128)
    kc, ks, pool = dev(codes), dev(scales), dev(d["pool"])
    before = kc.clone()
    jobs, _ = _fresh_jobs_and_refs(d, None, pool)
    with pytest.raises(L.CsaError, match="UNSUPPORTED"):
        L.csa_decode_index_topk_mxfp4(dev(d["q"]), dev(d["w"]), kc, ks, i32(d["n_ent"]),
                                      i64(d["q_pos0"]), 512, 4, jobs,
                                      block_pos0=i64(d["block_pos0"]))
    torch.cuda.synchronize()
    assert torch.equal(kc, before)


def test_decode_mxfp4_with_window_row_job():
    """The FP4 decode call with the step token's window row as a third job:
    the ring row equals csa_window_row's, and the selection and FP4 caches
    equal those of the two-job call on the same inputs."""
    d = _fresh_case("bf16", 3000, 1, [3000, 2999], False, seed=23)
    B, m, K, Di, D, R = d["B"], d["m"], 512, d["Di"], d["D"], d["R"]
    rng = np.random.default_rng(24)
    codes, scales = _rand_fp4(rng, B, 3000, Di)
    kv = dev(synth.Tensor(rng.standard_normal((B, 1, D)).astype(np.float32), "bf16"))
    wgain = dev((1 + 0.02 * rng.standard_normal(D)).astype(np.float32))
    L_win = 128
    outs = []
    for third in (False, True):
        kc, ks, pool = dev(codes), dev(scales), dev(d["pool"])
        ring = torch.zeros((B, L_win, D), dtype=torch.bfloat16, device="cuda")
        jobs, _ = _fresh_jobs_and_refs(d, None, pool)
        if third:
            jobs.append(dict(c_a=kv, gain=wgain, rope_dims=R, out=ring))
        idx, _, alls = L.csa_decode_index_topk_mxfp4(
            dev(d["q"]), dev(d["w"]), kc, ks, i32(d["n_ent"]), i64(d["q_pos0"]), K, m, jobs,
            block_pos0=i64(d["block_pos0"]), want_all_scores=True)
        outs.append((idx, alls, kc, ks, pool, ring))
    for k in (0, 2, 3, 4):   # selection and caches
        assert torch.equal(outs[0][k], outs[1][k]), k
    for b in range(B):       # scores of the visible entries (later columns are unspecified)
        nv = O.visible_count(int(d["q_pos0"][b]), m, int(d["n_ent"][b]))
        assert torch.equal(outs[0][1][b, :, :nv], outs[1][1][b, :, :nv]), b
    ring_ref = torch.zeros((B, L_win, D), dtype=torch.bfloat16, device="cuda")
    L.csa_window_row(kv, i64(d["q_pos0"]), ring_ref, gain=wgain, rope_dims=R)
    assert torch.equal(outs[1][5], ring_ref)
