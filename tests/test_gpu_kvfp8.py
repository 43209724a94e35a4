"""GPU parity of the mixed BF16 / FP8 KV storage against the CPU oracle.

The quantizer's packed rows must equal the oracle's bit for bit on identical
float inputs (f32 and bf16); the dequantizer (the hardware conversion the
attention uses) must reproduce the oracle's exact values for every code.
The compressor's FP8 output is pinned two ways: with float32 streams the
rows equal the oracle's quantization of the float32 entries the same call
writes unquantized (bit-exact); with bf16 streams each code equals the
oracle's quantization of its own float64 entry, or, next to a rounding
boundary, is within one step of it.  The attention over packed rows equals
the bf16 attention over the dequantized pool bitwise (the rows reach the
tile as the same bf16 values), and matches the oracle's attention on the
dequantized rows within the bf16 bar.
"""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_11_amd as L
from long_context_sparse_11_amd import synth
from oracle import csa_oracle as O
from tests.helpers import TOL_BF16, dev, host, rowwise_rel_err
from tests.test_gpu_parity import (ALL_KINDS, _fresh_case, _fresh_jobs_and_refs, _hca_step_case,
                                   _rand_sel, i32, i64)

pytestmark = pytest.mark.gpu

D, R = 512, 64
RB = 592


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    L.lib()


def _edge_rows(rng):
    """Rows hitting every rule: grid points and midpoints at several scales
    (block maximum 448 * 2^k fixes the scale), points next to midpoints,
    the subnormal range, saturation [448, 512), zero blocks, wide ranges."""
    grid = np.array(O.E4M3_GRID)
    mids = (grid[1:] + grid[:-1]) / 2
    rows = []
    for k in (-100, -20, -3, 0, 1, 7, 60, 100):
        pts = np.concatenate([[448.0], grid[1:], mids, mids * (1 + 2.0 ** -18),
                              mids * (1 - 2.0 ** -18), [500.0, 511.0, 449.0]])
        pts = pts * np.where(np.arange(len(pts)) % 3 == 1, -1, 1)
        body = np.resize(pts, 448)
        body[::32] = 448.0
        rows.append(np.concatenate([body * 2.0 ** k, rng.standard_normal(64) * 2.0 ** (k / 4)]))
    rows.append(np.zeros(512))
    one = np.zeros(512)
    one[37], one[300] = -3.0, 1e-3
    rows.append(one)
    for k in range(-30, 31, 6):
        rows.append(rng.standard_normal(512) * 2.0 ** k)
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_quantize_kv_fp8_bit_exact(dt):
    rng = np.random.default_rng(61)
    x = synth.Tensor(np.concatenate([_edge_rows(rng), rng.standard_normal((300, 512))
                                     .astype(np.float32)]), dt)
    got = host(L.csa_quantize_kv_fp8(dev(x), R))
    want = O.kv_fp8_quantize(x.f32.astype(np.float64), R)
    assert got.shape == want.shape == (x.shape[0], RB)
    assert np.array_equal(got, want)


def test_dequantize_kv_fp8_every_code():
    """Every code byte (but NaN) under several scale bytes: the hardware
    conversion gives the oracle's exact values."""
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    rows = np.zeros((8, RB), np.uint8)
    rng = np.random.default_rng(62)
    for r in range(8):
        rows[r, :448] = np.resize(np.roll(codes, 37 * r), 448)
        rows[r, 576:590] = [(100 + 5 * r + b) % 140 + 60 for b in range(14)]
        rows[r, 448:576] = rng.integers(0, 256, 128, dtype=np.uint8)
        rows[r, 448:576].view(np.uint16)[:] &= 0x7F7F   # finite bf16 RoPE channels
    got = host(L.csa_dequantize_kv_fp8(dev(rows), D, R))
    want = O.kv_fp8_dequantize(rows, D, R)
    assert np.array_equal(got, want)


def test_compress_kvfp8_f32_matches_quantized_f32_entries():
    """float32 streams: the packed rows equal the oracle's quantization of the
    float32 entries csa_compress writes for the same call (both the single
    workgroup path and the channel-split path with its finisher)."""
    rng = np.random.default_rng(63)
    for B, T, m, overlap in ((2, 64, 4, True), (16, 128, 128, False), (2, 2052, 4, True)):
        f = lambda *s: rng.standard_normal(s).astype(np.float32)
        kw = dict(z_a=dev(f(B, T, D)), bias_a=dev(0.02 * f(m, D)), gain=dev(1 + 0.02 * f(D)),
                  rope_dims=R, pos0=i64([4096] * B))
        if overlap:
            kw.update(c_b=dev(f(B, T, D)), z_b=dev(f(B, T, D)), bias_b=dev(0.02 * f(m, D)))
        c_a = dev(f(B, T, D))
        ref = host(L.csa_compress(c_a, m, **kw))
        got = host(L.csa_compress_kvfp8(c_a, m, **kw))
        assert np.array_equal(got, O.kv_fp8_quantize(ref.astype(np.float64), R)), (B, T, m)


def _near(x, rows):
    """Elements whose exact value sits next to a rounding boundary under the
    stored scale (a grid midpoint), or whose block maximum is next to a power
    of two (the scale choice): float32 pooling may fall on the other side."""
    grid = np.array(O.E4M3_GRID)
    mids = (grid[1:] + grid[:-1]) / 2
    X = np.repeat(np.exp2(rows[..., 576:590].astype(np.float64) - 127), 32, axis=-1)
    a = np.abs(x[..., :448]) / X
    near = np.min(np.abs(a[..., None] - mids), axis=-1) <= 1e-4 * np.maximum(a, 2.0 ** -6)
    amax = np.abs(x[..., :448]).reshape(x.shape[:-1] + (14, 32)).max(-1)
    f = amax / np.exp2(np.floor(np.log2(np.maximum(amax, 1e-300))))
    blk = np.minimum(np.abs(f - 1), np.abs(f - 2)) <= 1e-4
    return near | np.repeat(blk, 32, axis=-1)


def _check_fp8_entries(rows_gpu, exact):
    """Stored rows against the oracle's exact (float64) entries: the codes are
    the oracle's quantization, but next to a boundary the neighbouring code;
    the RoPE channels within the bf16 bar."""
    want = O.kv_fp8_quantize(exact, R)
    gd = O.kv_fp8_dequantize(rows_gpu, D, R)
    wd = O.kv_fp8_dequantize(want, D, R)
    near = _near(exact, want)
    assert np.array_equal(gd[..., :448][~near], wd[..., :448][~near])
    X = np.repeat(np.exp2(np.maximum(rows_gpu[..., 576:590], want[..., 576:590])
                          .astype(np.float64) - 127), 32, axis=-1)
    step = 32 * X   # a step of the largest binade: 2^(8-3) at the block's scale
    assert np.all(np.abs(gd[..., :448] - exact[..., :448])[near] <= step[near])
    assert rowwise_rel_err(gd[..., 448:], exact[..., 448:]) <= TOL_BF16


def test_compress_kvfp8_bf16_streams_against_oracle():
    """bf16 streams of the HCA closing block (16 x 128 rows, channel split)
    and a CSA chunk: rows against the oracle's entries."""
    rng = np.random.default_rng(64)
    for B, T, m, overlap in ((16, 128, 128, False), (2, 400, 4, True)):
        f = lambda *s: rng.standard_normal(s).astype(np.float32)
        bf = lambda *s: synth.Tensor(f(*s), "bf16")
        c_a, z_a = bf(B, T, D), bf(B, T, D)
        bias_a, gain = 0.02 * f(m, D), 1 + 0.02 * f(D)
        pos0 = np.array([1048576 - T] * B)
        kw = dict(z_a=dev(z_a), bias_a=dev(bias_a), gain=dev(gain), rope_dims=R, pos0=i64(pos0))
        okw = dict(gain=gain, rope_dims=R, pos0=pos0)
        if overlap:
            c_b, z_b, bias_b = bf(B, T, D), bf(B, T, D), 0.02 * f(m, D)
            kw.update(c_b=dev(c_b), z_b=dev(z_b), bias_b=dev(bias_b))
            okw.update(c_b=c_b.f32, z_b=z_b.f32, bias_b=bias_b)
        got = host(L.csa_compress_kvfp8(dev(c_a), m, **kw))
        ref = O.csa_compress(c_a.f32, z_a.f32, bias_a, m, **okw)
        _check_fp8_entries(got, ref)


@pytest.mark.parametrize("N,Tq,n_ent", [(3000, 1, [3000, 2999]), (20000, 3, [20000, 7001])])
def test_decode_with_fp8_kv_entry(N, Tq, n_ent):
    """The decode call with the KV job writing a packed row: the fresh row
    (row n_entries - 1) against the oracle's entry, every other row untouched;
    the key cache and the selection equal those of the bf16-KV call."""
    d = _fresh_case("bf16", N, Tq, n_ent, False, seed=N + Tq)
    B, m, K = d["B"], d["m"], 512
    rng = np.random.default_rng(65)
    pool8 = dev(O.kv_fp8_quantize(rng.standard_normal((B, N, D)).astype(np.float32)
                                  .astype(np.float64), R))
    before = pool8.clone()
    res = []
    for fp8 in (False, True):
        kidx, pool = dev(d["k_idx"]), dev(d["pool"])
        jobs, (kref, vref) = _fresh_jobs_and_refs(d, kidx, pool)
        if fp8:
            jobs[1]["out"], jobs[1]["out_kv_fp8"] = pool8, True
        idx, _, alls = L.csa_decode_index_topk(dev(d["q"]), dev(d["w"]), i32(d["n_ent"]),
                                               i64(d["q_pos0"]), K, m, jobs,
                                               block_pos0=i64(d["block_pos0"]),
                                               want_all_scores=True)
        res.append((idx, kidx))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    got = host(pool8)
    for b in range(B):
        r = int(d["n_ent"][b]) - 1
        keep = [i for i in range(N) if i != r]
        assert np.array_equal(got[b, keep], host(before)[b, keep])
        _check_fp8_entries(got[b, r][None], vref[b][None])


def _attn_case(rng, kind, N, K, W, Tq, H=64):
    B, m = 2, 4 if kind == "csa" else 128
    ctx = N * m
    q_pos0 = np.array([ctx - Tq, ctx - Tq - 3 * m])
    L_win = Tq + W - 1 + 3 * m
    win_pos0 = q_pos0 - W + 1 - 3 * m
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    q, win = synth.Tensor(f(B, Tq, H, D), "bf16"), synth.Tensor(f(B, L_win, D), "bf16")
    pool8 = O.kv_fp8_quantize(f(B, N, D).astype(np.float64), R)
    sink = 0.5 * f(H)
    return B, m, q, win, pool8, sink, q_pos0, win_pos0


@pytest.mark.parametrize("kind,N,K,W,Tq,H", [
    ("csa", 2000, 512, 128, 1, 64),      # decode: single-tile splits in head groups
    ("csa", 5000, 512, 128, 3, 64),      # few queries
    ("csa", 300, 64, 16, 24, 64),        # many queries, ragged
    ("csa", 9000, 2048, 128, 8, 64),     # multi-tile splits (selected indices staged)
    ("csa", 3000, 1024, 128, 1, 128),    # V4-Pro heads
    ("hca", 8192, 0, 128, 1, 64),        # HCA: multi-tile splits, a mixed FP8 / window tile
    ("hca", 300, 0, 16, 2, 64)])
def test_attn_kvfp8_equals_bf16_on_dequantized_pool_and_oracle(kind, N, K, W, Tq, H):
    rng = np.random.default_rng(N + K + Tq + H)
    B, m, q, win, pool8, sink, q_pos0, win_pos0 = _attn_case(rng, kind, N, K, W, Tq, H)
    deq = O.kv_fp8_dequantize(pool8, D, R)
    p8 = dev(pool8)
    pbf = L.csa_dequantize_kv_fp8(p8, D, R)
    assert np.array_equal(host(pbf), deq)
    scale = 1.0 / math.sqrt(D)
    if kind == "csa":
        nv = [[O.visible_count(q_pos0[b] + t, m, N) for t in range(Tq)] for b in range(B)]
        sel = _rand_sel(rng, B, Tq, K, nv, 3)
        o8, l8 = L.csa_sparse_attn_kvfp8(dev(q), p8, dev(sel), dev(win), i64(win_pos0), W,
                                         dev(sink), i64(q_pos0), rope_dims=R, want_lse=True)
        ob, lb = L.csa_sparse_attn(dev(q), pbf, dev(sel), dev(win), i64(win_pos0), W, dev(sink),
                                   i64(q_pos0), rope_dims=R, want_lse=True)
        ro, rl = O.csa_sparse_attn(q.f32, deq, sel, win.f32, win_pos0, W, sink, q_pos0, scale, R)
    else:
        n_ent = np.array([N, N - 7], np.int32)
        o8, l8 = L.hca_attn_kvfp8(dev(q), p8, i32(n_ent), m, dev(win), i64(win_pos0), W,
                                  dev(sink), i64(q_pos0), rope_dims=R, want_lse=True)
        ob, lb = L.hca_attn(dev(q), pbf, i32(n_ent), m, dev(win), i64(win_pos0), W, dev(sink),
                            i64(q_pos0), rope_dims=R, want_lse=True)
        ro, rl = O.hca_attn(q.f32, deq, n_ent, m, win.f32, win_pos0, W, sink, q_pos0, scale, R)
    assert torch.equal(o8, ob) and torch.equal(l8, lb)
    assert rowwise_rel_err(host(o8), ro) <= TOL_BF16
    assert np.abs(host(l8) - rl).max() <= 2e-2


def _run_hca_step_fp8(d, p8):
    return L.hca_decode_attn_kvfp8(dev(d["q"]), p8, i32(d["n_ent"]), d["m"], dev(d["c"]),
                                   dev(d["z"]), dev(d["bias"]), dev(d["gain"]),
                                   i64(d["block_pos0"]), dev(d["win"]), i64(d["win_pos0"]),
                                   d["W"], dev(d["sink"]), i64(d["q_pos0"]), rope_dims=R,
                                   want_lse=True)


@pytest.mark.parametrize("H,N,W,m,kinds", [
    (64, 300, 128, 128, ALL_KINDS),
    (64, 3000, 128, 128, ["close", "clamp", "open", "close"]),
    (128, 500, 128, 128, ["close", "open"]),
    (64, 12, 16, 16, ["close", "first", "empty", "open"]),   # one single-tile key split
])
def test_hca_decode_step_fused_fp8(H, N, W, m, kinds):
    """hca_decode_attn_kvfp8: the closing block's entry stored as a packed row
    (codes against the oracle's quantization of its exact entry) and the
    attention over the dequantized pool with it, against the oracle; and the
    same output as hca_attn_kvfp8 over the pool the call wrote."""
    d = _hca_step_case(kinds, H, N, W, m, seed=N + H + m + 1)
    pool8 = O.kv_fp8_quantize(d["pool"].f32.astype(np.float64), R)
    p8 = dev(pool8)
    out, lse = _run_hca_step_fp8(d, p8)
    got = host(p8)
    ref_pool = O.kv_fp8_dequantize(pool8, D, R)
    for b in range(d["B"]):
        if b in d["rows"]:
            row, ent = d["rows"][b]
            _check_fp8_entries(got[b, row][None], ent[None])
            keep = np.ones(N, bool)
            keep[row] = False
            assert np.array_equal(got[b, keep], pool8[b, keep])
            ref_pool[b, row] = O.kv_fp8_dequantize(O.kv_fp8_quantize(ent[None], R), D, R)[0]
        else:
            assert np.array_equal(got[b], pool8[b])
    ro, rl = O.hca_attn(d["q"].f32, ref_pool, d["n_ent"], m, d["win"].f32, d["win_pos0"], W,
                        d["sink"], d["q_pos0"], 1 / math.sqrt(D), R)
    assert rowwise_rel_err(host(out), ro) <= TOL_BF16
    assert np.abs(host(lse) - rl).max() <= 2e-2
    o2, l2 = L.hca_attn_kvfp8(dev(d["q"]), p8, i32(d["n_ent"]), m, dev(d["win"]),
                              i64(d["win_pos0"]), W, dev(d["sink"]), i64(d["q_pos0"]),
                              rope_dims=R, want_lse=True)
    assert rowwise_rel_err(host(out), host(o2).astype(np.float64)) <= 1e-2
    assert np.abs(host(lse) - host(l2)).max() <= 1e-2


def test_kvfp8_rejects_uncovered_shapes():
    q = torch.zeros((1, 1, 4, 64), dtype=torch.float32, device="cuda")
    pool = torch.zeros((1, 8, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        L.csa_sparse_attn_kvfp8(q, pool, torch.zeros((1, 1, 4), dtype=torch.int32, device="cuda"),
                                None, None, 0, torch.zeros(4, device="cuda"),
                                torch.zeros(1, dtype=torch.int64, device="cuda"), rope_dims=16)
    assert L.csa_kv_fp8_row_bytes(256, 64) == 0 and L.csa_kv_fp8_row_bytes(512, 48) == 0
    assert L.csa_kv_fp8_row_bytes(512, 64) == RB
