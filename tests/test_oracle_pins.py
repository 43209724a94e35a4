"""Pins for the CPU oracle: printed values from the pages, closed forms,
invariants, library special cases and brute force on tiny inputs.

Each test is chosen so that a plausible slip in the oracle (a flipped sign, a
wrong pair index, a dropped term, a transposed operand, the wrong overlap
direction, masking after instead of before top-k) fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import csa_oracle as O


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def test_rope_printed_pair(golden):
    g = golden("p1_rope_pair.txt")
    x = np.array(g["pair_in"])
    y = O.rope(x, g["position"], rope_dims=2)
    assert np.allclose(y, g["pair_out"], atol=1.5e-4)
    # the printed cos/sin are those of the frequency-1 pair
    assert np.allclose([math.cos(3), math.sin(3)], g["cos_sin"], atol=1e-4)


def test_rope_self_score_printed(golden):
    g = golden("p1_self_score.txt")
    q = np.array(g["q"]); k = np.array(g["k"])
    qr = O.rope(q, g["position"], int(g["rope_dims"]))
    kr = O.rope(k, g["position"], int(g["rope_dims"]))
    assert abs(qr @ kr - g["dot"]) < 1e-4
    # through the attention path: one key row (already rotated, as pool and
    # window rows are), sink far below -> lse equals the scaled logit
    _, lse = O.attend(q[None], int(g["position"]), kr[None], np.array([-1e300]),
                      g["scale"], int(g["rope_dims"]))
    assert abs(lse[0] - g["score"]) < 1e-4


def test_rope_matches_complex_rotation():
    """Interleaved pair (x_u, x_v) as the complex number x_u + i x_v times
    exp(i * pos * base**(-2j/R)) (the usual rotary-embedding frequencies)."""
    rng = np.random.default_rng(0)
    D, R, base = 24, 16, 10000.0
    x = rng.standard_normal((5, D))
    pos = np.array([0, 1, 7, 1000, 1048575])
    got = O.rope(x, pos, R, base)
    want = x.copy()
    z = x[:, D - R::2] + 1j * x[:, D - R + 1::2]
    freq = base ** (-np.arange(R // 2) * 2.0 / R)
    z = z * np.exp(1j * pos[:, None] * freq[None, :])
    want[:, D - R::2] = z.real
    want[:, D - R + 1::2] = z.imag
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    # channels before the rope slice are untouched
    assert np.array_equal(got[:, : D - R], x[:, : D - R])


def test_rope_norm_inverse_and_relative():
    rng = np.random.default_rng(1)
    D, R = 64, 16
    x = rng.standard_normal(D)
    y = rng.standard_normal(D)
    for p in [0, 3, 1234, 1048575]:
        xr = O.rope(x, p, R)
        assert abs(np.linalg.norm(xr) - np.linalg.norm(x)) < 1e-12
        assert np.allclose(O.rope(xr, -p, R), x, atol=1e-12)
    # dot products depend only on the position difference
    d1 = O.rope(x, 100, R) @ O.rope(y, 37, R)
    d2 = O.rope(x, 100 + 4096, R) @ O.rope(y, 37 + 4096, R)
    assert abs(d1 - d2) < 1e-10


# ---------------------------------------------------------------------------
# Sink softmax and attention
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["p1_sink_softmax_swa.txt", "p1_sink_softmax_csa.txt"])
def test_sink_softmax_printed(golden, name):
    g = golden(name)
    w, mass = O.sink_softmax_weights(g["logits"], g["sink"])
    assert np.allclose(w, g["weights"], atol=1e-4)
    assert abs(mass - g["sink_mass"]) < 6e-4
    if "denom" in g:
        e = np.exp(np.array(g["logits"] + [g["sink"]]))
        assert np.allclose(e, g["exp"], atol=1e-4)
        assert abs(e.sum() - g["denom"]) < 1e-4


@pytest.mark.parametrize("name", ["p1_sink_softmax_swa.txt", "p1_sink_softmax_csa.txt"])
def test_attend_exposes_printed_weights(golden, name):
    """Rows built so the output reveals the key weights: row j = [z_j, e_j],
    query = e_0, scale 1, no RoPE -> logit j = z_j and out[1 + j] = weight j."""
    g = golden(name)
    z = np.array(g["logits"])
    n = len(z)
    rows = np.zeros((n, 1 + n))
    rows[:, 0] = z
    rows[np.arange(n), 1 + np.arange(n)] = 1.0
    q = np.zeros((1, 1 + n)); q[0, 0] = 1.0
    out, lse = O.attend(q, 0, rows, np.array([g["sink"]]), 1.0, 0)
    assert np.allclose(out[0, 1:], g["weights"], atol=1e-4)
    assert abs(1.0 - out[0, 1:].sum() - g["sink_mass"]) < 6e-4


def test_sink_closed_form_equal_logits():
    for n, zval, sink in [(1, 0.3, -1.0), (7, -2.0, 0.5), (640, 1.25, 8.0)]:
        w, mass = O.sink_softmax_weights(np.full(n, zval), sink)
        assert np.allclose(w, 1.0 / (n + math.exp(sink - zval)), rtol=1e-12)
        assert abs(mass - math.exp(sink - zval) / (n + math.exp(sink - zval))) < 1e-12


def test_empty_key_set_is_all_sink():
    q = np.ones((3, 8))
    out, lse = O.attend(q, 5, np.zeros((0, 8)), np.array([0.1, -2.0, 4.0]), 0.5, 4)
    assert np.array_equal(out, np.zeros((3, 8)))
    assert np.allclose(lse, [0.1, -2.0, 4.0])


def test_attend_without_sink_is_textbook_mqa():
    """Sink -> -inf reduces to ordinary softmax attention; cross-check with
    torch's scaled_dot_product_attention (CPU, float64), one K=V head
    broadcast to every query head, RoPE applied around it."""
    rng = np.random.default_rng(2)
    H, D, R, n, t = 6, 32, 8, 23, 777
    q = rng.standard_normal((H, D))
    rows = rng.standard_normal((n, D))
    scale = 1 / math.sqrt(D)
    out, _ = O.attend(q, t, rows, np.full(H, -1e300), scale, R)
    qr = torch.from_numpy(O.rope(q, t, R))[None, :, None, :]
    kv = torch.from_numpy(rows)[None, None].expand(1, H, n, D)
    ref = torch.nn.functional.scaled_dot_product_attention(qr, kv, kv, scale=scale)[0, :, 0]
    ref = O.rope(ref.numpy(), -t, R)
    assert np.allclose(out, ref, atol=1e-12)


def test_attend_sink_equals_extra_zero_row():
    """A sink logit s behaves like one more key whose logit is s and whose
    value is the zero vector (library softmax on the extended logits)."""
    rng = np.random.default_rng(3)
    H, D, n = 4, 16, 9
    q = rng.standard_normal((H, D)); rows = rng.standard_normal((n, D))
    sink = rng.standard_normal(H)
    out, lse = O.attend(q, 0, rows, sink, 0.25, 0)
    z = 0.25 * q @ rows.T
    zz = np.concatenate([z, sink[:, None]], axis=1)
    p = scipy.special.softmax(zz, axis=1)
    assert np.allclose(out, p[:, :n] @ rows, atol=1e-12)
    assert np.allclose(lse, scipy.special.logsumexp(zz, axis=1), atol=1e-12)


# ---------------------------------------------------------------------------
# Visibility, window, sizes
# ---------------------------------------------------------------------------
def test_visibility_hca_printed(golden):
    g = golden("p4_visibility.txt")
    m, T = int(g["hca_m"]), int(g["hca_tokens"])
    first = [min(t for t in range(T) if O.visible_count(t, m, T // m) > w) for w in range(T // m)]
    assert first == [int(v) for v in g["hca_entry_first_visible"]]


def test_visibility_csa_sentinel_printed(golden):
    g = golden("p4_visibility.txt")
    m, k, T = int(g["csa_m"]), int(g["csa_k"]), int(g["csa_tokens"])
    rng = np.random.default_rng(4)
    scores = rng.standard_normal(T // m).astype(np.float32)
    filled = []
    for t in range(T):
        sel = O.select_topk(scores, O.visible_count(t, m, T // m), k)
        if t < m - 1:
            assert np.all(sel == int(g["sentinel"]))
        filled.append(int((sel >= 0).sum()))
        # only causally closed entries appear
        assert all(m * (s + 1) - 1 <= t for s in sel if s >= 0)
    assert filled == sorted(filled) and filled[-1] == k


def test_toy_csa_mask_before_topk(golden):
    g = golden("p1_csa_toy_select.txt")
    s = np.array(g["scores"], dtype=np.float32)
    k = int(g["k"])
    assert list(O.select_topk(s, len(s), k)) == [int(v) for v in g["unmasked_top2"]]
    assert list(O.select_topk(s, int(g["visible"]), k)) == [int(v) for v in g["selected"]]
    # keys for core attention: selected compressed + window tokens
    t = int(g["query_index"])
    n_keys = sum(1 for v in O.select_topk(s, int(g["visible"]), k) if v >= 0) + \
        len(O.window_positions(t, int(g["window"])))
    assert n_keys == int(g["n_keys"])
    assert list(O.window_positions(t, int(g["window"]))) == [t - 1, t]


def test_sizes_printed(golden):
    g = golden("p1_p3_sizes.txt")
    n = int(g["context"])
    K = int(g["index_topk"])
    W = int(g["swa_keys"])
    t = n - 1
    # CSA: 4:1 pool, top-k + window; HCA: 128:1 pool, all visible + window
    csa_sel = int((O.select_topk(np.zeros(O.visible_count(t, 4, n // 4), np.float32),
                                 O.visible_count(t, 4, n // 4), K) >= 0).sum())
    assert csa_sel + len(O.window_positions(t, W)) == int(g["csa_keys"])
    assert O.visible_count(t, 128, n // 128) + len(O.window_positions(t, W)) == int(g["hca_keys"])
    # toy cache after 8 tokens (m = 2 CSA, m' = 4 HCA, window 2)
    T = int(g["toy_tokens"])
    c = np.zeros((T, 4))
    assert O.compress(c, None, None, 2, c_b=c, z_b=c).shape[0] == int(g["toy_csa_entries"])
    assert O.compress(c, None, None, 4).shape[0] == int(g["toy_hca_entries"])
    assert len(O.window_positions(T - 1, int(g["toy_window"]))) == int(g["toy_window"])
    # dormant indexer: rows <= k are all kept
    for rows, kept in [(int(g["dormant_rows"]), int(g["dormant_rows"])),
                       (int(g["active_rows"]), K)]:
        s = np.random.default_rng(5).standard_normal(rows).astype(np.float32)
        assert int((O.select_topk(s, rows, K) >= 0).sum()) == kept


# ---------------------------------------------------------------------------
# Compressor
# ---------------------------------------------------------------------------
def _streams(rng, T, D):
    return [rng.standard_normal((T, D)) for _ in range(4)]


@pytest.mark.parametrize("T", [1, 3, 4, 5, 8, 13, 16])
def test_compress_pool_size(T):
    rng = np.random.default_rng(T)
    ca, za, cb, zb = _streams(rng, T, 6)
    for m in (1, 2, 4, 8):
        assert O.compress(ca, za, None, m, c_b=cb, z_b=zb).shape == (-(-T // m), 6)
        assert O.compress(ca, za, None, m).shape == (-(-T // m), 6)


def test_compress_zero_logits_is_uniform_mean():
    rng = np.random.default_rng(6)
    T, D, m = 14, 5, 4
    ca, _, cb, _ = _streams(rng, T, D)
    zero = np.zeros((T, D))
    out = O.compress(ca, zero, None, m, c_b=cb, z_b=zero)
    assert np.allclose(out[0], ca[0:4].mean(0))                       # no previous block
    assert np.allclose(out[1], np.concatenate([ca[4:8], cb[0:4]]).mean(0))
    assert np.allclose(out[3], np.concatenate([ca[12:14], cb[8:12]]).mean(0))  # partial block
    hca = O.compress(ca, zero, None, m)
    assert np.allclose(hca[2], ca[8:12].mean(0))


def test_compress_dominant_logit_selects_row():
    rng = np.random.default_rng(7)
    T, D, m = 8, 3, 4
    ca, za, cb, zb = _streams(rng, T, D)
    za = za.copy(); zb = zb.copy()
    zb[2, 1] = 80.0            # stream b, block 0, offset 2, channel 1 -> entry 1
    za[5, 0] = 80.0            # stream a, block 1, offset 1, channel 0 -> entry 1
    out = O.compress(ca, za, None, m, c_b=cb, z_b=zb)
    assert abs(out[1, 1] - cb[2, 1]) < 1e-12
    assert abs(out[1, 0] - ca[5, 0]) < 1e-12


def test_compress_bias_shifts_logits():
    """A bias on one in-block offset acts as that offset's extra logit."""
    rng = np.random.default_rng(8)
    T, D, m = 8, 4, 4
    ca, za, cb, zb = _streams(rng, T, D)
    ba = np.zeros((m, D)); ba[3] = 0.7
    bb = np.zeros((m, D)); bb[0] = -1.3
    za2 = za.copy(); za2[3::4] += 0.7
    zb2 = zb.copy(); zb2[0::4] -= 1.3
    a = O.compress(ca, za, ba, m, c_b=cb, z_b=zb, bias_b=bb)
    b = O.compress(ca, za2, None, m, c_b=cb, z_b=zb2)
    assert np.allclose(a, b, atol=1e-12)


def test_compress_matches_library_softmax_bruteforce():
    rng = np.random.default_rng(9)
    T, D, m = 11, 3, 4
    ca, za, cb, zb = _streams(rng, T, D)
    ba, bb = rng.standard_normal((m, D)), rng.standard_normal((m, D))
    pc, pz = rng.standard_normal((m, D)), rng.standard_normal((m, D))
    out = O.compress(ca, za, ba, m, c_b=cb, z_b=zb, bias_b=bb, prev_c_b=pc, prev_z_b=pz)
    for i in range(out.shape[0]):
        a_tok = [t for t in range(m * i, m * i + m) if t < T]
        logit = [za[t] + ba[t - m * i] for t in a_tok]
        val = [ca[t] for t in a_tok]
        if i == 0:
            logit += [pz[r] + bb[r] for r in range(m)]
            val += [pc[r] for r in range(m)]
        else:
            logit += [zb[t] + bb[t - m * (i - 1)] for t in range(m * (i - 1), m * i)]
            val += [cb[t] for t in range(m * (i - 1), m * i)]
        w = scipy.special.softmax(np.array(logit), axis=0)
        assert np.allclose(out[i], (w * np.array(val)).sum(0), atol=1e-12)


def test_compress_locality_and_overlap_direction():
    """Entry i depends on stream a of block i and stream b of block i-1 only."""
    rng = np.random.default_rng(10)
    T, D, m = 16, 4, 4
    ca, za, cb, zb = _streams(rng, T, D)
    base = O.compress(ca, za, None, m, c_b=cb, z_b=zb)
    for blk in range(4):
        for which in ("a", "b"):
            ca2, cb2 = ca.copy(), cb.copy()
            (ca2 if which == "a" else cb2)[m * blk: m * blk + m] += 1.0
            out = O.compress(ca2, za, None, m, c_b=cb2, z_b=zb)
            changed = [i for i in range(4) if not np.allclose(out[i], base[i])]
            want = [blk] if which == "a" else ([blk + 1] if blk + 1 < 4 else [])
            assert changed == want
    # HCA: no overlap, entry i only sees block i
    h = O.compress(ca, za, None, m)
    ca2 = ca.copy(); ca2[4:8] += 1
    h2 = O.compress(ca2, za, None, m)
    assert [i for i in range(4) if not np.allclose(h[i], h2[i])] == [1]


def test_compress_chunked_equals_whole():
    """Compressing a chunk with the previous block's b-stream as state and
    pos0 at the chunk start gives the same entries as one pass."""
    rng = np.random.default_rng(11)
    T, D, m, R = 24, 16, 4, 8
    ca, za, cb, zb = _streams(rng, T, D)
    ba, bb = 0.1 * rng.standard_normal((m, D)), 0.1 * rng.standard_normal((m, D))
    g = 1 + 0.1 * rng.standard_normal(D)
    kw = dict(gain=g, rope_dims=R)
    whole = O.compress(ca, za, ba, m, c_b=cb, z_b=zb, bias_b=bb, **kw)
    split = 12
    first = O.compress(ca[:split], za[:split], ba, m, c_b=cb[:split], z_b=zb[:split], bias_b=bb, **kw)
    second = O.compress(ca[split:], za[split:], ba, m, c_b=cb[split:], z_b=zb[split:], bias_b=bb,
                        prev_c_b=cb[split - m:split], prev_z_b=zb[split - m:split], pos0=split, **kw)
    assert np.allclose(np.concatenate([first, second]), whole, atol=1e-12)


def test_compress_rmsnorm_and_rope_position():
    rng = np.random.default_rng(12)
    T, D, m, R = 12, 32, 4, 8
    ca, za, cb, zb = _streams(rng, T, D)
    plain = O.compress(ca, za, None, m, c_b=cb, z_b=zb)
    normed = O.compress(ca, za, None, m, c_b=cb, z_b=zb, gain=np.ones(D), eps=0.0)
    assert np.allclose(np.sqrt((normed ** 2).mean(1)), 1.0)          # unit RMS
    assert np.allclose(normed / np.linalg.norm(normed, axis=1, keepdims=True),
                       plain / np.linalg.norm(plain, axis=1, keepdims=True))
    roped = O.compress(ca, za, None, m, c_b=cb, z_b=zb, gain=np.ones(D), eps=0.0,
                       rope_dims=R, pos0=100)
    for i in range(3):           # entry i rotated at its block's first token
        assert np.allclose(O.rope(roped[i], -(100 + m * i), R), normed[i], atol=1e-12)


def test_compress_m1_is_norm_and_rope_of_the_row():
    rng = np.random.default_rng(13)
    T, D, R = 10, 16, 4
    kv = rng.standard_normal((T, D))
    g = 1 + 0.02 * rng.standard_normal(D)
    rows = O.compress(kv, rng.standard_normal((T, D)), None, 1, gain=g, rope_dims=R, pos0=50)
    for j in range(T):
        unrot = O.rope(rows[j], -(50 + j), R) / g
        assert np.allclose(unrot / np.linalg.norm(unrot), kv[j] / np.linalg.norm(kv[j]))


# ---------------------------------------------------------------------------
# Indexer and selection
# ---------------------------------------------------------------------------
def test_index_single_head_unit_weight_is_relu_dot_topk():
    rng = np.random.default_rng(14)
    N, Di, K = 200, 16, 12
    q = rng.standard_normal((1, Di)); k = rng.standard_normal((N, Di))
    s = O.index_scores(q, np.ones(1), k)
    assert np.allclose(s, np.maximum(k @ q[0], 0))
    s32 = s.astype(np.float32)
    sel = O.select_topk(s32, N, K)
    ref = np.argsort(-s32.astype(np.float64), kind="stable")[:K]
    assert set(sel.tolist()) == set(ref.tolist())


def test_index_relu_before_head_weights():
    rng = np.random.default_rng(15)
    k = np.abs(rng.standard_normal((9, 4)))
    q = np.abs(rng.standard_normal((1, 4)))             # every dot positive
    assert np.all(O.index_scores(q, np.array([-1.0]), k) < 0)
    assert np.all(O.index_scores(-q, np.array([-1.0]), k) == 0)   # every dot negative


def test_index_head_weights_select_heads_linearly():
    rng = np.random.default_rng(16)
    Hi, Di, N = 5, 8, 30
    q = rng.standard_normal((Hi, Di)); k = rng.standard_normal((N, Di))
    w1, w2 = rng.standard_normal(Hi), rng.standard_normal(Hi)
    assert np.allclose(O.index_scores(q, w1 + w2, k),
                       O.index_scores(q, w1, k) + O.index_scores(q, w2, k))
    for h in range(Hi):
        e = np.zeros(Hi); e[h] = 1
        assert np.allclose(O.index_scores(q, e, k), np.maximum(k @ q[h], 0))


def test_select_ties_take_lower_index_and_descending_order():
    s = np.zeros(50, dtype=np.float32)
    assert list(O.select_topk(s, 50, 8)) == list(range(8))
    s = np.array([1, 3, 3, 2, 3, 0, 3], dtype=np.float32)
    assert list(O.select_topk(s, 7, 3)) == [1, 2, 4]
    assert list(O.select_topk(s, 7, 5)) == [1, 2, 3, 4, 6]
    rng = np.random.default_rng(17)
    s = rng.standard_normal(5000).astype(np.float32)
    sel = O.select_topk(s, 4000, 100)
    kth = np.sort(s[:4000])[-100]
    assert np.all(s[sel] >= kth) and len(set(sel.tolist())) == 100 and sel.max() < 4000


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------
def _toy_layer(seed, T=40, m=4, W=6, K=3, D=16, H=3, R=4, Hi=2, Di=8, pos_shift=0):
    rng = np.random.default_rng(seed)
    ca, za, cb, zb = [rng.standard_normal((1, T, D)) for _ in range(4)]
    ia, iza, ib, izb = [rng.standard_normal((1, T, Di)) for _ in range(4)]
    kv = rng.standard_normal((1, T, D))
    g = 1 + 0.02 * rng.standard_normal(D)
    q = rng.standard_normal((1, T, H, D))
    qi = rng.standard_normal((1, T, Hi, Di))
    wi = rng.standard_normal((1, T, Hi))
    sink = rng.standard_normal(H)
    pos0 = np.array([0])
    rpos = np.array([pos_shift])
    pool = O.csa_compress(ca, za, None, m, c_b=cb, z_b=zb, gain=g, rope_dims=R, pos0=rpos)
    keys = O.csa_compress(ia, iza, None, m, c_b=ib, z_b=izb, pos0=rpos)
    win = O.csa_compress(kv, None, None, 1, gain=g, rope_dims=R, pos0=rpos)
    n_ent = np.array([T // m])
    idx, _ = O.csa_index_topk(qi, wi, keys, n_ent, pos0, K, m)
    out, lse = O.csa_sparse_attn(q, pool, idx, win, pos0, W, sink, pos0, 1 / math.sqrt(D), R)
    return dict(out=out, lse=lse, idx=idx, pool=pool, win=win, q=q, sink=sink, D=D, R=R,
                W=W, m=m, T=T, n_ent=n_ent, pos0=pos0)


def test_layer_equals_masked_dense_attention():
    """Sparse attention over the selected rows + window equals dense attention
    over [all pool entries, window] with everything outside the selection
    masked (torch SDPA with a boolean mask, CPU float64)."""
    L = _toy_layer(18)
    D, R, W, T = L["D"], L["R"], L["W"], L["T"]
    for t in range(T):
        keys = np.concatenate([L["pool"][0], L["win"][0]])          # [N + T, D]
        allow = np.zeros(keys.shape[0], dtype=bool)
        allow[[s for s in L["idx"][0, t] if s >= 0]] = True
        allow[L["pool"].shape[1] + np.arange(max(0, t - W + 1), t + 1)] = True
        # the sink as an extra zero-valued key with logit = sink (per head)
        H = L["q"].shape[2]
        qr = O.rope(L["q"][0, t], t, R)
        zs = []
        kk = torch.from_numpy(keys)[None, None].expand(1, H, -1, D)
        mask = torch.from_numpy(allow)[None, None, None, :].expand(1, H, 1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qr)[None, :, None, :], kk, kk, attn_mask=mask, scale=1 / math.sqrt(D))
        # fold in the sink: out = ref * (1 - sink mass)
        z = (qr @ keys[allow].T) / math.sqrt(D)
        for h in range(H):
            zs.append(O.sink_softmax_weights(z[h], L["sink"][h])[1])
        ref = ref[0, :, 0].numpy() * (1 - np.array(zs))[:, None]
        assert np.allclose(O.rope(ref, -t, R), L["out"][0, t], atol=1e-12)


def test_layer_shift_invariance():
    """Rotating every row and the query by positions shifted by the same
    amount leaves the attention output unchanged: after the -t rotation only
    relative positions remain.  A wrong de-rotation sign breaks this."""
    a = _toy_layer(19)
    b = _toy_layer(19, pos_shift=4 * 1000)      # pool/window rotated at +4000
    D, R, W = a["D"], a["R"], a["W"]
    for t in [0, 5, 17, 39]:
        sel = [s for s in a["idx"][0, t] if s >= 0]
        win_r = list(range(max(0, t - W + 1), t + 1))
        rows_b = np.concatenate([b["pool"][0][sel].reshape(-1, D), b["win"][0][win_r]])
        out_b, lse_b = O.attend(a["q"][0, t], t + 4000, rows_b, a["sink"], 1 / math.sqrt(D), R)
        assert np.allclose(out_b, a["out"][0, t], atol=1e-9)
        assert np.allclose(lse_b, a["lse"][0, t], atol=1e-9)
        # de-rotating by the wrong sign gives a different answer
        bad = O.rope(O.rope(out_b, t + 4000, R), t + 4000, R)
        assert not np.allclose(bad, a["out"][0, t], atol=1e-3)


def test_layer_causality():
    """Perturbing every token after t changes nothing at query t."""
    T = 40
    base = _toy_layer(20, T=T)
    rng = np.random.default_rng(21)
    for t in [2, 3, 9, 22, 38]:
        # rebuild with the suffix replaced by fresh noise
        L = _toy_layer(20, T=T)
        out_ref = L["out"][0, t]
        rng2 = np.random.default_rng(20)
        arrs = [rng2.standard_normal((1, T, 16)) for _ in range(4)]
        idxs = [rng2.standard_normal((1, T, 8)) for _ in range(4)]
        kv = rng2.standard_normal((1, T, 16))
        g = 1 + 0.02 * rng2.standard_normal(16)
        q = rng2.standard_normal((1, T, 3, 16))
        qi = rng2.standard_normal((1, T, 2, 8))
        wi = rng2.standard_normal((1, T, 2))
        sink = rng2.standard_normal(3)
        for a in arrs + idxs + [kv]:
            a[0, t + 1:] = rng.standard_normal(a[0, t + 1:].shape)
        pos0 = np.array([0])
        pool = O.csa_compress(arrs[0], arrs[1], None, 4, c_b=arrs[2], z_b=arrs[3], gain=g, rope_dims=4)
        keys = O.csa_compress(idxs[0], idxs[1], None, 4, c_b=idxs[2], z_b=idxs[3])
        win = O.csa_compress(kv, None, None, 1, gain=g, rope_dims=4)
        idx, _ = O.csa_index_topk(qi, wi, keys, np.array([T // 4]), pos0, 3, 4, queries=[(0, t)])
        out, _ = O.csa_sparse_attn(q, pool, idx, win, pos0, 6, sink, pos0, 0.25, 4, queries=[(0, t)])
        assert np.allclose(out[0, t], out_ref, atol=1e-12)
        assert np.array_equal(idx[0, t], base["idx"][0, t])


def test_hca_equals_csa_with_all_visible_selected():
    rng = np.random.default_rng(22)
    B, Tq, H, D, R, N, m, W = 2, 5, 3, 16, 4, 12, 4, 3
    q = rng.standard_normal((B, Tq, H, D))
    pool = rng.standard_normal((B, N, D))
    win = rng.standard_normal((B, 20, D))
    q_pos0 = np.array([30, 40]); win_pos0 = np.array([25, 30])
    n_ent = np.array([N, 9])
    sink = rng.standard_normal(H)
    K = N
    idx = np.full((B, Tq, K), -1, dtype=np.int32)
    for b in range(B):
        for t in range(Tq):
            nv = O.visible_count(q_pos0[b] + t, m, n_ent[b])
            idx[b, t, :nv] = np.arange(nv)
    a, la = O.hca_attn(q, pool, n_ent, m, win, win_pos0, W, sink, q_pos0, 0.25, R)
    c, lc = O.csa_sparse_attn(q, pool, idx, win, win_pos0, W, sink, q_pos0, 0.25, R)
    assert np.allclose(a, c) and np.allclose(la, lc)


# ---------------------------------------------------------------------------
# MX FP4 storage of the indexer keys (reading: OCP Microscaling FP4, E2M1
# elements, E8M0 scale per 32 channels)
# ---------------------------------------------------------------------------
# (value at scale 1, E2M1 code) worked out by hand from the element grid
# 0, .5, 1, 1.5, 2, 3, 4, 6: exact grid points, the seven midpoints (ties go to
# the code with a clear lowest bit), points just off a midpoint, saturation.
_FP4_HAND = [(0.0, 0), (0.5, 1), (1.0, 2), (1.5, 3), (2.0, 4), (3.0, 5), (4.0, 6), (6.0, 7),
             (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
             (0.26, 1), (0.74, 1), (1.26, 3), (2.51, 5), (3.49, 5), (5.01, 7), (7.9, 7),
             (-6.0, 15), (-0.3, 9), (-2.5, 12), (-0.1, 8)]


def test_mxfp4_hand_codes():
    vals = [v for v, _ in _FP4_HAND] + [0.0] * (64 - len(_FP4_HAND))
    want = [c for _, c in _FP4_HAND] + [0] * (64 - len(_FP4_HAND))
    # amax 7.9: floor(log2 7.9) = 2, so the block's scale is 2^0 (byte 127)
    codes, scales = O.mxfp4_quantize(np.array(vals[:32] + vals[32:]).reshape(2, 32))
    assert scales[0, 0] == 127
    nib = [int(b) & 15 for b in codes.reshape(-1)]
    hi = [int(b) >> 4 for b in codes.reshape(-1)]
    got = [x for pair in zip(nib, hi) for x in pair]
    assert got[:32] == want[:32]


def test_mxfp4_packing_and_dequant_by_hand():
    x = np.zeros(32)
    x[0], x[1], x[2], x[3] = 1.0, -0.5, 6.0, -6.0
    codes, scales = O.mxfp4_quantize(x)
    assert scales[0] == 127
    assert codes[0] == (2 | (9 << 4)) and codes[1] == (7 | (15 << 4))
    assert np.all(codes[2:] == 0)
    # byte 0x7F with scale byte 129 (x4): channel 0 = -6*4, channel 1 = +6*4
    d = O.mxfp4_dequantize(np.array([0x7F] + [0] * 15, np.uint8), np.array([129], np.uint8))
    assert d[0] == -24.0 and d[1] == 24.0 and np.all(d[2:] == 0)


@pytest.mark.parametrize("k", [-20, -3, 0, 1, 7, 40])
def test_mxfp4_scale_exponent(k):
    # the scale byte is floor(log2 amax) - 2 + 127
    for amax, want in [(2.0 ** k, k + 125), (2.0 ** k * (1 - 2.0 ** -30), k + 124),
                       (1.5 * 2.0 ** k, k + 125)]:
        x = np.zeros(32)
        x[5] = -amax
        _, s = O.mxfp4_quantize(x)
        assert int(s[0]) == want, (amax, int(s[0]), want)
    z, s = O.mxfp4_quantize(np.zeros(64))
    assert np.all(s == 0) and np.all(z == 0)


def test_mxfp4_grid_values_round_trip_exactly():
    rng = np.random.default_rng(11)
    grid = np.array(O.E2M1_GRID)
    for trial in range(20):
        k = int(rng.integers(-30, 30))
        v = grid[rng.integers(0, 8, size=(3, 64))] * np.where(rng.random((3, 64)) < 0.5, -1, 1)
        v[:, 0], v[:, 32] = 6.0, -4.0   # block maxima fix the scale at 2^k
        x = v * 2.0 ** k
        codes, scales = O.mxfp4_quantize(x)
        assert np.array_equal(O.mxfp4_dequantize(codes, scales), x)


def test_mxfp4_error_within_half_grid_gap():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((40, 128)) * np.exp2(rng.integers(-8, 8, size=(40, 1)))
    codes, scales = O.mxfp4_quantize(x)
    d = O.mxfp4_dequantize(codes, scales)
    X = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=-1)
    a = np.abs(x) / X
    assert np.all(a < 8)
    # half the gap of the grid interval the scaled value falls in (values in
    # [6, 8) saturate to 6)
    half = np.where(a <= 2, 0.25, np.where(a <= 4, 0.5, np.where(a <= 6, 1.0, a - 6)))
    assert np.all(np.abs(d - x) <= half * X * (1 + 1e-12))
    assert np.all(np.sign(d) * np.sign(x) >= 0)
    # the block maximum keeps at least 2^(-1) of its value: scale choice sane
    amax = np.abs(x).reshape(40, 4, 32).max(-1)
    assert np.all(np.abs(d).reshape(40, 4, 32).max(-1) >= 0.5 * amax)


# ---------------------------------------------------------------------------
# Mixed BF16 / FP8 storage of the KV entries (reading: OCP Microscaling FP8,
# E4M3 elements, E8M0 scale per 32 channels; RoPE channels in bfloat16)
# ---------------------------------------------------------------------------
# E4M3 magnitudes worked out by hand from the format (bias 7, 3 mantissa bits,
# exponent field 0 subnormal in units of 2^-9, 0x7F not a number)
_E4M3_HAND = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
              0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x78: 256.0,
              0x79: 288.0, 0x7E: 448.0}
# (value at scale 1, code) by hand: grid points, midpoints (ties to the even
# code), points next to a midpoint, the subnormal range and its top,
# saturation of [448, 512) and signs
_FP8_HAND = [(1.0, 0x38), (1.0625, 0x38), (1.0626, 0x39), (1.1875, 0x3A), (1.125, 0x39),
             (300.0, 0x79), (304.0, 0x7A), (303.9, 0x79), (448.0, 0x7E), (460.0, 0x7E),
             (511.0, 0x7E), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (7.5 * 2.0 ** -9, 0x08),
             (2.0 ** -11, 0x00), (0.0, 0x00), (-1.0, 0xB8), (-300.0, 0xF9), (-2.0 ** -10, 0x80),
             (1.875, 0x3F), (1.9375, 0x40), (255.0, 0x78)]


def test_e4m3_grid_by_hand():
    for code, v in _E4M3_HAND.items():
        assert O.E4M3_GRID[code] == v, hex(code)
    assert len(O.E4M3_GRID) == 127 and all(np.diff(O.E4M3_GRID) > 0)


def test_fp8_hand_codes():
    # block maximum 511 (floor(log2) = 8): scale byte 127, scale 1
    vals = [v for v, _ in _FP8_HAND]
    x = np.zeros((1, 96))
    x[0, :len(vals)] = vals
    x[0, 32] = 1.0     # second block: amax 1 -> scale byte 119 (2^-8), 1 -> 256 = 0x78
    x[0, 33] = 2.0 ** -8   # -> 1.0 under that scale = 0x38
    rows = O.kv_fp8_quantize(x, 32)   # D = 96, R = 32: two FP8 blocks, channels 0-63
    assert rows.shape == (1, O.kv_fp8_row_bytes(96, 32)) == (1, 64 + 64 + 16)
    assert [int(c) for c in rows[0, :len(vals)]] == [c for _, c in _FP8_HAND]
    assert rows[0, 128] == 127 and rows[0, 129] == 119
    assert rows[0, 32] == 0x78 and rows[0, 33] == 0x38
    assert np.all(rows[0, 130:] == 0)       # scale padding


def test_fp8_codes_match_torch_float8_e4m3fn():
    """Library special case: at scale 1 (a block whose maximum lies in
    [256, 448)) the element codes equal torch's float32 -> float8_e4m3fn
    conversion (nearest, ties to even)."""
    import torch
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((50, 32)) * np.exp2(rng.integers(-12, 8, size=(50, 32))))
    x = np.clip(x, -440, 440).astype(np.float32)
    x[:, 0] = 300.0
    rows = O.kv_fp8_quantize(x.astype(np.float64), 0)
    assert np.all(rows[:, 32] == 127)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(rows[:, :32], want)


@pytest.mark.parametrize("k", [-20, -3, 0, 1, 7, 40])
def test_fp8_scale_exponent(k):
    # the scale byte is floor(log2 amax) - 8 + 127
    for amax, want in [(2.0 ** k, k + 119), (2.0 ** k * (1 - 2.0 ** -30), k + 118),
                       (1.5 * 2.0 ** k, k + 119)]:
        x = np.zeros(32)
        x[7] = -amax
        r = O.kv_fp8_quantize(x, 0)
        assert int(r[32]) == want, (amax, int(r[32]), want)
    z = O.kv_fp8_quantize(np.zeros(64), 0)
    assert np.all(z == 0)
    tiny = np.zeros(32)
    tiny[0] = 2.0 ** -130     # below 2^-119: the byte clamps at 0
    assert O.kv_fp8_quantize(tiny, 0)[32] == 0


def test_fp8_row_layout_and_rope_bf16():
    """D = 512, R = 64: 448 code bytes, the RoPE channels as bfloat16 bits
    (nearest even), 14 scale bytes padded to 16: 592 bytes."""
    assert O.kv_fp8_row_bytes(512, 64) == 592
    x = np.zeros(512)
    x[448] = 1.0                                  # bf16 0x3F80
    x[449] = 1.0 + 2.0 ** -8                      # tie -> even: 0x3F80
    x[450] = 1.0 + 3 * 2.0 ** -8                  # tie -> even: 0x3F82
    x[511] = -2.0                                 # 0xC000
    r = O.kv_fp8_quantize(x, 64)
    bits = r[448:576].view(np.uint16)
    assert bits[0] == 0x3F80 and bits[1] == 0x3F80 and bits[2] == 0x3F82 and bits[63] == 0xC000
    assert np.all(r[:448] == 0) and np.all(r[576:] == 0)
    d = O.kv_fp8_dequantize(r, 512, 64)
    assert d[448] == 1.0 and d[450] == 1.0 + 2.0 ** -6 and d[511] == -2.0


def test_fp8_grid_values_round_trip_exactly():
    rng = np.random.default_rng(14)
    grid = np.array(O.E4M3_GRID)
    for trial in range(20):
        k = int(rng.integers(-30, 30))
        v = grid[rng.integers(0, 127, size=(3, 448))] * np.where(rng.random((3, 448)) < 0.5, -1, 1)
        v[:, ::32] = 448.0          # every block's maximum fixes its scale at 2^k
        rope = rng.integers(-255, 256, size=(3, 64)) / 8.0    # 8 significant bits: exact in bfloat16
        x = np.concatenate([v * 2.0 ** k, rope], axis=1)
        r = O.kv_fp8_quantize(x, 64)
        assert np.array_equal(O.kv_fp8_dequantize(r, 512, 64), x)


def test_fp8_error_within_half_step():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((40, 512)) * np.exp2(rng.integers(-8, 8, size=(40, 1)))
    x = x.astype(np.float32).astype(np.float64)
    r = O.kv_fp8_quantize(x, 64)
    d = O.kv_fp8_dequantize(r, 512, 64)
    X = np.repeat(np.exp2(r[:, 576:590].astype(np.float64) - 127), 32, axis=-1)
    a = np.abs(x[:, :448]) / X
    assert np.all(a < 512)
    # half the local step: 2^(e-4) for a normal magnitude of exponent e, 2^-10
    # in the subnormal range; [448, 512) saturates to 448
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    half = np.where(a >= 448, a - 448, 2.0 ** (e - 4))
    assert np.all(np.abs(d[:, :448] - x[:, :448]) <= half * X * (1 + 1e-12))
    # the RoPE channels: bfloat16 rounding (half a unit: relative 2^-8 at most)
    assert np.all(np.abs(d[:, 448:] - x[:, 448:]) <= np.abs(x[:, 448:]) * 2.0 ** -8)


# ---------------------------------------------------------------------------
# Grouped low-rank output projection
# ---------------------------------------------------------------------------
def test_grouped_projection_is_block_diagonal_product():
    """Grouping = one product with a block-diagonal first matrix over the
    concatenated heads (scipy's block_diag builds it independently)."""
    import scipy.linalg
    rng = np.random.default_rng(31)
    H, D, g, r, d = 8, 16, 4, 12, 10
    o = rng.standard_normal((H, D))
    w_a = rng.standard_normal((g, r, (H // g) * D))
    w_b = rng.standard_normal((d, g * r))
    big = scipy.linalg.block_diag(*w_a)                 # [g r, H D]
    want = w_b @ (big @ o.reshape(-1))
    assert np.allclose(O.grouped_output_projection(o, w_a, w_b), want, rtol=1e-12, atol=1e-12)


def test_grouped_projection_one_group_is_two_plain_products():
    rng = np.random.default_rng(32)
    o = rng.standard_normal((4, 8))
    w_a = rng.standard_normal((1, 6, 32))
    w_b = rng.standard_normal((5, 6))
    want = torch.tensor(w_b) @ (torch.tensor(w_a[0]) @ torch.tensor(o).reshape(-1))
    assert np.allclose(O.grouped_output_projection(o, w_a, w_b), want.numpy(), rtol=1e-12)


def test_grouped_projection_group_locality():
    """Changing one head changes only its group's intermediate: with w_b
    reading a single group's slot, heads of other groups have no effect."""
    rng = np.random.default_rng(33)
    H, D, g, r = 8, 4, 4, 3
    o = rng.standard_normal((H, D))
    w_a = rng.standard_normal((g, r, (H // g) * D))
    w_b = np.zeros((r, g * r))
    w_b[:, 2 * r:3 * r] = np.eye(r)                    # reads group 2 only
    base = O.grouped_output_projection(o, w_a, w_b)
    o2 = o.copy()
    o2[[0, 1, 2, 3, 6, 7]] += 5.0                       # heads outside group 2 (heads 4, 5)
    assert np.allclose(O.grouped_output_projection(o2, w_a, w_b), base, rtol=0, atol=1e-12)
    o3 = o.copy()
    o3[5, 1] += 1.0                                     # head 5 = second head of group 2
    delta = O.grouped_output_projection(o3, w_a, w_b) - base
    assert np.allclose(delta, w_a[2][:, D + 1], atol=1e-12)


def test_compress_first_block_has_no_previous_block():
    """A block at the start of a sequence has no block before it: a given
    previous stream is not pooled there ([P2] section 3.2.2, eqs. 9-12 pool
    block i-1, which the first block lacks), while one block later it is."""
    rng = np.random.default_rng(41)
    m, D = 4, 8
    ca, za, cb, zb = (rng.standard_normal((m, D)) for _ in range(4))
    pc, pz = rng.standard_normal((m, D)), rng.standard_normal((m, D))
    bb = 0.1 * rng.standard_normal((m, D))
    kw = dict(c_b=cb, z_b=zb, bias_b=bb)
    alone = O.compress(ca, za, None, m, pos0=0, **kw)
    with_prev_at_0 = O.compress(ca, za, None, m, prev_c_b=pc, prev_z_b=pz, pos0=0, **kw)
    with_prev_at_m = O.compress(ca, za, None, m, prev_c_b=pc, prev_z_b=pz, pos0=m, **kw)
    assert np.array_equal(alone, with_prev_at_0)
    assert not np.allclose(alone, with_prev_at_m)
    # at pos0 = m the entry is the library softmax over all 2m rows
    logits = np.concatenate([za, pz + bb])
    wts = scipy.special.softmax(logits, axis=0)
    assert np.allclose(with_prev_at_m[0], (wts * np.concatenate([ca, pc])).sum(0), atol=1e-12)
