"""Plain float64 CPU oracle for DeepSeek-V4 Compressed Sparse Attention (CSA)
and Heavily Compressed Attention (HCA).

TEST INFRASTRUCTURE ONLY.  This module is the independent checker of the HIP
path: only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import it.  It imports nothing from the GPU package and shares
no code with it.  Every function is written for readability, not speed: plain
NumPy float64 (one library matmul or sort per step at most), loops where the
definition is a loop.

Sources (web pages on DeepSeek-V4; cited by page title and section):
  [P1] "DeepSeek V4 Inside: One Token Through Every Block"
  [P2] "DeepSeek-v4 Beyond Basics: A Practical Guide to mHC, CSA, HCA, and Muon"
  [P3] "07 The Model" (DS4 course, Phase 1 Module 1)
  [P4] Hugging Face transformers documentation page "DeepSeek-V4"

Readings taken where the pages are silent or ambiguous (each is listed in the
design notes of the repository):
  * overlap direction: entry i pools block i from stream a and block i-1 from
    stream b (the only direction under which a CSA query at t < m-1 sees no
    entry, as [P4] "Tata letak attention mask" states);
  * softmax per channel over the available rows, biases shaped [m, D];
  * a partial last block pools only the tokens that exist; a missing previous
    block contributes no rows;
  * an entry is RoPE-rotated at the position of its block's first token;
  * RoPE base 10000, no YaRN scaling; angles in float64;
  * RMSNorm eps 1e-6, a single gain shared by the head;
  * the indexer applies no scale, norm or RoPE; ReLU before the head weights;
  * mask first, then top-k; ties go to the lower entry index;
  * selected and window rows are concatenated without de-duplication;
  * an empty key set gives a zero output and lse equal to the sink logit;
  * all positions are 0-based;
  * FP4 indexer keys are stored in the OCP Microscaling (MX) FP4 format:
    E2M1 elements with one E8M0 power-of-two scale per 32 channels (the
    pages name FP4 for the indexer and give no format);
  * KV entries stored in mixed precision keep the RoPE channels in bfloat16
    and the others in the OCP MX FP8 format (E4M3 elements, one E8M0 scale
    per 32 channels); the pages name BF16 and FP8 and give no format.

Parity status: every function here is pinned by tests/test_oracle_pins.py
against printed values, closed forms, invariants or library routines, except
where a function docstring says "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "rope",
    "sink_softmax_weights",
    "compress",
    "visible_count",
    "window_positions",
    "index_scores",
    "select_topk",
    "attend",
    "csa_compress",
    "csa_index_topk",
    "csa_sparse_attn",
    "hca_attn",
    "E2M1_GRID",
    "mxfp4_quantize",
    "mxfp4_dequantize",
    "E4M3_GRID",
    "kv_fp8_row_bytes",
    "kv_fp8_quantize",
    "kv_fp8_dequantize",
    "grouped_output_projection",
]


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def rope(x, pos, rope_dims: int, base: float = 10000.0) -> np.ndarray:
    """Partial rotary embedding on interleaved pairs of the last ``rope_dims``
    channels.

    [P4] "Arsitektur": partial RoPE with interleaved pairs on the last
    qk_rope_head_dim channels of every head; the same rotation with position
    -i is applied to the rope slice of the attention output.  [P1] "What does
    layer 0 sliding-window attention do to p?": the pair (x, y) at position i
    becomes (x cos i - y sin i, x sin i + y cos i) for the pair whose
    frequency is 1.  [P2] section 3.3 (quoting the paper's section 2.3.3): RoPE
    acts on the last 64 dimensions.

    Pair j (0 <= j < R/2) covers channels u = D-R+2j and u+1 and turns with
    angle pos * base**(-2j/R), computed in float64.

    x: [..., D] array; pos: scalar or array broadcastable to x.shape[:-1].
    """
    x = np.array(x, dtype=np.float64, copy=True)
    if rope_dims == 0:
        return x
    D = x.shape[-1]
    R = int(rope_dims)
    assert R % 2 == 0 and 0 < R <= D
    half = R // 2
    j = np.arange(half, dtype=np.float64)
    theta = np.power(float(base), -2.0 * j / R)
    phi = np.asarray(pos, dtype=np.float64)[..., None] * theta
    u = D - R + 2 * np.arange(half)
    v = u + 1
    xu = x[..., u].copy()
    xv = x[..., v].copy()
    c = np.cos(phi)
    s = np.sin(phi)
    x[..., u] = xu * c - xv * s
    x[..., v] = xu * s + xv * c
    return x


# ---------------------------------------------------------------------------
# Softmax with a per-head sink in the denominator
# ---------------------------------------------------------------------------
def sink_softmax_weights(z, sink: float):
    """Weights exp(z_j) / (sum_k exp(z_k) + exp(sink)) and the left-over sink
    mass.  [P1] "What does layer 0 sliding-window attention do to p?", eq.(27):
    the sink logit enters the denominator only, so the key weights may sum to
    less than one and a head can put its mass on no key at all.

    The largest logit (sink included) is subtracted first; that changes no
    value of the quotient.
    """
    z = np.asarray(z, dtype=np.float64)
    mx = max(float(z.max()) if z.size else -math.inf, float(sink))
    e = np.exp(z - mx)
    es = math.exp(float(sink) - mx)
    denom = e.sum() + es
    return e / denom, es / denom


# ---------------------------------------------------------------------------
# Token-level compressor (CSA: m, overlapped, two streams; HCA: m', one stream)
# ---------------------------------------------------------------------------
def compress(c_a, z_a, bias_a, m: int, *, c_b=None, z_b=None, bias_b=None,
             prev_c_b=None, prev_z_b=None, gain=None, eps: float = 1e-6,
             rope_dims: int = 0, rope_base: float = 10000.0, pos0: int | None = None,
             overlap: bool | None = None) -> np.ndarray:
    """Compress one sequence's token streams into ceil(T/m) entries.

    [P2] section 3.2.2 (eqs. 9-12): two token streams C^a, C^b with logits
    Z^a, Z^b; every m tokens become one entry as a Hadamard (per-channel)
    softmax-weighted sum, the softmax running over the rows drawn from both
    Z^a and Z^b plus the learned position biases B^a, B^b.  [P1] "How does CSA
    compress 8 tokens into 4 KV entries?" (GOTCHA): 2m weights per block,
    normalised by a softmax, adjacent blocks overlap.  [P2] section 3.3
    (eqs. 20-23) and [P4] "Arsitektur": HCA uses m' = 128, one stream, no
    overlap.  [P2] section 3.3 (quoting section 2.3.3): RMSNorm on the single
    compressed KV head, then RoPE on its last 64 channels.

    Entry i (tokens m*i .. m*i+m-1 relative to ``pos0``) takes stream a from
    block i and, when overlapped, stream b from block i-1 (for i == 0 the
    b rows come from ``prev_*`` if given, otherwise block i has no b rows;
    a block that starts before token m is the sequence's first and has no
    block before it, so ``prev_*`` is not used when pos0 < m).  ``gain`` None
    means no RMSNorm; ``rope_dims`` 0 means no RoPE.  The entry is rotated at
    absolute position pos0 + m*i (pos0 None: positions unknown, taken as 0
    for RoPE, and ``prev_*`` used when given).

    Inputs are [T, D] (``prev_*`` [m, D]; biases [m, D]; gain [D]).
    The pages print no pooled value of the real operator, so the pins are
    closed forms, invariants and a library-softmax brute force on tiny inputs.
    Two parts rest on readings the pages do not fix and are parity unpinned
    against them (the tests pin them only to the reading): the overlap
    direction (stream b from block i-1) and the entry's RoPE position
    (pos0 + m*i).
    """
    c_a = np.asarray(c_a, dtype=np.float64)
    T, D = c_a.shape
    z_a = np.zeros((T, D)) if z_a is None else np.asarray(z_a, dtype=np.float64)
    bias_a = np.zeros((m, D)) if bias_a is None else np.asarray(bias_a, dtype=np.float64)
    if overlap is None:
        overlap = c_b is not None
    if overlap:
        c_b = np.asarray(c_b, dtype=np.float64)
        z_b = np.asarray(z_b, dtype=np.float64)
        bias_b = np.zeros((m, D)) if bias_b is None else np.asarray(bias_b, dtype=np.float64)
    n_entries = -(-T // m)
    out = np.zeros((n_entries, D))
    for i in range(n_entries):
        logits = []
        values = []
        for r in range(m):
            tok = m * i + r
            if tok < T:
                logits.append(z_a[tok] + bias_a[r])
                values.append(c_a[tok])
        if overlap:
            for r in range(m):
                if i >= 1:
                    tok = m * (i - 1) + r
                    logits.append(z_b[tok] + bias_b[r])
                    values.append(c_b[tok])
                elif prev_c_b is not None and (pos0 is None or pos0 >= m):
                    # the block before this chunk; a block that starts
                    # before token m is the first and has none
                    logits.append(np.asarray(prev_z_b[r], dtype=np.float64) + bias_b[r])
                    values.append(np.asarray(prev_c_b[r], dtype=np.float64))
        L = np.stack(logits)            # [rows, D]
        V = np.stack(values)            # [rows, D]
        w = np.exp(L - L.max(axis=0))   # per-channel softmax over the rows
        w = w / w.sum(axis=0)
        pooled = (w * V).sum(axis=0)
        if gain is not None:
            g = np.asarray(gain, dtype=np.float64)
            pooled = pooled / np.sqrt(np.mean(pooled * pooled) + eps) * g
        if rope_dims:
            pooled = rope(pooled, (pos0 or 0) + m * i, rope_dims, rope_base)
        out[i] = pooled
    return out


# ---------------------------------------------------------------------------
# Causal visibility and the sliding window
# ---------------------------------------------------------------------------
def visible_count(t_pos: int, m: int, n_entries: int) -> int:
    """Number of compressed entries a query at absolute position t may see.

    [P1] "How does CSA compress 8 tokens into 4 KV entries?": an entry is
    visible only when every token in it sits at or before the query.  [P4]
    "Tata letak attention mask": HCA entry w becomes visible once its window
    has closed, w < (t+1) // m; CSA queries before the first closed window
    (t < m-1) see nothing.  Entries beyond the cache (``n_entries``) do not
    exist.
    """
    return max(0, min(int(n_entries), (int(t_pos) + 1) // int(m)))


def window_positions(t_pos: int, W: int) -> range:
    """Absolute token positions of the uncompressed sliding-window branch for
    a query at t: the last W tokens up to and including t.  [P2] section 3.2.2:
    the most recent 128 uncompressed tokens; [P1] "What does layer 0
    sliding-window attention do to p?": the window includes the query's own
    token."""
    return range(max(0, int(t_pos) - int(W) + 1), int(t_pos) + 1)


# ---------------------------------------------------------------------------
# Lightning indexer and top-k selection
# ---------------------------------------------------------------------------
def index_scores(q_idx, w_idx, k_idx) -> np.ndarray:
    """Index scores of one query against every compressed indexer key.

    [P2] section 3.2.2 (eq. 16): I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . K[s]).
    [P3] "The indexer: a learned retrieval mechanism": every compressed row is
    scored against all 64 indexer query heads; each head's dot product passes
    a ReLU and the heads are mixed by learned per-head weights.

    q_idx [Hi, Di], w_idx [Hi], k_idx [N, Di] -> float64 [N].
    """
    q = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w_idx, dtype=np.float64)
    k = np.asarray(k_idx, dtype=np.float64)
    dots = q @ k.T                          # [Hi, N]
    return (w[:, None] * np.maximum(dots, 0.0)).sum(axis=0)


def select_topk(scores, n_visible: int, K: int) -> np.ndarray:
    """Top-k selector over the visible entries 0 .. n_visible-1.

    [P2] section 3.2.2 (eq. 17): keep the entries whose index score is among
    the top k.  [P1] "How does CSA compress 8 tokens into 4 KV entries?": the
    causal mask applies before the ranking.  [P3] "The indexer: a learned
    retrieval mechanism": with no more rows than k, every row is kept.  [P4]
    "Tata letak attention mask": empty slots carry the sentinel -1.

    The decision is taken on the scores as given (float32 for the parity
    rule); ties go to the lower index.  Returns int32 [K]: the chosen indices
    in ascending order, then -1 padding.
    """
    s = np.asarray(scores)
    n = int(n_visible)
    if n <= K:
        chosen = np.arange(n)
    else:
        idx = np.arange(n)
        vals = s[:n]
        # primary key: descending score; secondary: ascending index
        order = np.lexsort((idx, -vals.astype(np.float64)))
        chosen = np.sort(order[:K])
    out = np.full(K, -1, dtype=np.int32)
    out[: len(chosen)] = chosen
    return out


# ---------------------------------------------------------------------------
# Shared-K=V multi-query attention with a per-head sink
# ---------------------------------------------------------------------------
def attend(q, t_pos: int, rows, sink, scale: float, rope_dims: int,
           rope_base: float = 10000.0):
    """Core attention of one query token over a list of K=V rows.

    [P2] section 3.2.2 (eq. 19) and [P4] "Arsitektur": the selected compressed
    entries (concatenated with the window rows) serve as both key and value of
    a multi-query attention with one KV head.  [P1] "What does layer 0
    sliding-window attention do to p?": logits scaled by 1/sqrt(head_dim),
    sink logit in the denominator (eq. 27).  [P1] "How does CSA compress 8
    tokens into 4 KV entries?" and [P4] "Arsitektur": the rope slice of the
    output is rotated by position -t.

    q [H, D] (already RMS-normalised, not yet rotated), rows [n, D],
    sink [H] -> (out [H, D], lse [H]) in float64.  lse includes the sink.
    """
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64).reshape(-1, q.shape[-1])
    sink = np.asarray(sink, dtype=np.float64)
    H, D = q.shape
    if rows.shape[0] == 0:
        return np.zeros((H, D)), sink.copy()
    qr = rope(q, t_pos, rope_dims, rope_base)
    z = scale * (qr @ rows.T)                       # [H, n]
    mx = np.maximum(z.max(axis=1), sink)
    denom = np.exp(z - mx[:, None]).sum(axis=1) + np.exp(sink - mx)
    lse = mx + np.log(denom)
    p = np.exp(z - lse[:, None])                    # key weights
    o = p @ rows                                    # [H, D]
    return rope(o, -t_pos, rope_dims, rope_base), lse


# ---------------------------------------------------------------------------
# Batched drivers with the same argument meaning as the library's calls
# ---------------------------------------------------------------------------
def csa_compress(c_a, z_a, bias_a, m, *, c_b=None, z_b=None, bias_b=None,
                 prev_c_b=None, prev_z_b=None, gain=None, eps=1e-6,
                 rope_dims=0, rope_base=10000.0, pos0=None, overlap=None):
    """Batched ``compress``: streams [B, T, D], prev [B, m, D] -> [B, ceil(T/m), D]."""
    c_a = np.asarray(c_a)
    B = c_a.shape[0]
    pos0 = None if pos0 is None else np.asarray(pos0)
    outs = []
    for b in range(B):
        outs.append(compress(
            c_a[b], None if z_a is None else z_a[b], bias_a, m,
            c_b=None if c_b is None else c_b[b], z_b=None if z_b is None else z_b[b],
            bias_b=bias_b,
            prev_c_b=None if prev_c_b is None else prev_c_b[b],
            prev_z_b=None if prev_z_b is None else prev_z_b[b],
            gain=gain, eps=eps, rope_dims=rope_dims, rope_base=rope_base,
            pos0=None if pos0 is None else int(pos0[b]), overlap=overlap))
    return np.stack(outs)


def csa_index_topk(q_idx, w_idx, k_idx, n_entries, q_pos0, K, m, queries=None):
    """Scores and selections for every query (or the listed (b, t) pairs).

    q_idx [B, Tq, Hi, Di], w_idx [B, Tq, Hi], k_idx [B, N_cap, Di],
    n_entries [B], q_pos0 [B].  Returns (idx int32 [B, Tq, K] with -1 where not
    computed, scores float32 [B, Tq, N_cap] with NaN beyond the visible
    entries).  The float64 scores are rounded to float32 before selection.
    """
    q_idx = np.asarray(q_idx)
    B, Tq = q_idx.shape[:2]
    N_cap = np.asarray(k_idx).shape[1]
    idx = np.full((B, Tq, K), -1, dtype=np.int32)
    scores = np.full((B, Tq, N_cap), np.nan, dtype=np.float32)
    pairs = queries if queries is not None else [(b, t) for b in range(B) for t in range(Tq)]
    for b, t in pairs:
        t_pos = int(q_pos0[b]) + t
        n_vis = visible_count(t_pos, m, int(n_entries[b]))
        s64 = index_scores(q_idx[b, t], w_idx[b, t], k_idx[b, :n_vis])
        s32 = s64.astype(np.float32)
        scores[b, t, :n_vis] = s32
        idx[b, t] = select_topk(s32, n_vis, K)
    return idx, scores


def _window_rows(win, win_pos0, t_pos, W):
    r = [p - int(win_pos0) for p in window_positions(t_pos, W)]
    if r and (r[0] < 0 or r[-1] >= win.shape[0]):
        raise ValueError("window buffer does not cover the query's window")
    return np.asarray(win, dtype=np.float64)[r] if r else np.zeros((0, win.shape[1]))


def csa_sparse_attn(q, pool, idx, win, win_pos0, W, sink, q_pos0, scale,
                    rope_dims, rope_base=10000.0, queries=None):
    """Sparse attention over idx-selected pool rows and the window rows.

    q [B, Tq, H, D], pool [B, N_cap, D], idx [B, Tq, K] (-1 = empty slot),
    win [B, L_win, D] with win[b, r] the token at win_pos0[b] + r.
    Returns (out [B, Tq, H, D], lse [B, Tq, H]); entries not computed are NaN.
    """
    q = np.asarray(q)
    B, Tq, H, D = q.shape
    out = np.full((B, Tq, H, D), np.nan)
    lse = np.full((B, Tq, H), np.nan)
    pairs = queries if queries is not None else [(b, t) for b in range(B) for t in range(Tq)]
    for b, t in pairs:
        t_pos = int(q_pos0[b]) + t
        sel = [int(s) for s in idx[b, t] if s >= 0]
        rows = np.concatenate([np.asarray(pool[b][sel], dtype=np.float64).reshape(-1, D),
                               _window_rows(win[b], win_pos0[b], t_pos, W)])
        out[b, t], lse[b, t] = attend(q[b, t], t_pos, rows, sink, scale, rope_dims, rope_base)
    return out, lse


def hca_attn(q, pool, n_entries, m, win, win_pos0, W, sink, q_pos0, scale,
             rope_dims, rope_base=10000.0, queries=None):
    """Dense attention over every visible compressed entry and the window.

    [P2] section 3.3 (eq. 26): no top-k selection, every heavily compressed
    entry is attended.  [P1] "What does HCA change?": same MQA, window, RoPE
    and sink as CSA.  Argument meaning as ``csa_sparse_attn`` with the
    selection replaced by the entries w < visible_count(t, m, n_entries[b]).
    """
    q = np.asarray(q)
    B, Tq, H, D = q.shape
    out = np.full((B, Tq, H, D), np.nan)
    lse = np.full((B, Tq, H), np.nan)
    pairs = queries if queries is not None else [(b, t) for b in range(B) for t in range(Tq)]
    for b, t in pairs:
        t_pos = int(q_pos0[b]) + t
        n_vis = visible_count(t_pos, m, int(n_entries[b]))
        rows = np.concatenate([np.asarray(pool[b][:n_vis], dtype=np.float64).reshape(-1, D),
                               _window_rows(win[b], win_pos0[b], t_pos, W)])
        out[b, t], lse[b, t] = attend(q[b, t], t_pos, rows, sink, scale, rope_dims, rope_base)
    return out, lse


# ---------------------------------------------------------------------------
# FP4 storage of the indexer keys (reading)
# ---------------------------------------------------------------------------
# [P1] "What does HCA change?" names FP4 for the indexer's cache and gives no
# format.  Reading: the OCP Microscaling (MX) v1.0 FP4 format, blocks of 32
# channels.  Element: E2M1 (sign bit 3; 3-bit magnitude code c holding
# E2M1_GRID[c]).  Block scale: E8M0 byte s meaning 2**(s - 127), with
# s = floor(log2(max |x|)) - 2 + 127 clamped to [0, 254] (2 is the largest
# exponent of an E2M1 value); an all-zero block takes s = 0.  Each element is
# |x| / 2**(s-127) rounded to the nearest grid value, ties to the even code
# (the one whose lowest bit is 0); the scaled value is below 8, so the top
# grid value 6 also takes everything in [6, 8).  The sign bit is set for
# x < 0.  Packing: channel 2i in the low nibble of byte i.
# Parity unpinned against the pages (they print no FP4 value): the format is
# a reading; the functions below are pinned to its definition.
E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
MX_BLOCK = 32


def _e8m0_of_block(v) -> int:
    amax = max(abs(float(e)) for e in v)
    if amax == 0.0:
        return 0
    _, k = math.frexp(amax)          # amax = f * 2**k with 0.5 <= f < 1
    return min(max((k - 1) - 2 + 127, 0), 254)


def _e2m1_code(x: float, scale: float) -> int:
    a = abs(x) / scale
    best = min(range(8), key=lambda c: (abs(a - E2M1_GRID[c]), c & 1))
    return best | (8 if x < 0 else 0)


def mxfp4_quantize(x):
    """Keys [..., D] (D a multiple of 32) -> (codes uint8 [..., D/2],
    scales uint8 [..., D/32]) in the MX FP4 reading above.  Plain loops."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert D % MX_BLOCK == 0
    flat = x.reshape(-1, D)
    codes = np.zeros((flat.shape[0], D // 2), np.uint8)
    scales = np.zeros((flat.shape[0], D // MX_BLOCK), np.uint8)
    for r in range(flat.shape[0]):
        nib = []
        for blk in range(D // MX_BLOCK):
            v = flat[r, MX_BLOCK * blk: MX_BLOCK * (blk + 1)]
            s = _e8m0_of_block(v)
            scales[r, blk] = s
            nib += [_e2m1_code(e, 2.0 ** (s - 127)) for e in v]
        for i in range(D // 2):
            codes[r, i] = nib[2 * i] | (nib[2 * i + 1] << 4)
    return codes.reshape(x.shape[:-1] + (D // 2,)), scales.reshape(x.shape[:-1] + (D // MX_BLOCK,))


def mxfp4_dequantize(codes, scales) -> np.ndarray:
    """Exact values (float64 [..., D]) of MX FP4 keys stored as above."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[:-1] + (-1,))
    mag = np.asarray(E2M1_GRID, dtype=np.float64)[nib & 7]
    val = np.where(nib & 8, -mag, mag)
    scale = np.repeat(np.exp2(scales.astype(np.float64) - 127.0), MX_BLOCK, axis=-1)
    return val * scale


# ---------------------------------------------------------------------------
# Mixed BF16 / FP8 storage of the KV entries (reading)
# ---------------------------------------------------------------------------
# [P1] "What does HCA change?" (quoting the paper's section 2.3.4): the KV
# cache keeps the RoPE channels in BF16 and the other channels in FP8; the
# pages give no FP8 format.  Reading: the OCP Microscaling (MX) v1.0 FP8
# format on the D - R non-RoPE channels, blocks of 32 channels (the FP4
# reading's family).  Element: E4M3 as OCP defines it ("E4M3FN": sign bit 7,
# exponent field bits 3-6 with bias 7, mantissa bits 0-2; exponent field 0
# holds the subnormals m * 2**-9; magnitude code 0x7F is NaN, so the largest
# finite magnitude is 0x7E = 448).  Block scale: E8M0 byte s meaning
# 2**(s - 127), s = floor(log2(max |x|)) - 8 + 127 clamped to [0, 254] (8 is
# the largest exponent of an E4M3 value); an all-zero block takes s = 0.
# Each element is |x| / 2**(s-127) (below 512) rounded to the nearest finite
# E4M3 magnitude, ties to the even code, which saturates [448, 512) at 448;
# the sign bit is set for x < 0.  The R RoPE channels are rounded to
# bfloat16 (nearest, ties to even).  Packed row of one entry:
#   bytes [0, D-R)            E4M3 codes of channels 0 .. D-R-1
#   bytes [D-R, D+R)          bfloat16 of channels D-R .. D-1 (little endian)
#   bytes [D+R, D+R+P)        the (D-R)/32 scale bytes, zero-padded to P, the
#                             next multiple of 16
# (592 bytes for D = 512, R = 64, against 1,024 in bfloat16).
# Parity unpinned against the pages (they print no FP8 value): the format is
# a reading; the functions below are pinned to its definition.
E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Magnitude of E4M3 magnitude code 0..126 (exponent field 0: subnormal)."""
    e, m = code >> 3, code & 7
    if e == 0:
        return m * 2.0 ** -9
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_GRID = tuple(e4m3_value(c) for c in range(127))


def kv_fp8_row_bytes(D: int, rope_dims: int) -> int:
    nb = (D - rope_dims) // MX_BLOCK
    return (D - rope_dims) + 2 * rope_dims + 16 * ((nb + 15) // 16)


def _e8m0_fp8_of_block(v) -> int:
    amax = max(abs(float(e)) for e in v)
    if amax == 0.0:
        return 0
    _, k = math.frexp(amax)          # amax = f * 2**k with 0.5 <= f < 1
    return min(max((k - 1) - 8 + 127, 0), 254)


def _e4m3_codes(x, scale: float) -> np.ndarray:
    """Codes of the values x (one block) under one scale: the nearest finite
    E4M3 magnitude to |x| / scale, ties to the even code, plus the sign bit."""
    a = np.abs(np.asarray(x, dtype=np.float64)) / scale
    grid = np.asarray(E4M3_GRID)
    dist = np.abs(a[:, None] - grid[None, :])
    best = dist.min(axis=1, keepdims=True)
    tie_ok = dist == best
    # among the nearest (at most two adjacent codes) take the even one
    even = tie_ok & (np.arange(127)[None, :] % 2 == 0)
    code = np.where(even.any(axis=1), even.argmax(axis=1), tie_ok.argmax(axis=1))
    return (code | np.where(np.asarray(x) < 0, 0x80, 0)).astype(np.uint8)


def _bf16_bits(x) -> np.ndarray:
    """float64 -> bfloat16 bits, nearest with ties to even (via float32,
    exact for the float32 values the rows hold)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def kv_fp8_quantize(x, rope_dims: int) -> np.ndarray:
    """KV entries [..., D] (float values; the RoPE part must be float32
    values) -> packed rows uint8 [..., kv_fp8_row_bytes(D, R)] as above."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    R = rope_dims
    assert (D - R) % MX_BLOCK == 0 and 0 <= R <= D
    nb = (D - R) // MX_BLOCK
    rb = kv_fp8_row_bytes(D, R)
    flat = x.reshape(-1, D)
    out = np.zeros((flat.shape[0], rb), np.uint8)
    for r in range(flat.shape[0]):
        for blk in range(nb):
            v = flat[r, MX_BLOCK * blk: MX_BLOCK * (blk + 1)]
            s = _e8m0_fp8_of_block(v)
            out[r, D + R + blk] = s
            out[r, MX_BLOCK * blk: MX_BLOCK * (blk + 1)] = _e4m3_codes(v, 2.0 ** (s - 127))
        out[r, D - R: D + R] = _bf16_bits(flat[r, D - R:]).view(np.uint8)
    return out.reshape(x.shape[:-1] + (rb,))


def kv_fp8_dequantize(rows, D: int, rope_dims: int) -> np.ndarray:
    """Exact values (float64 [..., D]) of packed rows stored as above."""
    rows = np.asarray(rows, dtype=np.uint8)
    R = rope_dims
    nb = (D - R) // MX_BLOCK
    codes = rows[..., : D - R]
    mag = np.asarray(E4M3_GRID + (float("nan"),))[codes & 0x7F]
    val = np.where(codes & 0x80, -mag, mag)
    scale = np.repeat(np.exp2(rows[..., D + R: D + R + nb].astype(np.float64) - 127.0), MX_BLOCK,
                      axis=-1)
    bits = np.ascontiguousarray(rows[..., D - R: D + R]).view(np.uint16)
    rope = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.concatenate([val * scale, rope], axis=-1)


# ---------------------------------------------------------------------------
# Grouped low-rank output projection
# ---------------------------------------------------------------------------
def grouped_output_projection(o, w_a, w_b):
    """The attention output of one token mapped to the hidden size.

    [P2] section 3.3 (after eq. 26): the concatenated head outputs are too
    wide, so the heads are split into g groups; each group's outputs,
    concatenated, are projected to an intermediate vector, and the g
    intermediates, concatenated, are projected to the final attention
    output.  [P1] "What does layer 0 sliding-window attention do to p?" (the
    grouped W_O after the head concat; Flash: 64 heads in 8 groups) and [P4]
    "Arsitektur" (groups of heads -> a low rank per group -> hidden size).
    Group j holds heads j*H/g .. (j+1)*H/g - 1, in head order.

    o [H, D]; w_a [g, r, (H/g)*D] (group j's projection, one row per
    intermediate channel); w_b [d, g*r] -> float64 [d].
    """
    o = np.asarray(o, dtype=np.float64)
    w_a = np.asarray(w_a, dtype=np.float64)
    w_b = np.asarray(w_b, dtype=np.float64)
    H, D = o.shape
    g = w_a.shape[0]
    per = H // g
    mids = []
    for j in range(g):
        x_j = o[j * per:(j + 1) * per].reshape(-1)   # the group's heads, concatenated
        mids.append(w_a[j] @ x_j)
    return w_b @ np.concatenate(mids)
