"""Seeded synthetic inputs for the CSA / HCA workloads.

This module draws random numbers and rounds them to bfloat16; it holds none
of the method's arithmetic, so both the GPU tests and the CPU oracle can be
fed from it.  Every array is generated in float32 with NumPy's PCG64
(``default_rng(seed)``) in a fixed order, then (for bf16 workloads) rounded
once to bfloat16, round-to-nearest-even; the float32 view of the rounded
values and the raw uint16 bits describe the same numbers.

Workloads (shapes after DeepSeek-V4-Flash: 64 query heads x head_dim 512, one
shared K=V head, RoPE on the last 64 channels, indexer 64 heads x 128, top-k
512, window 128, CSA m = 4, HCA m' = 128):

  toy        fp32, T=256 causal tokens, 4 heads x 64 (RoPE 16), indexer 4 x 32,
             top-k 16, window 16, m = 4 -> pool 64
  csa64k     bf16, CSA decode, batch 4, one query each at position 65,535,
             16,384 pool entries
  prefill    bf16, CSA chunked prefill, batch 1, 4,096 queries at positions
             61,440 .. 65,535 (compressor over the chunk; 15,360-entry prefix)
  hca1m      bf16, HCA decode, batch 16 at position 1,048,575, 8,192 entries
  csa1m      bf16, CSA decode, batch 8 at position 1,048,575, 262,144 entries,
             indexer keys with 10% of rows scaled by 4 (heavy-tailed mixture)
"""
from __future__ import annotations

import numpy as np

FLASH = dict(H=64, D=512, R=64, Hi=64, Di=128, K=512, W=128)


# ---------------------------------------------------------------------------
# bfloat16 rounding (round to nearest even) of float32 inputs
# ---------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> uint16 bfloat16 bits, round-to-nearest-even (no NaNs here)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class Tensor:
    """A host array with its storage type: 'f32' keeps float32, 'bf16' keeps
    the uint16 bits; ``.f32`` gives the float32 values (computed on first use
    for bf16, so multi-GiB pools are not held twice unless asked for)."""

    def __init__(self, values: np.ndarray, dt: str):
        self.dt = dt
        self._f32 = None
        if dt == "bf16":
            self.bits = bf16_bits(values)
        else:
            self.bits = None
            self._f32 = np.ascontiguousarray(values, dtype=np.float32)

    @property
    def f32(self) -> np.ndarray:
        if self._f32 is None:
            self._f32 = bf16_to_f32(self.bits)
        return self._f32

    @property
    def shape(self):
        return self.bits.shape if self.dt == "bf16" else self._f32.shape

    @property
    def storage(self) -> np.ndarray:
        return self.bits if self.dt == "bf16" else self._f32


def _normal(rng, shape, std=1.0, mean=0.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------
def toy(seed: int = 0):
    """Toy CSA layer in fp32: every stream a full causal prefill of 256 tokens."""
    rng = np.random.default_rng(seed)
    T, H, D, R, Hi, Di, m, K, W = 256, 4, 64, 16, 4, 32, 4, 16, 16
    s = 1.0 / np.sqrt(D)
    si = 1.0 / np.sqrt(Di)
    d = dict(name="toy", dt="f32", B=1, T=T, Tq=T, H=H, D=D, R=R, Hi=Hi, Di=Di, m=m, K=K, W=W,
             q_pos0=np.array([0], np.int64), base=10000.0, eps=1e-6)
    d["q"] = Tensor(_normal(rng, (1, T, H, D), s), "f32")
    d["kv"] = Tensor(_normal(rng, (1, T, D), s), "f32")
    d["c_a"] = Tensor(_normal(rng, (1, T, D), s), "f32")
    d["c_b"] = Tensor(_normal(rng, (1, T, D), s), "f32")
    d["z_a"] = Tensor(_normal(rng, (1, T, D)), "f32")
    d["z_b"] = Tensor(_normal(rng, (1, T, D)), "f32")
    d["bias_a"] = _normal(rng, (m, D), 0.02)
    d["bias_b"] = _normal(rng, (m, D), 0.02)
    d["gain"] = _normal(rng, (D,), 0.02, 1.0)
    d["gain_win"] = _normal(rng, (D,), 0.02, 1.0)
    d["ic_a"] = Tensor(_normal(rng, (1, T, Di), si), "f32")
    d["ic_b"] = Tensor(_normal(rng, (1, T, Di), si), "f32")
    d["iz_a"] = Tensor(_normal(rng, (1, T, Di)), "f32")
    d["iz_b"] = Tensor(_normal(rng, (1, T, Di)), "f32")
    d["ibias_a"] = _normal(rng, (m, Di), 0.02)
    d["ibias_b"] = _normal(rng, (m, Di), 0.02)
    d["q_idx"] = Tensor(_normal(rng, (1, T, Hi, Di), si), "f32")
    d["w_idx"] = _normal(rng, (1, T, Hi), 0.02)
    d["sink"] = _normal(rng, (H,), 0.02)
    return d


def decode(kind: str, seed: int = 0, B: int | None = None, N: int | None = None,
           heavy_tail: bool | None = None):
    """Decode-step inputs (one new query per sequence) for 'csa64k', 'csa1m'
    or 'hca1m'.  ``B`` / ``N`` override the batch and the pool length for
    reduced-size parity cases; positions then follow from ``N``.

    The pool and window rows are drawn directly (they stand for already
    normalised, rotated entries); the closing block's compressor streams are
    drawn separately so the step can run the compressor too.
    """
    rng = np.random.default_rng(seed)
    F = FLASH
    H, D, R, Hi, Di, K, W = F["H"], F["D"], F["R"], F["Hi"], F["Di"], F["K"], F["W"]
    if kind == "csa64k":
        m, B0, N0, ht = 4, 4, 16384, False
    elif kind == "csa1m":
        m, B0, N0, ht = 4, 8, 262144, True
    elif kind == "hca1m":
        m, B0, N0, ht = 128, 16, 8192, False
    else:
        raise ValueError(kind)
    B = B0 if B is None else B
    N = N0 if N is None else N
    ht = ht if heavy_tail is None else heavy_tail
    ctx = N * m
    t = ctx - 1
    d = dict(name=kind, dt="bf16", B=B, Tq=1, H=H, D=D, R=R, Hi=Hi, Di=Di, m=m, K=K, W=W,
             N=N, base=10000.0, eps=1e-6,
             q_pos0=np.full(B, t, np.int64),
             n_entries=np.full(B, N, np.int32),
             win_pos0=np.full(B, ctx - W, np.int64),
             block_pos0=np.full(B, ctx - m, np.int64))
    d["q"] = Tensor(_normal(rng, (B, 1, H, D)), "bf16")
    d["pool"] = Tensor(_normal(rng, (B, N, D)), "bf16")
    d["win"] = Tensor(_normal(rng, (B, W, D)), "bf16")
    d["sink"] = _normal(rng, (H,), 0.02)
    # closing block of the compressor (entry N-1): block i (stream a) and,
    # for CSA, block i-1 (stream b) as the overlap state
    d["c_a"] = Tensor(_normal(rng, (B, m, D)), "bf16")
    d["z_a"] = Tensor(_normal(rng, (B, m, D)), "bf16")
    d["bias_a"] = _normal(rng, (m, D), 0.02)
    d["gain"] = _normal(rng, (D,), 0.02, 1.0)
    if kind != "hca1m":
        d["c_b"] = Tensor(_normal(rng, (B, m, D)), "bf16")
        d["z_b"] = Tensor(_normal(rng, (B, m, D)), "bf16")
        d["prev_c_b"] = Tensor(_normal(rng, (B, m, D)), "bf16")
        d["prev_z_b"] = Tensor(_normal(rng, (B, m, D)), "bf16")
        d["bias_b"] = _normal(rng, (m, D), 0.02)
        d["q_idx"] = Tensor(_normal(rng, (B, 1, Hi, Di)), "bf16")
        d["w_idx"] = _normal(rng, (B, 1, Hi), 0.02)
        kk = _normal(rng, (B, N, Di))
        if ht:
            n_heavy = int(0.1 * N)
            for b in range(B):
                rows = rng.permutation(N)[:n_heavy]
                kk[b, rows] *= np.float32(4.0)
        d["k_idx"] = Tensor(kk, "bf16")
        # indexer-key compressor streams for the closing block (Di wide)
        d["ic_a"] = Tensor(_normal(rng, (B, m, Di)), "bf16")
        d["iz_a"] = Tensor(_normal(rng, (B, m, Di)), "bf16")
        d["ic_b"] = Tensor(_normal(rng, (B, m, Di)), "bf16")
        d["iz_b"] = Tensor(_normal(rng, (B, m, Di)), "bf16")
        d["iprev_c_b"] = Tensor(_normal(rng, (B, m, Di)), "bf16")
        d["iprev_z_b"] = Tensor(_normal(rng, (B, m, Di)), "bf16")
        d["ibias_a"] = _normal(rng, (m, Di), 0.02)
        d["ibias_b"] = _normal(rng, (m, Di), 0.02)
    return d


def prefill(seed: int = 0, Tq: int = 4096, prefix: int = 15360):
    """CSA chunked prefill: ``Tq`` new tokens after a cached prefix of
    ``prefix`` entries (m = 4).  The chunk's compressor streams carry 4 extra
    leading rows: the previous block's b-stream (overlap state)."""
    rng = np.random.default_rng(seed)
    F = FLASH
    H, D, R, Hi, Di, K, W = F["H"], F["D"], F["R"], F["Hi"], F["Di"], F["K"], F["W"]
    m = 4
    p0 = prefix * m
    N = prefix + Tq // m
    L_win = Tq + W - 1
    d = dict(name="prefill", dt="bf16", B=1, Tq=Tq, H=H, D=D, R=R, Hi=Hi, Di=Di, m=m, K=K, W=W,
             N=N, prefix=prefix, base=10000.0, eps=1e-6,
             q_pos0=np.array([p0], np.int64), n_entries=np.array([N], np.int32),
             win_pos0=np.array([p0 - W + 1], np.int64), chunk_pos0=np.array([p0], np.int64))
    d["pool_prefix"] = Tensor(_normal(rng, (1, prefix, D)), "bf16")
    d["kidx_prefix"] = Tensor(_normal(rng, (1, prefix, Di)), "bf16")
    for name, width in (("c_a", D), ("z_a", D), ("c_b", D), ("z_b", D),
                        ("ic_a", Di), ("iz_a", Di), ("ic_b", Di), ("iz_b", Di)):
        d[name] = Tensor(_normal(rng, (1, Tq + m, width)), "bf16")
    d["bias_a"] = _normal(rng, (m, D), 0.02)
    d["bias_b"] = _normal(rng, (m, D), 0.02)
    d["ibias_a"] = _normal(rng, (m, Di), 0.02)
    d["ibias_b"] = _normal(rng, (m, Di), 0.02)
    d["gain"] = _normal(rng, (D,), 0.02, 1.0)
    d["win"] = Tensor(_normal(rng, (1, L_win, D)), "bf16")
    d["q"] = Tensor(_normal(rng, (1, Tq, H, D)), "bf16")
    d["q_idx"] = Tensor(_normal(rng, (1, Tq, Hi, Di)), "bf16")
    d["w_idx"] = _normal(rng, (1, Tq, Hi), 0.02)
    d["sink"] = _normal(rng, (H,), 0.02)
    return d
