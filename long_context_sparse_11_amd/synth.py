"""Seeded synthetic inputs for the CSA / HCA workloads.

This module draws random numbers and rounds them to bfloat16; it holds none
of the method's arithmetic, so both the GPU tests and the CPU oracle can be
fed from it.  Every array is generated in float32 with NumPy's PCG64 from its own stream,
``default_rng([seed, crc32(workload), crc32(array name)])``, so any subset of
a workload can be drawn without drawing the rest, then (for bf16 workloads)
rounded once to bfloat16, round-to-nearest-even; the float32 view of the
rounded values and the raw uint16 bits describe the same numbers.

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
  compress_stream
             bf16, the compressors alone over one 1,048,576-token sequence
             (KV entries 512 wide with RMSNorm + RoPE, indexer keys 128
             wide): 5.4 GiB of token streams, drawn on the device
  csa64k_fp4, csa1m_fp4
             as csa64k / csa1m with the indexer keys stored in MX FP4: code
             bytes drawn uniformly (every E2M1 code equally likely) and scale
             bytes uniformly from 125..127 (block scales 1/4, 1/2, 1), the
             heavy rows of csa1m_fp4 with scale bytes 2 higher (x4).  They
             are drawn as stored bytes: nothing here quantizes.
"""
from __future__ import annotations

import zlib

import numpy as np

FLASH = dict(H=64, D=512, R=64, Hi=64, Di=128, K=512, W=128)
# V4-Pro's attention and indexer ("DeepSeek-v4 Beyond Basics" section 3.2.2:
# m = 4, 64 indexer heads x 128, top-k 1024; section 3.3: 128 query heads x
# 512); RoPE and window as Flash (the page gives no other value)
PRO = dict(H=128, D=512, R=64, Hi=64, Di=128, K=1024, W=128)


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


def _rng(seed, workload, name):
    return np.random.default_rng([int(seed), zlib.crc32(workload.encode()), zlib.crc32(name.encode())])


class _Draw:
    """Per-array streams of one workload and seed."""

    def __init__(self, seed, workload):
        self.seed, self.workload = seed, workload

    def __call__(self, name, shape, std=1.0, mean=0.0):
        return _normal(_rng(self.seed, self.workload, name), shape, std, mean)

    def rng(self, name):
        return _rng(self.seed, self.workload, name)


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
    dr = _Draw(seed, "toy")
    T, H, D, R, Hi, Di, m, K, W = 256, 4, 64, 16, 4, 32, 4, 16, 16
    s = 1.0 / np.sqrt(D)
    si = 1.0 / np.sqrt(Di)
    d = dict(name="toy", dt="f32", B=1, T=T, Tq=T, H=H, D=D, R=R, Hi=Hi, Di=Di, m=m, K=K, W=W,
             N=T // m, q_pos0=np.array([0], np.int64), n_entries=np.array([T // m], np.int32),
             win_pos0=np.array([0], np.int64), base=10000.0, eps=1e-6)
    f = lambda n, shape, std=1.0: Tensor(dr(n, shape, std), "f32")
    d["q"] = f("q", (1, T, H, D), s)
    d["kv"] = f("kv", (1, T, D), s)
    for n in ("c_a", "c_b"):
        d[n] = f(n, (1, T, D), s)
    for n in ("z_a", "z_b"):
        d[n] = f(n, (1, T, D))
    d["bias_a"] = dr("bias_a", (m, D), 0.02)
    d["bias_b"] = dr("bias_b", (m, D), 0.02)
    d["gain"] = dr("gain", (D,), 0.02, 1.0)
    d["gain_win"] = dr("gain_win", (D,), 0.02, 1.0)
    for n in ("ic_a", "ic_b"):
        d[n] = f(n, (1, T, Di), si)
    for n in ("iz_a", "iz_b"):
        d[n] = f(n, (1, T, Di))
    d["ibias_a"] = dr("ibias_a", (m, Di), 0.02)
    d["ibias_b"] = dr("ibias_b", (m, Di), 0.02)
    d["q_idx"] = f("q_idx", (1, T, Hi, Di), si)
    d["w_idx"] = dr("w_idx", (1, T, Hi), 0.02)
    d["sink"] = dr("sink", (H,), 0.02)
    return d


DECODE = {  # m, batch, pool entries, heavy-tailed indexer keys
    "csa64k": (4, 4, 16384, False),
    "csa64k_pro": (4, 4, 16384, False),
    "csa1m": (4, 8, 262144, True),
    "hca1m": (128, 16, 8192, False),
    "csa64k_fp4": (4, 4, 16384, False),
    "csa1m_fp4": (4, 8, 262144, True),
}


def decode(kind: str, seed: int = 0, B: int | None = None, N: int | None = None,
           heavy_tail: bool | None = None, skip=()):
    """Decode-step inputs (one new query per sequence at the last position of
    a context of N*m tokens) for 'csa64k', 'csa1m', 'hca1m' or 'csa64k_pro'
    (V4-Pro shapes).  ``B`` / ``N``
    override batch and pool length for reduced-size cases; ``skip`` names
    arrays not to draw (e.g. the 2 GiB pool when only the indexer is tested).

    Pool and window rows are drawn directly (they stand for entries already
    normalised and rotated); the closing block's compressor streams are drawn
    separately so a step can run the compressor too.
    """
    dr = _Draw(seed, kind)
    F = PRO if kind.endswith("_pro") else FLASH
    H, D, R, Hi, Di, K, W = F["H"], F["D"], F["R"], F["Hi"], F["Di"], F["K"], F["W"]
    m, B0, N0, ht = DECODE[kind]
    B = B0 if B is None else B
    N = N0 if N is None else N
    ht = ht if heavy_tail is None else heavy_tail
    ctx = N * m
    d = dict(name=kind, dt="bf16", B=B, Tq=1, H=H, D=D, R=R, Hi=Hi, Di=Di, m=m, K=K, W=W,
             N=N, base=10000.0, eps=1e-6,
             q_pos0=np.full(B, ctx - 1, np.int64),
             n_entries=np.full(B, N, np.int32),
             win_pos0=np.full(B, ctx - W, np.int64),
             block_pos0=np.full(B, ctx - m, np.int64))

    def bf(name, shape, std=1.0):
        if name not in skip:
            d[name] = Tensor(dr(name, shape, std), "bf16")

    bf("q", (B, 1, H, D))
    bf("pool", (B, N, D))
    bf("win", (B, W, D))
    d["sink"] = dr("sink", (H,), 0.02)
    # closing block of the compressor (entry N-1): block i in stream a and,
    # for CSA, block i-1 in stream b (the overlap state)
    bf("c_a", (B, m, D))
    bf("z_a", (B, m, D))
    d["bias_a"] = dr("bias_a", (m, D), 0.02)
    d["gain"] = dr("gain", (D,), 0.02, 1.0)
    if kind == "hca1m":
        return d
    for n in ("c_b", "z_b", "prev_c_b", "prev_z_b"):
        bf(n, (B, m, D))
    d["bias_b"] = dr("bias_b", (m, D), 0.02)
    bf("q_idx", (B, 1, Hi, Di))
    d["w_idx"] = dr("w_idx", (B, 1, Hi), 0.02)
    if kind.endswith("_fp4"):
        if "k_idx" not in skip:
            d["k_codes"], d["k_scales"] = fp4_keys(dr, B, N, Di, ht)
    elif "k_idx" not in skip:
        kk = dr("k_idx", (B, N, Di))
        if ht:  # exactly floor(0.1 N) rows per sequence scaled by 4
            prng = dr.rng("heavy_rows")
            n_heavy = int(0.1 * N)
            for b in range(B):
                kk[b, prng.permutation(N)[:n_heavy]] *= np.float32(4.0)
        d["k_idx"] = Tensor(kk, "bf16")
    # indexer-key compressor streams of the closing block (Di wide)
    for n in ("ic_a", "iz_a", "ic_b", "iz_b", "iprev_c_b", "iprev_z_b"):
        bf(n, (B, m, Di))
    d["ibias_a"] = dr("ibias_a", (m, Di), 0.02)
    d["ibias_b"] = dr("ibias_b", (m, Di), 0.02)
    return d


def fp4_keys(dr, B, N, Di, heavy_tail):
    """MX FP4 indexer keys as stored bytes: codes [B, N, Di/2] uniform over
    all bytes, scale bytes [B, N, Di/32] uniform over 125..127; with
    ``heavy_tail`` exactly floor(0.1 N) rows per sequence get scale bytes 2
    higher (their values x4)."""
    codes = dr.rng("k_codes").integers(0, 256, size=(B, N, Di // 2), dtype=np.uint8)
    scales = dr.rng("k_scales").integers(125, 128, size=(B, N, Di // 32), dtype=np.uint8)
    if heavy_tail:
        prng = dr.rng("heavy_rows")
        n_heavy = int(0.1 * N)
        for b in range(B):
            scales[b, prng.permutation(N)[:n_heavy]] += np.uint8(2)
    return codes, scales


def swa_decode(seed: int = 0, B: int = 16, ctx: int = 1 << 20):
    """Sliding-window-only decode (the layers whose compression ratio is 0,
    "07 The Model", "The per-layer pattern"): each sequence's new token at
    position ctx - 1 attends to the raw window of the last W tokens and
    nothing else.  ``win`` holds window rows for tokens ctx - W .. ctx - 1;
    the last one is the new token's, which a step rebuilds from its KV row
    ``kv`` (m = 1: RMSNorm with the gain, RoPE at its position).  Shapes as
    the Flash decode workloads; no compressed entries (K = 0, N = 0)."""
    dr = _Draw(seed, "swa")
    F = FLASH
    H, D, R, W = F["H"], F["D"], F["R"], F["W"]
    d = dict(name="swa", dt="bf16", B=B, Tq=1, H=H, D=D, R=R, Hi=F["Hi"], Di=F["Di"], m=1, K=0,
             W=W, N=0, base=10000.0, eps=1e-6,
             q_pos0=np.full(B, ctx - 1, np.int64),
             n_entries=np.zeros(B, np.int32),
             win_pos0=np.full(B, ctx - W, np.int64))
    d["q"] = Tensor(dr("q", (B, 1, H, D)), "bf16")
    d["win"] = Tensor(dr("win", (B, W, D)), "bf16")
    d["kv"] = Tensor(dr("kv", (B, 1, D)), "bf16")
    d["gain"] = dr("gain", (D,), 0.02, 1.0)
    d["sink"] = dr("sink", (H,), 0.02)
    return d


def oproj(seed: int = 0, T: int = 4):
    """Grouped output projection after a decode step (Flash: 64 heads x 512
    in 8 groups, rank 1024 per group, hidden 4096): T tokens' attention
    outputs ~N(0, 1) and weights ~N(0, 1/fan_in), bf16."""
    dr = _Draw(seed, "oproj")
    F = FLASH
    H, D, G, r, dm = F["H"], F["D"], 8, 1024, 4096
    ka = (H // G) * D
    d = dict(name="oproj", dt="bf16", B=T, Tq=1, H=H, D=D, R=F["R"], Hi=F["Hi"], Di=F["Di"],
             m=1, K=0, W=0, G=G, r=r, d_model=dm)
    d["o"] = Tensor(dr("o", (T, H, D)), "bf16")
    d["w_a"] = Tensor(dr("w_a", (G, r, ka), 1.0 / np.sqrt(ka)), "bf16")
    d["w_b"] = Tensor(dr("w_b", (dm, G * r), 1.0 / np.sqrt(G * r)), "bf16")
    return d


def prefill(seed: int = 0, Tq: int = 4096, prefix: int = 15360, skip=()):
    """CSA chunked prefill: ``Tq`` new tokens after a cached prefix of
    ``prefix`` entries (m = 4).  The chunk's compressor streams carry m extra
    leading rows: the previous block's b-stream (overlap state)."""
    dr = _Draw(seed, "prefill")
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

    def bf(name, shape, std=1.0):
        if name not in skip:
            d[name] = Tensor(dr(name, shape, std), "bf16")

    bf("pool_prefix", (1, prefix, D))
    bf("kidx_prefix", (1, prefix, Di))
    for name, width in (("c_a", D), ("z_a", D), ("c_b", D), ("z_b", D),
                        ("ic_a", Di), ("iz_a", Di), ("ic_b", Di), ("iz_b", Di)):
        bf(name, (1, Tq + m, width))
    d["bias_a"] = dr("bias_a", (m, D), 0.02)
    d["bias_b"] = dr("bias_b", (m, D), 0.02)
    d["ibias_a"] = dr("ibias_a", (m, Di), 0.02)
    d["ibias_b"] = dr("ibias_b", (m, Di), 0.02)
    d["gain"] = dr("gain", (D,), 0.02, 1.0)
    bf("win", (1, L_win, D))
    bf("q", (1, Tq, H, D))
    bf("q_idx", (1, Tq, Hi, Di))
    d["w_idx"] = dr("w_idx", (1, Tq, Hi), 0.02)
    d["sink"] = dr("sink", (H,), 0.02)
    return d


def compress_stream(seed: int = 0, T: int = 1 << 20, device: str = "cuda"):
    """The compressors alone over one long sequence (a prefill's compressor
    pass, or the standalone streaming measurement): T tokens from position 0,
    the KV compressor (D = 512, overlap, RMSNorm gain, RoPE 64) and the
    indexer-key compressor (Di = 128, overlap) over the same blocks.  The
    eight token streams [1, T, D] / [1, T, Di] (5.4 GiB at T = 2^20) are drawn
    on the device, N(0, 1) in bfloat16 from torch's generator seeded with
    (seed, crc32 of the stream name): a host draw of that size would take
    minutes.  Biases and gain follow the host recipe (N(0, 0.02), 1 +
    N(0, 0.02)).  ``device=None`` skips the streams (their parameters only)."""
    dr = _Draw(seed, "compress_stream")
    F = FLASH
    D, R, Di, m = F["D"], F["R"], F["Di"], 4
    d = dict(name="compress_stream", dt="bf16", B=1, Tq=T, T=T, H=F["H"], D=D, R=R, Hi=F["Hi"],
             Di=Di, m=m, K=F["K"], W=F["W"], N=T // m, base=10000.0, eps=1e-6,
             pos0=np.array([0], np.int64))
    d["bias_a"] = dr("bias_a", (m, D), 0.02)
    d["bias_b"] = dr("bias_b", (m, D), 0.02)
    d["gain"] = dr("gain", (D,), 0.02, 1.0)
    d["ibias_a"] = dr("ibias_a", (m, Di), 0.02)
    d["ibias_b"] = dr("ibias_b", (m, Di), 0.02)
    if device is None:
        return d
    import torch
    for name, width in (("c_a", D), ("z_a", D), ("c_b", D), ("z_b", D),
                        ("ic_a", Di), ("iz_a", Di), ("ic_b", Di), ("iz_b", Di)):
        g = torch.Generator(device=device)
        g.manual_seed(int(seed) * 1000003 + zlib.crc32(name.encode()))
        d[name] = torch.randn((1, T, width), generator=g, device=device, dtype=torch.bfloat16)
    return d
