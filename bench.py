"""Benchmark of one decode step of DeepSeek-V4 Compressed Sparse Attention on
one MI355X.

Default workload (the headline metric's configuration): CSA decode, batch 4,
one new query per sequence at context 65,536 (16,384 compressed entries),
64 heads x 512, RoPE 64, indexer 64 x 128, top-k 512, window 128.  A step is
the whole hot path for that batch: compress the closing block (KV entry and
indexer key, written in place into the caches; one launch with the indexer
scoring), lightning-indexer scores + top-512 selection, sparse gather
attention with the sink.  Other workloads
(--workload): csa1m (batch 8, context 1,048,576), hca1m (HCA decode, batch
16, context 1,048,576: one hca_decode_attn call, the closing block's entry
and the attention), prefill (CSA chunk of 4,096
queries on a 61,440-token prefix), csa64k_pro (V4-Pro attention: 128 heads,
top-1024), csa64k_fp4 / csa1m_fp4 (as csa64k / csa1m with the indexer keys
stored in MX FP4; the fresh key is quantized inside the step), swa
(sliding-window-only layers, batch 16: one swa_decode_attn call, the new
token's window row and the attention over the 128-token window alone), oproj (the grouped low-rank output
projection of the csa64k batch's 4 tokens: 64 heads in 8 groups -> 8 x 1024
-> 4096), csa64k_stream (the csa64k step as a streaming loop: positions and
entry counts advanced on the device, the new token's window row written into
a ring by the indexer launch, a block closing every 4th step), oproj_prefill (the same projection for a 4,096-token prefill chunk: a
tiled GEMM).

Timing: inputs resident in HBM; the step is captured once per input copy in
a HIP graph and replayed; enough copies of the inputs are rotated that no
step finds its data in the 256 MB Infinity Cache.  Warmup steps are untimed,
then exactly --steps steps are timed, bracketed by device synchronisation.
Per-call durations come from HIP events on the library's stream.  The CPU
oracle is timed on a bounded sample of the same workload (rank 0, N = 1).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA/HCA attention decode tokens/s at 64K & 1M ctx; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
CAL_BYTES = 512 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="csa64k",
                   choices=["csa64k", "csa1m", "hca1m", "prefill", "csa64k_pro", "csa64k_fp4",
                            "csa1m_fp4", "swa", "oproj", "oproj_prefill", "csa64k_stream",
                            "compress_stream", "csa64k_fp8", "csa1m_fp8", "hca1m_fp8"])
    p.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graph replay")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-oracle sample budget")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--only", action="store_true",
                   help="measure the named workload alone (the default csa64k run also measures "
                        "the 1M-context decodes, csa1m and hca1m)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# workload setup
# ---------------------------------------------------------------------------
CSA_DECODE = ("csa64k", "csa1m", "csa64k_pro", "csa64k_fp4", "csa1m_fp4", "csa64k_stream",
              "csa64k_fp8", "csa1m_fp8")
# KV pools stored as packed mixed BF16 / FP8 rows (the pool is quantized on
# the device once, before timing)
KV_FP8 = ("csa64k_fp8", "csa1m_fp8", "hca1m_fp8")
HCA = ("hca1m", "hca1m_fp8")
# a streaming run starts this many entries below the 16,384-entry cache (a
# block closes every 4th step, so 2,048 steps fit before the cache is full)
STREAM_HEADROOM = 512


def upload(d, torch):
    from long_context_sparse_11_amd.device import to_device
    out = {}
    for k, v in d.items():
        if isinstance(v, torch.Tensor):   # drawn on the device already
            out[k] = v
        elif hasattr(v, "storage") or isinstance(v, np.ndarray):
            out[k] = to_device(v)
        else:
            out[k] = v
    return out


class Step:
    """Buffers of one input copy plus the closure that runs one step."""

    def __init__(self, kind, g, L, torch):
        self.kind, self.g, self.L, self.torch = kind, g, L, torch
        self._cws = {}
        B, D, m = g["B"], g["D"], g["m"]
        self.B = B
        if kind in CSA_DECODE:
            N, K, W = g["N"], g["K"], g["W"]
            self.idx = torch.empty((B, 1, K), dtype=torch.int32, device="cuda")
            self.out = torch.empty_like(g["q"])
            self.ws_i = torch.empty(L.csa_index_topk_ws_bytes(B, 1, g["Hi"], N, K),
                                    dtype=torch.uint8, device="cuda")
            n = L.csa_attn_ws_bytes(B, 1, g["H"], D, K + W)
            self.ws_a = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
            if kind == "csa64k_stream":
                # device state of the loop: the first step is token 4 n - 1
                n0 = N - STREAM_HEADROOM
                self.q_pos = torch.full((B,), 4 * n0 - 2, dtype=torch.int64, device="cuda")
                self.n_ent = torch.full((B,), n0 - 1, dtype=torch.int32, device="cuda")
                self.blk = torch.full((B,), -1, dtype=torch.int64, device="cuda")
                self.kv = g["c_a"][:, :1].contiguous()
        elif kind in ("oproj", "oproj_prefill"):
            T = g["B"]
            self.out = torch.empty((T, g["d_model"]), dtype=torch.bfloat16, device="cuda")
            self.mid = torch.empty((T, g["G"] * g["r"]), dtype=torch.bfloat16, device="cuda")
        elif kind == "swa":
            W = g["W"]
            self.out = torch.empty_like(g["q"])
            n = L.swa_decode_attn_ws_bytes(B, g["H"], D, W)
            self.ws_a = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
        elif kind == "compress_stream":
            self.pool = torch.empty((B, g["N"], D), dtype=torch.bfloat16, device="cuda")
            self.keys = torch.empty((B, g["N"], g["Di"]), dtype=torch.bfloat16, device="cuda")
        elif kind in HCA:
            N, W = g["N"], g["W"]
            self.out = torch.empty_like(g["q"])
            n = L.hca_decode_attn_ws_bytes(B, g["H"], D, N + W)
            self.ws_a = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
        else:  # prefill
            Tq, N, K, W = g["Tq"], g["N"], g["K"], g["W"]
            self.idx = torch.empty((1, Tq, K), dtype=torch.int32, device="cuda")
            self.out = torch.empty_like(g["q"])
            self.ws_i = torch.empty(L.csa_index_topk_ws_bytes(1, Tq, g["Hi"], N, K), dtype=torch.uint8,
                                    device="cuda")
            n = L.csa_attn_ws_bytes(1, Tq, g["H"], D, K + W)
            self.ws_a = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")

    def cws(self, c, m, overlap=True):
        """Preallocated compressor workspace for stream tensor c [B, T, D]."""
        key = (tuple(c.shape), m, overlap)
        if key not in self._cws:
            B, T, D = c.shape
            n = self.L.csa_compress_ws_bytes(1, B, T, D, m, overlap)
            self._cws[key] = self.torch.empty(max(n, 1), dtype=self.torch.uint8, device="cuda")
        return self._cws[key]

    def dominant(self):
        """(name, thunk) of the unit that carries most of the step's
        algorithmic bytes (flops for prefill), launched exactly as inside the
        step: for CSA decode the fused launch of the closing block's
        compressors and the indexer scoring (csa_decode_index_scores: the
        step's first launch without the selection that follows it); for
        prefill the indexer scoring kernel (csa_index_scores launches the
        step's index_prefill grid); for HCA and window-only decode the
        attention call; for the output projection its call."""
        g, L = self.g, self.L
        if self.kind in HCA or self.kind == "swa":
            return self.calls()[-1]
        if self.kind in ("oproj", "oproj_prefill", "compress_stream"):
            return self.calls()[0]
        if not hasattr(self, "scores"):
            B, Tq, N = g["B"], g["Tq"], g["N"]
            self.scores = self.torch.empty((B, Tq, N), dtype=self.torch.float32, device="cuda")
        if self.kind == "prefill":
            return ("index_scores", lambda: L.csa_index_scores(
                g["q_idx"], g["w_idx"], g["k_idx"], g["n_entries"], g["q_pos0"], g["m"],
                out=self.scores))
        if self.kind == "csa64k_stream":
            return ("index_decode_fresh", lambda: L.csa_decode_index_scores(
                g["q_idx"], g["w_idx"], self.n_ent, self.q_pos, g["m"], self.stream_jobs(),
                block_pos0=self.blk, out=self.scores))
        if self.kind.endswith("_fp4"):
            return ("index_decode_fresh", lambda: L.csa_decode_index_scores_mxfp4(
                g["q_idx"], g["w_idx"], g["k_codes"], g["k_scales"], g["n_entries"], g["q_pos0"],
                g["m"], self.decode_jobs(fp4=True), block_pos0=g["block_pos0"], out=self.scores))
        return ("index_decode_fresh", lambda: L.csa_decode_index_scores(
            g["q_idx"], g["w_idx"], g["n_entries"], g["q_pos0"], g["m"], self.decode_jobs(),
            block_pos0=g["block_pos0"], out=self.scores))

    def decode_jobs(self, fp4=False):
        """The closing block's compressor jobs of a CSA decode step: the
        indexer key (into k_idx, or quantized into the FP4 caches) and the KV
        entry, both to row n_entries - 1 of their pools."""
        g = self.g
        key = dict(c_a=g["ic_a"], z_a=g["iz_a"], c_b=g["ic_b"], z_b=g["iz_b"],
                   prev_c_b=g["iprev_c_b"], prev_z_b=g["iprev_z_b"], bias_a=g["ibias_a"],
                   bias_b=g["ibias_b"])
        if not fp4:
            key["out"] = g["k_idx"]
        kv = dict(c_a=g["c_a"], z_a=g["z_a"], c_b=g["c_b"], z_b=g["z_b"], prev_c_b=g["prev_c_b"],
                  prev_z_b=g["prev_z_b"], bias_a=g["bias_a"], bias_b=g["bias_b"], gain=g["gain"],
                  rope_dims=g["R"], out=g["pool"], out_kv_fp8=self.kind in KV_FP8)
        return [key, kv]

    def stream_jobs(self):
        """The streaming step's jobs: key and KV entries of a closing block
        and the token's window row (third job, written to its ring slot)."""
        g = self.g
        return self.decode_jobs() + [dict(c_a=self.kv, gain=g["gain"], rope_dims=g["R"],
                                          out=g["win"])]

    def calls(self):
        """The step as a list of (name, thunk) library calls."""
        g, L = self.g, self.L
        kind = self.kind
        if kind in CSA_DECODE:
            N, m = g["N"], g["m"]
            pool = g["pool"]
            attn_fn = L.csa_sparse_attn_kvfp8 if kind in KV_FP8 else L.csa_sparse_attn
            attn = ("sparse_attn", lambda: attn_fn(g["q"], pool, self.idx, g["win"],
                                                   g["win_pos0"], g["W"], g["sink"],
                                                   g["q_pos0"], rope_dims=g["R"],
                                                   out=self.out, ws=self.ws_a))
            if kind == "csa64k_stream":
                # the key and KV entries of a closing block and the token's
                # window row (third job, written to its ring slot) in the
                # indexer launch
                st = self.stream_jobs()
                return [
                    ("advance", lambda: L.csa_decode_advance(self.q_pos, self.n_ent, self.blk,
                                                             m, N)),
                    ("compress_index_topk", lambda: L.csa_decode_index_topk(
                        g["q_idx"], g["w_idx"], self.n_ent, self.q_pos, g["K"], m, st,
                        block_pos0=self.blk, ws=self.ws_i, idx_out=self.idx)),
                    ("sparse_attn", lambda: L.csa_sparse_attn(g["q"], pool, self.idx, g["win"],
                                                              None, g["W"], g["sink"],
                                                              self.q_pos, rope_dims=g["R"],
                                                              out=self.out, ws=self.ws_a)),
                ]
            if kind.endswith("_fp4"):
                # indexer keys stored in MX FP4: the fresh key is quantized
                # by the fused launch into row n_entries - 1
                jobs = self.decode_jobs(fp4=True)
                return [("compress_index_topk", lambda: L.csa_decode_index_topk_mxfp4(
                    g["q_idx"], g["w_idx"], g["k_codes"], g["k_scales"], g["n_entries"],
                    g["q_pos0"], g["K"], m, jobs, block_pos0=g["block_pos0"],
                    ws=self.ws_i, idx_out=self.idx)), attn]
            jobs = self.decode_jobs()
            return [
                # the indexer key and the KV entry of the closing block (row
                # n_entries - 1 of their pools; a packed FP8 row for the _fp8
                # workloads), then the indexer top-K: the compressors run
                # inside the indexer launch
                ("compress_index_topk", lambda: L.csa_decode_index_topk(
                    g["q_idx"], g["w_idx"], g["n_entries"], g["q_pos0"], g["K"], m, jobs,
                    block_pos0=g["block_pos0"], ws=self.ws_i, idx_out=self.idx)),
                attn,
            ]
        if kind in ("oproj", "oproj_prefill"):
            return [("output_proj", lambda: L.csa_output_proj(g["o"], g["w_a"], g["w_b"],
                                                              mid=self.mid, out=self.out))]
        if kind == "compress_stream":
            # both compressors over the whole sequence, one launch
            jobs = [dict(c_a=g["c_a"], z_a=g["z_a"], c_b=g["c_b"], z_b=g["z_b"],
                         bias_a=g["bias_a"], bias_b=g["bias_b"], gain=g["gain"],
                         rope_dims=g["R"], out=self.pool),
                    dict(c_a=g["ic_a"], z_a=g["iz_a"], c_b=g["ic_b"], z_b=g["iz_b"],
                         bias_a=g["ibias_a"], bias_b=g["ibias_b"], out=self.keys)]
            return [("compress", lambda: L.csa_compress_batch(jobs, g["m"], pos0=g["pos0"]))]
        if kind == "swa":
            # one call: the new token's window row (m = 1), written over the
            # last row of the window by the attention launch's last split,
            # and the attention over the window alone
            W, win = g["W"], g["win"]
            return [
                ("swa_step", lambda: L.swa_decode_attn(g["q"], g["kv"], g["gain"], win,
                                                       g["win_pos0"], W, g["sink"], g["q_pos0"],
                                                       rope_dims=g["R"], out=self.out,
                                                       ws=self.ws_a)),
            ]
        if kind in HCA:
            # one call: the closing block's entry (pooled by the attention
            # launch's last split, stored to row N - 1: bf16, or a packed
            # BF16 / FP8 row) and the attention
            m, pool = g["m"], g["pool"]
            fn = L.hca_decode_attn_kvfp8 if kind == "hca1m_fp8" else L.hca_decode_attn
            return [
                ("hca_step", lambda: fn(
                    g["q"], pool, g["n_entries"], m, g["c_a"], g["z_a"], g["bias_a"], g["gain"],
                    g["block_pos0"], g["win"], g["win_pos0"], g["W"], g["sink"], g["q_pos0"],
                    rope_dims=g["R"], out=self.out, ws=self.ws_a)),
            ]
        # prefill
        N, D, Di, m, P = g["N"], g["D"], g["Di"], g["m"], g["prefix"]
        pool, kidx = g["pool"], g["k_idx"]
        return [
            # the chunk's KV entries and indexer keys, one launch
            ("compress", lambda: L.csa_compress_batch([
                dict(c_a=g["c_a"][:, m:], z_a=g["z_a"][:, m:], c_b=g["c_b"][:, m:],
                     z_b=g["z_b"][:, m:], prev_c_b=g["c_b"][:, :m], prev_z_b=g["z_b"][:, :m],
                     bias_a=g["bias_a"], bias_b=g["bias_b"], gain=g["gain"], rope_dims=g["R"],
                     out=pool[:, P:], out_bstride=N * D),
                dict(c_a=g["ic_a"][:, m:], z_a=g["iz_a"][:, m:], c_b=g["ic_b"][:, m:],
                     z_b=g["iz_b"][:, m:], prev_c_b=g["ic_b"][:, :m], prev_z_b=g["iz_b"][:, :m],
                     bias_a=g["ibias_a"], bias_b=g["ibias_b"], out=kidx[:, P:],
                     out_bstride=N * Di)],
                m, pos0=g["chunk_pos0"])),
            ("index_topk", lambda: L.csa_index_topk(g["q_idx"], g["w_idx"], kidx, g["n_entries"],
                                                    g["q_pos0"], g["K"], m, ws=self.ws_i,
                                                    idx_out=self.idx)),
            ("sparse_attn", lambda: L.csa_sparse_attn(g["q"], pool, self.idx, g["win"],
                                                      g["win_pos0"], g["W"], g["sink"],
                                                      g["q_pos0"], rope_dims=g["R"], out=self.out,
                                                      ws=self.ws_a)),
        ]


def make_inputs(kind):
    from long_context_sparse_11_amd import synth
    if kind == "prefill":
        d = synth.prefill(0)
    elif kind == "swa":
        d = synth.swa_decode(0)
    elif kind == "oproj":
        d = synth.oproj(0)
    elif kind == "oproj_prefill":
        d = synth.oproj(0, T=4096)
    elif kind == "compress_stream":
        d = synth.compress_stream(0)
    elif kind in KV_FP8:
        # the bf16 workload's inputs; its pool is quantized on the device
        d = synth.decode(kind[:-4], 0)
        d["name"] = kind
    elif kind == "csa64k_stream":
        # the 64K caches; the loop itself starts STREAM_HEADROOM entries lower
        d = synth.decode("csa64k", 0)
        d["name"] = kind
    else:
        d = synth.decode(kind, 0)
    return d


def prefill_buffers(g, torch):
    """Pool / key caches of the prefill workload: cached prefix + room for the chunk."""
    B, P, N, D, Di = 1, g["prefix"], g["N"], g["D"], g["Di"]
    pool = torch.empty((B, N, D), dtype=torch.bfloat16, device="cuda")
    pool[:, :P] = g.pop("pool_prefix")
    kidx = torch.empty((B, N, Di), dtype=torch.bfloat16, device="cuda")
    kidx[:, :P] = g.pop("kidx_prefix")
    g["pool"], g["k_idx"] = pool, kidx


# ---------------------------------------------------------------------------
# algorithmic work per step (what the method must move / compute)
# ---------------------------------------------------------------------------
def algorithmic(kind, d):
    H, D, Hi, Di, K, W, m = d["H"], d["D"], d["Hi"], d["Di"], d["K"], d["W"], d["m"]
    B, Tq = d["B"], d["Tq"]
    bf = 2
    out = {}
    # bytes of one stored KV entry: bf16, or a packed mixed BF16 / FP8 row
    R = d["R"]
    vb = (D - R) + 2 * R + 16 * (((D - R) // 32 + 15) // 16) if kind in KV_FP8 else D * bf
    if kind in CSA_DECODE:
        N = d["N"]
        # bytes of one stored indexer key: bf16, or MX FP4 codes + scale bytes
        kb = Di // 2 + Di // 32 if kind.endswith("_fp4") else Di * bf
        comp = B * ((4 * m) * D * bf + vb + (4 * m) * Di * bf + kb)
        idx_bytes = B * (N * kb + Hi * Di * bf + Hi * 4 + K * 4)
        # the step's first launch without the selection: the closing block's
        # compressors (their streams in, the two entries out) and the scoring
        # (visible keys, query heads and weights)
        out["index_decode_fresh"] = {"bytes": comp + B * (N * kb + Hi * Di * bf + Hi * 4),
                                     "flops": B * 2 * Hi * Di * N}
        rows = min(K, N) + W
        attn_bytes = B * (min(K, N) * vb + W * D * bf + 2 * H * D * bf + K * 4)
        out["bytes"] = {"compress_index_topk": comp + idx_bytes, "sparse_attn": attn_bytes}
        out["flops"] = {"compress_index_topk": B * 2 * Hi * Di * N,
                        "sparse_attn": B * 4 * H * D * rows}
    elif kind in ("oproj", "oproj_prefill"):
        G, r, dm = d["G"], d["r"], d["d_model"]
        ka = (H // G) * D
        # both weights once, the tokens' outputs in, the intermediates out and
        # back in, the projected tokens out
        byt = (G * r * ka + dm * G * r) * bf + B * (H * D + 2 * G * r + dm) * bf
        fl = 2 * B * (G * r * ka + dm * G * r)
        out["bytes"] = {"output_proj": byt}
        out["flops"] = {"output_proj": fl}
        out["output_proj"] = {"bytes": byt, "flops": fl}
    elif kind == "compress_stream":
        T, N = d["T"], d["N"]
        # four token streams of each compressor in, the entries out
        byt = 4 * T * (D + Di) * bf + N * (D + Di) * bf
        out["bytes"] = {"compress": byt}
        out["flops"] = {}
        out["compress"] = {"bytes": byt, "flops": 0}
    elif kind == "swa":
        # the token's kv row in and its window row out, then the window, the
        # query and the output (one call does both)
        byt = B * 2 * D * bf + B * (W * D * bf + 2 * H * D * bf)
        fl = B * 4 * H * D * W
        out["bytes"] = {"swa_step": byt}
        out["flops"] = {"swa_step": fl}
        out["swa_step"] = {"bytes": byt, "flops": fl}
    elif kind in HCA:
        N = d["N"]
        # the closing block's two streams in, its entry out (the bias, shared
        # by the batch, is not counted)
        comp = B * (2 * m * D * bf + vb)
        rows = N + W
        attn = B * (N * vb + W * D * bf + 2 * H * D * bf)
        fl = B * 4 * H * D * rows
        # one call does both
        out["bytes"] = {"hca_step": comp + attn}
        out["flops"] = {"hca_step": fl}
        out["hca_step"] = {"bytes": comp + attn, "flops": fl}
    else:
        N, P = d["N"], d["prefix"]
        T = Tq + m
        comp = 4 * T * D * bf + (Tq // m) * D * bf + 4 * T * Di * bf + (Tq // m) * Di * bf
        p0 = P * m
        vis = [min(N, (p0 + t + 1) // m) for t in range(Tq)]
        idx_bytes = N * Di * bf + Tq * (Hi * Di * bf + Hi * 4 + K * 4)
        attn_bytes = Tq * (2 * H * D * bf + K * 4) + (Tq + W - 1) * D * bf + N * D * bf
        out["bytes"] = {"compress": comp, "index_topk": idx_bytes, "sparse_attn": attn_bytes}
        out["flops"] = {"index_topk": 2 * Hi * Di * sum(vis),
                        "sparse_attn": 4 * H * D * (K + W) * Tq}
        out["index_scores"] = {"bytes": N * Di * bf + Tq * (Hi * Di * bf + Hi * 4),
                               "flops": 2 * Hi * Di * sum(vis)}
    return out


def per_call_rate(kind, work, call_us):
    out = {}
    for name, us in call_us.items():
        if us <= 0:
            continue
        r = {}
        if name in work["bytes"]:
            r["GB/s"] = round(work["bytes"][name] / (us * 1e-6) / 1e9, 1)
        fl = work.get("flops", {}).get(name)
        if fl and kind in ("prefill", "oproj_prefill"):
            r["TFLOP/s"] = round(fl / (us * 1e-6) / 1e12, 1)
        if r:
            out[name] = r
    return out


# ---------------------------------------------------------------------------
# measured HBM traffic of the dominant kernel (hardware counters, committed)
# ---------------------------------------------------------------------------
DOMINANT_KERNELS = {
    "index_decode_fresh": ["index_decode<true, *> (closing-block compressors + scoring, "
                           "the step's first launch)"],
    "index_scores": ["index_prefill"],
    "hca_step": ["attn_hs<false, true, 4> (its last split pools the closing block)",
                 "attn_combine<bf16>"],
    "swa_step": ["attn_hs<false, false, 2> (its last split builds the token's window row)",
                 "attn_combine<bf16>"],
    "sparse_attn": ["attn_hs<true, *> (+ attn_combine<bf16> when split)"],
    "output_proj": ["proj_rows<4>", "proj_rows<8>"],
    "output_proj_gemm": ["proj_gemm<0>", "proj_gemm<1>"],
    "compress": ["compress_kernel<bf16, 8> (both compressors, one launch)"],
}
KERNEL_SOURCES = {
    "index_decode_fresh": ["indexer.hip", "common.h", "kernels.h"],
    "index_scores": ["indexer.hip", "common.h", "kernels.h"],
    "hca_step": ["attn.hip", "common.h", "kernels.h"],
    "swa_step": ["attn.hip", "common.h", "kernels.h"],
    "sparse_attn": ["attn.hip", "common.h", "kernels.h"],
    "output_proj": ["oproj.hip", "oproj.h", "common.h", "kernels.h"],
    "compress": ["compress.hip", "common.h", "kernels.h"],
}
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def kernel_source_hash(dom):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[dom]:
        with open(os.path.join(ROOT, "long_context_sparse_11_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kind, dom):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, each scaled by what it
    reads for the calibration kernel), from the committed counter record of
    this workload; None when there is none or the kernel source changed since."""
    try:
        with open(COUNTERS) as fh:
            rec = json.load(fh).get(kind)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel") != dom or rec.get("source_sha256") != kernel_source_hash(dom):
        return None
    return int(rec["hbm_bytes_per_launch"])


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the same step)
# ---------------------------------------------------------------------------
def cpu_baseline(kind, d, budget_s):
    from long_context_sparse_11_amd.synth import bf16_to_f32
    from oracle import csa_oracle as O

    def rows_of(t, b, sel):  # float32 rows of one sequence, converted on demand
        return bf16_to_f32(t.bits[b][sel]) if t.dt == "bf16" else t.f32[b][sel]

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    B, Tq = d["B"], d["Tq"]
    scale = 1.0 / math.sqrt(d["D"])
    done = 0
    t0 = time.perf_counter()
    if kind == "prefill":
        # compress the chunk once, then queries one at a time
        m = d["m"]
        pool = np.concatenate([d["pool_prefix"].f32[0], O.compress(
            d["c_a"].f32[0, m:], d["z_a"].f32[0, m:], d["bias_a"], m, c_b=d["c_b"].f32[0, m:],
            z_b=d["z_b"].f32[0, m:], bias_b=d["bias_b"], prev_c_b=d["c_b"].f32[0, :m],
            prev_z_b=d["z_b"].f32[0, :m], gain=d["gain"], rope_dims=d["R"],
            pos0=int(d["chunk_pos0"][0]))])
        keys = np.concatenate([d["kidx_prefix"].f32[0], O.compress(
            d["ic_a"].f32[0, m:], d["iz_a"].f32[0, m:], d["ibias_a"], m, c_b=d["ic_b"].f32[0, m:],
            z_b=d["iz_b"].f32[0, m:], bias_b=d["ibias_b"], prev_c_b=d["ic_b"].f32[0, :m],
            prev_z_b=d["iz_b"].f32[0, :m])])
        t = 0
        while time.perf_counter() - t0 < budget_s and t < Tq:
            tp = int(d["q_pos0"][0]) + t
            nv = O.visible_count(tp, m, d["N"])
            s = O.index_scores(d["q_idx"].f32[0, t], d["w_idx"][0, t], keys[:nv]).astype(np.float32)
            sel = O.select_topk(s, nv, d["K"])
            rows = np.concatenate([pool[[v for v in sel if v >= 0]],
                                   d["win"].f32[0][[p - int(d["win_pos0"][0]) for p in O.window_positions(tp, d["W"])]]])
            O.attend(d["q"].f32[0, t], tp, rows, d["sink"], scale, d["R"])
            t += 1
            done += 1
        sample = f"chunk compress + {done} of {Tq} queries"
    elif kind == "compress_stream":
        # entries one block at a time, from host copies of the streams' first
        # tokens (the device draw), both compressors per entry; the sample
        # wraps around its first 4,096 entries until the time budget is spent
        m, n = d["m"], 0
        T_s = 1 << 14
        h = {k: d[k][0, :T_s].float().cpu().numpy() for k in
             ("c_a", "z_a", "c_b", "z_b", "ic_a", "iz_a", "ic_b", "iz_b")}
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s or n == 0:
            i = n % (T_s // m)
            lo = max(0, (i - 1) * m)
            prev = {} if i == 0 else dict(c_b=h["c_b"][lo:i * m], z_b=h["z_b"][lo:i * m])
            iprev = {} if i == 0 else dict(c_b=h["ic_b"][lo:i * m], z_b=h["iz_b"][lo:i * m])
            blk = slice(i * m, (i + 1) * m)
            O.compress(h["c_a"][blk], h["z_a"][blk], d["bias_a"], m, bias_b=d["bias_b"],
                       prev_c_b=prev.get("c_b"), prev_z_b=prev.get("z_b"),
                       c_b=h["c_b"][blk], z_b=h["z_b"][blk], gain=d["gain"],
                       rope_dims=d["R"], pos0=i * m)
            O.compress(h["ic_a"][blk], h["iz_a"][blk], d["ibias_a"], m, bias_b=d["ibias_b"],
                       prev_c_b=iprev.get("c_b"), prev_z_b=iprev.get("z_b"),
                       c_b=h["ic_b"][blk], z_b=h["iz_b"][blk])
            n += 1
        done = n * m
        sample = f"{n} entries of both compressors ({done} tokens) from the sequence start"
    elif kind in ("oproj", "oproj_prefill"):
        wa, wb = d["w_a"].f32, d["w_b"].f32
        while time.perf_counter() - t0 < budget_s or done == 0:
            O.grouped_output_projection(d["o"].f32[done % B], wa, wb)
            done += 1
        sample = f"{done} tokens' projections of batch {B}"
    elif kind == "swa":
        W = d["W"]
        while time.perf_counter() - t0 < budget_s or done == 0:
            bb = done % B
            tp = int(d["q_pos0"][bb])
            row = O.csa_compress(d["kv"].f32[bb:bb + 1], None, None, 1, gain=d["gain"],
                                 rope_dims=d["R"], pos0=[tp])[0, 0]
            rows = d["win"].f32[bb].astype(np.float64)
            rows[W - 1] = row
            O.attend(d["q"].f32[bb, 0], tp, rows, d["sink"], scale, d["R"])
            done += 1
        sample = f"{done} decode queries (window row + window attention per query) of batch {B}"
    else:
        b = 0
        hca = kind in ("hca1m", "hca1m_fp8")
        D, R = d["D"], d["R"]
        # packed mixed BF16 / FP8 pools: the rows the step reads, stored and read back
        kvq = ((lambda r: O.kv_fp8_dequantize(O.kv_fp8_quantize(r, R), D, R))
               if kind.endswith("_fp8") else (lambda r: r))
        while time.perf_counter() - t0 < budget_s or done == 0:
            bb = b % B
            m = d["m"]
            tp = int(d["q_pos0"][bb])
            kv = O.compress(d["c_a"].f32[bb], d["z_a"].f32[bb], d["bias_a"], m,
                            c_b=None if hca else d["c_b"].f32[bb],
                            z_b=None if hca else d["z_b"].f32[bb],
                            bias_b=d.get("bias_b"),
                            prev_c_b=None if hca else d["prev_c_b"].f32[bb],
                            prev_z_b=None if hca else d["prev_z_b"].f32[bb],
                            gain=d["gain"], rope_dims=d["R"], pos0=int(d["block_pos0"][bb]))
            win = d["win"].f32[bb]
            wr = [p - int(d["win_pos0"][bb]) for p in O.window_positions(tp, d["W"])]
            if hca:
                nv = O.visible_count(tp, m, d["N"])
                pool = rows_of(d["pool"], bb, slice(0, nv)).astype(np.float64)
                pool[-1] = kv[0]
                rows = np.concatenate([kvq(pool), win[wr]])
            else:
                ik = O.compress(d["ic_a"].f32[bb], d["iz_a"].f32[bb], d["ibias_a"], m,
                           c_b=d["ic_b"].f32[bb], z_b=d["iz_b"].f32[bb], bias_b=d["ibias_b"],
                           prev_c_b=d["iprev_c_b"].f32[bb], prev_z_b=d["iprev_z_b"].f32[bb])
                nv = O.visible_count(tp, m, d["N"])
                if kind.endswith("_fp4"):
                    keys = O.mxfp4_dequantize(d["k_codes"][bb, :nv], d["k_scales"][bb, :nv])
                    keys[-1] = O.mxfp4_dequantize(*O.mxfp4_quantize(ik[0]))
                else:
                    keys = rows_of(d["k_idx"], bb, slice(0, nv))
                s = O.index_scores(d["q_idx"].f32[bb, 0], d["w_idx"][bb, 0],
                                   keys).astype(np.float32)
                sel = O.select_topk(s, nv, d["K"])
                rows = np.concatenate([kvq(rows_of(d["pool"], bb, [v for v in sel if v >= 0])
                                           .astype(np.float64)), win[wr]])
            O.attend(d["q"].f32[bb, 0], tp, rows, d["sink"], scale, d["R"])
            done += 1
            b += 1
        sample = f"{done} decode queries (full step per query) of batch {B}"
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": sample, "seconds": round(el, 2),
            "host_cpus": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


# ---------------------------------------------------------------------------
WORKLOAD_CONFIG = {
    "csa64k": dict(workload="csa_decode_64k", batch=4, context=65536, entries=16384),
    "csa64k_pro": dict(workload="csa_decode_64k_v4pro", batch=4, context=65536, entries=16384),
    "csa1m": dict(workload="csa_decode_1m", batch=8, context=1048576, entries=262144),
    "csa64k_fp4": dict(workload="csa_decode_64k_mxfp4_keys", batch=4, context=65536,
                       entries=16384, index_key_format="mxfp4"),
    "csa1m_fp4": dict(workload="csa_decode_1m_mxfp4_keys", batch=8, context=1048576,
                      entries=262144, index_key_format="mxfp4"),
    "hca1m": dict(workload="hca_decode_1m", batch=16, context=1048576, entries=8192),
    "swa": dict(workload="swa_decode_1m", batch=16, context=1048576, entries=0),
    "oproj": dict(workload="output_proj_decode", batch=4, groups=8, group_rank=1024, hidden=4096),
    "csa64k_stream": dict(workload="csa_decode_64k_streaming", batch=4,
                          context="63,488 upward (16,384-entry cache)", entries=15872,
                          window="ring"),
    "oproj_prefill": dict(workload="output_proj_prefill_4k", batch=4096, groups=8,
                          group_rank=1024, hidden=4096),
    "prefill": dict(workload="csa_prefill_4k_on_60k", batch=1, queries=4096, context=65536,
                    entries=16384),
    "compress_stream": dict(workload="compress_stream_1m", batch=1, tokens=1048576,
                            entries=262144, key_width=128),
    "csa64k_fp8": dict(workload="csa_decode_64k_fp8_kv", batch=4, context=65536, entries=16384,
                       kv_format="bf16 rope + mx fp8"),
    "csa1m_fp8": dict(workload="csa_decode_1m_fp8_kv", batch=8, context=1048576, entries=262144,
                      kv_format="bf16 rope + mx fp8"),
    "hca1m_fp8": dict(workload="hca_decode_1m_fp8_kv", batch=16, context=1048576, entries=8192,
                      kv_format="bf16 rope + mx fp8"),
}
# workloads measured after the headline in the default run (the metric's 1M
# context), with their timed steps capped so the whole run stays short
ALSO = ("csa1m", "hca1m")
ALSO_STEPS = 20


def measure(kind, steps, warmup, use_graph, cpu_seconds, torch, L):
    """Run one workload: warmup + timed steps (graph replays), per-call and
    dominant-unit timing with HIP events, the roofline fields and, when
    cpu_seconds is set, the CPU oracle's rate.  Returns the result dict."""
    d = make_inputs(kind)
    work = algorithmic(kind, d)
    step_bytes = sum(work["bytes"].values())
    n_copies = max(1, min(64, math.ceil(2 * MALL_BYTES / max(step_bytes, 1)) + 1))

    # one copy uploaded from host, the rest cloned on the device
    base = upload({k: v for k, v in d.items() if k not in ("name", "dt")}, torch)
    if kind == "prefill":
        prefill_buffers(base, torch)
    if kind in KV_FP8:
        base["pool"] = L.csa_quantize_kv_fp8(base["pool"], d["R"])
        torch.cuda.synchronize()
    copies = [base]
    big = [k for k, v in base.items() if isinstance(v, torch.Tensor) and v.numel() * v.element_size() > 4096]
    for _ in range(n_copies - 1):
        c = dict(base)
        for k in big:
            c[k] = base[k].clone()
        copies.append(c)
    steps_l = [Step(kind, c, L, torch) for c in copies]

    # calibration kernel of known traffic for the hardware byte counters
    # (reads and writes 512 MiB; also flushes the Infinity Cache)
    cal_src = torch.zeros(CAL_BYTES, dtype=torch.uint8, device="cuda")
    cal_dst = torch.empty_like(cal_src)
    torch.bitwise_not(cal_src, out=cal_dst)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    stream = torch.cuda.current_stream()
    names = [n for n, _ in steps_l[0].calls()]
    # eager warm-up (loads the code objects)
    for st in steps_l[:2]:
        for _, f in st.calls():
            f()
    torch.cuda.synchronize()
    # steps per graph replay: several decode steps are captured together
    # (each on its own input copy), as a serving loop would capture them
    per_graph = next(p for p in (10, 8, 5, 4, 2, 1) if steps % p == 0 and warmup % p == 0) \
        if use_graph else 1
    reps_call = 20  # repetitions of one call per timing graph (distinct copies)
    graphs, call_graphs = [], []
    if use_graph:
        for gi in range(n_copies):
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gph):
                for r in range(per_graph):
                    for _, f in steps_l[(gi * per_graph + r) % n_copies].calls():
                        f()
            graphs.append(gph)
        for k in range(len(names)):
            cg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(cg):
                for r in range(reps_call):
                    steps_l[r % n_copies].calls()[k][1]()
            call_graphs.append(cg)
        dom_graph = torch.cuda.CUDAGraph()
        for st in steps_l[:2]:
            st.dominant()[1]()   # allocates its output before capture
        torch.cuda.synchronize()
        with torch.cuda.graph(dom_graph):
            for r in range(reps_call):
                steps_l[r % n_copies].dominant()[1]()
        torch.cuda.synchronize()

    def run(i):  # replay i covers steps i*per_graph .. (i+1)*per_graph-1
        if use_graph:
            graphs[i % n_copies].replay()
        else:
            for _, f in steps_l[i % n_copies].calls():
                f()

    for i in range(warmup // per_graph):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps // per_graph):
        run(warmup // per_graph + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / steps
    tokens = d["B"] * d["Tq"]
    value = tokens * steps / elapsed

    # device time per step and per library call: HIP events on the library's
    # stream around graph replays, queued behind a spin kernel so the device
    # never waits for the host between them
    def timed(thunks):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in thunks]
        torch.cuda._sleep(20_000_000)
        for (e0, e1), th in zip(evs, thunks):
            e0.record(stream)
            th()
            e1.record(stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]  # us

    if use_graph:
        dev_step_us = float(np.median(timed([(lambda i=i: run(i)) for i in range(20)]))) / per_graph
        call_us = {n: float(np.median(timed([call_graphs[k].replay] * 10))) / reps_call
                   for k, n in enumerate(names)}
    else:
        dev_step_us = float(np.median(timed([(lambda i=i: run(i)) for i in range(20)])))
        call_us = {n: float(np.median(timed([(lambda i=i, k=k: steps_l[i % n_copies].calls()[k][1]())
                                             for i in range(20)]))) for k, n in enumerate(names)}

    # roofline of the dominant unit: its per-launch duration from HIP events
    # around replays of a graph of reps_call launches (rotating input
    # copies), on the library's stream
    dom = steps_l[0].dominant()[0]
    if use_graph:
        dom_us = float(np.median(timed([dom_graph.replay] * 10))) / reps_call
    else:
        dom_us = float(np.median(timed([(lambda i=i: steps_l[i % n_copies].dominant()[1]())
                                        for i in range(20)])))
    dw = work[dom]
    if kind in ("prefill", "oproj_prefill"):
        ach = dw["flops"] / (dom_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        ach = dw["bytes"] / (dom_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(kind, dom)
    roof["kernel"] = dom
    roof["device_kernels"] = DOMINANT_KERNELS["output_proj_gemm" if kind == "oproj_prefill" else dom]
    roof["algorithmic_bytes_per_launch"] = int(dw["bytes"])
    roof["algorithmic_flops_per_launch"] = int(dw["flops"])
    roof["avg_launch_us"] = round(dom_us, 2)

    # the whole step against the HBM roofline: its algorithmic bytes over the
    # wall-clock time per step (and over the device time per step)
    step_roof = {"algorithmic_bytes": int(step_bytes),
                 "achieved_GBs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                 "frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "frac_device_time": round(step_bytes / (dev_step_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                           4)}

    cpu = cpu_baseline(kind, d, cpu_seconds) if cpu_seconds else None

    cfg = dict(WORKLOAD_CONFIG[kind])
    cfg.update(heads=d["H"], head_dim=d["D"], rope_dims=d["R"], index_heads=d["Hi"],
               index_dim=d["Di"], index_topk=d["K"], window=d["W"], m=d["m"], step_calls=names,
               graph=use_graph, steps_per_graph=per_graph, input_copies=n_copies)
    res = dict(value=round(value, 1), ms_per_step=round(ms_per_step, 5), config=cfg,
               roofline=roof, step_roofline=step_roof, cpu_baseline=cpu,
               device_us_per_step=round(dev_step_us, 2),
               per_call_us={k: round(v, 2) for k, v in call_us.items()},
               # each call's algorithmic rate: HBM GB/s, and TFLOP/s where the
               # call is a large contraction (the prefill indexer and
               # attention, the prefill projection)
               per_call_rate=per_call_rate(kind, work, call_us),
               step_algorithmic_bytes=int(step_bytes))
    del graphs, call_graphs, steps_l, copies, base
    if use_graph:
        del dom_graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {a.gpus}); the path shards by sequence "
              "across GPUs with no exchange, so the whole-job rate is N times this line", file=sys.stderr)
        sys.exit(2)
    import torch
    import long_context_sparse_11_amd as L
    L.lib()
    if not torch.cuda.is_available():
        print("no GPU", file=sys.stderr)
        sys.exit(1)

    use_graph = not a.no_graph
    kind = a.workload
    r = measure(kind, a.steps, a.warmup, use_graph, None if a.no_cpu else a.cpu_seconds, torch, L)
    line = {
        "metric": METRIC, "value": r["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": r["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": r["config"], "roofline": r["roofline"],
        "step_roofline": r["step_roofline"], "cpu_baseline": r["cpu_baseline"],
        "device_us_per_step": r["device_us_per_step"], "per_call_us": r["per_call_us"],
        "per_call_rate": r["per_call_rate"], "step_algorithmic_bytes": r["step_algorithmic_bytes"],
    }
    # the metric's 1M-context decode workloads, measured in the same run
    if kind == "csa64k" and not a.only:
        also = {}
        for k in ALSO:
            n, w = max(min(a.steps, ALSO_STEPS), 1), min(a.warmup, ALSO_STEPS)
            ra = measure(k, n, w, use_graph, None, torch, L)
            also[ra["config"]["workload"]] = {
                "value": ra["value"], "unit": "tokens/s", "steps": n, "warmup": w,
                "ms_per_step": ra["ms_per_step"], "device_us_per_step": ra["device_us_per_step"],
                "per_call_us": ra["per_call_us"], "per_call_rate": ra["per_call_rate"],
                "roofline": ra["roofline"], "step_roofline": ra["step_roofline"],
                "config": ra["config"]}
        line["also"] = also
    print(json.dumps(line))


if __name__ == "__main__":
    main()
