"""Thin ctypes binding of libcsa.so (declared in include/csa.h).

Argument marshalling only: every step runs in the HIP library.  Tensors are
torch tensors on the GPU (PyTorch supplies device memory and the current HIP
stream); outputs and workspaces are allocated here with torch and handed to
the library.  There is no fallback: if the library is missing or a call
fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")
_lib = None

CSA_F32, CSA_BF16 = 0, 1

_c = ctypes
_SIGS = {
    "csa_compress": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                _c.c_void_p, _c.c_float, _c.c_int, _c.c_double, _c.c_void_p,
                                _c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_size_t,
                                _c.c_void_p]),
    "csa_compress_ws_bytes": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                            _c.c_int]),
    "csa_compress_batch": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                      _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p]),
    "csa_index_topk": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                  _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                  _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                  _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "csa_decode_index_topk": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                          _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_void_p,
                                          _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_void_p,
                                          _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                          _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "csa_index_scores": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                     _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                     _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "csa_quantize_mxfp4": (_c.c_int, [_c.c_int, _c.c_int64, _c.c_int, _c.c_void_p, _c.c_void_p,
                                      _c.c_void_p, _c.c_void_p]),
    "csa_index_topk_mxfp4": (_c.c_int, [_c.c_int] * 7 + [_c.c_void_p] * 10 + [_c.c_size_t,
                                                                               _c.c_void_p]),
    "csa_index_scores_mxfp4": (_c.c_int, [_c.c_int] * 6 + [_c.c_void_p] * 8),
    "csa_decode_index_topk_mxfp4": (_c.c_int, [_c.c_int] * 8 + [_c.c_void_p, _c.c_void_p, _c.c_int]
                                    + [_c.c_void_p] * 10 + [_c.c_size_t, _c.c_void_p]),
    "csa_decode_index_topk_noalloc": (_c.c_int, [_c.c_int] * 9 + [_c.c_void_p, _c.c_void_p,
                                                                    _c.c_int]
                                      + [_c.c_void_p] * 8),
    "csa_decode_index_scores": (_c.c_int, [_c.c_int] * 8 + [_c.c_void_p, _c.c_void_p, _c.c_int]
                                + [_c.c_void_p] * 6),
    "csa_decode_index_scores_mxfp4": (_c.c_int, [_c.c_int] * 7
                                      + [_c.c_void_p, _c.c_void_p, _c.c_int]
                                      + [_c.c_void_p] * 8),
    "csa_output_proj": (_c.c_int, [_c.c_int] * 6 + [_c.c_void_p] * 6),
    "csa_kv_fp8_row_bytes": (_c.c_size_t, [_c.c_int, _c.c_int]),
    "csa_quantize_kv_fp8": (_c.c_int, [_c.c_int, _c.c_int64, _c.c_int, _c.c_int, _c.c_void_p,
                                       _c.c_void_p, _c.c_void_p]),
    "csa_dequantize_kv_fp8": (_c.c_int, [_c.c_int64, _c.c_int, _c.c_int, _c.c_void_p,
                                         _c.c_void_p, _c.c_void_p]),
    "csa_compress_kvfp8": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                      _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                      _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                      _c.c_void_p, _c.c_float, _c.c_int, _c.c_double,
                                      _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p,
                                      _c.c_size_t, _c.c_void_p]),
    "csa_sparse_attn_kvfp8": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                         _c.c_double, _c.c_float, _c.c_void_p, _c.c_void_p,
                                         _c.c_int, _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int,
                                         _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_void_p,
                                         _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_size_t,
                                         _c.c_void_p]),
    "hca_attn_kvfp8": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_double,
                                  _c.c_float, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p,
                                  _c.c_int, _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int,
                                  _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                  _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "csa_window_row": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p,
                                  _c.c_float, _c.c_int, _c.c_double, _c.c_void_p, _c.c_void_p,
                                  _c.c_int, _c.c_void_p]),
    "csa_decode_advance": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p,
                                      _c.c_void_p, _c.c_void_p]),
    "csa_index_topk_ws_bytes": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int]),
    "csa_sparse_attn": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                   _c.c_double, _c.c_float, _c.c_void_p, _c.c_void_p, _c.c_int,
                                   _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_void_p,
                                   _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                   _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "hca_attn": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                            _c.c_double, _c.c_float, _c.c_void_p, _c.c_void_p, _c.c_int,
                            _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int,
                            _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                            _c.c_size_t, _c.c_void_p]),
    "csa_attn_ws_bytes": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int]),
    "hca_decode_attn": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_double,
                                   _c.c_float, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p,
                                   _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                   _c.c_void_p, _c.c_float, _c.c_void_p, _c.c_void_p, _c.c_int,
                                   _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_void_p,
                                   _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_size_t,
                                   _c.c_void_p]),
    "hca_decode_attn_kvfp8": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_double,
                                   _c.c_float, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p,
                                   _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                   _c.c_void_p, _c.c_float, _c.c_void_p, _c.c_void_p, _c.c_int,
                                   _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_void_p,
                                   _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_size_t,
                                   _c.c_void_p]),
    "hca_decode_attn_ws_bytes": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int, _c.c_int]),
    "swa_decode_attn": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_double,
                                   _c.c_float, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                   _c.c_float, _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int,
                                   _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                   _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "swa_decode_attn_ws_bytes": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int, _c.c_int]),
    "csa_status_string": (_c.c_char_p, [_c.c_int]),
}


class CsaError(RuntimeError):
    pass


def lib():
    """Load libcsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise CsaError(f"{_LIB_PATH} is missing; run long_context_sparse_11_amd.build.build()")
        h = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def _check(status: int, what: str):
    if status != 0:
        msg = lib().csa_status_string(status).decode()
        raise CsaError(f"{what} failed: {msg}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t) -> int:
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    if t.dtype == torch.float32:
        return CSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _f32(t):
    if t is not None and t.dtype != torch.float32:
        raise TypeError("parameter vectors are float32")
    return t


def _i64(t):
    if t is not None and t.dtype != torch.int64:
        raise TypeError("positions are int64")
    return t


# ---------------------------------------------------------------------------
def csa_compress(c_a, m, *, z_a=None, c_b=None, z_b=None, prev_c_b=None, prev_z_b=None,
                 bias_a=None, bias_b=None, gain=None, eps=1e-6, rope_dims=0,
                 rope_base=10000.0, pos0=None, out=None, out_bstride=0, ws=None, stream=None):
    """Compressor (see include/csa.h).  c_a [B, T, D]; returns out [B, ceil(T/m), D]
    (or writes the caller's ``out`` with batch stride ``out_bstride``).  ``ws``: a
    device byte tensor of csa_compress_ws_bytes(...) bytes, allocated here when
    the call can use one and none is given; an empty tensor means no workspace."""
    B, T, D = c_a.shape
    overlap = c_b is not None
    _dev(c_a, z_a, c_b, z_b, prev_c_b, prev_z_b, bias_a, bias_b, gain, pos0)
    _f32(bias_a), _f32(bias_b), _f32(gain), _i64(pos0)
    n_out = -(-T // m)
    if out is None:
        out = torch.empty((B, n_out, D), dtype=c_a.dtype, device=c_a.device)
    else:  # may be a view into a larger cache: [B, n_out, D] with batch stride out_bstride
        bs = out_bstride if out_bstride else n_out * D
        if (tuple(out.shape) != (B, n_out, D) or out.dtype != c_a.dtype or not out.is_cuda
                or out.stride(2) != 1 or (n_out > 1 and out.stride(1) != D)
                or (B > 1 and out.stride(0) != bs)):
            raise ValueError("out must be [B, ceil(T/m), D] with row stride D and batch stride "
                             "out_bstride")
    need = csa_compress_ws_bytes(_dt(c_a), B, T, D, m, overlap)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=c_a.device)
    if ws is not None and ws.numel() == 0:
        ws = None
    if ws is not None:
        _dev(ws)
    st = lib().csa_compress(_dt(c_a), B, T, D, m, int(overlap), _p(c_a), _p(z_a), _p(c_b), _p(z_b),
                            _p(prev_c_b), _p(prev_z_b), _p(bias_a), _p(bias_b), _p(gain),
                            float(eps), int(rope_dims), float(rope_base), _p(pos0), _p(out),
                            int(out_bstride), _p(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                            _stream(stream))
    _check(st, "csa_compress")
    return out


class CompressJob(ctypes.Structure):
    """Mirror of csa_compress_job (include/csa.h)."""
    _fields_ = [("D", _c.c_int), ("c_a", _c.c_void_p), ("z_a", _c.c_void_p),
                ("c_b", _c.c_void_p), ("z_b", _c.c_void_p), ("prev_c_b", _c.c_void_p),
                ("prev_z_b", _c.c_void_p), ("bias_a", _c.c_void_p), ("bias_b", _c.c_void_p),
                ("gain", _c.c_void_p), ("eps", _c.c_float), ("rope_dims", _c.c_int),
                ("rope_base", _c.c_double), ("out", _c.c_void_p), ("out_bstride", _c.c_int64),
                ("out_kv_fp8", _c.c_int)]


def _job_array(jobs, B, T, overlap, out_shape, first_out_none=False):
    """ctypes array of csa_compress_job from job dicts; out_shape(D) is the
    shape each job's ``out`` must have (row stride D, batch stride
    ``out_bstride`` or the rows times D).  first_out_none: job 0 has no
    ``out`` (its entries go elsewhere)."""
    arr = (CompressJob * len(jobs))()
    for k, j in enumerate(jobs):
        c_a, out = j["c_a"], j.get("out")
        Bj, Tj, D = c_a.shape
        if k == 2:   # the step token's window row into its ring
            if Tj != 1 or Bj != B or out is None or out.dim() != 3 or out.shape[0] != B \
                    or out.shape[2] != D or not out.is_contiguous() or out.dtype != c_a.dtype:
                raise ValueError("jobs[2]: c_a [B, 1, D] and out the ring [B, L_win, D]")
            _dev(c_a, j.get("gain"))
            _f32(j.get("gain"))
            p = lambda t: t.data_ptr() if t is not None else None
            arr[k] = CompressJob(D, p(c_a), None, None, None, None, None, None, None,
                                 p(j.get("gain")), float(j.get("eps", 1e-6)),
                                 int(j.get("rope_dims", 0)), float(j.get("rope_base", 10000.0)),
                                 out.data_ptr(), out.shape[1] * D)
            continue
        if (Bj, Tj) != (B, T) or (j.get("c_b") is not None) != overlap or c_a.dtype != jobs[0]["c_a"].dtype:
            raise ValueError("jobs must share B, T, dtype and overlap")
        ts = [j.get(n) for n in ("z_a", "c_b", "z_b", "prev_c_b", "prev_z_b", "bias_a", "bias_b", "gain")]
        _dev(c_a, *ts)
        _f32(j.get("bias_a")), _f32(j.get("bias_b")), _f32(j.get("gain"))
        shape = out_shape(D)
        fp8 = bool(j.get("out_kv_fp8", False))
        if fp8:   # packed mixed BF16 / FP8 rows: [B, rows, row_bytes] uint8
            rb = csa_kv_fp8_row_bytes(D, int(j.get("rope_dims", 0)))
            shape = (shape[0], shape[1], rb)
            bs = j.get("out_bstride", 0) or shape[1] * rb
            if (out is None or tuple(out.shape) != shape or out.dtype != torch.uint8
                    or not out.is_cuda or out.stride(2) != 1
                    or (shape[1] > 1 and out.stride(1) != rb) or (B > 1 and out.stride(0) != bs)):
                raise ValueError(f"out must be uint8 {list(shape)} with row stride {rb} and "
                                 "batch stride out_bstride (bytes)")
        else:
            bs = j.get("out_bstride", 0) or shape[1] * D
        if fp8:
            pass
        elif k == 0 and first_out_none:
            if out is not None or j.get("out_bstride", 0):
                raise ValueError("job 0 takes no out here")
        elif (tuple(out.shape) != shape or out.dtype != c_a.dtype or not out.is_cuda
                or out.stride(2) != 1 or (shape[1] > 1 and out.stride(1) != D)
                or (B > 1 and out.stride(0) != bs)):
            raise ValueError(f"out must be {list(shape)} with row stride D and batch stride "
                             "out_bstride")
        p = lambda t: t.data_ptr() if t is not None else None
        arr[k] = CompressJob(D, p(c_a), p(j.get("z_a")), p(j.get("c_b")), p(j.get("z_b")),
                             p(j.get("prev_c_b")), p(j.get("prev_z_b")), p(j.get("bias_a")),
                             p(j.get("bias_b")), p(j.get("gain")), float(j.get("eps", 1e-6)),
                             int(j.get("rope_dims", 0)), float(j.get("rope_base", 10000.0)),
                             None if out is None else out.data_ptr(),
                             int(j.get("out_bstride", 0)), int(fp8))
    return arr


def csa_compress_batch(jobs, m, *, pos0=None, stream=None):
    """Up to two compressors over the same token block in one launch (see
    include/csa.h).  ``jobs``: dicts with the keyword arguments of
    csa_compress plus ``c_a`` and ``out`` (both required here); every job's
    streams share B, T and, with ``c_b`` given, the overlap."""
    if not 1 <= len(jobs) <= 2:
        raise ValueError("one or two jobs")
    B, T, _ = jobs[0]["c_a"].shape
    overlap = jobs[0].get("c_b") is not None
    _i64(pos0)
    _dev(pos0)
    arr = _job_array(jobs, B, T, overlap, lambda D: (B, -(-T // m), D))
    st = lib().csa_compress_batch(_dt(jobs[0]["c_a"]), B, T, m, int(overlap), _p(pos0),
                                  ctypes.cast(arr, ctypes.c_void_p), len(jobs), _stream(stream))
    _check(st, "csa_compress_batch")
    return [j["out"] for j in jobs]


def csa_compress_ws_bytes(dt, B, T, D, m, overlap=False):
    """Workspace bytes csa_compress can use (dt: 0 float32, 1 bfloat16)."""
    return int(lib().csa_compress_ws_bytes(dt, B, T, D, m, int(bool(overlap))))


def csa_index_topk_ws_bytes(B, Tq, Hi, N_cap, K):
    return int(lib().csa_index_topk_ws_bytes(B, Tq, Hi, N_cap, K))


def csa_index_topk(q_idx, w_idx, k_idx, n_entries, q_pos0, K, m, *, want_scores=False,
                   want_all_scores=False, ws=None, idx_out=None, stream=None):
    """Indexer scores + top-K.  Returns (idx [B,Tq,K] int32, score_out or None,
    all_scores or None)."""
    B, Tq, Hi, Di = q_idx.shape
    N_cap = k_idx.shape[1]
    _dev(q_idx, w_idx, k_idx, n_entries, q_pos0)
    _f32(w_idx), _i64(q_pos0)
    if n_entries.dtype != torch.int32:
        raise TypeError("n_entries is int32")
    dev = q_idx.device
    if idx_out is None:
        idx_out = torch.empty((B, Tq, K), dtype=torch.int32, device=dev)
    score_out = torch.empty((B, Tq, K), dtype=torch.float32, device=dev) if want_scores else None
    all_scores = (torch.empty((B, Tq, N_cap), dtype=torch.float32, device=dev)
                  if want_all_scores else None)
    need = csa_index_topk_ws_bytes(B, Tq, Hi, N_cap, K)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib().csa_index_topk(_dt(q_idx), B, Tq, Hi, Di, N_cap, K, m, _p(q_idx), _p(w_idx),
                              _p(k_idx), _p(n_entries), _p(q_pos0), _p(idx_out), _p(score_out),
                              _p(all_scores), _p(ws), 0 if ws is None else ws.numel(),
                              _stream(stream))
    _check(st, "csa_index_topk")
    return idx_out, score_out, all_scores


def csa_decode_index_topk(q_idx, w_idx, n_entries, q_pos0, K, m, jobs, *, block_pos0=None,
                          want_scores=False, want_all_scores=False, ws=None, idx_out=None,
                          stream=None):
    """A decode step's compressors and indexer in one call (see include/csa.h).
    ``jobs``: one or two dicts as for csa_compress_batch over the closing
    block (c_a [B, m, D]); each ``out`` is the whole pool [B, N_cap, D] and
    the new entry of sequence b lands in row min(n_entries[b], N_cap) - 1;
    jobs[0] is the indexer-key compressor, its pool the indexer's keys.
    Returns (idx, score_out or None, all_scores or None) as csa_index_topk."""
    B, Tq, Hi, Di = q_idx.shape
    k_idx = jobs[0]["out"]
    N_cap = k_idx.shape[1]
    overlap = jobs[0].get("c_b") is not None
    _dev(q_idx, w_idx, n_entries, q_pos0, block_pos0)
    _f32(w_idx), _i64(q_pos0), _i64(block_pos0)
    if n_entries.dtype != torch.int32:
        raise TypeError("n_entries is int32")
    if jobs[0]["c_a"].shape[1] != m:
        raise ValueError("the jobs' streams hold one block of m tokens")
    arr = _job_array(jobs, B, m, overlap, lambda D: (B, N_cap, D))
    dev = q_idx.device
    if idx_out is None:
        idx_out = torch.empty((B, Tq, K), dtype=torch.int32, device=dev)
    score_out = torch.empty((B, Tq, K), dtype=torch.float32, device=dev) if want_scores else None
    all_scores = (torch.empty((B, Tq, N_cap), dtype=torch.float32, device=dev)
                  if want_all_scores else None)
    need = csa_index_topk_ws_bytes(B, Tq, Hi, N_cap, K)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib().csa_decode_index_topk(_dt(q_idx), B, Tq, Hi, Di, N_cap, K, m, int(overlap),
                                     _p(block_pos0), ctypes.cast(arr, ctypes.c_void_p), len(jobs),
                                     _p(q_idx), _p(w_idx), _p(n_entries), _p(q_pos0), _p(idx_out),
                                     _p(score_out), _p(all_scores), _p(ws),
                                     0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "csa_decode_index_topk")
    return idx_out, score_out, all_scores


def csa_decode_index_topk_noalloc(q_idx, w_idx, n_entries, q_pos0, K, m, jobs, *,
                                  block_pos0=None, want_scores=False, want_all_scores=False,
                                  idx_out=None, stream=None):
    """csa_decode_index_topk working in the library's own device scratch
    (no workspace argument; see include/csa.h).  The outputs are allocated
    here unless given: pass idx_out (and nothing else to allocate) where the
    caller must not allocate."""
    B, Tq, Hi, Di = q_idx.shape
    k_idx = jobs[0]["out"]
    N_cap = k_idx.shape[1]
    overlap = jobs[0].get("c_b") is not None
    _dev(q_idx, w_idx, n_entries, q_pos0, block_pos0)
    _f32(w_idx), _i64(q_pos0), _i64(block_pos0)
    if n_entries.dtype != torch.int32:
        raise TypeError("n_entries is int32")
    if jobs[0]["c_a"].shape[1] != m:
        raise ValueError("the jobs' streams hold one block of m tokens")
    arr = _job_array(jobs, B, m, overlap, lambda D: (B, N_cap, D))
    dev = q_idx.device
    if idx_out is None:
        idx_out = torch.empty((B, Tq, K), dtype=torch.int32, device=dev)
    score_out = torch.empty((B, Tq, K), dtype=torch.float32, device=dev) if want_scores else None
    all_scores = (torch.empty((B, Tq, N_cap), dtype=torch.float32, device=dev)
                  if want_all_scores else None)
    st = lib().csa_decode_index_topk_noalloc(
        _dt(q_idx), B, Tq, Hi, Di, N_cap, K, m, int(overlap), _p(block_pos0),
        ctypes.cast(arr, ctypes.c_void_p), len(jobs), _p(q_idx), _p(w_idx), _p(n_entries),
        _p(q_pos0), _p(idx_out), _p(score_out), _p(all_scores), _stream(stream))
    _check(st, "csa_decode_index_topk_noalloc")
    return idx_out, score_out, all_scores


def _fp4_keys(k_codes, k_scales, Di):
    B, N_cap, nb = k_codes.shape
    if (k_codes.dtype != torch.uint8 or k_scales.dtype != torch.uint8 or nb * 2 != Di
            or tuple(k_scales.shape) != (B, N_cap, Di // 32) or not k_codes.is_contiguous()
            or not k_scales.is_contiguous()):
        raise ValueError("k_codes uint8 [B, N_cap, Di/2] and k_scales uint8 [B, N_cap, Di/32], "
                         "contiguous")
    return N_cap


def csa_quantize_mxfp4(x, *, codes=None, scales=None, stream=None):
    """[..., D] float32/bf16 -> (codes uint8 [..., D/2], scales uint8
    [..., D/32]) in MX FP4 (see include/csa.h)."""
    _dev(x)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    lead = tuple(x.shape[:-1])
    if codes is None:
        codes = torch.empty(lead + (D // 2,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(lead + (D // 32,), dtype=torch.uint8, device=x.device)
    st = lib().csa_quantize_mxfp4(_dt(x), rows, D, _p(x), _p(codes), _p(scales), _stream(stream))
    _check(st, "csa_quantize_mxfp4")
    return codes, scales


def csa_index_topk_mxfp4(q_idx, w_idx, k_codes, k_scales, n_entries, q_pos0, K, m, *,
                         want_scores=False, want_all_scores=False, ws=None, idx_out=None,
                         stream=None):
    """csa_index_topk with MX FP4 keys (q_idx bf16)."""
    B, Tq, Hi, Di = q_idx.shape
    _dev(q_idx, w_idx, k_codes, k_scales, n_entries, q_pos0)
    _f32(w_idx), _i64(q_pos0)
    N_cap = _fp4_keys(k_codes, k_scales, Di)
    dev = q_idx.device
    if idx_out is None:
        idx_out = torch.empty((B, Tq, K), dtype=torch.int32, device=dev)
    score_out = torch.empty((B, Tq, K), dtype=torch.float32, device=dev) if want_scores else None
    all_scores = (torch.empty((B, Tq, N_cap), dtype=torch.float32, device=dev)
                  if want_all_scores else None)
    need = csa_index_topk_ws_bytes(B, Tq, Hi, N_cap, K)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib().csa_index_topk_mxfp4(B, Tq, Hi, Di, N_cap, K, m, _p(q_idx), _p(w_idx),
                                    _p(k_codes), _p(k_scales), _p(n_entries), _p(q_pos0),
                                    _p(idx_out), _p(score_out), _p(all_scores), _p(ws),
                                    0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "csa_index_topk_mxfp4")
    return idx_out, score_out, all_scores


def csa_index_scores_mxfp4(q_idx, w_idx, k_codes, k_scales, n_entries, q_pos0, m, *, out=None,
                           stream=None):
    """csa_index_scores with MX FP4 keys (q_idx bf16)."""
    B, Tq, Hi, Di = q_idx.shape
    _dev(q_idx, w_idx, k_codes, k_scales, n_entries, q_pos0)
    _f32(w_idx), _i64(q_pos0)
    N_cap = _fp4_keys(k_codes, k_scales, Di)
    if out is None:
        out = torch.empty((B, Tq, N_cap), dtype=torch.float32, device=q_idx.device)
    st = lib().csa_index_scores_mxfp4(B, Tq, Hi, Di, N_cap, m, _p(q_idx), _p(w_idx), _p(k_codes),
                                      _p(k_scales), _p(n_entries), _p(q_pos0), _p(out),
                                      _stream(stream))
    _check(st, "csa_index_scores_mxfp4")
    return out


def csa_decode_index_topk_mxfp4(q_idx, w_idx, k_codes, k_scales, n_entries, q_pos0, K, m, jobs,
                                *, block_pos0=None, want_scores=False, want_all_scores=False,
                                ws=None, idx_out=None, stream=None):
    """csa_decode_index_topk with the indexer keys in MX FP4: jobs[0] (the
    key compressor, no ``out``) writes its fresh entry quantized into row
    min(n_entries[b], N_cap) - 1 of k_codes / k_scales."""
    B, Tq, Hi, Di = q_idx.shape
    _dev(q_idx, w_idx, k_codes, k_scales, n_entries, q_pos0, block_pos0)
    _f32(w_idx), _i64(q_pos0), _i64(block_pos0)
    N_cap = _fp4_keys(k_codes, k_scales, Di)
    if jobs[0]["c_a"].shape[1] != m:
        raise ValueError("the jobs' streams hold one block of m tokens")
    overlap = jobs[0].get("c_b") is not None
    arr = _job_array(jobs, B, m, overlap, lambda D: (B, N_cap, D), first_out_none=True)
    dev = q_idx.device
    if idx_out is None:
        idx_out = torch.empty((B, Tq, K), dtype=torch.int32, device=dev)
    score_out = torch.empty((B, Tq, K), dtype=torch.float32, device=dev) if want_scores else None
    all_scores = (torch.empty((B, Tq, N_cap), dtype=torch.float32, device=dev)
                  if want_all_scores else None)
    need = csa_index_topk_ws_bytes(B, Tq, Hi, N_cap, K)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib().csa_decode_index_topk_mxfp4(
        B, Tq, Hi, Di, N_cap, K, m, int(overlap), _p(block_pos0),
        ctypes.cast(arr, ctypes.c_void_p), len(jobs), _p(q_idx), _p(w_idx), _p(k_codes),
        _p(k_scales), _p(n_entries), _p(q_pos0), _p(idx_out), _p(score_out), _p(all_scores),
        _p(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "csa_decode_index_topk_mxfp4")
    return idx_out, score_out, all_scores


def csa_decode_index_scores(q_idx, w_idx, n_entries, q_pos0, m, jobs, *, block_pos0=None,
                            out=None, stream=None):
    """The scoring half of csa_decode_index_topk: the closing block's fresh
    entries (jobs as there), then the scores [B, Tq, N_cap] float32 of every
    visible entry (later columns as they were).  Returns the scores."""
    B, Tq, Hi, Di = q_idx.shape
    N_cap = jobs[0]["out"].shape[1]
    overlap = jobs[0].get("c_b") is not None
    _dev(q_idx, w_idx, n_entries, q_pos0, block_pos0)
    _f32(w_idx), _i64(q_pos0), _i64(block_pos0)
    if n_entries.dtype != torch.int32:
        raise TypeError("n_entries is int32")
    if jobs[0]["c_a"].shape[1] != m:
        raise ValueError("the jobs' streams hold one block of m tokens")
    arr = _job_array(jobs, B, m, overlap, lambda D: (B, N_cap, D))
    out = _scores_out(out, B, Tq, N_cap, q_idx.device)
    st = lib().csa_decode_index_scores(_dt(q_idx), B, Tq, Hi, Di, N_cap, m, int(overlap),
                                       _p(block_pos0), ctypes.cast(arr, ctypes.c_void_p),
                                       len(jobs), _p(q_idx), _p(w_idx), _p(n_entries),
                                       _p(q_pos0), _p(out), _stream(stream))
    _check(st, "csa_decode_index_scores")
    return out


def csa_decode_index_scores_mxfp4(q_idx, w_idx, k_codes, k_scales, n_entries, q_pos0, m, jobs,
                                  *, block_pos0=None, out=None, stream=None):
    """csa_decode_index_scores with the indexer keys in MX FP4 (jobs[0] has
    no ``out``; its fresh entry goes quantized into k_codes / k_scales)."""
    B, Tq, Hi, Di = q_idx.shape
    _dev(q_idx, w_idx, k_codes, k_scales, n_entries, q_pos0, block_pos0)
    _f32(w_idx), _i64(q_pos0), _i64(block_pos0)
    N_cap = _fp4_keys(k_codes, k_scales, Di)
    if jobs[0]["c_a"].shape[1] != m:
        raise ValueError("the jobs' streams hold one block of m tokens")
    overlap = jobs[0].get("c_b") is not None
    arr = _job_array(jobs, B, m, overlap, lambda D: (B, N_cap, D), first_out_none=True)
    out = _scores_out(out, B, Tq, N_cap, q_idx.device)
    st = lib().csa_decode_index_scores_mxfp4(
        B, Tq, Hi, Di, N_cap, m, int(overlap), _p(block_pos0), ctypes.cast(arr, ctypes.c_void_p),
        len(jobs), _p(q_idx), _p(w_idx), _p(k_codes), _p(k_scales), _p(n_entries), _p(q_pos0),
        _p(out), _stream(stream))
    _check(st, "csa_decode_index_scores_mxfp4")
    return out


def _scores_out(out, B, Tq, N_cap, device):
    if out is None:
        return torch.empty((B, Tq, N_cap), dtype=torch.float32, device=device)
    if tuple(out.shape) != (B, Tq, N_cap) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out is a contiguous float32 [B, Tq, N_cap] tensor")
    return out


def csa_index_scores(q_idx, w_idx, k_idx, n_entries, q_pos0, m, *, out=None, stream=None):
    """Indexer scores of the visible entries (no selection).  Returns scores
    [B, Tq, N_cap] float32; columns past a query's visible count are left as
    they were (uninitialised when ``out`` is not given)."""
    B, Tq, Hi, Di = q_idx.shape
    N_cap = k_idx.shape[1]
    _dev(q_idx, w_idx, k_idx, n_entries, q_pos0)
    _f32(w_idx), _i64(q_pos0)
    if n_entries.dtype != torch.int32:
        raise TypeError("n_entries is int32")
    if out is None:
        out = torch.empty((B, Tq, N_cap), dtype=torch.float32, device=q_idx.device)
    elif tuple(out.shape) != (B, Tq, N_cap) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out is a contiguous float32 [B, Tq, N_cap] tensor")
    st = lib().csa_index_scores(_dt(q_idx), B, Tq, Hi, Di, N_cap, m, _p(q_idx), _p(w_idx),
                                _p(k_idx), _p(n_entries), _p(q_pos0), _p(out), _stream(stream))
    _check(st, "csa_index_scores")
    return out


def csa_window_row(kv, pos, win, *, gain=None, eps=1e-6, rope_dims=0, rope_base=10000.0,
                   stream=None):
    """The new token's window row written into the ring win [B, L_win, D]
    at row pos[b] % L_win (see include/csa.h).  kv [B, 1, D]."""
    B, _, D = kv.shape
    _dev(kv, gain, pos, win)
    _f32(gain), _i64(pos)
    if win.dtype != kv.dtype or tuple(win.shape[::2]) != (B, D) or not win.is_contiguous():
        raise ValueError("win must be a contiguous [B, L_win, D] tensor of kv's dtype")
    st = lib().csa_window_row(_dt(kv), B, D, _p(kv), _p(gain), float(eps), int(rope_dims),
                              float(rope_base), _p(pos), _p(win), win.shape[1], _stream(stream))
    _check(st, "csa_window_row")
    return win


def csa_decode_advance(q_pos, n_entries, block_pos0, m, N_cap, *, stream=None):
    """One token forward on the device (see include/csa.h)."""
    _dev(q_pos, n_entries, block_pos0)
    _i64(q_pos), _i64(block_pos0)
    if n_entries.dtype != torch.int32:
        raise TypeError("n_entries is int32")
    st = lib().csa_decode_advance(q_pos.shape[0], int(m), int(N_cap), _p(q_pos), _p(n_entries),
                                  _p(block_pos0), _stream(stream))
    _check(st, "csa_decode_advance")


def csa_output_proj(o, w_a, w_b, *, mid=None, out=None, stream=None):
    """Grouped low-rank output projection (see include/csa.h).  o [T, H, D]
    bf16, w_a [G, r, (H/G) D], w_b [d, G r]; returns (out [T, d], mid [T, G r])."""
    T, H, D = o.shape
    G, r, ka = w_a.shape
    d = w_b.shape[0]
    _dev(o, w_a, w_b)
    for t in (o, w_a, w_b):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("o, w_a, w_b are contiguous bf16 tensors")
    if ka * G != H * D or w_b.shape[1] != G * r:
        raise ValueError("w_a must be [G, r, (H/G) D] and w_b [d, G r]")
    if mid is None:
        mid = torch.empty((T, G * r), dtype=torch.bfloat16, device=o.device)
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=o.device)
    st = lib().csa_output_proj(T, H, D, G, r, d, _p(o), _p(w_a), _p(w_b), _p(mid), _p(out),
                               _stream(stream))
    _check(st, "csa_output_proj")
    return out, mid


def csa_attn_ws_bytes(B, Tq, H, D, keys_per_query):
    return int(lib().csa_attn_ws_bytes(B, Tq, H, D, keys_per_query))


def csa_sparse_attn(q, pool, idx, win, win_pos0, W, sink, q_pos0, *, rope_dims, rope_base=10000.0,
                    scale=None, want_lse=False, out=None, ws=None, stream=None):
    """Sparse attention over idx-selected pool rows + window.  Returns (out, lse)."""
    B, Tq, H, D = q.shape
    N_cap = pool.shape[1]
    K = idx.shape[2]
    L_win = 0 if win is None else win.shape[1]
    _dev(q, pool, idx, win, win_pos0, sink, q_pos0)
    _f32(sink), _i64(q_pos0), _i64(win_pos0)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device) if want_lse else None
    need = csa_attn_ws_bytes(B, Tq, H, D, K + W)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib().csa_sparse_attn(_dt(q), B, Tq, H, D, int(rope_dims), float(rope_base), float(scale),
                               _p(q), _p(pool), N_cap, _p(idx), K, _p(win), L_win, _p(win_pos0),
                               int(W), _p(sink), _p(q_pos0), _p(out), _p(lse), _p(ws),
                               0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "csa_sparse_attn")
    return out, lse


def hca_attn(q, pool, n_entries, m, win, win_pos0, W, sink, q_pos0, *, rope_dims,
             rope_base=10000.0, scale=None, want_lse=False, out=None, ws=None, stream=None):
    """Dense attention over every visible pool entry + window.  Returns (out, lse)."""
    B, Tq, H, D = q.shape
    N_cap = pool.shape[1]
    L_win = 0 if win is None else win.shape[1]
    _dev(q, pool, n_entries, win, win_pos0, sink, q_pos0)
    _f32(sink), _i64(q_pos0), _i64(win_pos0)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device) if want_lse else None
    need = csa_attn_ws_bytes(B, Tq, H, D, N_cap + W)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib().hca_attn(_dt(q), B, Tq, H, D, int(rope_dims), float(rope_base), float(scale), _p(q),
                        _p(pool), N_cap, _p(n_entries), int(m), _p(win), L_win, _p(win_pos0),
                        int(W), _p(sink), _p(q_pos0), _p(out), _p(lse), _p(ws),
                        0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "hca_attn")
    return out, lse


def hca_decode_attn_ws_bytes(B, H, D, keys_per_query):
    return int(lib().hca_decode_attn_ws_bytes(B, H, D, keys_per_query))


def hca_decode_attn(q, pool, n_entries, m, c, z, bias, gain, block_pos0, win, win_pos0, W, sink,
                    q_pos0, *, rope_dims, rope_base=10000.0, eps=1e-6, scale=None,
                    want_lse=False, out=None, ws=None, stream=None, _fn="hca_decode_attn"):
    """One HCA decode step (see include/csa.h): the closing block c, z [B, m, D]
    is pooled into pool row min(n_entries, N_cap) - 1 where block_pos0 >= 0,
    and the query q [B, 1, H, D] attends to every visible entry + window.
    Returns (out, lse)."""
    B, Tq, H, D = q.shape
    if Tq != 1:
        raise ValueError("hca_decode_attn takes one query per sequence")
    if _fn == "hca_decode_attn_kvfp8":
        _fp8_pool(pool, D, rope_dims)
    elif pool.dtype != torch.bfloat16:
        raise TypeError("pool is bf16")
    N_cap = pool.shape[1]
    L_win = 0 if win is None else win.shape[1]
    _dev(q, pool, n_entries, c, z, bias, gain, block_pos0, win, win_pos0, sink, q_pos0)
    _f32(sink), _f32(bias), _f32(gain), _i64(q_pos0), _i64(win_pos0), _i64(block_pos0)
    for t in (q, c, z):
        if t is not None and t.dtype != torch.bfloat16:
            raise TypeError("q, c and z are bf16")
    if tuple(c.shape) != (B, m, D) or (z is not None and tuple(z.shape) != (B, m, D)):
        raise ValueError("c and z must be [B, m, D]")
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device) if want_lse else None
    need = hca_decode_attn_ws_bytes(B, H, D, N_cap + W)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = getattr(lib(), _fn)(B, H, D, int(rope_dims), float(rope_base), float(scale), _p(q),
                             _p(pool), N_cap, _p(n_entries), int(m), _p(c), _p(z), _p(bias),
                             _p(gain), float(eps), _p(block_pos0), _p(win), L_win,
                             _p(win_pos0), int(W), _p(sink), _p(q_pos0), _p(out), _p(lse),
                             _p(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(st, _fn)
    return out, lse


def hca_decode_attn_kvfp8(q, pool, n_entries, m, c, z, bias, gain, block_pos0, win, win_pos0, W,
                          sink, q_pos0, **kw):
    """hca_decode_attn with the pool as packed mixed BF16 / FP8 rows (uint8
    [B, N_cap, row_bytes]): the new entry is stored packed and attended as
    the values read back from its row."""
    return hca_decode_attn(q, pool, n_entries, m, c, z, bias, gain, block_pos0, win, win_pos0, W,
                           sink, q_pos0, _fn="hca_decode_attn_kvfp8", **kw)


def swa_decode_attn_ws_bytes(B, H, D, W):
    return int(lib().swa_decode_attn_ws_bytes(B, H, D, W))


def swa_decode_attn(q, kv, gain, win, win_pos0, W, sink, q_pos0, *, rope_dims,
                    rope_base=10000.0, eps=1e-6, scale=None, want_lse=False, out=None, ws=None,
                    stream=None):
    """One window-only decode step (see include/csa.h): the token's window
    row from kv [B, 1, D] is written into win (its ring slot when win_pos0 is
    None, else row q_pos0 - win_pos0), and q [B, 1, H, D] attends to the
    window.  Returns (out, lse)."""
    B, Tq, H, D = q.shape
    if Tq != 1:
        raise ValueError("swa_decode_attn takes one query per sequence")
    L_win = win.shape[1]
    _dev(q, kv, gain, win, win_pos0, sink, q_pos0)
    _f32(sink), _f32(gain), _i64(q_pos0), _i64(win_pos0)
    for t in (q, kv, win):
        if t.dtype != torch.bfloat16:
            raise TypeError("q, kv and win are bf16")
    if tuple(kv.shape) != (B, 1, D):
        raise ValueError("kv must be [B, 1, D]")
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device) if want_lse else None
    need = swa_decode_attn_ws_bytes(B, H, D, W)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib().swa_decode_attn(B, H, D, int(rope_dims), float(rope_base), float(scale), _p(q),
                               _p(kv), _p(gain), float(eps), _p(win), L_win, _p(win_pos0),
                               int(W), _p(sink), _p(q_pos0), _p(out), _p(lse), _p(ws),
                               0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "swa_decode_attn")
    return out, lse


# ------------------------------------------------- mixed BF16 / FP8 KV rows
def csa_kv_fp8_row_bytes(D, rope_dims):
    """Bytes of one packed mixed BF16 / FP8 KV row (0: shape not covered)."""
    return int(lib().csa_kv_fp8_row_bytes(int(D), int(rope_dims)))


def _fp8_pool(pool, D, rope_dims):
    rb = csa_kv_fp8_row_bytes(D, rope_dims)
    if rb == 0:
        raise ValueError("packed FP8 rows need D = 512 and rope_dims a multiple of 32")
    if pool.dtype != torch.uint8 or pool.dim() != 3 or pool.shape[2] != rb or not pool.is_contiguous():
        raise ValueError(f"pool must be contiguous uint8 [B, N_cap, {rb}]")
    return rb


def csa_quantize_kv_fp8(x, rope_dims, *, out=None, stream=None):
    """[..., D] float32/bf16 KV entries -> packed rows uint8 [..., row_bytes]."""
    _dev(x)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    D = x.shape[-1]
    rb = csa_kv_fp8_row_bytes(D, rope_dims)
    rows = x.numel() // D if D else 0
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (rb,), dtype=torch.uint8, device=x.device)
    st = lib().csa_quantize_kv_fp8(_dt(x), rows, D, int(rope_dims), _p(x), _p(out),
                                   _stream(stream))
    _check(st, "csa_quantize_kv_fp8")
    return out


def csa_dequantize_kv_fp8(rows_in, D, rope_dims, *, out=None, stream=None):
    """Packed rows [..., row_bytes] -> their values as bf16 [..., D]."""
    _dev(rows_in)
    rb = csa_kv_fp8_row_bytes(D, rope_dims)
    if rows_in.dtype != torch.uint8 or rows_in.shape[-1] != rb or not rows_in.is_contiguous():
        raise ValueError(f"rows must be contiguous uint8 [..., {rb}]")
    n = rows_in.numel() // rb
    if out is None:
        out = torch.empty(tuple(rows_in.shape[:-1]) + (D,), dtype=torch.bfloat16,
                          device=rows_in.device)
    st = lib().csa_dequantize_kv_fp8(n, int(D), int(rope_dims), _p(rows_in), _p(out),
                                     _stream(stream))
    _check(st, "csa_dequantize_kv_fp8")
    return out


def csa_compress_kvfp8(c_a, m, *, z_a=None, c_b=None, z_b=None, prev_c_b=None, prev_z_b=None,
                       bias_a=None, bias_b=None, gain=None, eps=1e-6, rope_dims=0,
                       rope_base=10000.0, pos0=None, out=None, out_bstride=0, ws=None,
                       stream=None):
    """csa_compress writing packed mixed BF16 / FP8 rows: returns out uint8
    [B, ceil(T/m), row_bytes] (or writes the caller's ``out``, batch stride
    ``out_bstride`` bytes)."""
    B, T, D = c_a.shape
    overlap = c_b is not None
    _dev(c_a, z_a, c_b, z_b, prev_c_b, prev_z_b, bias_a, bias_b, gain, pos0)
    _f32(bias_a), _f32(bias_b), _f32(gain), _i64(pos0)
    n_out = -(-T // m)
    rb = csa_kv_fp8_row_bytes(D, rope_dims)
    if out is None:
        out = torch.empty((B, n_out, rb), dtype=torch.uint8, device=c_a.device)
    else:
        bs = out_bstride if out_bstride else n_out * rb
        if (tuple(out.shape) != (B, n_out, rb) or out.dtype != torch.uint8 or not out.is_cuda
                or out.stride(2) != 1 or (n_out > 1 and out.stride(1) != rb)
                or (B > 1 and out.stride(0) != bs)):
            raise ValueError(f"out must be uint8 [B, ceil(T/m), {rb}] with batch stride "
                             "out_bstride (bytes)")
    need = csa_compress_ws_bytes(_dt(c_a), B, T, D, m, overlap)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=c_a.device)
    if ws is not None and ws.numel() == 0:
        ws = None
    st = lib().csa_compress_kvfp8(_dt(c_a), B, T, D, m, int(overlap), _p(c_a), _p(z_a), _p(c_b),
                                  _p(z_b), _p(prev_c_b), _p(prev_z_b), _p(bias_a), _p(bias_b),
                                  _p(gain), float(eps), int(rope_dims), float(rope_base),
                                  _p(pos0), _p(out), int(out_bstride), _p(ws),
                                  0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "csa_compress_kvfp8")
    return out


def csa_sparse_attn_kvfp8(q, pool, idx, win, win_pos0, W, sink, q_pos0, *, rope_dims,
                          rope_base=10000.0, scale=None, want_lse=False, out=None, ws=None,
                          stream=None):
    """csa_sparse_attn over packed mixed BF16 / FP8 pool rows."""
    B, Tq, H, D = q.shape
    _fp8_pool(pool, D, rope_dims)
    N_cap = pool.shape[1]
    K = idx.shape[2]
    L_win = 0 if win is None else win.shape[1]
    _dev(q, pool, idx, win, win_pos0, sink, q_pos0)
    _f32(sink), _i64(q_pos0), _i64(win_pos0)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device) if want_lse else None
    need = csa_attn_ws_bytes(B, Tq, H, D, K + W)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib().csa_sparse_attn_kvfp8(B, Tq, H, D, int(rope_dims), float(rope_base), float(scale),
                                     _p(q), _p(pool), N_cap, _p(idx), K, _p(win), L_win,
                                     _p(win_pos0), int(W), _p(sink), _p(q_pos0), _p(out), _p(lse),
                                     _p(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "csa_sparse_attn_kvfp8")
    return out, lse


def hca_attn_kvfp8(q, pool, n_entries, m, win, win_pos0, W, sink, q_pos0, *, rope_dims,
                   rope_base=10000.0, scale=None, want_lse=False, out=None, ws=None, stream=None):
    """hca_attn over packed mixed BF16 / FP8 pool rows."""
    B, Tq, H, D = q.shape
    _fp8_pool(pool, D, rope_dims)
    N_cap = pool.shape[1]
    L_win = 0 if win is None else win.shape[1]
    _dev(q, pool, n_entries, win, win_pos0, sink, q_pos0)
    _f32(sink), _i64(q_pos0), _i64(win_pos0)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device) if want_lse else None
    need = csa_attn_ws_bytes(B, Tq, H, D, N_cap + W)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib().hca_attn_kvfp8(B, Tq, H, D, int(rope_dims), float(rope_base), float(scale), _p(q),
                              _p(pool), N_cap, _p(n_entries), int(m), _p(win), L_win,
                              _p(win_pos0), int(W), _p(sink), _p(q_pos0), _p(out), _p(lse),
                              _p(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "hca_attn_kvfp8")
    return out, lse
