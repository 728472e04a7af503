"""GPU fill of the large synthetic tensors (same bits as ``synth.rng``).

Used by the tests and the benchmark to put the hash tables, hidden states and
projection weights straight into device memory; a host slice of any of them
is regenerated with ``synth.workloads.*_values``.
"""
from __future__ import annotations

import ctypes
import os

from . import rng
from .workloads import Workload, hidden_rows_per_token

_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libngram_synth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing; run synth/build.py (or __graft_entry__.build())")
        L = ctypes.CDLL(path)
        L.synth_fill_normal.restype = ctypes.c_int
        L.synth_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                        ctypes.c_uint64, ctypes.c_int64, ctypes.c_float,
                                        ctypes.c_void_p]
        L.synth_fill_normal_fp8.restype = ctypes.c_int
        L.synth_fill_normal_fp8.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                            ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                                            ctypes.c_void_p]
        _LIB = L
    return _LIB


def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def fill_normal(t, seed: int, sigma: float, offset: int = 0, stream=None):
    """Fill a contiguous fp32/bf16 CUDA tensor with normal draws ``offset..``."""
    import torch
    assert t.is_cuda and t.is_contiguous()
    dtype = {torch.float32: 0, torch.bfloat16: 1}[t.dtype]
    rc = lib().synth_fill_normal(ctypes.c_void_p(t.data_ptr()), dtype, t.numel(),
                                 ctypes.c_uint64(seed & ((1 << 64) - 1)), offset,
                                 ctypes.c_float(float(rng.normal_scale(sigma))),
                                 _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal failed ({rc})")
    return t


def fill_normal_fp8(t, seed: int, sigma: float, inv_scale: float, offset: int = 0, stream=None):
    """Fill a contiguous uint8 CUDA tensor with E4M3 codes of normal draws * inv_scale."""
    import torch
    assert t.is_cuda and t.is_contiguous() and t.dtype == torch.uint8
    rc = lib().synth_fill_normal_fp8(ctypes.c_void_p(t.data_ptr()), t.numel(),
                                     ctypes.c_uint64(seed & ((1 << 64) - 1)), offset,
                                     ctypes.c_float(float(rng.normal_scale(sigma))),
                                     ctypes.c_float(float(inv_scale)), _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal_fp8 failed ({rc})")
    return t


def torch_dtype(w: Workload):
    import torch
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def make_tables(w: Workload, device="cuda"):
    import torch
    out = []
    for j, r in enumerate(w.rows()):
        if w.tdtype == "fp8":
            t = torch.empty((r, w.row_dim), dtype=torch.uint8, device=device)
            out.append(fill_normal_fp8(t, w.table_seed(j), w.table_sigma, 1.0 / w.table_scale))
        else:
            t = torch.empty((r, w.row_dim), dtype=torch_dtype(w), device=device)
            out.append(fill_normal(t, w.table_seed(j), w.table_sigma))
    return out


def make_hidden(w: Workload, n_tokens: int, batch_id: int = 0, device="cuda"):
    import torch
    nbh = hidden_rows_per_token(w)
    t = torch.empty((n_tokens, nbh, w.hidden), dtype=torch_dtype(w), device=device)
    return fill_normal(t, w.hidden_seed(batch_id), w.hidden_sigma)


def make_weights(w: Workload, device="cuda", layout: str = "mem_d"):
    """(W_K, W_V) on the device: [nb, mem, d] and [mem, d] for layout
    'mem_d'; the same matrices stored transposed ([nb, d, mem], [d, mem])
    for layout 'd_mem'."""
    import torch
    wk = torch.empty((w.n_branches, w.mem_dim, w.hidden), dtype=torch_dtype(w), device=device)
    for b in range(w.n_branches):
        fill_normal(wk[b], w.wk_seed(b), w.w_sigma)
    wv = torch.empty((w.mem_dim, w.hidden), dtype=torch_dtype(w), device=device)
    fill_normal(wv, w.wv_seed(), w.w_sigma)
    if layout == "d_mem":
        wk = wk.transpose(1, 2).contiguous()
        wv = wv.t().contiguous()
    elif layout != "mem_d":
        raise ValueError(layout)
    return wk, wv
