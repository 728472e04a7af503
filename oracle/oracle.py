"""ORACLE wrapper -- TEST INFRASTRUCTURE ONLY.

ctypes access to ``oracle/libngram_oracle.so`` (plain C, fp64, see
``ngram_oracle.c`` for the definition of every step and the passages it
follows) plus the composition of those steps into the layer's forward pass.
Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this module; the GPU library never does and shares nothing with it.

Inputs are numpy arrays in storage form: float32 arrays for fp32 tensors,
uint16 bit patterns for bf16 tensors (``dtype`` says which).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Callable, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libngram_oracle.so")
_DT = {"f32": 0, "bf16": 1, "fp8": 2}
_lib = None

_p = ctypes.c_void_p
_i32, _i64, _u64, _f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Temporarily route every step through another build of the oracle
    source (the mutation tests plant mistakes in a copy)."""
    global _lib
    saved = lib()
    _lib = _load(path)
    try:
        yield
    finally:
        _lib = saved


def _load(path: str):
    L = ctypes.CDLL(path)
    L.orc_num_threads.restype = ctypes.c_int
    L.orc_set_num_threads.argtypes = [ctypes.c_int]
    L.orc_compress.restype = _i64
    L.orc_compress.argtypes = [_p, _i64, _p, _i32, _i32, _i32, _p]
    L.orc_hash.argtypes = [_p, _i32, _i32, _p, _i32, _i32, _i32, _p, _i32, _p, _p, _p]
    L.orc_gather.argtypes = [_p, _i64, _i32, _p, _i32, _i32, _p, _p]
    L.orc_fp8_e4m3_value.restype = _f64
    L.orc_fp8_e4m3_value.argtypes = [ctypes.c_uint32]
    L.orc_project.argtypes = [_p, _i64, _i32, _p, _i32, _i32, _p]
    L.orc_gate.argtypes = [_p, _i32, _i64, _i64, _p, _i64, _i32, _i32, _p, _p, _f64, _p]
    L.orc_gated_value.argtypes = [_p, _p, _i64, _i32, _i32, _p]
    L.orc_conv_block.argtypes = [_p, _i32, _i32, _i32, _i32, _p, _i32, _i32, _i32, _p,
                                 _f64, _p, _p]
    L.orc_conv_block_backward.argtypes = [_p, _i32, _i32, _i32, _i32, _p, _i32, _i32, _i32, _p,
                                          _f64, _p, _p, _p, _p, _p]
    L.orc_gated_value_backward.argtypes = [_p, _p, _p, _i64, _i32, _i32, _p, _p]
    L.orc_gate_backward.argtypes = [_p, _i32, _i64, _i64, _p, _i64, _i32, _i32, _p, _p, _f64, _p,
                                    _p, _p, _p, _p]
    L.orc_project_backward.argtypes = [_p, _i64, _i32, _p, _i32, _i32, _p, _p, _p]
    L.orc_scatter_add.argtypes = [_p, _i64, _i32, _p, _i32, _p]
    L.orc_normalise_rows.argtypes = [_p, _i64, _i32, _p, _i32, _f64, _p]
    return L


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype=None):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


def _storage(a, dtype: str) -> np.ndarray:
    return _c(a, {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dtype])


def fp8_e4m3_value(byte: int) -> float:
    """The value an OCP FP8 E4M3 byte encodes."""
    return float(lib().orc_fp8_e4m3_value(int(byte)))


# ---------------------------------------------------------------------------
# the steps
# ---------------------------------------------------------------------------

def compress(raw, lut, vocab: int, vocab_c: int, pad_id: int = 0):
    raw, lut = _c(raw, np.int32), _c(lut, np.int32)
    out = np.empty_like(raw)
    bad = lib().orc_compress(_ptr(raw), raw.size, _ptr(lut), vocab, vocab_c, pad_id, _ptr(out))
    return out, int(bad)


def hash_rows(comp, hist, orders: Sequence[int], heads: int, rows: Sequence[int], mult,
              pad_id: int = 0) -> np.ndarray:
    """comp int32[B, T]; hist int32[B, H] compressed ids or None -> int32[B*T, n_tables]."""
    comp = _c(comp, np.int32)
    B, T = comp.shape
    hist = _c(hist, np.int32)
    H = 0 if hist is None else hist.shape[1]
    orders_a = _c(list(orders), np.int32)
    rows_a = _c(list(rows), np.int64)
    mult = _c(mult, np.uint64).reshape(-1, 4)
    nt = len(orders) * heads
    out = np.empty((B * T, nt), dtype=np.int32)
    lib().orc_hash(_ptr(comp), B, T, _ptr(hist), H, pad_id, len(orders), _ptr(orders_a), heads,
                   _ptr(rows_a), _ptr(mult), _ptr(out))
    return out


def gather(row_idx, tables: Sequence[np.ndarray], dtype: str, scales=None) -> np.ndarray:
    """row_idx int32[n, nt]; tables[j] [rows_j, row_dim] storage -> float64[n, mem].
    ``dtype`` "fp8" takes uint8 E4M3 tables and one float32 scale per table."""
    row_idx = _c(row_idx, np.int32)
    n, nt = row_idx.shape
    tabs = [_storage(t, dtype) for t in tables]
    row_dim = tabs[0].shape[1]
    ptrs = (ctypes.c_void_p * nt)(*[t.ctypes.data for t in tabs])
    sc = None if scales is None else _c(list(scales), np.float32)
    if dtype == "fp8" and (sc is None or sc.size < nt):
        raise ValueError("fp8 tables need one scale per table")
    e = np.empty((n, nt * row_dim), dtype=np.float64)
    lib().orc_gather(_ptr(row_idx), n, nt, ptrs, _DT[dtype], row_dim, _ptr(sc), _ptr(e))
    return e


def gather_from_rows(row_idx, provider: Callable[[int, np.ndarray], np.ndarray],
                     dtype: str, scales=None) -> np.ndarray:
    """Gather when the tables are too large to hold: ``provider(j, rows)`` returns
    the storage of rows ``rows`` of table j; the oracle indexes a compact copy."""
    row_idx = _c(row_idx, np.int32)
    compact, remap = [], np.empty_like(row_idx)
    for j in range(row_idx.shape[1]):
        uniq, inv = np.unique(row_idx[:, j], return_inverse=True)
        compact.append(provider(j, uniq))
        remap[:, j] = inv.reshape(-1)
    return gather(remap, compact, dtype, scales)


def project(e, w, dtype: str) -> np.ndarray:
    e = _c(e, np.float64)
    w = _storage(w, dtype)
    mem, d = w.shape
    out = np.empty((e.shape[0], d), dtype=np.float64)
    lib().orc_project(_ptr(e), e.shape[0], mem, _ptr(w), _DT[dtype], d, _ptr(out))
    return out


def gate(hidden, dtype: str, k, gamma_q=None, gamma_k=None, eps: float = 1e-6) -> np.ndarray:
    """hidden [n, nbh, d] storage (nbh = 1: shared query); k float64[n, nb, d]."""
    hidden = _storage(hidden, dtype)
    k = _c(k, np.float64)
    n, nb, d = k.shape
    nbh = hidden.shape[1]
    bstride = 0 if nbh == 1 else d
    out = np.empty((n, nb), dtype=np.float64)
    lib().orc_gate(_ptr(hidden), _DT[dtype], nbh * d, bstride, _ptr(k), n, nb, d,
                   _ptr(_storage(gamma_q, dtype) if gamma_q is not None else None),
                   _ptr(_storage(gamma_k, dtype) if gamma_k is not None else None),
                   eps, _ptr(out))
    return out


def gated_value(g, v) -> np.ndarray:
    g, v = _c(g, np.float64), _c(v, np.float64)
    n, nb = g.shape
    d = v.shape[1]
    u = np.empty((n, nb, d), dtype=np.float64)
    lib().orc_gated_value(_ptr(g), _ptr(v), n, nb, d, _ptr(u))
    return u


def conv_block(u, conv_w, dtype: str, dilation: int, gamma_u=None, eps: float = 1e-6,
               state=None) -> np.ndarray:
    """u float64[B, T, nb, d]; conv_w [kernel, d] storage; state float64
    [B, (kernel-1)*dilation, nb, d] of normalised rows or None."""
    u = _c(u, np.float64)
    B, T, nb, d = u.shape
    w = _storage(conv_w, dtype)
    kernel = w.shape[0]
    st = _c(state, np.float64)
    out = np.empty_like(u)
    lib().orc_conv_block(_ptr(u), B, T, nb, d, _ptr(w), _DT[dtype], kernel, dilation,
                         _ptr(_storage(gamma_u, dtype) if gamma_u is not None else None),
                         eps, _ptr(st), _ptr(out))
    return out


def normalised_rows(u, gamma_u=None, dtype: str = "f32", eps: float = 1e-6) -> np.ndarray:
    """RMSNorm of each row of u (float64[..., d]): gamma_u (.) u / rms(u), the
    rows the convolution reads (and a conv-state ring holds)."""
    u = _c(u, np.float64)
    d = u.shape[-1]
    out = np.empty_like(u)
    lib().orc_normalise_rows(_ptr(u), u.size // d, d,
                             _ptr(_storage(gamma_u, dtype) if gamma_u is not None else None),
                             _DT[dtype], eps, _ptr(out))
    return out


# ---------------------------------------------------------------------------
# the layer's forward pass, step by step
# ---------------------------------------------------------------------------

def forward(raw, hist_raw, lut, vocab: int, vocab_c: int, orders, heads: int, rows, mult,
            tables_or_provider, hidden, wk, wv, conv_w, dtype: str, *, gamma_q=None,
            gamma_k=None, gamma_u=None, eps: float = 1e-6, conv_state=None, pad_id: int = 0,
            table_dtype: Optional[str] = None, table_scales=None):
    """Full forward on raw ids int32[B, T] (history raw int32[B, H] or None).

    ``tables_or_provider``: list of full tables, or ``provider(j, rows)``, in
    ``table_dtype`` (default ``dtype``; "fp8" with ``table_scales``).
    hidden: [B*T, nbh, d] storage; wk: [nb, mem, d]; wv: [mem, d]; conv_w: [4, d].
    Returns a dict with every intermediate (float64 where floating point).
    """
    raw = _c(raw, np.int32)
    B, T = raw.shape
    comp, bad = compress(raw, lut, vocab, vocab_c, pad_id)
    hist_c = None
    if hist_raw is not None:
        hist_c, bad_h = compress(hist_raw, lut, vocab, vocab_c, pad_id)
        bad += bad_h
    r = hash_rows(comp, hist_c, orders, heads, rows, mult, pad_id)
    tdt = table_dtype or dtype
    if callable(tables_or_provider):
        e = gather_from_rows(r, tables_or_provider, tdt, table_scales)
    else:
        e = gather(r, tables_or_provider, tdt, table_scales)
    wk = np.asarray(wk)
    nb = wk.shape[0]
    k = np.stack([project(e, wk[b], dtype) for b in range(nb)], axis=1)
    v = project(e, wv, dtype)
    g = gate(hidden, dtype, k, gamma_q, gamma_k, eps)
    u = gated_value(g, v)
    d = v.shape[1]
    delta = conv_block(u.reshape(B, T, nb, d), conv_w, dtype, max(orders), gamma_u, eps,
                       conv_state)
    return {"comp": comp, "bad": bad, "row_idx": r, "e": e, "k": k, "v": v, "gate": g,
            "u": u, "delta": delta.reshape(B * T, nb, d)}


# ---------------------------------------------------------------------------
# the layer's backward pass (gradients of L = sum(d_out * out))
# ---------------------------------------------------------------------------

def conv_block_backward(u, conv_w, dtype: str, dilation: int, d_delta, gamma_u=None,
                        eps: float = 1e-6, state=None):
    """u, d_delta float64[B, T, nb, d] -> (d_u, d_conv_w [kernel, d], d_gamma_u [d])."""
    u, dd = _c(u, np.float64), _c(d_delta, np.float64)
    B, T, nb, d = u.shape
    w = _storage(conv_w, dtype)
    kernel = w.shape[0]
    st = _c(state, np.float64)
    d_u = np.empty_like(u)
    d_w = np.zeros((kernel, d), dtype=np.float64)
    d_g = np.zeros(d, dtype=np.float64)
    lib().orc_conv_block_backward(_ptr(u), B, T, nb, d, _ptr(w), _DT[dtype], kernel, dilation,
                                  _ptr(_storage(gamma_u, dtype) if gamma_u is not None else None),
                                  eps, _ptr(st), _ptr(dd), _ptr(d_u), _ptr(d_w), _ptr(d_g))
    return d_u, d_w, d_g


def gated_value_backward(g, v, d_u):
    """g [n, nb], v [n, d], d_u [n, nb, d] -> (d_gate [n, nb], d_v [n, d])."""
    g, v, d_u = _c(g, np.float64), _c(v, np.float64), _c(d_u, np.float64)
    n, nb = g.shape
    d = v.shape[1]
    d_g = np.empty((n, nb), dtype=np.float64)
    d_v = np.empty((n, d), dtype=np.float64)
    lib().orc_gated_value_backward(_ptr(g), _ptr(v), _ptr(d_u), n, nb, d, _ptr(d_g), _ptr(d_v))
    return d_g, d_v


def gate_backward(hidden, dtype: str, k, d_gate, gamma_q=None, gamma_k=None, eps: float = 1e-6):
    """hidden [n, nbh, d] storage; k float64[n, nb, d]; d_gate [n, nb] ->
    (d_k [n, nb, d], d_hidden [n, nbh, d], d_gamma_q [d], d_gamma_k [d])."""
    hidden = _storage(hidden, dtype)
    k, dg = _c(k, np.float64), _c(d_gate, np.float64)
    n, nb, d = k.shape
    nbh = hidden.shape[1]
    bstride = 0 if nbh == 1 else d
    d_k = np.empty_like(k)
    d_h = np.zeros((n, nbh, d), dtype=np.float64)
    d_gq = np.zeros(d, dtype=np.float64)
    d_gk = np.zeros(d, dtype=np.float64)
    lib().orc_gate_backward(_ptr(hidden), _DT[dtype], nbh * d, bstride, _ptr(k), n, nb, d,
                            _ptr(_storage(gamma_q, dtype) if gamma_q is not None else None),
                            _ptr(_storage(gamma_k, dtype) if gamma_k is not None else None),
                            eps, _ptr(dg), _ptr(d_k), _ptr(d_h), _ptr(d_gq), _ptr(d_gk))
    return d_k, d_h, d_gq, d_gk


def project_backward(e, w, dtype: str, d_out, d_e):
    """out = e @ w (w [mem, d] storage): adds d_out @ w.T into d_e [n, mem] and
    returns d_w = e.T @ d_out [mem, d]."""
    e, d_out = _c(e, np.float64), _c(d_out, np.float64)
    w = _storage(w, dtype)
    mem, d = w.shape
    assert d_e.flags.c_contiguous and d_e.dtype == np.float64
    d_w = np.zeros((mem, d), dtype=np.float64)
    lib().orc_project_backward(_ptr(e), e.shape[0], mem, _ptr(w), _DT[dtype], d, _ptr(d_out),
                               _ptr(d_e), _ptr(d_w))
    return d_w


def scatter_add(row_idx, d_e, row_dim: int):
    """Table gradients of the gather: for each table j, (rows, grads): the
    distinct rows its tokens hit and the summed d_e slices [len(rows), row_dim]."""
    row_idx = _c(row_idx, np.int32)
    d_e = _c(d_e, np.float64)
    n, nt = row_idx.shape
    rows, compact, remap = [], [], np.empty_like(row_idx)
    for j in range(nt):
        uniq, inv = np.unique(row_idx[:, j], return_inverse=True)
        rows.append(uniq)
        compact.append(np.zeros((len(uniq), row_dim), dtype=np.float64))
        remap[:, j] = inv.reshape(-1)
    ptrs = (ctypes.c_void_p * nt)(*[c.ctypes.data for c in compact])
    lib().orc_scatter_add(_ptr(remap), n, nt, _ptr(d_e), row_dim, ptrs)
    return list(zip(rows, compact))


def backward(raw, hist_raw, lut, vocab: int, vocab_c: int, orders, heads: int, rows, mult,
             tables_or_provider, hidden, wk, wv, conv_w, dtype: str, d_out, *, gamma_q=None,
             gamma_k=None, gamma_u=None, eps: float = 1e-6, conv_state=None, pad_id: int = 0,
             table_dtype: Optional[str] = None, table_scales=None, add_residual: bool = False):
    """Gradients of L = sum(d_out * out) for the forward above (out = Delta, or
    hidden + Delta with ``add_residual``).  d_out: [B*T, nb, d].  Returns the
    forward's dict plus d_tables (per table: rows hit, summed gradients),
    d_wk [nb, mem, d], d_wv [mem, d], d_conv_w [kernel, d], d_hidden [B*T, nbh, d],
    d_gamma_q, d_gamma_k, d_gamma_u [d] (float64)."""
    f = forward(raw, hist_raw, lut, vocab, vocab_c, orders, heads, rows, mult, tables_or_provider,
                hidden, wk, wv, conv_w, dtype, gamma_q=gamma_q, gamma_k=gamma_k, gamma_u=gamma_u,
                eps=eps, conv_state=conv_state, pad_id=pad_id, table_dtype=table_dtype,
                table_scales=table_scales)
    raw = _c(raw, np.int32)
    B, T = raw.shape
    wk = np.asarray(wk)
    nb = wk.shape[0]
    d = wk.shape[2]
    d_out = _c(d_out, np.float64).reshape(B * T, nb, d)
    d_u, d_conv_w, d_gamma_u = conv_block_backward(f["u"].reshape(B, T, nb, d), conv_w, dtype,
                                                   max(orders), d_out.reshape(B, T, nb, d),
                                                   gamma_u, eps, conv_state)
    d_gate, d_v = gated_value_backward(f["gate"], f["v"], d_u.reshape(B * T, nb, d))
    d_k, d_hidden, d_gamma_q, d_gamma_k = gate_backward(hidden, dtype, f["k"], d_gate, gamma_q,
                                                        gamma_k, eps)
    if add_residual:  # out[t, b] = hidden row of branch b (or the shared row) + Delta
        if d_hidden.shape[1] == 1:
            d_hidden[:, 0] += d_out.sum(axis=1)
        else:
            d_hidden += d_out
    e = f["e"]
    d_e = np.zeros_like(e)
    d_wk = np.stack([project_backward(e, wk[b], dtype, d_k[:, b], d_e) for b in range(nb)])
    d_wv = project_backward(e, wv, dtype, d_v, d_e)
    d_tables = scatter_add(f["row_idx"], d_e, e.shape[1] // len(rows))
    f.update(d_tables=d_tables, d_wk=d_wk, d_wv=d_wv, d_conv_w=d_conv_w, d_hidden=d_hidden,
             d_gamma_q=d_gamma_q, d_gamma_k=d_gamma_k, d_gamma_u=d_gamma_u, d_e=d_e,
             d_k=d_k, d_v=d_v, d_gate=d_gate, d_u=d_u)
    return f
