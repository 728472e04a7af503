"""Thin ctypes binding of ``libngram.so`` (declared in ``include/ngram.h``).

Each function has the name of the C entry point it calls and only marshals
arguments: torch CUDA tensors become device pointers, the current torch
stream becomes the HIP stream, and a negative status raises ``NgramError``.
Every step of the layer runs in the library's HIP kernels; there is no other
code path.  If the library is missing the import fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

MAX_TABLES = 16
MAX_ORDER = 4
MAX_BRANCHES = 4
ADD_RESIDUAL = 1
UPDATE_STATE = 2
PREFETCHED = 4
KEEP_FOR_BACKWARD = 8    # the workspace holds the call's row ids and E (ngram_forward_prefetch)
MEM_ROWS, MEM_TILES16 = 0, 1  # layouts of E in the forward workspace
F32, BF16, FP8_E4M3 = 0, 1, 2  # FP8_E4M3: table storage only
W_MEM_D, W_D_MEM = 0, 1  # projection storage: [mem, d] or [d, mem] (fast path)

_HERE = os.path.dirname(os.path.abspath(__file__))
# NGRAM_LIBRARY names another build of the library (a variant under test);
# by default the in-tree build next to this file is loaded.
LIB_PATH = os.environ.get("NGRAM_LIBRARY") or os.path.join(_HERE, "libngram.so")


class NgramError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


class NgramConfig(ctypes.Structure):
    """Mirror of ``ngram_config`` (include/ngram.h)."""
    _fields_ = [
        ("n_orders", ctypes.c_int32),
        ("orders", ctypes.c_int32 * MAX_ORDER),
        ("heads_per_order", ctypes.c_int32),
        ("n_tables", ctypes.c_int32),
        ("rows", ctypes.c_int64 * MAX_TABLES),
        ("hash_mult", (ctypes.c_uint64 * MAX_ORDER) * MAX_TABLES),
        ("row_dim", ctypes.c_int32),
        ("mem_dim", ctypes.c_int32),
        ("hidden_dim", ctypes.c_int32),
        ("n_branches", ctypes.c_int32),
        ("conv_kernel", ctypes.c_int32),
        ("conv_dilation", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("vocab_compressed", ctypes.c_int32),
        ("pad_id", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("table_dtype", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("w_layout", ctypes.c_int32),
        ("table_scale", ctypes.c_float * MAX_TABLES),
        ("tune_proj_plan", ctypes.c_int32),
        ("tune_decode_ni", ctypes.c_int32),
        ("tune_decode_split", ctypes.c_int32),
    ]


class NgramWorkspaceView(ctypes.Structure):
    """Mirror of ``ngram_workspace_view`` (include/ngram.h)."""
    _fields_ = [
        ("row_idx_offset", ctypes.c_int64),
        ("mem_offset", ctypes.c_int64),
        ("mem_layout", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


def make_config(*, orders: Sequence[int], heads: int, rows: Sequence[int], hash_mult,
                row_dim: int, hidden_dim: int, n_branches: int, vocab: int,
                vocab_compressed: int, dtype: int, pad_id: int = 0, rms_eps: float = 1e-6,
                conv_kernel: int = 4, conv_dilation: Optional[int] = None,
                w_layout: int = W_MEM_D, table_dtype: Optional[int] = None,
                table_scales: Optional[Sequence[float]] = None, proj_plan: Optional[int] = None,
                decode_plan: Optional[Sequence[int]] = None) -> NgramConfig:
    """Fill an NgramConfig; ``hash_mult`` is indexable as [table][slot].
    ``dtype`` is the activation dtype and, unless ``table_dtype`` says
    otherwise (FP8_E4M3 with one scale per table), the tables' too.
    ``proj_plan`` (a prefill projection tile plan id) and ``decode_plan``
    ((ni, split) of the decode projection) override the library's tiling."""
    c = NgramConfig()
    c.n_orders = len(orders)
    for i, o in enumerate(orders):
        c.orders[i] = int(o)
    c.heads_per_order = heads
    c.n_tables = len(orders) * heads
    for j, r in enumerate(rows):
        c.rows[j] = int(r)
    for j in range(min(len(hash_mult), MAX_TABLES)):
        for i in range(MAX_ORDER):
            c.hash_mult[j][i] = int(hash_mult[j][i])
    c.row_dim = row_dim
    c.mem_dim = c.n_tables * row_dim
    c.hidden_dim = hidden_dim
    c.n_branches = n_branches
    c.conv_kernel = conv_kernel
    c.conv_dilation = max(orders) if conv_dilation is None else conv_dilation
    c.vocab = vocab
    c.vocab_compressed = vocab_compressed
    c.pad_id = pad_id
    c.rms_eps = rms_eps
    c.table_dtype = dtype if table_dtype is None else table_dtype
    c.act_dtype = dtype
    c.w_layout = w_layout
    for j, sc in enumerate(table_scales or ()):
        c.table_scale[j] = float(sc)
    c.tune_proj_plan = 0 if proj_plan is None else int(proj_plan) + 1
    if decode_plan is not None:
        c.tune_decode_ni, c.tune_decode_split = int(decode_plan[0]), int(decode_plan[1])
    return c


_lib = None
_p, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_cfgp = ctypes.POINTER(NgramConfig)

_SIGS = {
    "ngram_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "ngram_abi_version": (ctypes.c_int, []),
    "ngram_config_validate": (ctypes.c_int, [_cfgp]),
    "ngram_compress_ids": (ctypes.c_int, [_cfgp, _p, _i64, _p, _p, _p, _p]),
    "ngram_hash": (ctypes.c_int, [_cfgp, _p, _i32, _i32, _p, _p, _p]),
    "ngram_gather": (ctypes.c_int, [_cfgp, _p, _i64, _p, _p, _p]),
    "ngram_gate_workspace_size": (_sz, [_cfgp, _i64]),
    "ngram_gate": (ctypes.c_int, [_cfgp, _p, _i64, _p, _p, _p, _p, _p, _i64, _p, _p, _p, _sz, _p]),
    "ngram_causal_conv": (ctypes.c_int, [_cfgp, _p, _i32, _i32, _p, _p, _p, _p, _i32, _p, _p]),
    "ngram_forward_workspace_size": (_sz, [_cfgp, _i32, _i32]),
    "ngram_forward_workspace_view": (ctypes.c_int, [_cfgp, _i32, _i32,
                                                    ctypes.POINTER(NgramWorkspaceView)]),
    "ngram_backward_workspace_size": (_sz, [_cfgp, _i32, _i32]),
}
_FWD_ARGS = [_cfgp, _p, _i32, _i32, _p, _p, _p, _p, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _i32,
             _p, _p, _p, _p, _sz, _p]
_BWD_ARGS = [_cfgp, _p, _i32, _i32, _p, _p, _p, _p, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _i32,
             _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]
_SIGS["ngram_forward"] = (ctypes.c_int, _FWD_ARGS)
_SIGS["ngram_forward_timed"] = (ctypes.c_int, _FWD_ARGS + [_p, _p])
_SIGS["ngram_forward_noalloc"] = (ctypes.c_int, _FWD_ARGS[:-3] + [_p])
# cfg, raw_ids, B, T, history, lut, tables, err_flag, workspace, bytes, stream
_SIGS["ngram_forward_prefetch"] = (ctypes.c_int, [_cfgp, _p, _i32, _i32, _p, _p, _p, _p, _p,
                                                  ctypes.c_size_t, _p])
NOALLOC_SCRATCH_BYTES = 64 << 20  # NGRAM_NOALLOC_SCRATCH_BYTES
_SIGS["ngram_backward"] = (ctypes.c_int, _BWD_ARGS)
_SIGS["ngram_backward_timed"] = (ctypes.c_int, _BWD_ARGS + [_p, _p])


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().ngram_status_str(status).decode()


def abi_version() -> int:
    return lib().ngram_abi_version()


def ngram_config_validate(cfg: NgramConfig) -> int:
    return lib().ngram_config_validate(ctypes.byref(cfg))


N_STAGES = 4
STAGE_NAMES = ("hash", "gather", "projection", "gate_conv")


def _event_array(events):
    """2 * N_STAGES torch.cuda.Event (enable_timing=True) -> a HOST array of
    their hipEvent_t handles (torch creates a handle on its first record)."""
    if len(events) != 2 * N_STAGES:
        raise ValueError(f"need {2 * N_STAGES} events")
    for e in events:
        if not e.cuda_event:
            e.record()
    return (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not t.is_contiguous():
        raise ValueError("tensors passed to libngram must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise NgramError(status, where)


def _table_array(tables):
    arr = (ctypes.c_void_p * MAX_TABLES)()
    for j, t in enumerate(tables):
        arr[j] = t if isinstance(t, int) else (t.data_ptr() if t is not None else None)
    return arr


def _workspace(nbytes: int, device):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def ngram_compress_ids(cfg, raw_ids, lut, comp_ids, err_flag=None, stream=None):
    _check(lib().ngram_compress_ids(ctypes.byref(cfg), _ptr(raw_ids), raw_ids.numel(), _ptr(lut),
                                    _ptr(comp_ids), _ptr(err_flag), _stream(stream)),
           "ngram_compress_ids")
    return comp_ids


def ngram_hash(cfg, comp_ids, row_idx, history=None, stream=None):
    B, T = comp_ids.shape
    _check(lib().ngram_hash(ctypes.byref(cfg), _ptr(comp_ids), B, T, _ptr(history),
                            _ptr(row_idx), _stream(stream)), "ngram_hash")
    return row_idx


def ngram_gather(cfg, row_idx, tables, mem, stream=None):
    n_tok = row_idx.numel() // cfg.n_tables
    _check(lib().ngram_gather(ctypes.byref(cfg), _ptr(row_idx), n_tok, _table_array(tables),
                              _ptr(mem), _stream(stream)), "ngram_gather")
    return mem


def ngram_gate_workspace_size(cfg, n_tok: int) -> int:
    return int(lib().ngram_gate_workspace_size(ctypes.byref(cfg), n_tok))


def ngram_gate(cfg, hidden, hidden_branch_stride, mem, w_k, w_v, gates, u=None, gamma_q=None,
               gamma_k=None, workspace=None, stream=None):
    n_tok = mem.shape[0]
    need = ngram_gate_workspace_size(cfg, n_tok)
    if workspace is None:
        workspace = _workspace(need, mem.device)
    _check(lib().ngram_gate(ctypes.byref(cfg), _ptr(hidden), hidden_branch_stride, _ptr(mem),
                            _ptr(w_k), _ptr(w_v), _ptr(gamma_q), _ptr(gamma_k), n_tok,
                            _ptr(gates), _ptr(u), _ptr(workspace), workspace.numel(),
                            _stream(stream)), "ngram_gate")
    return gates, u


def ngram_causal_conv(cfg, u, B: int, T: int, conv_w, out, gamma_u=None, conv_state=None,
                      state_pos=None, flags: int = 0, stream=None):
    _check(lib().ngram_causal_conv(ctypes.byref(cfg), _ptr(u), B, T, _ptr(conv_w), _ptr(gamma_u),
                                   _ptr(conv_state), _ptr(state_pos), flags, _ptr(out),
                                   _stream(stream)), "ngram_causal_conv")
    return out


def ngram_forward_workspace_size(cfg, B: int, T: int) -> int:
    return int(lib().ngram_forward_workspace_size(ctypes.byref(cfg), B, T))


def ngram_forward_workspace_view(cfg, B: int, T: int) -> NgramWorkspaceView:
    """Where ngram_forward leaves the call's row ids and memory vector E in
    its workspace (byte offsets and the layout of E)."""
    v = NgramWorkspaceView()
    _check(lib().ngram_forward_workspace_view(ctypes.byref(cfg), B, T, ctypes.byref(v)),
           "ngram_forward_workspace_view")
    return v


def _forward_args(cfg, raw_ids, lut, tables, hidden, hidden_branch_stride, w_k, w_v, conv_w, out,
                  history, gamma_q, gamma_k, gamma_u, conv_state, state_pos, flags, gates,
                  err_flag, workspace, stream):
    B, T = raw_ids.shape
    if workspace is None:
        workspace = _workspace(ngram_forward_workspace_size(cfg, B, T), raw_ids.device)
    return (ctypes.byref(cfg), _ptr(raw_ids), B, T, _ptr(history), _ptr(lut), _table_array(tables),
            _ptr(hidden), hidden_branch_stride, _ptr(w_k), _ptr(w_v), _ptr(conv_w), _ptr(gamma_q),
            _ptr(gamma_k), _ptr(gamma_u), _ptr(conv_state), _ptr(state_pos), flags, _ptr(out),
            _ptr(gates), _ptr(err_flag), _ptr(workspace), workspace.numel(), _stream(stream))


def ngram_forward(cfg, raw_ids, lut, tables, hidden, hidden_branch_stride, w_k, w_v, conv_w, out,
                  history=None, gamma_q=None, gamma_k=None, gamma_u=None, conv_state=None,
                  state_pos=None, flags: int = 0, gates=None, err_flag=None, workspace=None,
                  stream=None):
    _check(lib().ngram_forward(*_forward_args(cfg, raw_ids, lut, tables, hidden,
                                              hidden_branch_stride, w_k, w_v, conv_w, out,
                                              history, gamma_q, gamma_k, gamma_u, conv_state,
                                              state_pos, flags, gates, err_flag, workspace,
                                              stream)), "ngram_forward")
    return out


def ngram_forward_prefetch(cfg, raw_ids, lut, tables, workspace, history=None, err_flag=None,
                           stream=None):
    """Steps 1-4 of ngram_forward into ``workspace`` (row ids and E), for a
    later ngram_forward(..., flags=PREFETCHED, workspace=workspace)."""
    B, T = raw_ids.shape
    _check(lib().ngram_forward_prefetch(ctypes.byref(cfg), _ptr(raw_ids), B, T, _ptr(history),
                                        _ptr(lut), _table_array(tables), _ptr(err_flag),
                                        _ptr(workspace), workspace.numel(), _stream(stream)),
           "ngram_forward_prefetch")
    return workspace


def ngram_forward_noalloc(cfg, raw_ids, lut, tables, hidden, hidden_branch_stride, w_k, w_v,
                          conv_w, out, history=None, gamma_q=None, gamma_k=None, gamma_u=None,
                          conv_state=None, state_pos=None, flags: int = 0, gates=None,
                          err_flag=None, stream=None):
    """ngram_forward without a workspace: the library's static per-GPU
    scratch serves instead (calls on one GPU must not overlap)."""
    B, T = raw_ids.shape
    _check(lib().ngram_forward_noalloc(ctypes.byref(cfg), _ptr(raw_ids), B, T, _ptr(history),
                                       _ptr(lut), _table_array(tables), _ptr(hidden),
                                       hidden_branch_stride, _ptr(w_k), _ptr(w_v), _ptr(conv_w),
                                       _ptr(gamma_q), _ptr(gamma_k), _ptr(gamma_u),
                                       _ptr(conv_state), _ptr(state_pos), flags, _ptr(out),
                                       _ptr(gates), _ptr(err_flag), _stream(stream)),
           "ngram_forward_noalloc")
    return out


def ngram_forward_timed(events, cfg, raw_ids, lut, tables, hidden, hidden_branch_stride, w_k, w_v,
                        conv_w, out, history=None, gamma_q=None, gamma_k=None, gamma_u=None,
                        conv_state=None, state_pos=None, flags: int = 0, gates=None,
                        err_flag=None, workspace=None, stream=None) -> int:
    """ngram_forward with each stage's kernels timed into ``events`` (2 *
    N_STAGES torch.cuda.Event); returns the mask of the stages that ran."""
    mask = ctypes.c_int32(0)
    _check(lib().ngram_forward_timed(*_forward_args(cfg, raw_ids, lut, tables, hidden,
                                                    hidden_branch_stride, w_k, w_v, conv_w, out,
                                                    history, gamma_q, gamma_k, gamma_u,
                                                    conv_state, state_pos, flags, gates, err_flag,
                                                    workspace, stream),
                                     _event_array(events), ctypes.byref(mask)),
           "ngram_forward_timed")
    return int(mask.value)


def ngram_backward_workspace_size(cfg, B: int, T: int) -> int:
    return int(lib().ngram_backward_workspace_size(ctypes.byref(cfg), B, T))


def _backward_args(cfg, raw_ids, lut, tables, hidden, hidden_branch_stride, w_k, w_v, conv_w,
                   d_out, d_tables, d_w_k, d_w_v, d_conv_w, history, gamma_q, gamma_k, gamma_u,
                   conv_state, state_pos, flags, d_hidden, d_gammas, workspace, stream):
    B, T = raw_ids.shape
    if workspace is None:
        workspace = _workspace(ngram_backward_workspace_size(cfg, B, T), raw_ids.device)
    return (ctypes.byref(cfg), _ptr(raw_ids), B, T, _ptr(history), _ptr(lut), _table_array(tables),
            _ptr(hidden), hidden_branch_stride, _ptr(w_k), _ptr(w_v), _ptr(conv_w), _ptr(gamma_q),
            _ptr(gamma_k), _ptr(gamma_u), _ptr(conv_state), _ptr(state_pos), flags, _ptr(d_out),
            _table_array(d_tables), _ptr(d_w_k), _ptr(d_w_v), _ptr(d_conv_w), _ptr(d_hidden),
            _ptr(d_gammas), _ptr(workspace), workspace.numel(), _stream(stream))


def ngram_backward(cfg, raw_ids, lut, tables, hidden, hidden_branch_stride, w_k, w_v, conv_w,
                   d_out, d_tables, d_w_k, d_w_v, d_conv_w, history=None, gamma_q=None,
                   gamma_k=None, gamma_u=None, conv_state=None, state_pos=None, flags: int = 0,
                   d_hidden=None, d_gammas=None, workspace=None, stream=None):
    """Gradients of sum(d_out * out); ``d_tables`` (fp32, one per table) are
    accumulated, the other gradient tensors written."""
    _check(lib().ngram_backward(*_backward_args(cfg, raw_ids, lut, tables, hidden,
                                                hidden_branch_stride, w_k, w_v, conv_w, d_out,
                                                d_tables, d_w_k, d_w_v, d_conv_w, history,
                                                gamma_q, gamma_k, gamma_u, conv_state, state_pos,
                                                flags, d_hidden, d_gammas, workspace, stream)),
           "ngram_backward")


def ngram_backward_timed(events, cfg, raw_ids, lut, tables, hidden, hidden_branch_stride, w_k,
                         w_v, conv_w, d_out, d_tables, d_w_k, d_w_v, d_conv_w, history=None,
                         gamma_q=None, gamma_k=None, gamma_u=None, conv_state=None,
                         state_pos=None, flags: int = 0, d_hidden=None, d_gammas=None,
                         workspace=None, stream=None) -> int:
    """ngram_backward with its four stages timed into ``events``; returns the
    mask of the stages that ran."""
    mask = ctypes.c_int32(0)
    _check(lib().ngram_backward_timed(*_backward_args(cfg, raw_ids, lut, tables, hidden,
                                                      hidden_branch_stride, w_k, w_v, conv_w,
                                                      d_out, d_tables, d_w_k, d_w_v, d_conv_w,
                                                      history, gamma_q, gamma_k, gamma_u,
                                                      conv_state, state_pos, flags, d_hidden,
                                                      d_gammas, workspace, stream),
                                      _event_array(events), ctypes.byref(mask)),
           "ngram_backward_timed")
    return int(mask.value)
