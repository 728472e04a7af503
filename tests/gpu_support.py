"""Shared helpers for the GPU parity tests: device inputs built from the seeded
generator, the library's configuration for a workload, oracle references
computed from the same generator on the host, and the error metric."""
from __future__ import annotations

import numpy as np
import torch

from synth import device as SD
from synth import workloads as W

_TABLES = {}
_WEIGHTS = {}


def H():
    import hashed_gram_embedding_amd as H
    return H


def config(w: W.Workload, layout: str = "mem_d", **over):
    kw = W.layer_config(w, layout)
    kw.update(over)
    return H().make_config(**kw)


def tdtype(w: W.Workload):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def to_device(values: np.ndarray, w: W.Workload):
    """Host storage (f32 or bf16 bits) -> device tensor of the workload dtype."""
    if w.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32)).cuda()
    bits = np.ascontiguousarray(values, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(bits).cuda().view(torch.bfloat16)


def to_storage(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host storage (f32 array or bf16 bits)."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.double().cpu().numpy()


def tables(w: W.Workload):
    key = (w.param_seed, tuple(w.rows()), w.row_dim, w.tdtype)
    if key not in _TABLES:
        # the Qwen-scale set is 95 GiB: keep at most one large set resident
        if sum(w.rows()) * w.row_dim > 1e9:
            for k in [k for k in _TABLES if sum(k[1]) * k[2] > 1e9]:
                del _TABLES[k]
            torch.cuda.empty_cache()
        _TABLES[key] = SD.make_tables(w)
    return _TABLES[key]


def weights(w: W.Workload, layout: str = "mem_d"):
    key = (w.param_seed, w.mem_dim, w.hidden, w.n_branches, w.dtype, layout)
    if key not in _WEIGHTS:
        _WEIGHTS[key] = SD.make_weights(w, layout=layout)
    return _WEIGHTS[key]


def host_weights(wk: torch.Tensor, wv: torch.Tensor, layout: str):
    """Device weights -> host storage in the oracle's [mem, d] orientation."""
    k, v = to_storage(wk), to_storage(wv)
    if layout == "d_mem":
        k, v = np.ascontiguousarray(k.transpose(0, 2, 1)), np.ascontiguousarray(v.T)
    return k, v


def conv_w(w):
    return to_device(W.conv_weight_values(w), w)


def gammas(w, random: bool):
    return {k: to_device(W.gamma_values(w, k, random), w) for k in "qku"}


def rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((y - ref).ravel()) / (den if den > 0 else 1.0))


TOL = 2e-3  # normwise relative error bound for floating-point outputs


def oracle_table_kw(w: W.Workload) -> dict:
    """The oracle's table arguments for a workload (storage dtype, scales)."""
    return dict(table_dtype=w.tdtype, table_scales=w.table_scales())


def oracle_rows(w: W.Workload):
    """Row provider for the oracle: rows regenerated on the host."""
    return lambda j, rows: W.table_row_values(w, j, rows)


def oracle_forward_window(orc, w, ids, hist, b, start, length, hidden_fn, wk_host, wv_host,
                          conv_host, gam=None, conv_state=None):
    """Oracle forward for positions [start, start+length) of sequence b,
    computed on the extended window [start-9, start+length) (the conv's halo)
    with the two ids before it as history."""
    halo = 3 * w.max_order
    s0 = max(0, start - halo)
    sub = ids[b:b + 1, s0:start + length]
    h0 = max(0, s0 - (w.max_order - 1))
    if s0 > 0:
        hist_sub = ids[b:b + 1, h0:s0]
    elif hist is not None:
        hist_sub = hist[b:b + 1]
    else:
        hist_sub = None
    T = ids.shape[1]
    toks = b * T + np.arange(s0, start + length)
    hid = hidden_fn(toks)
    kw = {}
    if gam is not None:
        kw = dict(gamma_q=gam["q"], gamma_k=gam["k"], gamma_u=gam["u"])
    out = orc.forward(sub, hist_sub, W.make_lut(w), w.vocab, w.vocab_compressed, w.orders,
                      w.heads, w.rows(), W.hash_multipliers(w), oracle_rows(w), hid, wk_host,
                      wv_host, conv_host, w.dtype, eps=w.rms_eps, conv_state=conv_state,
                      **oracle_table_kw(w), **kw)
    keep = slice(start - s0, start - s0 + length)
    return {k: (v[keep] if isinstance(v, np.ndarray) and v.ndim >= 2 and v.shape[0] == len(toks)
                else v) for k, v in out.items()}


def oracle_backward(orc, w, ids, hist, hidden_storage, wk_host, wv_host, conv_host, gam_storage,
                    d_out, conv_state, residual):
    """Oracle gradients for a whole (small) batch: hidden [n, nbh, d] storage,
    weights in the oracle's [mem, d] orientation, d_out float64 [n, nb, d]."""
    return orc.backward(ids, hist, W.make_lut(w), w.vocab, w.vocab_compressed, w.orders, w.heads,
                        w.rows(), W.hash_multipliers(w), oracle_rows(w), hidden_storage, wk_host,
                        wv_host, conv_host, w.dtype, d_out, gamma_q=gam_storage["q"],
                        gamma_k=gam_storage["k"], gamma_u=gam_storage["u"], eps=w.rms_eps,
                        conv_state=conv_state, add_residual=residual, **oracle_table_kw(w))
