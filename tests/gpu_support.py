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
# Per row (one token and branch) and per element: bf16 keeps 8 significand
# bits, so rounding to nearest moves an element by at most half an ulp, at
# most 2^-8 = 3.9e-3 of its own magnitude (at the bottom of a binade; 1.66e-3
# rms over a uniform spread of significands).  No row's normwise error, and no
# element's error relative to the largest reference element, can exceed that
# beyond the fp32 arithmetic's error (~1e-6); an element whose fp32 value
# lies next to a rounding midpoint rounds to the neighbour of the exact
# value's rounding, still within half an ulp plus that error.
ROW_TOL = 4e-3    # max over rows of the row's normwise relative error
MAX_TOL = 4e-3    # max |y - ref| / max |ref|


def errors(got, want):
    """(normwise, worst row's normwise, max-abs over max |ref|) errors of got
    against want; rows run along the last axis."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    e = rel_err(got, want)
    g2 = got.reshape(-1, want.shape[-1]) if want.ndim else got.reshape(1, 1)
    w2 = want.reshape(g2.shape)
    den = np.linalg.norm(w2, axis=1)
    num = np.linalg.norm(g2 - w2, axis=1)
    row = float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1.0), num)))
    peak = float(np.max(np.abs(want))) if want.size else 0.0
    mx = float(np.max(np.abs(got - want)) / (peak if peak > 0 else 1.0)) if want.size else 0.0
    return e, row, mx


def check(got, want, label: str = "", tol: float = TOL, row_tol: float = ROW_TOL,
          max_tol: float = MAX_TOL):
    """Assert the normwise, per-row and per-element bounds above."""
    e, row, mx = errors(got, want)
    print(f"   {label} rel_err {e:.3e} worst row {row:.3e} max-abs/max {mx:.3e}")
    assert e < tol and row < row_tol and mx < max_tol, (label, e, row, mx)


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


# ---------------------------------------------------------------------------
# the row ids and memory vector ngram_forward itself produced
# ---------------------------------------------------------------------------

def forward_ids_and_memory(cfg, w: W.Workload, B: int, T: int, ws: torch.Tensor):
    """Row ids [n, n_tables] (int32) and E [n, mem_dim] (the memory dtype) that
    the last ngram_forward left in its workspace ``ws`` (a uint8 tensor), as
    ngram_forward_workspace_view places them; decode's 16-token MFMA tiles
    are put back into rows."""
    v = H().ngram_forward_workspace_view(cfg, B, T)
    n = B * T
    rows = ws[v.row_idx_offset:v.row_idx_offset + 4 * n * w.n_tables].view(torch.int32)
    rows = rows.view(n, w.n_tables)
    mdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    es = 4 if w.dtype == "f32" else 2
    if v.mem_layout == H().MEM_TILES16:
        nblk = (n + 15) // 16
        raw = ws[v.mem_offset:v.mem_offset + nblk * 16 * w.mem_dim * es].view(mdt)
        # element ((blk * K/32 + kk) * 4 + q) * 128 + r * 8 + c holds token
        # 16 blk + r, value 32 kk + 8 q + c
        e = raw.view(nblk, w.mem_dim // 32, 4, 16, 8).permute(0, 3, 1, 2, 4)
        e = e.reshape(nblk * 16, w.mem_dim)[:n]
    else:
        e = ws[v.mem_offset:v.mem_offset + n * w.mem_dim * es].view(mdt).view(n, w.mem_dim)
    return rows, e


def oracle_row_ids(orc, w: W.Workload, ids, hist):
    """The oracle's compression and hashing of raw ids [B, T] (history raw
    [B, H] or None): row ids [B*T, n_tables]."""
    lut = W.make_lut(w)
    comp, _ = orc.compress(ids, lut, w.vocab, w.vocab_compressed)
    hc = orc.compress(hist, lut, w.vocab, w.vocab_compressed)[0] if hist is not None else None
    return orc.hash_rows(comp, hc, w.orders, w.heads, w.rows(), W.hash_multipliers(w))


def check_forward_ids_and_memory(orc, w: W.Workload, ids, hist, cfg, ws, sample: int = 160):
    """Bit-exact check of what the forward's own kernels produced: every
    token's row ids equal the oracle's hashing of its raw ids (compression,
    n-gram windows, history, pad); every token's E equals the concatenation
    of the table rows at those ids (fetched by torch on the device; fp8 rows
    decoded and scaled by torch's float8_e4m3fn conversion, then rounded to
    bf16); and a sample of tokens equals the oracle's own gather of rows
    regenerated on the host."""
    B, T = ids.shape
    got_rows, e = forward_ids_and_memory(cfg, w, B, T, ws)
    ref_rows = oracle_row_ids(orc, w, ids, hist)
    assert np.array_equal(got_rows.cpu().numpy(), ref_rows), "row ids"
    tabs = tables(w)
    d_rows = torch.from_numpy(ref_rows).cuda()
    bits = torch.int32 if w.dtype == "f32" else torch.int16
    for j in range(w.n_tables):
        want = tabs[j].index_select(0, d_rows[:, j].long())
        if w.tdtype == "fp8":
            want = (want.view(torch.float8_e4m3fn).float() * float(w.table_scales()[j])).bfloat16()
        got = e[:, j * w.row_dim:(j + 1) * w.row_dim]
        assert torch.equal(got.contiguous().view(bits), want.view(bits)), f"E table {j}"
    n = ref_rows.shape[0]
    rs = np.random.default_rng(11)
    pick = np.unique(np.concatenate([[0, n - 1], rs.integers(0, n, sample)]))
    e_ref = orc.gather_from_rows(ref_rows[pick], oracle_rows(w), w.tdtype,
                                 w.table_scales() if w.tdtype == "fp8" else None)
    assert np.array_equal(to_f64(e[torch.from_numpy(pick).cuda()]), e_ref), "E sample"
    print(f"   row ids and E of all {n} tokens bit-exact ({len(pick)} also against host rows)")
