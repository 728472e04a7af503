"""Op-level parity of the C-ABI entry points against the oracle: compressed
ids, hash rows and gathered memory bit-exact on every token of every
workload; gates, U and the conv block within the normwise tolerance."""
import numpy as np
import pytest
import torch

import gpu_support as G
from synth import rng
from synth import workloads as W

pytestmark = pytest.mark.gpu

ALL = ["tiny", "engram_small", "qwen_decode", "qwen_prefill", "qwen_multibranch_uniform",
       "qwen_multibranch_zipf13"]


def _ids(w):
    ids, hist = W.make_ids(w)
    return ids, hist


@pytest.mark.parametrize("name", ALL)
def test_compress_and_hash_bit_exact(orc, name):
    H = G.H()
    w = W.get(name)
    print(f"[compress+hash] {name}", flush=True)
    cfg = G.config(w)
    ids, hist = _ids(w)
    lut = W.make_lut(w)
    d_ids = torch.from_numpy(ids).cuda()
    d_lut = torch.from_numpy(lut).cuda()
    comp = torch.empty_like(d_ids)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    H.ngram_compress_ids(cfg, d_ids, d_lut, comp, err)
    ref_comp, bad = orc.compress(ids, lut, w.vocab, w.vocab_compressed)
    assert bad == 0 and err.item() == 0
    assert np.array_equal(comp.cpu().numpy(), ref_comp)
    d_hist = None
    ref_hist = None
    if hist is not None:
        ref_hist, _ = orc.compress(hist, lut, w.vocab, w.vocab_compressed)
        d_hist = torch.from_numpy(ref_hist).cuda()
    rows = torch.empty((ids.size, w.n_tables), dtype=torch.int32, device="cuda")
    H.ngram_hash(cfg, comp, rows, history=d_hist)
    ref = orc.hash_rows(ref_comp, ref_hist, w.orders, w.heads, w.rows(), W.hash_multipliers(w))
    assert np.array_equal(rows.cpu().numpy(), ref)


def test_compress_invalid_ids_flag_and_pad(orc):
    H = G.H()
    w = W.get("tiny")
    cfg = G.config(w)
    lut = W.make_lut(w)
    ids = np.array([5, -3, 999, 1000, 123456, 0, 17], dtype=np.int32)
    comp = torch.empty(7, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    H.ngram_compress_ids(cfg, torch.from_numpy(ids).cuda(), torch.from_numpy(lut).cuda(), comp, err)
    ref, bad = orc.compress(ids, lut, w.vocab, w.vocab_compressed)
    assert bad == 3 and err.item() == 1
    assert np.array_equal(comp.cpu().numpy(), ref)


@pytest.mark.parametrize("name", ["tiny", "engram_small", "qwen_decode", "qwen_prefill",
                                  "qwen_multibranch_uniform", "qwen_multibranch_zipf13"])
def test_gather_bit_exact(orc, name):
    """Every token's memory vector equals the concatenation of the table rows
    at the oracle's row ids (checked on the device for all tokens with torch
    indexing, and against host-regenerated rows on a sample)."""
    H = G.H()
    w = W.get(name)
    print(f"[gather] {name}", flush=True)
    cfg = G.config(w)
    ids, hist = _ids(w)
    lut = W.make_lut(w)
    comp, _ = orc.compress(ids, lut, w.vocab, w.vocab_compressed)
    hc = orc.compress(hist, lut, w.vocab, w.vocab_compressed)[0] if hist is not None else None
    ref_rows = orc.hash_rows(comp, hc, w.orders, w.heads, w.rows(), W.hash_multipliers(w))
    tabs = G.tables(w)
    d_rows = torch.from_numpy(ref_rows).cuda()
    n = ref_rows.shape[0]
    mem = torch.empty((n, w.mem_dim), dtype=G.tdtype(w), device="cuda")
    H.ngram_gather(cfg, d_rows, tabs, mem)
    torch.cuda.synchronize()
    # all tokens: the rows the oracle names, fetched by torch
    for j in range(w.n_tables):
        want = tabs[j].index_select(0, d_rows[:, j].long())
        got = mem[:, j * w.row_dim:(j + 1) * w.row_dim]
        assert torch.equal(got.view(torch.int16) if w.dtype == "bf16" else got.view(torch.int32),
                           want.view(torch.int16) if w.dtype == "bf16" else want.view(torch.int32)), j
    # sample: the oracle's own gather of host-regenerated rows
    rs = np.random.default_rng(3)
    sample = np.unique(np.concatenate([[0, n - 1], rs.integers(0, n, 200)]))
    e_ref = orc.gather_from_rows(ref_rows[sample], G.oracle_rows(w), w.dtype)
    assert np.array_equal(G.to_f64(mem[torch.from_numpy(sample).cuda()]), e_ref)


@pytest.mark.parametrize("name", ["engram_small_fp8", "qwen_decode_fp8"])
def test_gather_fp8_bit_exact(orc, name):
    """FP8 tables: every token's E equals the E4M3 values at the oracle's row
    ids times the table's scale, rounded to bf16 (torch's conversions on the
    device, all tokens), and the oracle's own gather on a sample."""
    H = G.H()
    w = (W.get("engram_small").replace(table_dtype="fp8") if name == "engram_small_fp8"
         else W.get(name))
    print(f"[gather fp8] {name}", flush=True)
    cfg = G.config(w)
    ids, hist = _ids(w)
    lut = W.make_lut(w)
    comp, _ = orc.compress(ids, lut, w.vocab, w.vocab_compressed)
    hc = orc.compress(hist, lut, w.vocab, w.vocab_compressed)[0] if hist is not None else None
    ref_rows = orc.hash_rows(comp, hc, w.orders, w.heads, w.rows(), W.hash_multipliers(w))
    tabs = G.tables(w)
    d_rows = torch.from_numpy(ref_rows).cuda()
    n = ref_rows.shape[0]
    mem = torch.empty((n, w.mem_dim), dtype=torch.bfloat16, device="cuda")
    H.ngram_gather(cfg, d_rows, tabs, mem)
    torch.cuda.synchronize()
    scale = torch.tensor(w.table_scale, dtype=torch.float32, device="cuda")
    for j in range(w.n_tables):
        codes = tabs[j].index_select(0, d_rows[:, j].long())
        want = (codes.view(torch.float8_e4m3fn).float() * scale).bfloat16()
        got = mem[:, j * w.row_dim:(j + 1) * w.row_dim]
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), j
    rs = np.random.default_rng(4)
    sample = np.unique(np.concatenate([[0, n - 1], rs.integers(0, n, 200)]))
    e_ref = orc.gather_from_rows(ref_rows[sample], G.oracle_rows(w), "fp8", w.table_scales())
    assert np.array_equal(G.to_f64(mem[torch.from_numpy(sample).cuda()]), e_ref)


def _synthetic_memory(w, n, seed):
    """E for op-level gate tests: N(0, 0.02) values of the table dtype."""
    return rng.normal_values(seed, np.arange(n * w.mem_dim), 0.02, w.dtype).reshape(n, w.mem_dim)


@pytest.mark.parametrize("name,n,shared,random_gamma,layout", [
    ("tiny", 256, True, False, "mem_d"),
    ("tiny", 37, True, True, "d_mem"),
    ("engram_small", 300, True, False, "mem_d"),
    ("engram_small", 1500, True, True, "mem_d"),
    ("engram_small", 700, True, True, "d_mem"),
    ("qwen_decode", 256, True, False, "mem_d"),
    ("qwen_decode", 256, True, False, "d_mem"),
    ("qwen_decode", 1091, True, True, "mem_d"),
    ("qwen_decode", 1091, True, True, "d_mem"),
    ("qwen_decode", 4133, True, False, "d_mem"),
    ("qwen_multibranch_zipf13", 200, False, False, "mem_d"),
    ("qwen_multibranch_zipf13", 1029, False, True, "mem_d"),
    ("qwen_multibranch_zipf13", 1029, False, True, "d_mem"),
])
def test_gate_op(orc, name, n, shared, random_gamma, layout):
    H = G.H()
    w = W.get(name)
    print(f"[gate] {name} n={n} shared={shared} gamma={random_gamma} layout={layout}", flush=True)
    cfg = G.config(w, layout)
    e = _synthetic_memory(w, n, 77 + n)
    nbh = 1 if shared else w.n_branches
    hid = rng.normal_values(91 + n, np.arange(n * nbh * w.hidden), 1.0, w.dtype).reshape(
        n, nbh, w.hidden)
    wk, wv = G.weights(w, layout)
    gam = G.gammas(w, random_gamma)
    gates = torch.empty((n, w.n_branches), dtype=torch.float32, device="cuda")
    u = torch.empty((n, w.n_branches, w.hidden), dtype=G.tdtype(w), device="cuda")
    H.ngram_gate(cfg, G.to_device(hid, w), 0 if shared else w.hidden, G.to_device(e, w), wk, wv,
                 gates, u, gamma_q=gam["q"], gamma_k=gam["k"])
    torch.cuda.synchronize()
    e64 = W.to_f64(e, w.dtype)
    wk_h, wv_h = G.host_weights(wk, wv, layout)
    k = np.stack([orc.project(e64, wk_h[b], w.dtype) for b in range(w.n_branches)], axis=1)
    v = orc.project(e64, wv_h, w.dtype)
    g_ref = orc.gate(hid, w.dtype, k, G.to_storage(gam["q"]), G.to_storage(gam["k"]), w.rms_eps)
    u_ref = orc.gated_value(g_ref, v)
    G.check(gates.cpu().numpy(), g_ref, "gates")
    G.check(G.to_f64(u), u_ref, "U")
    assert bool(((gates > 0) & (gates < 1)).all())


@pytest.mark.parametrize("name,B,T,with_state,random_gamma", [
    ("tiny", 1, 256, False, False),
    ("tiny", 3, 70, True, True),
    ("engram_small", 2, 133, False, True),
    ("qwen_decode", 256, 1, True, False),
    ("qwen_decode", 2, 200, False, False),
    ("qwen_multibranch_zipf13", 2, 97, True, True),
    ("qwen_multibranch_zipf13", 1, 5, False, False),
])
def test_causal_conv_op(orc, name, B, T, with_state, random_gamma):
    H = G.H()
    w = W.get(name)
    print(f"[conv] {name} B={B} T={T} state={with_state}", flush=True)
    cfg = G.config(w)
    nb, d, halo = w.n_branches, w.hidden, 3 * w.max_order
    u = rng.normal_values(5 + T, np.arange(B * T * nb * d), 0.01, w.dtype).reshape(B, T, nb, d)
    gam = G.gammas(w, random_gamma)
    state = None
    d_state = None
    if with_state:
        state = rng.normal_f32(6 + T, np.arange(B * halo * nb * d), 1.0).reshape(B, halo, nb, d)
        d_state = torch.from_numpy(state).cuda()
    out = torch.empty((B, T, nb, d), dtype=G.tdtype(w), device="cuda")
    H.ngram_causal_conv(cfg, G.to_device(u, w), B, T, G.conv_w(w), out, gamma_u=gam["u"],
                        conv_state=d_state)
    torch.cuda.synchronize()
    ref = orc.conv_block(W.to_f64(u, w.dtype), W.conv_weight_values(w), w.dtype, w.max_order,
                         G.to_storage(gam["u"]), w.rms_eps,
                         None if state is None else state.astype(np.float64))
    G.check(G.to_f64(out), ref, "conv")
