"""Fused ngram_forward against the oracle: every workload at its full size in
the launch configuration the benchmark uses, outputs compared on sampled
windows (each with its 11-token context) or in full where the oracle is
quick, plus edge cases (ragged and short sequences, history, conv state,
residual flag, other order sets, invalid ids, empty batches)."""
import numpy as np
import pytest
import torch

import gpu_support as G
from synth import device as SD
from synth import rng
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _device_inputs(w, ids, hist, random_gamma=False, layout="mem_d"):
    n = ids.size
    d = dict(
        layout=layout,
        ids=torch.from_numpy(ids).cuda(),
        hist=None if hist is None else torch.from_numpy(hist).cuda(),
        lut=torch.from_numpy(W.make_lut(w)).cuda(),
        tables=G.tables(w),
        hidden=SD.make_hidden(w, n),
        conv_w=G.conv_w(w),
        gam=G.gammas(w, random_gamma),
    )
    d["wk"], d["wv"] = G.weights(w, layout)
    return d


def _run(w, inp, flags=0, conv_state=None):
    """One ngram_forward; its configuration and workspace stay in ``inp``
    for _check_ids."""
    H = G.H()
    B, T = inp["ids"].shape
    cfg = G.config(w, inp["layout"])
    out = torch.empty((B, T, w.n_branches, w.hidden), dtype=G.tdtype(w), device="cuda")
    gates = torch.empty((B, T, w.n_branches), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(H.ngram_forward_workspace_size(cfg, B, T), 1), dtype=torch.uint8,
                     device="cuda")
    hbs = 0 if w.n_branches == 1 else w.hidden
    g = inp["gam"]
    H.ngram_forward(cfg, inp["ids"], inp["lut"], inp["tables"], inp["hidden"], hbs, inp["wk"],
                    inp["wv"], inp["conv_w"], out, history=inp["hist"], gamma_q=g["q"],
                    gamma_k=g["k"], gamma_u=g["u"], conv_state=conv_state, flags=flags,
                    gates=gates, err_flag=err, workspace=ws)
    torch.cuda.synchronize()
    inp["cfg"], inp["ws"] = cfg, ws
    return out, gates, err.item()


def _check_ids(orc, w, ids, hist, inp):
    """The row ids and E that this forward's own kernels produced, bit-exact
    on every token."""
    G.check_forward_ids_and_memory(orc, w, ids, hist, inp["cfg"], inp["ws"])


def _host_params(w, inp):
    wk, wv = G.host_weights(inp["wk"], inp["wv"], inp["layout"])
    return wk, wv, W.conv_weight_values(w), {k: G.to_storage(v) for k, v in inp["gam"].items()}


def _check_windows(orc, w, ids, hist, inp, out, gates, windows, flags=0, state=None):
    wk, wv, cw, gam = _host_params(w, inp)
    T = ids.shape[1]
    for b, start, length in windows:
        st = None if state is None or start > 0 else state[b:b + 1]
        ref = G.oracle_forward_window(orc, w, ids, hist, b, start, length,
                                      lambda toks: W.hidden_values(w, toks), wk, wv, cw, gam,
                                      conv_state=st)
        toks = b * T + np.arange(start, start + length)
        got = G.to_f64(out.reshape(-1, w.n_branches, w.hidden)[torch.from_numpy(toks).cuda()])
        want = ref["delta"]
        if flags:
            want = want + W.to_f64(W.hidden_values(w, toks), w.dtype)
        G.check(got, want, f"window b={b} [{start},{start + length}) out")
        G.check(gates.reshape(-1, w.n_branches)[torch.from_numpy(toks).cuda()].cpu().numpy(),
                ref["gate"], "gates")


@pytest.mark.parametrize("random_gamma,flags", [(False, 0), (True, 1)])
def test_forward_tiny_full(orc, random_gamma, flags):
    w = W.get("tiny")
    print(f"[forward] tiny gamma={random_gamma} flags={flags}", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, random_gamma)
    out, gates, err = _run(w, inp, flags)
    assert err == 0
    _check_ids(orc, w, ids, hist, inp)
    _check_windows(orc, w, ids, hist, inp, out, gates, [(0, 0, w.seq_len)], flags)


@pytest.mark.parametrize("layout", ["mem_d", "d_mem"])
def test_forward_engram_small(orc, layout):
    w = W.get("engram_small")
    print(f"[forward] engram_small {layout}", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, random_gamma=True, layout=layout)
    out, gates, err = _run(w, inp)
    assert err == 0
    _check_ids(orc, w, ids, hist, inp)
    T = w.seq_len
    _check_windows(orc, w, ids, hist, inp, out, gates,
                   [(0, 0, 40), (0, 1000, 40), (7, 2049, 40), (7, T - 40, 40)])


@pytest.mark.parametrize("layout", ["mem_d", "d_mem"])
def test_forward_qwen_decode_full(orc, layout):
    w = W.get("qwen_decode")
    print(f"[forward] qwen_decode {layout}", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, layout=layout)
    out, gates, err = _run(w, inp)
    assert err == 0
    _check_ids(orc, w, ids, hist, inp)
    wk, wv, cw, gam = _host_params(w, inp)
    ref = orc.forward(ids, hist, W.make_lut(w), w.vocab, w.vocab_compressed, w.orders, w.heads,
                      w.rows(), W.hash_multipliers(w), G.oracle_rows(w),
                      W.hidden_values(w, np.arange(ids.size)), wk, wv, cw, w.dtype,
                      gamma_q=gam["q"], gamma_k=gam["k"], gamma_u=gam["u"], eps=w.rms_eps)
    G.check(G.to_f64(out).reshape(ref["delta"].shape), ref["delta"], "decode out")
    G.check(gates.cpu().numpy().reshape(ref["gate"].shape), ref["gate"], "decode gates")


def test_forward_qwen_decode_fp8_full(orc):
    """FP8 tables on the decode route: hash + gather widens the rows to bf16
    E (times each table's scale) for the weight-stationary projection."""
    w = W.get("qwen_decode_fp8")
    print("[forward] qwen_decode_fp8", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, layout="d_mem")
    out, gates, err = _run(w, inp)
    assert err == 0
    _check_ids(orc, w, ids, hist, inp)
    wk, wv, cw, gam = _host_params(w, inp)
    ref = orc.forward(ids, hist, W.make_lut(w), w.vocab, w.vocab_compressed, w.orders, w.heads,
                      w.rows(), W.hash_multipliers(w), G.oracle_rows(w),
                      W.hidden_values(w, np.arange(ids.size)), wk, wv, cw, w.dtype,
                      eps=w.rms_eps, **G.oracle_table_kw(w))
    G.check(G.to_f64(out).reshape(ref["delta"].shape), ref["delta"], "decode fp8 out")
    G.check(gates.cpu().numpy().reshape(ref["gate"].shape), ref["gate"], "decode fp8 gates")


@pytest.mark.parametrize("layout", ["mem_d", "d_mem"])
def test_forward_engram_small_fp8(orc, layout):
    """FP8 tables on the prefill routes: gather to bf16 E, then the
    projection kernel of the layout (E materialised)."""
    w = W.get("engram_small").replace(table_dtype="fp8", batch=2, seq_len=1000)
    print(f"[forward] engram_small fp8 {layout}", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, layout=layout)
    out, gates, err = _run(w, inp)
    assert err == 0
    _check_ids(orc, w, ids, hist, inp)
    _check_windows(orc, w, ids, hist, inp, out, gates, [(0, 0, 300), (1, 650, 350)])


def test_forward_qwen_prefill_fp8(orc):
    w = W.get("qwen_prefill_fp8")
    print("[forward] qwen_prefill_fp8 262144 tokens", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, layout="d_mem")
    out, gates, err = _run(w, inp)
    assert err == 0
    _check_ids(orc, w, ids, hist, inp)
    T = w.seq_len
    _check_windows(orc, w, ids, hist, inp, out, gates, [(0, 0, 24), (0, 98765, 24), (0, T - 24, 24)])


@pytest.mark.parametrize("layout", ["mem_d", "d_mem"])
def test_forward_qwen_decode_conv_state_and_residual(orc, layout):
    """A populated conv state (the last 9 normalised rows of each sequence)."""
    w = W.get("qwen_decode").replace(batch=16)
    print(f"[forward] qwen_decode state+residual {layout}", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, layout=layout)
    halo = 3 * w.max_order
    state = rng.normal_f32(4242, np.arange(w.batch * halo * w.hidden), 1.0).reshape(
        w.batch, halo, 1, w.hidden)
    out, gates, err = _run(w, inp, flags=1, conv_state=torch.from_numpy(state).cuda())
    assert err == 0
    _check_windows(orc, w, ids, hist, inp, out, gates, [(b, 0, 1) for b in range(w.batch)],
                   flags=1, state=state.astype(np.float64))


@pytest.mark.parametrize("layout", ["mem_d", "d_mem"])
def test_forward_chunk_with_conv_state(orc, layout):
    """A prefill chunk that continues earlier ones: a populated conv state,
    the residual flag and 150 positions per sequence (three conv tiles, the
    first of which starts its taps on the state rows)."""
    w = W.get("engram_small").replace(batch=2, seq_len=150, hidden=256, heads=2,
                                      row_start=10007)
    print(f"[forward] chunk with conv state, {layout}", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, layout=layout, random_gamma=True)
    halo = 3 * w.max_order
    state = rng.normal_f32(4343, np.arange(w.batch * halo * w.hidden), 1.0).reshape(
        w.batch, halo, 1, w.hidden)
    out, gates, err = _run(w, inp, flags=1, conv_state=torch.from_numpy(state).cuda())
    assert err == 0
    _check_windows(orc, w, ids, hist, inp, out, gates, [(b, 0, w.seq_len) for b in range(w.batch)],
                   flags=1, state=state.astype(np.float64))


@pytest.mark.parametrize("layout", ["mem_d", "d_mem"])
def test_forward_qwen_prefill(orc, layout):
    w = W.get("qwen_prefill")
    print(f"[forward] qwen_prefill 262144 tokens {layout}", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, layout=layout)
    out, gates, err = _run(w, inp)
    assert err == 0
    _check_ids(orc, w, ids, hist, inp)
    T = w.seq_len
    _check_windows(orc, w, ids, hist, inp, out, gates,
                   [(0, 0, 24), (0, 7, 24), (0, 131071, 24), (0, T - 24, 24)])
    assert bool(((gates > 0) & (gates < 1)).all())


@pytest.mark.parametrize("name,layout", [("qwen_multibranch_uniform", "d_mem"),
                                         ("qwen_multibranch_zipf13", "d_mem"),
                                         ("qwen_multibranch_zipf13", "mem_d")])
def test_forward_multibranch(orc, name, layout):
    """Four branches: four key segments and per-branch queries."""
    w = W.get(name)
    print(f"[forward] {name} {layout}", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, layout=layout)
    out, gates, err = _run(w, inp)
    assert err == 0
    _check_ids(orc, w, ids, hist, inp)
    T = w.seq_len
    _check_windows(orc, w, ids, hist, inp, out, gates, [(0, 0, 16), (9, 4000, 16), (15, T - 16, 16)])


@pytest.mark.parametrize("B,T", [(3, 77), (4, 5), (1, 1), (2, 64), (1, 65)])
def test_forward_ragged_and_short(orc, B, T):
    w = W.get("tiny").replace(batch=B, seq_len=T)
    print(f"[forward] tiny B={B} T={T}", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, random_gamma=True)
    out, gates, err = _run(w, inp)
    _check_ids(orc, w, ids, hist, inp)
    _check_windows(orc, w, ids, hist, inp, out, gates, [(b, 0, T) for b in range(B)])


@pytest.mark.parametrize("variant", ["orders234", "orders12_bf16", "order2_only",
                                     "rowdim96_bf16_dmem", "tables16x160_bf16_dmem"])
def test_forward_other_order_sets(orc, variant):
    """Dilation follows the largest order (4, 2, 2)."""
    if variant == "orders234":
        w = W.get("tiny").replace(orders=(2, 3, 4), explicit_rows=(), batch=2, seq_len=90)
    elif variant == "orders12_bf16":
        w = W.get("engram_small").replace(orders=(1, 2), heads=4, batch=2, seq_len=300,
                                          hidden=256)
    elif variant == "order2_only":
        w = W.get("tiny").replace(orders=(2,), heads=3, explicit_rows=(), batch=2, seq_len=50)
    elif variant == "rowdim96_bf16_dmem":  # the projection cannot gather K steps itself
        w = W.get("engram_small").replace(heads=2, row_dim=96, batch=2, seq_len=200,
                                          hidden=128)
    else:  # 16 tables x 160 values: 8 heads per order, E of 2560 (320-byte rows)
        w = W.get("engram_small").replace(heads=8, row_dim=160, row_start=10007, batch=2,
                                          seq_len=200, hidden=256)
    print(f"[forward] {variant}", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, layout="d_mem" if "dmem" in variant else "mem_d")
    out, gates, err = _run(w, inp)
    _check_ids(orc, w, ids, hist, inp)
    _check_windows(orc, w, ids, hist, inp, out, gates,
                   [(b, 0, w.seq_len) for b in range(w.batch)])


@pytest.mark.parametrize("d,T", [(4096, 96), (4096, 1), (4160, 1)])
def test_forward_wide_hidden(orc, d, T):
    """The widest hidden sizes the kernels specialise for: d = 4,096 fills the
    register-resident decode finalize (four column groups per thread) and the
    prefill conv; d = 4,160 takes the decode finalize that streams columns
    through L2.  T = 1 with a history is the decode route."""
    w = W.get("engram_small").replace(hidden=d, heads=2, row_start=10007, batch=3, seq_len=T,
                                      history_len=2 if T == 1 else 0)
    print(f"[forward] d={d} T={T}", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, random_gamma=True, layout="d_mem")
    out, gates, err = _run(w, inp, flags=1)
    assert err == 0
    _check_ids(orc, w, ids, hist, inp)
    _check_windows(orc, w, ids, hist, inp, out, gates, [(b, 0, T) for b in range(w.batch)],
                   flags=1)


def test_forward_invalid_ids_are_pad(orc):
    w = W.get("tiny").replace(batch=2, seq_len=40)
    ids, hist = W.make_ids(w)
    ids[0, 5] = -7
    ids[1, 30] = w.vocab + 3
    inp = _device_inputs(w, ids, hist)
    out, gates, err = _run(w, inp)
    assert err == 1
    _check_ids(orc, w, ids, hist, inp)
    _check_windows(orc, w, ids, hist, inp, out, gates, [(0, 0, 40), (1, 0, 40)])


def test_forward_empty_batch():
    H = G.H()
    w = W.get("tiny")
    cfg = G.config(w)
    ids = torch.empty((0, 16), dtype=torch.int32, device="cuda")
    inp = _device_inputs(w, np.zeros((1, 16), dtype=np.int32), None)
    out = torch.empty((0, 16, 1, w.hidden), dtype=torch.float32, device="cuda")
    H.ngram_forward(cfg, ids, inp["lut"], inp["tables"], inp["hidden"], 0, inp["wk"], inp["wv"],
                    inp["conv_w"], out, workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()


def test_forward_qwen_decode_16x160_full(orc):
    """The page's own table geometry at full scale: 16 tables of ~20M rows x
    160 bf16 (320-byte rows across 128-byte lines), 256 decode tokens."""
    w = W.get("qwen_decode_16x160")
    print("[forward] qwen_decode_16x160", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, layout="d_mem")
    out, gates, err = _run(w, inp)
    assert err == 0
    _check_ids(orc, w, ids, hist, inp)
    wk, wv, cw, gam = _host_params(w, inp)
    ref = orc.forward(ids, hist, W.make_lut(w), w.vocab, w.vocab_compressed, w.orders, w.heads,
                      w.rows(), W.hash_multipliers(w), G.oracle_rows(w),
                      W.hidden_values(w, np.arange(ids.size)), wk, wv, cw, w.dtype,
                      eps=w.rms_eps)
    G.check(G.to_f64(out).reshape(ref["delta"].shape), ref["delta"], "decode 16x160 out")
    G.check(gates.cpu().numpy().reshape(ref["gate"].shape), ref["gate"], "decode 16x160 gates")


def test_forward_qwen_prefill_16x160(orc):
    w = W.get("qwen_prefill_16x160")
    print("[forward] qwen_prefill_16x160 262144 tokens", flush=True)
    ids, hist = W.make_ids(w)
    inp = _device_inputs(w, ids, hist, layout="d_mem")
    out, gates, err = _run(w, inp)
    assert err == 0
    _check_ids(orc, w, ids, hist, inp)
    T = w.seq_len
    _check_windows(orc, w, ids, hist, inp, out, gates, [(0, 0, 24), (0, 77777, 24), (0, T - 24, 24)])
