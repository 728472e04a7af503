"""Every tile plan of the projection kernel that streams operands straight
into LDS (W stored [d, mem]) against the oracle, at ragged token counts: the
op-level gate on a dense memory matrix and the forward pass.  The
configuration's tuning fields select the plan."""
import numpy as np
import pytest
import torch

import gpu_support as G
from synth import device as SD
from synth import rng
from synth import workloads as W

pytestmark = pytest.mark.gpu

PLANS = list(range(13))


@pytest.mark.parametrize("plan", PLANS)
@pytest.mark.parametrize("n", [77, 1000, 4133])
def test_gate_each_plan(orc, plan, n):
    H = G.H()
    w = W.get("qwen_multibranch_zipf13")
    print(f"[plan {plan}] gate n={n}", flush=True)
    cfg = G.config(w, "d_mem", proj_plan=plan)
    e = rng.normal_values(31 + n, np.arange(n * w.mem_dim), 0.02, "bf16").reshape(n, w.mem_dim)
    hid = rng.normal_values(32 + n, np.arange(n * 4 * w.hidden), 1.0, "bf16").reshape(n, 4, w.hidden)
    wk, wv = G.weights(w, "d_mem")
    gates = torch.empty((n, 4), dtype=torch.float32, device="cuda")
    u = torch.empty((n, 4, w.hidden), dtype=torch.bfloat16, device="cuda")
    H.ngram_gate(cfg, G.to_device(hid, w), w.hidden, G.to_device(e, w), wk, wv, gates, u)
    torch.cuda.synchronize()
    e64 = W.to_f64(e, "bf16")
    wk_h, wv_h = G.host_weights(wk, wv, "d_mem")
    k = np.stack([orc.project(e64, wk_h[b], "bf16") for b in range(4)], axis=1)
    v = orc.project(e64, wv_h, "bf16")
    g_ref = orc.gate(hid, "bf16", k, eps=w.rms_eps)
    G.check(gates.cpu().numpy(), g_ref, "gates")
    G.check(G.to_f64(u), orc.gated_value(g_ref, v), "U")


@pytest.mark.parametrize("plan", [8, 11, 12])
def test_gate_ragged_hidden(orc, plan):
    """A hidden size that is not a multiple of the column tile (2,080 =
    8 x 256 + 32 = 16 x 128 + 32): the last column tile's waves hold columns
    past d, which are computed from clamped weight rows and never stored."""
    H = G.H()
    w = W.get("qwen_multibranch_zipf13").replace(hidden=2080)
    n = 777
    print(f"[plan {plan}] gate d=2080 n={n}", flush=True)
    cfg = G.config(w, "d_mem", proj_plan=plan)
    e = rng.normal_values(91, np.arange(n * w.mem_dim), 0.02, "bf16").reshape(n, w.mem_dim)
    hid = rng.normal_values(92, np.arange(n * 4 * w.hidden), 1.0, "bf16").reshape(n, 4, w.hidden)
    wk, wv = G.weights(w, "d_mem")
    gates = torch.empty((n, 4), dtype=torch.float32, device="cuda")
    u = torch.empty((n, 4, w.hidden), dtype=torch.bfloat16, device="cuda")
    H.ngram_gate(cfg, G.to_device(hid, w), w.hidden, G.to_device(e, w), wk, wv, gates, u)
    torch.cuda.synchronize()
    e64 = W.to_f64(e, "bf16")
    wk_h, wv_h = G.host_weights(wk, wv, "d_mem")
    k = np.stack([orc.project(e64, wk_h[b], "bf16") for b in range(4)], axis=1)
    v = orc.project(e64, wv_h, "bf16")
    g_ref = orc.gate(hid, "bf16", k, eps=w.rms_eps)
    G.check(gates.cpu().numpy(), g_ref, "gates")
    G.check(G.to_f64(u), orc.gated_value(g_ref, v), "U")


@pytest.mark.parametrize("plan", PLANS)
def test_forward_each_plan(orc, plan):
    """Every tile plan in the forward pass (hash, gather to E, projection,
    conv)."""
    H = G.H()
    w = W.get("qwen_prefill").replace(batch=3, seq_len=1100)
    print(f"[plan {plan}] forward", flush=True)
    cfg = G.config(w, "d_mem", proj_plan=plan)
    ids, _ = W.make_ids(w)
    wk, wv = G.weights(w, "d_mem")
    hidden = SD.make_hidden(w, ids.size)
    out = torch.empty((3, 1100, 1, w.hidden), dtype=torch.bfloat16, device="cuda")
    gates = torch.empty((3, 1100, 1), dtype=torch.float32, device="cuda")
    H.ngram_forward(cfg, torch.from_numpy(ids).cuda(), torch.from_numpy(W.make_lut(w)).cuda(),
                    G.tables(w), hidden, 0, wk, wv, G.conv_w(w), out, gates=gates)
    torch.cuda.synchronize()
    wk_h, wv_h = G.host_weights(wk, wv, "d_mem")
    for b, start in [(0, 0), (1, 517), (2, 1100 - 20)]:
        ref = G.oracle_forward_window(orc, w, ids, None, b, start, 20,
                                      lambda toks: W.hidden_values(w, toks), wk_h, wv_h,
                                      W.conv_weight_values(w))
        got = G.to_f64(out[b, start:start + 20])
        G.check(got.reshape(ref["delta"].shape), ref["delta"], f"b={b} [{start}, +20)")
        G.check(gates[b, start:start + 20].cpu().numpy().reshape(ref["gate"].shape), ref["gate"],
                "gates")


# (ni, split): 16*ni weight columns per workgroup (ni 2..6), K slices (each a
# multiple of 128 wide).  With K = 2560: 3 (48 columns) leaves a ragged last
# column tile, 6 (96) another one; splits 2..20 give 40- down to 4-step slices.
DECODE_PLANS = [None, (5, 4), (4, 4), (6, 4), (2, 2), (3, 5), (5, 10), (4, 20)]


@pytest.mark.parametrize("plan", DECODE_PLANS, ids=lambda p: "default" if p is None else
                         f"{p[0]}x{p[1]}")
@pytest.mark.parametrize("name,batch", [("qwen_decode", 64), ("qwen_decode", 300),
                                        ("qwen_multibranch_zipf13", 64)])
def test_decode_path_plans(orc, plan, name, batch):
    """One new token per sequence (T = 1): hash+gather, the weight-stationary
    projection and the decode finalize, with a populated conv state, the
    residual flag and random RMSNorm gains (300 rows: two ragged passes)."""
    print(f"[decode plan {plan}] {name} batch {batch}", flush=True)
    _decode_case(orc, name, batch, plan=plan)


def test_decode_1100_sequences(orc):
    """More than 1,024 sequences: the hash+gather kernel splits each token
    over two waves instead of four, and the projection makes several passes."""
    print("[decode] 1100 sequences", flush=True)
    _decode_case(orc, "qwen_decode", 1100)


@pytest.mark.parametrize("batch", [1, 17])
def test_decode_small_batches(orc, batch):
    """A single sequence and 17 (one full 16-row block and one row of the
    next): most of the projection's sixteen waves then compute clamped
    copies of the last row block, which they never store."""
    print(f"[decode] {batch} sequences", flush=True)
    _decode_case(orc, "qwen_decode", batch)


def test_decode_invalid_ids_are_pad(orc):
    """Ids outside the vocabulary, in the new tokens and in the history, hash
    as the pad id and set the error flag."""
    print("[decode invalid ids]", flush=True)
    _decode_case(orc, "qwen_decode", 300, bad_ids=True)


def _decode_case(orc, name, batch, bad_ids=False, plan=None):
    H = G.H()
    w = W.get(name).replace(batch=batch, seq_len=1, history_len=2)
    cfg = G.config(w, "d_mem", decode_plan=plan)
    ids, hist = W.make_ids(w)
    if bad_ids:
        ids[3, 0], ids[290, 0] = -5, w.vocab + 11
        hist[7, 1], hist[260, 0] = w.vocab, -1
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wk, wv = G.weights(w, "d_mem")
    nb, d, halo = w.n_branches, w.hidden, 3 * w.max_order
    hidden = SD.make_hidden(w, ids.size)
    gam = G.gammas(w, True)
    state = rng.normal_f32(77, np.arange(w.batch * halo * nb * d), 1.0).reshape(w.batch, halo, nb, d)
    out = torch.empty((w.batch, 1, nb, d), dtype=torch.bfloat16, device="cuda")
    gates = torch.empty((w.batch, 1, nb), dtype=torch.float32, device="cuda")
    ws = torch.empty(H.ngram_forward_workspace_size(cfg, w.batch, 1), dtype=torch.uint8,
                     device="cuda")
    H.ngram_forward(cfg, torch.from_numpy(ids).cuda(), torch.from_numpy(W.make_lut(w)).cuda(),
                    G.tables(w), hidden, 0 if nb == 1 else d, wk, wv, G.conv_w(w), out,
                    history=torch.from_numpy(hist).cuda(), gamma_q=gam["q"], gamma_k=gam["k"],
                    gamma_u=gam["u"], conv_state=torch.from_numpy(state).cuda(), flags=1,
                    gates=gates, err_flag=err, workspace=ws)
    torch.cuda.synchronize()
    assert err.item() == (1 if bad_ids else 0)
    G.check_forward_ids_and_memory(orc, w, ids, hist, cfg, ws)
    wk_h, wv_h = G.host_weights(wk, wv, "d_mem")
    gh = {k: G.to_storage(v) for k, v in gam.items()}
    ref = orc.forward(ids, hist, W.make_lut(w), w.vocab, w.vocab_compressed, w.orders, w.heads,
                      w.rows(), W.hash_multipliers(w), G.oracle_rows(w),
                      W.hidden_values(w, np.arange(ids.size)), wk_h, wv_h,
                      W.conv_weight_values(w), "bf16", gamma_q=gh["q"], gamma_k=gh["k"],
                      gamma_u=gh["u"], eps=w.rms_eps, conv_state=state.astype(np.float64))
    want = ref["delta"] + W.to_f64(W.hidden_values(w, np.arange(ids.size)), "bf16").reshape(
        w.batch, -1, d)[:, :1 if nb == 1 else nb]
    got = G.to_f64(out).reshape(want.shape)
    G.check(got, want, "decode out")
    G.check(gates.cpu().numpy().reshape(ref["gate"].shape), ref["gate"], "decode gates")


def test_single_token_large_batch_takes_prefill_route(orc):
    """T = 1 with more sequences than the decode route serves: the prefill
    route (hash with history, gather, projection, conv) gives the same
    result."""
    w = W.get("engram_small").replace(batch=2100, seq_len=1, history_len=2, heads=2,
                                      hidden=128)
    print("[single token, 2100 sequences]", flush=True)
    H = G.H()
    cfg = G.config(w, "d_mem")
    ids, hist = W.make_ids(w)
    wk, wv = G.weights(w, "d_mem")
    hidden = SD.make_hidden(w, ids.size)
    out = torch.empty((w.batch, 1, 1, w.hidden), dtype=torch.bfloat16, device="cuda")
    gates = torch.empty((w.batch, 1, 1), dtype=torch.float32, device="cuda")
    H.ngram_forward(cfg, torch.from_numpy(ids).cuda(), torch.from_numpy(W.make_lut(w)).cuda(),
                    G.tables(w), hidden, 0, wk, wv, G.conv_w(w), out,
                    history=torch.from_numpy(hist).cuda(), gates=gates)
    torch.cuda.synchronize()
    wk_h, wv_h = G.host_weights(wk, wv, "d_mem")
    ref = orc.forward(ids, hist, W.make_lut(w), w.vocab, w.vocab_compressed, w.orders, w.heads,
                      w.rows(), W.hash_multipliers(w), G.oracle_rows(w),
                      W.hidden_values(w, np.arange(ids.size)), wk_h, wv_h,
                      W.conv_weight_values(w), "bf16", eps=w.rms_eps)
    G.check(G.to_f64(out).reshape(ref["delta"].shape), ref["delta"], "out")
    G.check(gates.cpu().numpy().reshape(ref["gate"].shape), ref["gate"], "gates")
