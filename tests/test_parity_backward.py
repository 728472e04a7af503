"""ngram_backward against the oracle's backward (itself pinned to the oracle
forward by finite differences): table gradients (scatter-add), W_K, W_V,
conv taps, query rows and RMSNorm gains, on bf16 configurations with one and
several branches, shared and per-branch queries, a populated conv state, the
residual flag, fp8 tables, and the Qwen-scale dimensions (2560-wide E and d).

Tolerances (normwise relative error): dK and dV enter the dE and dW products
as bf16 -- one rounding of one operand, 2^-9 relative at most, ~1.1e-3 rms --
so the table, W_K and W_V gradients are held to 5e-3; the conv, query and
gain gradients are fp32 end to end and held to 1e-4."""
import numpy as np
import pytest
import torch

import gpu_support as G
from synth import device as SD
from synth import rng
from synth import workloads as W

pytestmark = pytest.mark.gpu

TOL_GEMM = 5e-3
TOL_F32 = 1e-4


def _bf16(x):
    return torch.from_numpy(rng.f32_to_bf16_bits(np.asarray(x, np.float32)).view(np.int16)).cuda().view(torch.bfloat16)


def _case(orc, w, nbh, with_state, residual, random_gamma, seed):
    H = G.H()
    ids, hist = W.make_ids(w)
    n, nb, d = ids.size, w.n_branches, w.hidden
    cfg = G.config(w, "d_mem")
    tabs = G.tables(w)
    wk, wv = G.weights(w, "d_mem")
    conv = G.conv_w(w)
    gam = G.gammas(w, random_gamma)
    rs = np.random.default_rng(seed)
    hidden_f = rs.standard_normal((n, nbh, d)).astype(np.float32)
    hidden = _bf16(hidden_f)
    d_out_f = rs.standard_normal((n, nb, d)).astype(np.float32)
    d_out = _bf16(d_out_f)
    state = (rs.standard_normal((w.batch, 3 * w.max_order, nb, d)).astype(np.float32)
             if with_state else None)
    d_tabs = [torch.zeros((r, w.row_dim), dtype=torch.float32, device="cuda") for r in w.rows()]
    d_wk = torch.empty((nb, d, w.mem_dim), dtype=torch.float32, device="cuda")
    d_wv = torch.empty((d, w.mem_dim), dtype=torch.float32, device="cuda")
    d_cw = torch.empty((4, d), dtype=torch.float32, device="cuda")
    d_h = torch.empty((n, nbh, d), dtype=torch.float32, device="cuda")
    d_g = torch.empty((3, d), dtype=torch.float32, device="cuda")
    H.ngram_backward(cfg, torch.from_numpy(ids).cuda(), torch.from_numpy(W.make_lut(w)).cuda(),
                     tabs, hidden, 0 if nbh == 1 else d, wk, wv, conv, d_out, d_tabs, d_wk, d_wv,
                     d_cw, history=None if hist is None else torch.from_numpy(hist).cuda(),
                     gamma_q=gam["q"], gamma_k=gam["k"], gamma_u=gam["u"],
                     conv_state=None if state is None else torch.from_numpy(state).cuda(),
                     flags=1 if residual else 0, d_hidden=d_h, d_gammas=d_g)
    torch.cuda.synchronize()
    wk_h, wv_h = G.host_weights(wk, wv, "d_mem")
    gh = {k: G.to_storage(v) for k, v in gam.items()}
    ref = G.oracle_backward(orc, w, ids, hist, G.to_storage(hidden).reshape(n, nbh, d), wk_h, wv_h,
                            G.to_storage(conv), gh,
                            G.to_f64(d_out).reshape(n, nb, d),
                            None if state is None else state.astype(np.float64), residual)
    errs = {
        "d_wk": G.rel_err(d_wk.double().cpu().numpy(), ref["d_wk"].transpose(0, 2, 1)),
        "d_wv": G.rel_err(d_wv.double().cpu().numpy(), ref["d_wv"].T),
        "d_conv_w": G.rel_err(d_cw.double().cpu().numpy(), ref["d_conv_w"]),
        "d_hidden": G.rel_err(d_h.double().cpu().numpy(), ref["d_hidden"]),
    }
    if gam["q"] is not None:
        errs["d_gammas"] = G.rel_err(d_g.double().cpu().numpy(),
                                     np.stack([ref["d_gamma_q"], ref["d_gamma_k"], ref["d_gamma_u"]]))
    got_rows, want_rows = [], []
    for j, (rows_j, grads_j) in enumerate(ref["d_tables"]):
        got_rows.append(d_tabs[j][torch.from_numpy(rows_j).cuda().long()].double().cpu().numpy())
        want_rows.append(grads_j)
        # rows no token named stay zero
        assert float(d_tabs[j].abs().sum()) == pytest.approx(float(np.abs(got_rows[-1]).sum()), rel=1e-6)
    errs["d_tables"] = G.rel_err(np.concatenate(got_rows), np.concatenate(want_rows))
    print("   backward rel_err " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k in ("d_wk", "d_wv", "d_tables"):
        assert errs[k] < TOL_GEMM, (k, errs[k])
    for k in ("d_conv_w", "d_hidden", "d_gammas"):
        if k in errs:
            assert errs[k] < TOL_F32, (k, errs[k])


SMALL = W.get("engram_small").replace(batch=2, seq_len=300, hidden=256, heads=2,
                                      row_start=10007)


@pytest.mark.parametrize("nb,nbh,with_state,residual,random_gamma,tables", [
    (1, 1, False, False, False, "bf16"),
    (1, 1, True, True, True, "bf16"),
    (2, 1, False, True, True, "bf16"),
    (3, 3, True, False, True, "bf16"),
    (1, 1, True, True, True, "fp8"),
])
def test_backward_small(orc, nb, nbh, with_state, residual, random_gamma, tables):
    w = SMALL.replace(n_branches=nb, table_dtype="fp8" if tables == "fp8" else None)
    print(f"[backward] small nb={nb} nbh={nbh} state={with_state} residual={residual} "
          f"{tables}", flush=True)
    _case(orc, w, nbh, with_state, residual, random_gamma, seed=nb * 7 + nbh)


def test_backward_qwen_dims(orc):
    """The Qwen-scale product shapes (8 tables x 320 -> E of 2560, d = 2560),
    64 sequences of a new token with a 2-token history; small prime tables so
    that the fp32 table gradients fit beside them."""
    w = W.get("qwen_decode").replace(batch=64, row_start=100003)
    print("[backward] qwen dims, 64 tokens", flush=True)
    _case(orc, w, 1, False, True, True, seed=5)


@pytest.mark.parametrize("nb", [1, 2])
def test_backward_split_k_weight_gradients(orc, nb):
    """4,500 tokens (71 K steps of 64 after padding): the dW product splits
    its K steps over 4 workgroups per tile, raggedly (17/18/18/18), and the
    summed splits land in d_w_k and d_w_v on either side of the boundary."""
    w = SMALL.replace(batch=3, seq_len=1500, n_branches=nb)
    print(f"[backward] split-K dW, 3 x 1500 tokens, nb={nb}", flush=True)
    _case(orc, w, 1, False, True, True, seed=20 + nb)


def test_backward_8400_tokens(orc):
    """8,400 tokens (from 8,192 rows the K / V recompute and the dE product
    take the 256 x 256 tile, here 33 row tiles with a ragged last one of 208
    rows) at small dimensions, so that the oracle's backward stays quick."""
    w = SMALL.replace(batch=2, seq_len=4200)
    print("[backward] 2 x 4200 tokens", flush=True)
    _case(orc, w, 1, True, True, True, seed=30)


def test_backward_widest_hidden(orc):
    """d = 4,096, the widest hidden size the backward takes (four column
    groups per thread in the per-row kernels)."""
    w = SMALL.replace(hidden=4096, batch=2, seq_len=70)
    print("[backward] d=4096, 2 x 70 tokens", flush=True)
    _case(orc, w, 1, True, True, True, seed=31)


def test_backward_single_token_sequences_and_ragged(orc):
    """T = 1 (every conv tap outside the sequence) and a ragged token count."""
    w = SMALL.replace(batch=37, seq_len=1, history_len=2)
    print("[backward] 37 sequences x 1 token", flush=True)
    _case(orc, w, 1, True, False, True, seed=9)
    w = SMALL.replace(batch=3, seq_len=77)
    print("[backward] 3 x 77 tokens", flush=True)
    _case(orc, w, 1, False, True, False, seed=10)


def test_backward_wide_rows(orc):
    """576-wide table rows (E of 2,304): the table gradient's wavefronts take
    each row in two column passes, the second ragged (64 of 512 columns)."""
    w = SMALL.replace(row_dim=576, batch=2, seq_len=200)
    print("[backward] 576-wide rows, 2 x 200 tokens", flush=True)
    _case(orc, w, 1, True, True, True, seed=51)


@pytest.mark.parametrize("orders", [(1,), (2,), (2, 3, 4)])
def test_backward_other_dilations(orc, orders):
    """The conv block's backward at dilations 1, 2 and 4 (the largest order),
    with a conv state and a ragged last tile of positions (150 = 64 + 64 + 22)."""
    w = SMALL.replace(orders=orders, batch=2, seq_len=150)
    print(f"[backward] orders {orders}", flush=True)
    _case(orc, w, 1, True, True, True, seed=40 + len(orders) + max(orders))


def test_backward_rejects_unsupported():
    H = G.H()
    w = W.get("tiny")  # fp32 activations, W stored [mem, d]
    cfg = G.config(w)
    ids, _ = W.make_ids(w)
    x = torch.zeros(16, device="cuda")
    with pytest.raises(H.NgramError) as e:
        H.ngram_backward(cfg, torch.from_numpy(ids).cuda(), torch.from_numpy(W.make_lut(w)).cuda(),
                         G.tables(w), x, 0, x, x, x, x, [x] * w.n_tables, x, x, x,
                         workspace=torch.empty(1 << 20, dtype=torch.uint8, device="cuda"))
    assert e.value.status == -3  # NGRAM_EDTYPE


def test_backward_deterministic_gradients_run_to_run():
    """Two identical backward calls give bit-identical gradients: W_K, W_V,
    the conv taps, the query rows and the gains (fixed-order sums, no float
    atomics), and the tables, whose rows named by several tokens add their
    contributions in ascending token order.  The id stream repeats rows often
    (Zipf ids over small tables), so many rows take several terms."""
    H = G.H()
    w = W.get("engram_small").replace(batch=3, seq_len=300, hidden=512, heads=2,
                                      row_start=10007, n_branches=2)
    print("[backward] run-to-run determinism", flush=True)
    ids, hist = W.make_ids(w)
    n, nb, d = ids.size, w.n_branches, w.hidden
    cfg = G.config(w, "d_mem")
    wk, wv = G.weights(w, "d_mem")
    gam = G.gammas(w, True)
    rs = np.random.default_rng(21)
    hidden = _bf16(rs.standard_normal((n, nb, d)).astype(np.float32))
    d_out = _bf16(rs.standard_normal((n, nb, d)).astype(np.float32))
    state = torch.from_numpy(rs.standard_normal((w.batch, 3 * w.max_order, nb, d))
                             .astype(np.float32)).cuda()
    runs = []
    for _ in range(2):
        g = dict(tabs=[torch.zeros((r, w.row_dim), dtype=torch.float32, device="cuda")
                       for r in w.rows()],
                 wk=torch.empty((nb, d, w.mem_dim), dtype=torch.float32, device="cuda"),
                 wv=torch.empty((d, w.mem_dim), dtype=torch.float32, device="cuda"),
                 cw=torch.empty((4, d), dtype=torch.float32, device="cuda"),
                 h=torch.empty((n, nb, d), dtype=torch.float32, device="cuda"),
                 gm=torch.empty((3, d), dtype=torch.float32, device="cuda"))
        H.ngram_backward(cfg, torch.from_numpy(ids).cuda(),
                         torch.from_numpy(W.make_lut(w)).cuda(), G.tables(w), hidden, d, wk, wv,
                         G.conv_w(w), d_out, g["tabs"], g["wk"], g["wv"], g["cw"],
                         gamma_q=gam["q"], gamma_k=gam["k"], gamma_u=gam["u"], conv_state=state,
                         flags=1, d_hidden=g["h"], d_gammas=g["gm"])
        torch.cuda.synchronize()
        runs.append(g)
    a, b = runs
    for k in ("wk", "wv", "cw", "h", "gm"):
        assert torch.equal(a[k], b[k]), k
    shared = 0
    for ta, tb in zip(a["tabs"], b["tabs"]):
        assert torch.equal(ta, tb)
    for ta in a["tabs"]:
        shared += int((ta != 0).any(dim=1).sum().item())
    # fewer touched rows than (token, table) pairs: rows were shared
    assert shared < n * w.n_tables
