"""The conv-state ring (decode, and prefill in chunks) through the C-ABI.

The layer's formula ("Qwen3.8-Flash-Next 深度研究" §2.3) applies the dilated
causal conv over RMSNorm(U) along the sequence, so a sequence that arrives in
pieces needs the last 3 * dil normalised rows of the earlier pieces.  With
NGRAM_UPDATE_STATE ngram_forward writes them into the caller's ring: these
tests feed sequences one token (or one chunk) per call, carrying only the ring
and its positions (which the library advances) from call to call, and compare with one call over the whole
sequence and with the oracle -- outputs within the parity tolerance, row ids
bit-identical, the ring's rows against the oracle's normalised rows."""
import numpy as np
import pytest
import torch

import gpu_support as G
from synth import device as SD
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _small(nb=1, **over):
    """A bf16 layer small enough to build in a moment: 4 tables of 64 values,
    d = 256, W stored [d, mem] (the decode route serves T = 1)."""
    kw = dict(heads=2, row_start=10007, hidden=256, n_branches=nb, history_len=0)
    kw.update(over)
    return W.get("engram_small").replace(**kw)


class Layer:
    """Device parameters of a workload and one ngram_forward per call."""

    def __init__(self, w, layout="d_mem", random_gamma=True):
        self.w = w
        self.H = G.H()
        self.cfg = G.config(w, layout)
        self.tabs = G.tables(w)
        self.wk, self.wv = G.weights(w, layout)
        self.conv = G.conv_w(w)
        self.gam = G.gammas(w, random_gamma)
        self.lut = torch.from_numpy(W.make_lut(w)).cuda()
        self.layout = layout

    def run(self, ids, hist, hidden, ring=None, pos=None, flags=0):
        """ids raw int32 [B, T] (host), hist raw [B, max_order - 1] or None,
        hidden device [B*T, nbh, d]; returns out, gates, workspace."""
        w, H = self.w, self.H
        B, T = ids.shape
        out = torch.empty((B, T, w.n_branches, w.hidden), dtype=torch.bfloat16, device="cuda")
        gates = torch.empty((B, T, w.n_branches), dtype=torch.float32, device="cuda")
        ws = torch.empty(H.ngram_forward_workspace_size(self.cfg, B, T), dtype=torch.uint8,
                         device="cuda")
        H.ngram_forward(self.cfg, torch.from_numpy(np.ascontiguousarray(ids)).cuda(), self.lut,
                        self.tabs, hidden, 0 if w.n_branches == 1 else w.hidden, self.wk, self.wv,
                        self.conv, out, history=None if hist is None else
                        torch.from_numpy(np.ascontiguousarray(hist)).cuda(),
                        gamma_q=self.gam["q"], gamma_k=self.gam["k"], gamma_u=self.gam["u"],
                        conv_state=ring, state_pos=pos, flags=flags, gates=gates, workspace=ws)
        return out, gates, ws

    def row_ids(self, ws, B, T):
        rows, _ = G.forward_ids_and_memory(self.cfg, self.w, B, T, ws)
        return rows.cpu().numpy()


def _history(ids, t0, n_hist):
    """Raw ids of the n_hist positions before t0 (raw 0, the pad id's
    preimage, before the sequence start), oldest first."""
    B = ids.shape[0]
    h = np.zeros((B, n_hist), dtype=np.int32)
    for k in range(n_hist):
        p = t0 - n_hist + k
        if p >= 0:
            h[:, k] = ids[:, p]
    return h


def _nan_ring(w, B):
    R = 3 * w.max_order
    return torch.full((B, R, w.n_branches, w.hidden), float("nan"), dtype=torch.float32,
                      device="cuda")


def _oracle(orc, layer, ids, hidden_host):
    w = layer.w
    wk, wv = G.host_weights(layer.wk, layer.wv, layer.layout)
    gam = {k: G.to_storage(v) for k, v in layer.gam.items()}
    return orc.forward(ids, None, W.make_lut(w), w.vocab, w.vocab_compressed, w.orders, w.heads,
                       w.rows(), W.hash_multipliers(w), G.oracle_rows(w), hidden_host, wk, wv,
                       W.conv_weight_values(w), "bf16", gamma_q=gam["q"], gamma_k=gam["k"],
                       gamma_u=gam["u"], eps=w.rms_eps)


def _check_ring(orc, layer, ring, ref, L):
    """After positions [0, L) the ring holds N_p (the oracle's normalised U
    rows) of the last R positions, position p in slot p mod R."""
    w = layer.w
    B, R = ring.shape[0], ring.shape[1]
    u = ref["u"].reshape(B, L, w.n_branches, w.hidden)
    n = orc.normalised_rows(u, G.to_storage(layer.gam["u"]), "bf16", w.rms_eps)
    got = ring.double().cpu().numpy()
    for p in range(max(0, L - R), L):
        # fp32 arithmetic against fp64: well inside 1e-5 of the row's norm
        G.check(got[:, p % R], n[:, p], f"ring slot of position {p}", tol=1e-5, row_tol=1e-5,
                max_tol=1e-5)


@pytest.mark.parametrize("name,nb,B,L,flags", [("small", 1, 6, 20, 0),
                                               ("small", 4, 3, 17, 1),
                                               ("qwen", 1, 32, 14, 1)])
def test_decode_steps_equal_prefill(orc, name, nb, B, L, flags):
    """L calls of one token each, carrying the ring (initially NaN: positions
    before the start must not be read) and its positions, equal one call over
    the L tokens: outputs and gates within the tolerance of each other and of
    the oracle, row ids bit-identical, and the ring ends holding the last
    3 * dil normalised rows."""
    H = G.H()
    if name == "small":
        w = _small(nb=nb, batch=B, seq_len=L)
    else:
        w = W.get("qwen_decode").replace(batch=B, seq_len=L, history_len=0)
    print(f"[ring] decode steps = prefill, {name} nb={nb} B={B} L={L} flags={flags}", flush=True)
    layer = Layer(w)
    ids, _ = W.make_ids(w)
    hidden = SD.make_hidden(w, B * L)                    # token b*L + t
    nbh = hidden.shape[1]
    out_p, gates_p, ws_p = layer.run(ids, None, hidden, flags=flags & 1)
    rows_p = layer.row_ids(ws_p, B, L)
    ring = _nan_ring(w, B)
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    hv = hidden.view(B, L, nbh, w.hidden)
    outs, gates, rows = [], [], []
    for t in range(L):
        o, g, ws = layer.run(ids[:, t:t + 1], _history(ids, t, w.max_order - 1),
                             hv[:, t].contiguous(), ring, pos, flags | H.UPDATE_STATE)
        torch.cuda.synchronize()
        outs.append(o)
        gates.append(g)
        rows.append(layer.row_ids(ws, B, 1))
    assert torch.equal(pos, torch.full_like(pos, L))      # advanced by the library
    out_d = torch.cat(outs, dim=1)
    gates_d = torch.cat(gates, dim=1)
    rows_d = np.stack(rows, axis=1).reshape(B * L, -1)
    assert np.array_equal(rows_d, rows_p)
    G.check(G.to_f64(out_d), G.to_f64(out_p), "decode steps against one prefill call")
    G.check(gates_d.cpu().numpy(), gates_p.cpu().numpy(), "gates against prefill")
    ref = _oracle(orc, layer, ids, W.hidden_values(w, np.arange(B * L)))
    want = ref["delta"].reshape(B, L, nb, w.hidden)
    if flags & 1:
        want = want + W.to_f64(W.hidden_values(w, np.arange(B * L)), "bf16").reshape(
            B, L, nbh, w.hidden)
    G.check(G.to_f64(out_d), want, "decode steps against the oracle")
    G.check(gates_d.cpu().numpy(), ref["gate"].reshape(B, L, nb), "gates against the oracle")
    _check_ring(orc, layer, ring, ref, L)


@pytest.mark.parametrize("layout", ["d_mem", "mem_d"])
def test_chunks_then_decode_equal_prefill(orc, layout):
    """Prefill in three chunks (12 positions: one conv tile; 150: three tiles,
    whose ring update runs after the conv; 70) and then three decode steps,
    each call carrying the ring: equal to one call over the 235 tokens."""
    w = _small(batch=2, seq_len=235)
    print(f"[ring] chunks 12 + 150 + 70 + 3 x 1, {layout}", flush=True)
    H = G.H()
    layer = Layer(w, layout)
    ids, _ = W.make_ids(w)
    B, L = 2, 235
    hidden = SD.make_hidden(w, B * L)
    hv = hidden.view(B, L, 1, w.hidden)
    out_p, gates_p, ws_p = layer.run(ids, None, hidden, flags=1)
    rows_p = layer.row_ids(ws_p, B, L).reshape(B, L, -1)
    ring = _nan_ring(w, B)
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    outs, t0 = [], 0
    for T in (12, 150, 70, 1, 1, 1):
        o, _, ws = layer.run(ids[:, t0:t0 + T], _history(ids, t0, w.max_order - 1),
                             hv[:, t0:t0 + T].reshape(B * T, 1, w.hidden).contiguous(), ring, pos,
                             1 | H.UPDATE_STATE)
        torch.cuda.synchronize()
        assert np.array_equal(layer.row_ids(ws, B, T).reshape(B, T, -1), rows_p[:, t0:t0 + T])
        outs.append(o)
        t0 += T
        assert torch.equal(pos, torch.full_like(pos, t0))
    G.check(G.to_f64(torch.cat(outs, dim=1)), G.to_f64(out_p), "chunks against one call")
    ref = _oracle(orc, layer, ids, W.hidden_values(w, np.arange(B * L)))
    want = ref["delta"].reshape(B, L, 1, w.hidden) + W.to_f64(
        W.hidden_values(w, np.arange(B * L)), "bf16").reshape(B, L, 1, w.hidden)
    G.check(G.to_f64(torch.cat(outs, dim=1)), want, "chunks against the oracle")
    _check_ring(orc, layer, ring, ref, L)


@pytest.mark.parametrize("T", [1, 40])
def test_fresh_sequence_ignores_ring_contents(T):
    """state_pos = 0: every position before the start reads zero, whatever the
    ring holds, so the output equals a call without a ring, bit for bit."""
    w = _small(batch=3, seq_len=T)
    print(f"[ring] fresh sequence T={T}", flush=True)
    H = G.H()
    layer = Layer(w)
    ids, _ = W.make_ids(w)
    hidden = SD.make_hidden(w, 3 * T)
    out_a, gates_a, _ = layer.run(ids, None, hidden)
    ring = torch.full((3, 3 * w.max_order, 1, w.hidden), 1e30, dtype=torch.float32,
                      device="cuda")
    pos = torch.zeros(3, dtype=torch.int32, device="cuda")
    out_b, gates_b, _ = layer.run(ids, None, hidden, ring, pos, H.UPDATE_STATE)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(gates_a, gates_b)


@pytest.mark.parametrize("T", [1, 30])
def test_rotated_ring_equals_oldest_first_state(T):
    """The same rows held oldest first (state_pos NULL) or rotated by a ring
    position: identical outputs bit for bit, in the forward and in the
    backward's deterministic gradients."""
    w = _small(batch=2, seq_len=T)
    print(f"[ring] rotated ring T={T}", flush=True)
    H = G.H()
    layer = Layer(w)
    ids, _ = W.make_ids(w)
    hist = _history(np.concatenate([np.full((2, 5), 7, np.int32), ids], axis=1), 5, 2)
    hidden = SD.make_hidden(w, 2 * T)
    R = 3 * w.max_order
    legacy = torch.randn((2, R, 1, w.hidden), dtype=torch.float32, device="cuda",
                         generator=torch.Generator("cuda").manual_seed(5))
    p = np.array([R + 4, 3 * R + 7], dtype=np.int32)     # ring positions, both full rings
    rotated = torch.empty_like(legacy)
    for b in range(2):
        for q in range(-R, 0):
            rotated[b, (p[b] + q) % R] = legacy[b, R + q]
    pos = torch.from_numpy(p).cuda()
    out_a, gates_a, _ = layer.run(ids, hist, hidden, legacy, None, 1)
    out_b, gates_b, _ = layer.run(ids, hist, hidden, rotated, pos, 1)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(gates_a, gates_b)
    if T == 1:
        return
    d_out = torch.randn(out_a.shape, device="cuda", generator=torch.Generator("cuda").manual_seed(6)
                        ).bfloat16()
    grads = []
    for ring, pp in ((legacy, None), (rotated, pos)):
        d_tabs = [torch.zeros((r, w.row_dim), dtype=torch.float32, device="cuda")
                  for r in w.rows()]
        g = dict(wk=torch.empty((1, w.hidden, w.mem_dim), dtype=torch.float32, device="cuda"),
                 wv=torch.empty((w.hidden, w.mem_dim), dtype=torch.float32, device="cuda"),
                 cw=torch.empty((4, w.hidden), dtype=torch.float32, device="cuda"),
                 h=torch.empty((2 * T, 1, w.hidden), dtype=torch.float32, device="cuda"))
        H.ngram_backward(layer.cfg, torch.from_numpy(ids).cuda(), layer.lut, layer.tabs, hidden, 0,
                         layer.wk, layer.wv, layer.conv, d_out, d_tabs, g["wk"], g["wv"], g["cw"],
                         history=torch.from_numpy(hist).cuda(), gamma_q=layer.gam["q"],
                         gamma_k=layer.gam["k"], gamma_u=layer.gam["u"], conv_state=ring,
                         state_pos=pp, flags=1, d_hidden=g["h"])
        torch.cuda.synchronize()
        grads.append(g)
    for k in ("cw", "h", "wk", "wv"):
        assert torch.equal(grads[0][k], grads[1][k]), k


@pytest.mark.parametrize("chunks", [(5, 7, 1, 1), (70, 130, 1)])
def test_op_conv_chunks_equal_one_call(orc, chunks):
    """ngram_causal_conv over a U stream in chunks, the ring updated by each
    call (in its kernel or, for chunks of several conv tiles, by the update
    kernel after it), equals one call over the whole stream."""
    H = G.H()
    w = W.get("qwen_multibranch_zipf13")
    cfg = G.config(w)
    B, nb, d = 2, w.n_branches, w.hidden
    L = sum(chunks)
    print(f"[ring] op conv chunks {chunks}", flush=True)
    from synth import rng
    u = rng.normal_values(8 + L, np.arange(B * L * nb * d), 0.01, "bf16").reshape(B, L, nb, d)
    gam = G.gammas(w, True)
    full = torch.empty((B, L, nb, d), dtype=torch.bfloat16, device="cuda")
    H.ngram_causal_conv(cfg, G.to_device(u, w), B, L, G.conv_w(w), full, gamma_u=gam["u"])
    ring = _nan_ring(w, B)
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    outs, t0 = [], 0
    for T in chunks:
        o = torch.empty((B, T, nb, d), dtype=torch.bfloat16, device="cuda")
        H.ngram_causal_conv(cfg, G.to_device(np.ascontiguousarray(u[:, t0:t0 + T]), w), B, T,
                            G.conv_w(w), o, gamma_u=gam["u"], conv_state=ring, state_pos=pos,
                            flags=H.UPDATE_STATE)
        outs.append(o)
        t0 += T
    torch.cuda.synchronize()
    assert torch.equal(pos, torch.full_like(pos, L))
    G.check(G.to_f64(torch.cat(outs, dim=1)), G.to_f64(full), "chunks against one call")
    ref = orc.conv_block(W.to_f64(u, "bf16"), W.conv_weight_values(w), "bf16", w.max_order,
                         G.to_storage(gam["u"]), w.rms_eps)
    G.check(G.to_f64(torch.cat(outs, dim=1)), ref, "chunks against the oracle")
    n = orc.normalised_rows(W.to_f64(u, "bf16"), G.to_storage(gam["u"]), "bf16", w.rms_eps)
    R = 3 * w.max_order
    got = ring.double().cpu().numpy()
    for p in range(L - R, L):
        G.check(got[:, p % R], n[:, p], f"ring slot of position {p}", tol=1e-5, row_tol=1e-5,
                max_tol=1e-5)
