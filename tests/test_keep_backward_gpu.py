"""Training without the recompute, through the C-ABI: ngram_forward with
NGRAM_KEEP_FOR_BACKWARD leaves its row ids, E and fp32 K / V in a backward
workspace, and ngram_backward with the same flag uses them instead of
recomputing them ("Qwen3.8-Flash-Next 深度研究" §2.3: the backward is the
chain rule of the forward's steps, whose intermediates are the same either
way).

- The forward's outputs and gates with the flag equal the plain call's bit for
  bit when the plain call takes the same (prefill) route, and to rounding when
  it takes the decode route (a different product kernel).
- Every gradient of the backward on the kept intermediates equals the
  recomputing backward's to rounding (the two product kernels accumulate in
  the same order, so in practice bit for bit; the bound allows last bits),
  and the recomputing backward is held to the oracle by the backward parity
  tests.
- A second backward on the same workspace gives the same bits: the backward
  leaves what the forward kept intact."""
import numpy as np
import pytest
import torch

import gpu_support as G
from synth import device as SD
from synth import rng
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _bf16(x):
    return torch.from_numpy(rng.f32_to_bf16_bits(np.asarray(x, np.float32)).view(np.int16)).cuda().view(torch.bfloat16)


class _Layer:
    def __init__(self, w, seed, with_state):
        self.H, self.w = G.H(), w
        self.cfg = G.config(w, "d_mem")
        ids, hist = W.make_ids(w, batch_id=seed)
        self.n = ids.size
        self.B, self.T = ids.shape
        self.ids = torch.from_numpy(ids).cuda()
        self.hist = None if hist is None else torch.from_numpy(hist).cuda()
        self.lut = torch.from_numpy(W.make_lut(w)).cuda()
        self.tabs = G.tables(w)
        self.wk, self.wv = G.weights(w, "d_mem")
        self.conv = G.conv_w(w)
        self.gam = G.gammas(w, True)
        rs = np.random.default_rng(seed)
        nb, d = w.n_branches, w.hidden
        self.hidden = _bf16(rs.standard_normal((self.n, nb, d)).astype(np.float32))
        self.d_out = _bf16(rs.standard_normal((self.n, nb, d)).astype(np.float32))
        self.state = (torch.from_numpy(rs.standard_normal((self.B, 3 * w.max_order, nb, d))
                                       .astype(np.float32)).cuda() if with_state else None)
        self.pos = (torch.full((self.B,), 4, dtype=torch.int32, device="cuda")
                    if with_state else None)
        self.hbs = 0 if nb == 1 else d

    def forward(self, flags, ws):
        w = self.w
        out = torch.empty((self.B, self.T, w.n_branches, w.hidden), dtype=torch.bfloat16,
                          device="cuda")
        gates = torch.empty((self.B, self.T, w.n_branches), dtype=torch.float32, device="cuda")
        self.H.ngram_forward(self.cfg, self.ids, self.lut, self.tabs, self.hidden, self.hbs,
                             self.wk, self.wv, self.conv, out, history=self.hist,
                             gamma_q=self.gam["q"], gamma_k=self.gam["k"], gamma_u=self.gam["u"],
                             conv_state=self.state, state_pos=self.pos, flags=flags, gates=gates,
                             workspace=ws)
        torch.cuda.synchronize()
        return out, gates

    def backward(self, flags, ws):
        w = self.w
        nb, d = w.n_branches, w.hidden
        g = dict(tabs=[torch.zeros((r, w.row_dim), dtype=torch.float32, device="cuda")
                       for r in w.rows()],
                 wk=torch.empty((nb, d, w.mem_dim), dtype=torch.float32, device="cuda"),
                 wv=torch.empty((d, w.mem_dim), dtype=torch.float32, device="cuda"),
                 cw=torch.empty((4, d), dtype=torch.float32, device="cuda"),
                 h=torch.empty((self.n, nb, d), dtype=torch.float32, device="cuda"),
                 gm=torch.empty((3, d), dtype=torch.float32, device="cuda"))
        self.H.ngram_backward(self.cfg, self.ids, self.lut, self.tabs, self.hidden, self.hbs,
                              self.wk, self.wv, self.conv, self.d_out, g["tabs"], g["wk"],
                              g["wv"], g["cw"], history=self.hist, gamma_q=self.gam["q"],
                              gamma_k=self.gam["k"], gamma_u=self.gam["u"],
                              conv_state=self.state, state_pos=self.pos, flags=flags,
                              d_hidden=g["h"], d_gammas=g["gm"], workspace=ws)
        torch.cuda.synchronize()
        return g


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _close(a, b, what, tol=1e-5):
    a, b = a.double().cpu().numpy(), b.double().cpu().numpy()
    e = G.rel_err(a, b)
    assert e <= tol, (what, e)


CASES = [
    ("qwen_dims", W.get("qwen_train").replace(batch=2, seq_len=640), False, 0),
    ("branches", W.get("engram_small").replace(batch=2, seq_len=300, hidden=256, heads=2,
                                               row_start=10007, n_branches=2), True, 1),
    ("fp8_tables", W.get("engram_small").replace(batch=2, seq_len=300, hidden=256, heads=2,
                                                 row_start=10007, table_dtype="fp8"), True, 1),
    # 8,400 tokens: the forward's projection takes the default 256 x 256 plan
    # on 16x16 MFMAs, whose epilogue then also stores K and V for the backward
    ("rows_8400", W.get("engram_small").replace(batch=2, seq_len=4200, hidden=256, heads=2,
                                                row_start=10007), True, 1),
]


@pytest.mark.parametrize("name,w,with_state,flags", CASES, ids=[c[0] for c in CASES])
def test_kept_forward_and_backward(name, w, with_state, flags):
    H = G.H()
    print(f"[keep] {name} {w.batch} x {w.seq_len}", flush=True)
    L = _Layer(w, 3, with_state)
    size = H.ngram_backward_workspace_size(L.cfg, L.B, L.T)
    ws_plain = torch.empty(H.ngram_forward_workspace_size(L.cfg, L.B, L.T), dtype=torch.uint8,
                           device="cuda")
    ws_keep = torch.full((size,), 0x7F, dtype=torch.uint8, device="cuda")
    out0, gates0 = L.forward(flags, ws_plain)
    out1, gates1 = L.forward(flags | H.KEEP_FOR_BACKWARD, ws_keep)
    assert torch.equal(_bits(out0), _bits(out1)) and torch.equal(gates0, gates1)

    ws_re = torch.empty(size, dtype=torch.uint8, device="cuda")
    ref = L.backward(flags, ws_re)                           # recomputes
    got = L.backward(flags | H.KEEP_FOR_BACKWARD, ws_keep)   # the kept intermediates
    again = L.backward(flags | H.KEEP_FOR_BACKWARD, ws_keep)
    for k in ("wk", "wv", "cw", "h", "gm"):
        _close(got[k], ref[k], k)
        assert torch.equal(got[k], again[k]), k
    for j, (a, b, c) in enumerate(zip(got["tabs"], ref["tabs"], again["tabs"])):
        _close(a, b, f"table {j}")
        assert torch.equal(a, c), j


def test_kept_forward_on_a_decode_shaped_call():
    """One token per sequence: the plain call takes the decode route, the kept
    one the prefill route; outputs agree to rounding, and the backward on the
    kept intermediates matches the recomputing one."""
    H = G.H()
    w = W.get("qwen_train").replace(batch=96, seq_len=1, history_len=2)
    print("[keep] decode-shaped 96 x 1", flush=True)
    L = _Layer(w, 5, True)
    size = H.ngram_backward_workspace_size(L.cfg, L.B, L.T)
    ws_plain = torch.empty(H.ngram_forward_workspace_size(L.cfg, L.B, L.T), dtype=torch.uint8,
                           device="cuda")
    ws_keep = torch.empty(size, dtype=torch.uint8, device="cuda")
    out0, gates0 = L.forward(0, ws_plain)
    out1, gates1 = L.forward(H.KEEP_FOR_BACKWARD, ws_keep)
    G.check(G.to_f64(out1), G.to_f64(out0), "kept vs decode route", tol=1e-3, row_tol=2e-3,
            max_tol=4e-3)
    _close(gates1, gates0, "gates", tol=1e-5)
    ref = L.backward(0, torch.empty(size, dtype=torch.uint8, device="cuda"))
    got = L.backward(H.KEEP_FOR_BACKWARD, ws_keep)
    for k in ("wk", "wv", "cw", "h", "gm"):
        _close(got[k], ref[k], k)


def test_kept_forward_advances_the_ring_alike():
    """With NGRAM_UPDATE_STATE as well, the kept forward writes the same ring
    rows and positions as the plain one."""
    H = G.H()
    w = W.get("engram_small").replace(batch=2, seq_len=100, hidden=256, heads=2, row_start=10007)
    print("[keep] ring update, 2 x 100", flush=True)
    L = _Layer(w, 7, True)
    ring0, pos0 = L.state.clone(), L.pos.clone()
    ws_plain = torch.empty(H.ngram_forward_workspace_size(L.cfg, L.B, L.T), dtype=torch.uint8,
                           device="cuda")
    ws_keep = torch.empty(H.ngram_backward_workspace_size(L.cfg, L.B, L.T), dtype=torch.uint8,
                          device="cuda")
    out0, gates0 = L.forward(H.UPDATE_STATE, ws_plain)
    ring1, pos1 = L.state.clone(), L.pos.clone()
    L.state.copy_(ring0)
    L.pos.copy_(pos0)
    out1, gates1 = L.forward(H.UPDATE_STATE | H.KEEP_FOR_BACKWARD, ws_keep)
    assert torch.equal(_bits(out0), _bits(out1)) and torch.equal(gates0, gates1)
    assert torch.equal(L.state, ring1) and torch.equal(L.pos, pos1)
    assert not torch.equal(ring1, ring0)


def test_kept_refusals():
    H = G.H()
    w = W.get("engram_small").replace(batch=1, seq_len=64, hidden=256, heads=2, row_start=10007)
    L = _Layer(w, 1, False)
    small = torch.empty(H.ngram_forward_workspace_size(L.cfg, 1, 64), dtype=torch.uint8,
                        device="cuda")
    with pytest.raises(H.NgramError) as e:
        L.forward(H.KEEP_FOR_BACKWARD, small)
    assert e.value.status == -7  # NGRAM_EWORKSPACE: a backward workspace is needed
    big = torch.empty(H.ngram_backward_workspace_size(L.cfg, 1, 64), dtype=torch.uint8,
                      device="cuda")
    with pytest.raises(H.NgramError) as e:
        L.forward(H.KEEP_FOR_BACKWARD | H.PREFETCHED, big)
    assert e.value.status == -1
    out = torch.empty((1, 64, 1, w.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(H.NgramError) as e:
        H.ngram_forward_noalloc(L.cfg, L.ids, L.lut, L.tabs, L.hidden, 0, L.wk, L.wv, L.conv, out,
                                flags=H.KEEP_FOR_BACKWARD)
    assert e.value.status == -1
