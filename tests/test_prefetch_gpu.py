"""The lookup run ahead of the layer (ngram_forward_prefetch, then
ngram_forward with NGRAM_PREFETCHED), through the C-ABI.

The n-gram hash ids depend on the token ids alone ("Qwen3.8-Flash-Next 深度研究"
§2.3), so the lookup can run before the layer's input is ready, on another
stream.  The forward that then skips its lookup must give exactly what one
plain call gives: the same kernels on the same values, so outputs, gates, row
ids and E are compared bit for bit, on the decode route (E in MFMA tiles,
history ids, a ring) and on the prefill route, with the prefetch on a second
stream ordered by an event and the workspace filled with garbage first."""
import numpy as np
import pytest
import torch

import gpu_support as G
from synth import device as SD
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _layer_inputs(w, B, T, seed):
    ids, hist = W.make_ids(w.replace(batch=B, seq_len=T), batch_id=seed)
    hidden = SD.make_hidden(w, B * T)
    return ids, hist, hidden


@pytest.mark.parametrize("name,B,T", [("qwen_decode", 256, 1), ("qwen_decode", 17, 1),
                                      ("engram_small", 2, 700)])
def test_prefetched_forward_equals_plain(name, B, T):
    H = G.H()
    w = W.get(name)
    print(f"[prefetch] {name} B={B} T={T}", flush=True)
    cfg = G.config(w, "d_mem")
    ids, hist, hidden = _layer_inputs(w, B, T, 5)
    ids_d = torch.from_numpy(ids).cuda()
    hist_d = None if hist is None else torch.from_numpy(hist).cuda()
    lut = torch.from_numpy(W.make_lut(w)).cuda()
    tabs = G.tables(w)
    wk, wv = G.weights(w, "d_mem")
    conv = G.conv_w(w)
    gam = G.gammas(w, True)
    nbh = 0 if w.n_branches == 1 else w.hidden
    size = H.ngram_forward_workspace_size(cfg, B, T)
    R = 3 * w.max_order

    def run(flags, ws, stream=None):
        out = torch.empty((B, T, w.n_branches, w.hidden), dtype=torch.bfloat16, device="cuda")
        gates = torch.empty((B, T, w.n_branches), dtype=torch.float32, device="cuda")
        ring = torch.zeros((B, R, w.n_branches, w.hidden), dtype=torch.float32, device="cuda")
        pos = torch.full((B,), 5, dtype=torch.int32, device="cuda")
        H.ngram_forward(cfg, ids_d, lut, tabs, hidden, nbh, wk, wv, conv, out, history=hist_d,
                        gamma_q=gam["q"], gamma_k=gam["k"], gamma_u=gam["u"], conv_state=ring,
                        state_pos=pos, flags=flags | H.UPDATE_STATE, gates=gates, workspace=ws,
                        stream=stream)
        return out, gates, ring, pos

    ws0 = torch.empty(size, dtype=torch.uint8, device="cuda")
    ref = run(0, ws0)
    torch.cuda.synchronize()

    ws1 = torch.full((size,), 0xA5, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        H.ngram_forward_prefetch(cfg, ids_d, lut, tabs, ws1, history=hist_d, stream=side)
        done = side.record_event()
    main = torch.cuda.current_stream()
    main.wait_event(done)
    got = run(H.PREFETCHED, ws1, stream=main)
    torch.cuda.synchronize()

    for a, b, what in zip(ref, got, ("out", "gates", "ring", "ring positions")):
        assert torch.equal(a, b), what
    r0, e0 = G.forward_ids_and_memory(cfg, w, B, T, ws0)
    r1, e1 = G.forward_ids_and_memory(cfg, w, B, T, ws1)
    assert torch.equal(r0, r1) and torch.equal(e0, e1)
