"""Concurrent calls on two streams, through the C-ABI.

The library keeps no state between calls: everything a call needs lives in
its arguments and its own workspace.  Two forwards with different inputs and
workspaces, issued together on two streams so that their kernels can overlap
on the device, must each give exactly what the same call gives alone: a
decode step with its conv-state ring beside a prefill chunk, and two decode
steps of different batches."""
import pytest
import torch

import gpu_support as G
from synth import device as SD
from synth import workloads as W

pytestmark = pytest.mark.gpu


class _Call:
    """One ngram_forward with its own inputs, outputs, ring and workspace."""

    def __init__(self, w, seed, ring: bool):
        H = G.H()
        self.H, self.w = H, w
        self.cfg = G.config(w, "d_mem")
        ids, hist = W.make_ids(w, batch_id=seed)
        self.ids = torch.from_numpy(ids).cuda()
        self.hist = None if hist is None else torch.from_numpy(hist).cuda()
        self.lut = torch.from_numpy(W.make_lut(w)).cuda()
        self.tables = G.tables(w)
        self.hidden = SD.make_hidden(w, ids.size, batch_id=seed)
        self.wk, self.wv = G.weights(w, "d_mem")
        self.conv = G.conv_w(w)
        self.gam = G.gammas(w, True)
        B, T = ids.shape
        self.ws = torch.empty(H.ngram_forward_workspace_size(self.cfg, B, T), dtype=torch.uint8,
                              device="cuda")
        self.out = torch.empty((B, T, w.n_branches, w.hidden), dtype=torch.bfloat16,
                               device="cuda")
        self.gates = torch.empty((B, T, w.n_branches), dtype=torch.float32, device="cuda")
        self.ring0 = self.pos0 = None
        if ring:
            R = 3 * w.max_order
            self.ring0 = torch.randn((B, R, w.n_branches, w.hidden), device="cuda",
                                     generator=torch.Generator("cuda").manual_seed(seed))
            self.pos0 = torch.full((B,), 9, dtype=torch.int32, device="cuda")

    def run(self, stream=None):
        H = self.H
        ring = None if self.ring0 is None else self.ring0.clone()
        pos = None if self.pos0 is None else self.pos0.clone()
        flags = H.ADD_RESIDUAL | (H.UPDATE_STATE if ring is not None else 0)
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())  # the clones above
        H.ngram_forward(self.cfg, self.ids, self.lut, self.tables, self.hidden, 0, self.wk,
                        self.wv, self.conv, self.out, history=self.hist,
                        gamma_q=self.gam["q"], gamma_k=self.gam["k"], gamma_u=self.gam["u"],
                        conv_state=ring, state_pos=pos, flags=flags, gates=self.gates,
                        workspace=self.ws, stream=stream)
        return ring, pos

    def snapshot(self, ring, pos):
        return [t.clone() for t in (self.out, self.gates) + ((ring, pos) if ring is not None
                                                             else ())]


@pytest.mark.parametrize("a,b", [(("qwen_decode", 256, 1, True), ("engram_small", 2, 1500, False)),
                                 (("qwen_decode", 256, 1, True), ("qwen_decode", 33, 1, True))],
                         ids=["decode_beside_prefill", "two_decode_batches"])
def test_two_streams_match_calls_alone(a, b):
    print(f"[streams] {a} beside {b}", flush=True)
    calls = []
    for i, (name, B, T, ring) in enumerate((a, b)):
        w = W.get(name).replace(batch=B, seq_len=T)
        calls.append(_Call(w, 20 + i, ring))
    alone = []
    for c in calls:
        r = c.run()
        torch.cuda.synchronize()
        alone.append(c.snapshot(*r))
    for c in calls:
        c.out.fill_(0)
        c.gates.fill_(0)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    states = []
    for rep in range(3):
        # both calls queued before either is waited for
        states = [c.run(s) for c, s in zip(calls, streams)]
        torch.cuda.synchronize()
        for c, st, want in zip(calls, states, alone):
            got = c.snapshot(*st)
            for g, x in zip(got, want):
                gb = g.view(torch.int16) if g.dtype == torch.bfloat16 else g
                xb = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
                assert torch.equal(gb, xb), (rep, c.w.name)
