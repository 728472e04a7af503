"""Properties of the GPU path that hold at any size: run-to-run bit identity
(no float atomics, so a race would show), identical outputs for an identical
context in another batch slot, causality and the 12-token receptive field."""
import numpy as np
import pytest
import torch

import gpu_support as G
from synth import device as SD
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _forward(w, ids, hidden):
    H = G.H()
    B, T = ids.shape
    cfg = G.config(w, "d_mem")
    wk, wv = G.weights(w, "d_mem")
    out = torch.empty((B, T, w.n_branches, w.hidden), dtype=G.tdtype(w), device="cuda")
    gates = torch.empty((B, T, w.n_branches), dtype=torch.float32, device="cuda")
    H.ngram_forward(cfg, torch.from_numpy(ids).cuda(), torch.from_numpy(W.make_lut(w)).cuda(),
                    G.tables(w), hidden, 0 if w.n_branches == 1 else w.hidden, wk, wv, G.conv_w(w),
                    out, gates=gates)
    torch.cuda.synchronize()
    return out, gates


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("name", ["engram_small", "qwen_multibranch_zipf13"])
def test_run_to_run_bit_identical(name):
    w = W.get(name).replace(batch=2, seq_len=2048)
    print(f"[invariant] determinism {name}", flush=True)
    ids, _ = W.make_ids(w)
    hidden = SD.make_hidden(w, ids.size)
    a, ga = _forward(w, ids, hidden)
    b, gb = _forward(w, ids, hidden)
    assert torch.equal(_bits(a), _bits(b)) and torch.equal(ga.view(torch.int32), gb.view(torch.int32))


def test_same_context_other_slot_identical():
    w = W.get("qwen_prefill").replace(batch=3, seq_len=700)
    print("[invariant] batch-slot invariance", flush=True)
    ids, _ = W.make_ids(w)
    ids[2] = ids[0]
    hidden = SD.make_hidden(w, ids.size).view(3, 700, 1, w.hidden)
    hidden[2] = hidden[0]
    out, gates = _forward(w, ids, hidden.view(-1, 1, w.hidden))
    assert torch.equal(_bits(out[2]), _bits(out[0])) and torch.equal(gates[2], gates[0])


def test_causality_and_receptive_field():
    w = W.get("qwen_prefill").replace(batch=1, seq_len=500)
    print("[invariant] causality", flush=True)
    ids, _ = W.make_ids(w)
    hidden = SD.make_hidden(w, ids.size)
    base, _ = _forward(w, ids, hidden)
    s = 250
    ids2 = ids.copy()
    lut = W.make_lut(w)
    ids2[0, s] = next(x for x in range(1, w.vocab) if lut[x] != lut[ids[0, s]])
    pert, _ = _forward(w, ids2, hidden)
    changed = [(not torch.equal(_bits(pert[0, t]), _bits(base[0, t]))) for t in range(500)]
    assert not any(changed[:s])
    assert changed[s] and changed[s + 11]
    assert not any(changed[s + 12:])
