"""ngram_forward_noalloc (the forward for callers that cannot allocate: the
library's static per-GPU scratch instead of a workspace) against
ngram_forward through the C-ABI: identical outputs, gates, error flags and
ring updates, bit for bit, on two calls in a row whose second is smaller (the
scratch keeps the first call's contents), on the decode route and on the
prefill route; a call larger than the scratch is refused before any launch."""
import numpy as np
import pytest
import torch

import gpu_support as G
from synth import device as SD
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _inputs(w, layout, seed_batch=0):
    ids, hist = W.make_ids(w, batch_id=seed_batch)
    d = dict(ids=torch.from_numpy(ids).cuda(),
             hist=None if hist is None else torch.from_numpy(hist).cuda(),
             lut=torch.from_numpy(W.make_lut(w)).cuda(), tables=G.tables(w),
             hidden=SD.make_hidden(w, ids.size, batch_id=seed_batch), conv_w=G.conv_w(w),
             gam=G.gammas(w, True))
    d["wk"], d["wv"] = G.weights(w, layout)
    return d


def _both(w, layout, inp, ring0=None, pos=None, flags=1):
    """The same call through ngram_forward (own workspace) and
    ngram_forward_noalloc; each gets its own copy of the ring."""
    H = G.H()
    cfg = G.config(w, layout)
    B, T = inp["ids"].shape
    hbs = 0 if w.n_branches == 1 else w.hidden
    res = []
    for noalloc in (False, True):
        out = torch.empty((B, T, w.n_branches, w.hidden), dtype=G.tdtype(w), device="cuda")
        gates = torch.empty((B, T, w.n_branches), dtype=torch.float32, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        ring = None if ring0 is None else ring0.clone()
        p = None if pos is None else pos.clone()
        kw = dict(history=inp["hist"], gamma_q=inp["gam"]["q"], gamma_k=inp["gam"]["k"],
                  gamma_u=inp["gam"]["u"], conv_state=ring, state_pos=p, flags=flags,
                  gates=gates, err_flag=err)
        args = (cfg, inp["ids"], inp["lut"], inp["tables"], inp["hidden"], hbs, inp["wk"],
                inp["wv"], inp["conv_w"], out)
        if noalloc:
            H.ngram_forward_noalloc(*args, **kw)
        else:
            H.ngram_forward(*args, **kw)
        torch.cuda.synchronize()
        res.append((out, gates, err, ring, p))
    return res


def _same(res):
    (o1, g1, e1, r1, p1), (o2, g2, e2, r2, p2) = res
    bits = torch.int16 if o1.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(o1.view(bits), o2.view(bits)), "out"
    assert torch.equal(g1, g2), "gates"
    assert e1.item() == e2.item()
    if r1 is not None:
        assert torch.equal(r1, r2), "ring"
    if p1 is not None:
        assert torch.equal(p1, p2), "ring positions"


def test_noalloc_decode_route_two_calls():
    """Qwen-scale decode (256 sequences, a ring updated in place, residual),
    then 17 sequences: the second call finds the first one's E and partials
    in the scratch."""
    H = G.H()
    print("[noalloc] decode 256 then 17 sequences", flush=True)
    for batch, seed in ((256, 0), (17, 3)):
        w = W.get("qwen_decode").replace(batch=batch)
        inp = _inputs(w, "d_mem", seed)
        R = 3 * w.max_order
        ring = torch.randn((batch, R, 1, w.hidden), device="cuda",
                           generator=torch.Generator("cuda").manual_seed(batch))
        pos = torch.full((batch,), 40, dtype=torch.int32, device="cuda")
        _same(_both(w, "d_mem", inp, ring, pos, flags=1 | H.UPDATE_STATE))


def test_noalloc_prefill_route_two_calls():
    """Prefill (hash, gather, projection, conv): 2 x 1,500 tokens, then one
    sequence of 300 with invalid ids (the error flag must match too)."""
    print("[noalloc] prefill 2 x 1500 then 1 x 300", flush=True)
    w = W.get("engram_small").replace(batch=2, seq_len=1500)
    _same(_both(w, "d_mem", _inputs(w, "d_mem"), flags=0))
    w = W.get("engram_small").replace(batch=1, seq_len=300)
    inp = _inputs(w, "d_mem", 5)
    inp["ids"][0, 7] = -3
    res = _both(w, "d_mem", inp, flags=1)
    assert res[0][2].item() == 1
    _same(res)


def test_noalloc_refuses_more_than_its_scratch():
    H = G.H()
    w = W.get("engram_small").replace(batch=1, seq_len=8192)
    cfg = G.config(w, "d_mem")
    assert H.ngram_forward_workspace_size(cfg, 1, 8192) > H.ngram.NOALLOC_SCRATCH_BYTES
    inp = _inputs(w, "d_mem")
    out = torch.empty((1, 8192, 1, w.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(H.NgramError) as e:
        H.ngram_forward_noalloc(cfg, inp["ids"], inp["lut"], inp["tables"], inp["hidden"], 0,
                                inp["wk"], inp["wv"], inp["conv_w"], out)
    assert e.value.status == -8
