"""The forward replayed from a HIP graph, through the C-ABI.

A serving loop captures one decode step once and replays it.  The captured
launches must then give, replay after replay, exactly what the same calls
give eagerly: each replay re-runs every kernel on the buffers captured (the
library issues no memset and keeps no host state between calls), the conv-state
ring advancing in place as it does between eager calls ("Qwen3.8-Flash-Next
深度研究" §2.3: the causal convolution over the normalised gated values, whose
taps reach three positions back).  Eager work and synchronisations run between
the replays, and every replay is compared bit for bit with its eager
counterpart: on the decode route with the ring, and on the prefill route
through the no-allocation entry point, whose static scratch an eager call with
other inputs overwrites between the replays."""
import pytest
import torch

import gpu_support as G
from synth import device as SD
from synth import workloads as W

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _inputs(w, seed):
    ids, hist = W.make_ids(w, batch_id=seed)
    d = dict(ids=torch.from_numpy(ids).cuda(),
             hist=None if hist is None else torch.from_numpy(hist).cuda(),
             lut=torch.from_numpy(W.make_lut(w)).cuda(), tables=G.tables(w),
             hidden=SD.make_hidden(w, ids.size, batch_id=seed), conv_w=G.conv_w(w),
             gam=G.gammas(w, True))
    d["wk"], d["wv"] = G.weights(w, "d_mem")
    return d


def _other_work():
    """Eager work of the program's own between two replays."""
    x = torch.randn((512, 512), device="cuda", dtype=torch.float32)
    (x @ x).sum().item()
    torch.cuda.synchronize()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_graph_replays_decode_steps_with_ring():
    H = G.H()
    w = W.get("qwen_decode")
    B = w.batch
    print(f"[graph] decode {B} sequences, ring, {REPLAYS} replays", flush=True)
    cfg = G.config(w, "d_mem")
    inp = _inputs(w, 2)
    R = 3 * w.max_order
    ring0 = torch.randn((B, R, 1, w.hidden), device="cuda",
                        generator=torch.Generator("cuda").manual_seed(11))
    pos0 = torch.full((B,), 7, dtype=torch.int32, device="cuda")
    ws = torch.empty(H.ngram_forward_workspace_size(cfg, B, 1), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((B, 1, 1, w.hidden), dtype=torch.bfloat16, device="cuda")
    gates = torch.empty((B, 1, 1), dtype=torch.float32, device="cuda")
    ring = ring0.clone()
    pos = pos0.clone()

    def step():
        H.ngram_forward(cfg, inp["ids"], inp["lut"], inp["tables"], inp["hidden"], 0, inp["wk"],
                        inp["wv"], inp["conv_w"], out, history=inp["hist"],
                        gamma_q=inp["gam"]["q"], gamma_k=inp["gam"]["k"],
                        gamma_u=inp["gam"]["u"], conv_state=ring, state_pos=pos,
                        flags=H.UPDATE_STATE | H.ADD_RESIDUAL, gates=gates, workspace=ws)

    eager = []
    for _ in range(REPLAYS):
        step()
        torch.cuda.synchronize()
        eager.append((out.clone(), gates.clone(), ring.clone(), pos.clone()))

    ring.copy_(ring0)
    pos.copy_(pos0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()
    # capture launches nothing: the ring is still at its start
    assert torch.equal(ring, ring0) and torch.equal(pos, pos0)
    out.fill_(0)
    for i in range(REPLAYS):
        _other_work()
        g.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((out, gates, ring, pos), eager[i],
                                   ("out", "gates", "ring", "ring positions")):
            assert torch.equal(_bits(got), _bits(want)), (i, what)
    del g


def test_graph_replays_noalloc_prefill():
    H = G.H()
    w = W.get("engram_small").replace(batch=2, seq_len=700)
    print(f"[graph] noalloc prefill 2 x 700, {REPLAYS} replays", flush=True)
    cfg = G.config(w, "d_mem")
    inp = _inputs(w, 4)
    B, T = inp["ids"].shape
    args = (cfg, inp["ids"], inp["lut"], inp["tables"], inp["hidden"], 0, inp["wk"], inp["wv"],
            inp["conv_w"])
    kw = dict(history=inp["hist"], gamma_q=inp["gam"]["q"], gamma_k=inp["gam"]["k"],
              gamma_u=inp["gam"]["u"], flags=H.ADD_RESIDUAL)

    ref = torch.empty((B, T, 1, w.hidden), dtype=torch.bfloat16, device="cuda")
    ref_g = torch.empty((B, T, 1), dtype=torch.float32, device="cuda")
    H.ngram_forward(*args, ref, gates=ref_g, **kw)
    torch.cuda.synchronize()

    # a different, smaller call that overwrites the static scratch between replays
    w2 = W.get("engram_small").replace(batch=1, seq_len=300)
    inp2 = _inputs(w2, 9)
    out2 = torch.empty((1, 300, 1, w2.hidden), dtype=torch.bfloat16, device="cuda")

    def scribble():
        H.ngram_forward_noalloc(cfg, inp2["ids"], inp2["lut"], inp2["tables"], inp2["hidden"], 0,
                                inp2["wk"], inp2["wv"], inp2["conv_w"], out2,
                                history=inp2["hist"])
        torch.cuda.synchronize()

    out = torch.empty_like(ref)
    gates = torch.empty_like(ref_g)
    H.ngram_forward_noalloc(*args, out, gates=gates, **kw)  # the scratch's set-up, eagerly
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref)) and torch.equal(gates, ref_g)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            H.ngram_forward_noalloc(*args, out, gates=gates, **kw)
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        scribble()
        _other_work()
        out.fill_(0)
        gates.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), (i, "out")
        assert torch.equal(gates, ref_g), (i, "gates")
    del g
