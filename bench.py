#!/usr/bin/env python3
"""Benchmark of the fused N-gram embedding forward (ngram_forward) on one
MI355X.

Default workload: the Qwen-scale decode step -- 256 sequences x 1 new token
with a 2-token history, 8 prime tables of ~20M rows x 320 bf16 (95.37 GiB
resident in HBM), hidden = memory = 2560.  One step is one ngram_forward
call (compression, hashing, gather, projections, gate, conv) over one batch;
consecutive steps cycle over a pool of distinct pre-generated batches whose
inputs are resident in HBM before timing starts.

Prints one JSON line: tokens/s, the step's share of the HBM roofline, the
roofline of the dominant kernel (HIP-event timing of each stage, measured in
this run), the attainable HBM bandwidth of a plain device copy, and the CPU
oracle timed on this host on a bounded sample (all cores and one thread).
Extra keys of the same line: the decode step with a conv-state ring (the
realistic long-running decode), the step replayed from a HIP graph and the
host cost of one call, and -- over the same resident tables -- the long
prefill and the multi-branch sweep under both id distributions (with their
row-reuse fractions), each with its own roofline figures.

``--pass backward`` measures a training step of the layer instead
(ngram_forward then ngram_backward, default workload qwen_train: 16 x 4,096
tokens at the Qwen dimensions, 8 tables of ~2M rows) and prints its own line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "N-gram-embedding tokens/sec (fused forward) and % of HBM peak GB/s, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="2000 forward, 100 backward")
    ap.add_argument("--warmup", type=int, default=None, help="100 forward, 10 backward")
    ap.add_argument("--pass", dest="pass_", choices=("forward", "backward"), default="forward")
    ap.add_argument("--workload", default=None,
                    help="qwen_decode (forward), qwen_train (backward)")
    ap.add_argument("--pool", type=int, default=64, help="distinct batches (decode)")
    ap.add_argument("--stage-steps", type=int, default=200,
                    help="steps of the per-stage event timing region")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time on all threads (a one-thread run takes 0.4x more)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the ring / graph / host extras and the other workloads")
    ap.add_argument("--other-steps", type=int, default=6,
                    help="timed steps of each other workload (long prefill, multi-branch)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--proj-plan", type=int, default=None, metavar="ID",
                    help="prefill projection tile plan id (the library picks one by default)")
    ap.add_argument("--profile-region", action="store_true",
                    help="for a profiler's kernel trace: a few warmup steps, then only the "
                         "timed region, held behind a spin long enough for a profiled host to "
                         "enqueue it, so the trace averages back-to-back kernels as the line does")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# workload setup
# ---------------------------------------------------------------------------

_TABLES = {}


def shared_tables(w):
    """Device tables of a workload, built once per parameter set (the Qwen
    workloads share one 95 GiB set; the 16 x 160 geometry has its own)."""
    from synth import device as SD
    import torch
    key = (w.param_seed, tuple(w.rows()), w.row_dim, w.tdtype)
    if key not in _TABLES:
        _TABLES.clear()  # one 95 GiB set resident at a time
        torch.cuda.empty_cache()
        _TABLES[key] = SD.make_tables(w)
    return _TABLES[key]


class Setup:
    def __init__(self, name: str, pool: int, proj_plan=None):
        import torch

        import hashed_gram_embedding_amd as H
        from synth import device as SD
        from synth import workloads as W

        self.H, self.W = H, W
        w = W.get(name)
        self.w = w
        # projection weights stored [d, mem] (torch.nn.Linear layout): the
        # library's fast path
        self.cfg = H.make_config(**W.layer_config(w, "d_mem"), proj_plan=proj_plan)
        self.pool = pool if w.history_len else 1
        dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        self.tables = shared_tables(w)
        self.wk, self.wv = SD.make_weights(w, layout="d_mem")
        conv = W.conv_weight_values(w)
        self.conv = (torch.from_numpy(conv).cuda() if w.dtype == "f32" else
                     torch.from_numpy(conv.view(np.int16)).cuda().view(torch.bfloat16))
        self.lut = torch.from_numpy(W.make_lut(w)).cuda()
        ids, hists = [], []
        for p in range(self.pool):
            i, h = W.make_ids(w, batch_id=p)
            ids.append(i)
            hists.append(h)
        self.ids_host, self.hist_host = ids, hists
        self.ids = [torch.from_numpy(i).cuda() for i in ids]
        self.hist = [None if h is None else torch.from_numpy(h).cuda() for h in hists]
        n = w.n_tokens
        # one hidden pool; batch p uses tokens [p*n, (p+1)*n) of the stream
        self.hidden_all = SD.make_hidden(w, n * self.pool)
        self.hidden = [self.hidden_all[p * n:(p + 1) * n] for p in range(self.pool)]
        self.out = torch.empty((w.batch, w.seq_len, w.n_branches, w.hidden), dtype=dt,
                               device="cuda")
        ws = H.ngram_forward_workspace_size(self.cfg, w.batch, w.seq_len)
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        self.hbs = 0 if w.n_branches == 1 else w.hidden
        # the conv-state ring of a long-running decode (step_ring): the last
        # 3 * dil normalised rows of every sequence, updated in place
        self.ring = None
        self.ring_pos = None
        torch.cuda.synchronize()

    def step(self, p: int):
        s = self
        s.H.ngram_forward(s.cfg, s.ids[p], s.lut, s.tables, s.hidden[p], s.hbs, s.wk, s.wv,
                          s.conv, s.out, history=s.hist[p], workspace=s.ws)

    def step_timed(self, p: int, events) -> int:
        """One step with each stage's kernels timed into ``events``."""
        s = self
        return s.H.ngram_forward_timed(events, s.cfg, s.ids[p], s.lut, s.tables, s.hidden[p],
                                       s.hbs, s.wk, s.wv, s.conv, s.out, history=s.hist[p],
                                       workspace=s.ws)

    def step_ring(self, p: int):
        """One decode step of a long-running sequence batch: the ring supplies
        the conv taps of the three earlier positions and receives this one's
        normalised row (NGRAM_UPDATE_STATE, which also advances the
        positions), and the output is the residual stream plus Delta
        (NGRAM_ADD_RESIDUAL)."""
        import torch
        s = self
        if s.ring is None:
            w = s.w
            s.ring = torch.zeros((w.batch, 3 * w.max_order, w.n_branches, w.hidden),
                                 dtype=torch.float32, device="cuda")
            s.ring_pos = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
        s.H.ngram_forward(s.cfg, s.ids[p], s.lut, s.tables, s.hidden[p], s.hbs, s.wk, s.wv,
                          s.conv, s.out, history=s.hist[p], conv_state=s.ring,
                          state_pos=s.ring_pos, flags=s.H.ADD_RESIDUAL | s.H.UPDATE_STATE,
                          workspace=s.ws)

    def row_reuse(self) -> float:
        """Of the last step's row lookups, the fraction that named a row some
        earlier token of the step had already named (per table, averaged over
        the tables): the locality the caches can exploit.  The row ids are the
        ones the forward itself left in its workspace."""
        import torch
        w = self.w
        v = self.H.ngram_forward_workspace_view(self.cfg, w.batch, w.seq_len)
        n = w.n_tokens
        rows = self.ws[v.row_idx_offset:v.row_idx_offset + 4 * n * w.n_tables]
        rows = rows.view(torch.int32).view(n, w.n_tables)
        uniq = [int(torch.unique(rows[:, j]).numel()) for j in range(w.n_tables)]
        return float(np.mean([1.0 - u / n for u in uniq]))


# ---------------------------------------------------------------------------
# algorithmic bytes / flops (what the method must move, not the design's
# intermediates): ids in, gathered rows, query in, output out, weights once
# ---------------------------------------------------------------------------

def algorithmic(w, ring: bool = False):
    """Algorithmic bytes and FLOPs of one step, and their split over the
    stages by the kernel that moves them: ids and gathered rows to the
    hash / gather kernels, the weights to the projection, the query rows,
    the output, the conv taps (and a ring's three taps read and one row
    written, fp32) to the gate + conv kernel.  Intermediates of this design
    (E, V, partial sums) are not algorithmic bytes."""
    es = 4 if w.dtype == "f32" else 2              # activations, weights, E
    tes = {"f32": 4, "bf16": 2, "fp8": 1}[w.tdtype]  # table storage
    n = w.n_tokens
    nbh = w.n_branches if w.n_branches > 1 else 1
    ids_b = 4 * (n + w.batch * w.history_len)
    rows_b = n * w.n_tables * w.row_dim * tes
    hid_b = n * nbh * w.hidden * es
    out_b = n * w.n_branches * w.hidden * es
    w_b = (w.n_branches + 1) * w.mem_dim * w.hidden * es
    conv_b = 4 * w.hidden * es
    ring_b = 4 * 4 * n * w.n_branches * w.hidden if ring else 0
    flops = 2.0 * n * w.mem_dim * w.hidden * (w.n_branches + 1)
    stages = {
        "hash": dict(bytes=ids_b, flops=0.0),
        "gather": dict(bytes=rows_b, flops=0.0),
        "projection": dict(bytes=w_b, flops=flops),
        "gate_conv": dict(bytes=hid_b + out_b + conv_b + ring_b, flops=0.0),
    }
    if route(w) == "decode":  # one kernel hashes and gathers
        stages["gather"]["bytes"] += ids_b
        stages["hash"]["bytes"] = 0
    total = dict(bytes=ids_b + rows_b + hid_b + out_b + w_b + conv_b + ring_b, flops=flops,
                 per_token=(ids_b + rows_b + hid_b + out_b + ring_b) / n,
                 weights=w_b + conv_b)
    return stages, total


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_CS = "hashed_gram_embedding_amd/csrc/"
# kernel sources of each stage, per route (see route())
STAGE_SOURCES = {
    ("gather", "decode"): [_CS + "gather.hip", _CS + "hashing.h", _CS + "internal.h"],
    ("projection", "decode"): [_CS + "project_decode.hip"],
    ("gate_conv", "decode"): [_CS + "finalize.hip"],
    ("hash", "f32"): [_CS + "ids.hip", _CS + "hashing.h"],
    ("gather", "f32"): [_CS + "gather.hip"],
    ("projection", "f32"): [_CS + "project.hip"],
    ("gate_conv", "f32"): [_CS + "finalize.hip"],
    ("hash", "materialised"): [_CS + "ids.hip", _CS + "hashing.h"],
    ("gather", "materialised"): [_CS + "gather.hip", _CS + "internal.h"],
    ("projection", "materialised"): [_CS + "project_async.hip", _CS + "epilogue.h"],
    ("gate_conv", "materialised"): [_CS + "finalize.hip"],
}


def route(w) -> str:
    """Kernel route of a workload's forward: fp32; decode (one new token per
    sequence); materialised (hash, gather to E, then the projection)."""
    if w.dtype == "f32":
        return "f32"
    if w.seq_len == 1:
        return "decode"
    return "materialised"


def stage_source_sha(stage: str, w):
    srcs = STAGE_SOURCES.get((stage, route(w)))
    return None if srcs is None else source_sha(srcs)


def counter_record(stage: str, w):
    """The committed rocprofv3 record of the stage's kernel at this workload
    (profiles/counters.json), or None when none was taken for this kernel
    source and workload."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        data = json.load(f)
    rec = data.get(f"{stage}:{w.name}")
    sha = stage_source_sha(stage, w)
    if not rec or sha is None or rec.get("source_sha") != sha:
        return None
    return rec


def counter_traffic(stage: str, w):
    """HBM bytes per launch of the stage's kernel from the committed rocprofv3
    counter runs (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for
    a plain copy of known size), or None."""
    rec = counter_record(stage, w)
    return None if rec is None else float(rec["traffic_bytes"])


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def cpu_baseline(setup: Setup, seconds: float):
    """The oracle on all of the host's threads, then on one thread (for 40 %
    of that time)."""
    from oracle import oracle as O
    O.lib()
    cores = O.num_threads()
    res = cpu_baseline_run(setup, seconds)
    O.set_num_threads(1)
    try:
        one = cpu_baseline_run(setup, max(1.0, 0.4 * seconds))
    finally:
        O.set_num_threads(cores)
    res["value_1thread"] = one["value"]
    res["sample_1thread"] = one["sample"]
    return res


def cpu_baseline_run(setup: Setup, seconds: float):
    from oracle import oracle as O

    W, w = setup.W, setup.w
    wk = np.stack([W.weight_values(w, "k", b) for b in range(w.n_branches)])
    wv = W.weight_values(w, "v")
    conv = W.conv_weight_values(w)
    lut = W.make_lut(w)
    mult = W.hash_multipliers(w)
    rows = w.rows()
    units = []  # (ids [B,T], hist, first flat token, n_out)
    if w.history_len:  # decode: whole batches
        for p in range(setup.pool):
            units.append((setup.ids_host[p], setup.hist_host[p], p * w.n_tokens, w.n_tokens,
                          "batch"))
        desc = f"whole {w.batch}-token decode batches"
    else:  # prefill-like: 256-token windows of each sequence, with their context
        L = 256
        rs = np.random.default_rng(0)
        for k in range(64):
            b = int(rs.integers(0, w.batch))
            start = int(rs.integers(0, w.seq_len - L))
            units.append((b, start, L))
        desc = "256-token windows (plus 11-token context) at seeded offsets"
    O.lib()
    done_tokens, elapsed, used = 0, 0.0, 0
    halo = 3 * w.max_order
    for u in units:
        if w.history_len:
            ids, hist, tok0, n_out, _ = u
            toks = tok0 + np.arange(n_out)
            sub, hsub, keep = ids, hist, slice(0, n_out)
        else:
            b, start, L = u
            ids_full = setup.ids_host[0]
            s0 = max(0, start - halo)
            h0 = max(0, s0 - (w.max_order - 1))
            sub = ids_full[b:b + 1, s0:start + L]
            hsub = ids_full[b:b + 1, h0:s0] if s0 > 0 else None
            toks = b * w.seq_len + np.arange(s0, start + L)
            n_out = L
        hid = W.hidden_values(w, toks)
        comp, _ = O.compress(sub, lut, w.vocab, w.vocab_compressed)
        hc = O.compress(hsub, lut, w.vocab, w.vocab_compressed)[0] if hsub is not None else None
        r = O.hash_rows(comp, hc, w.orders, w.heads, rows, mult)
        cache = {j: {int(x): W.table_row_values(w, j, np.array([x]))[0]
                     for x in np.unique(r[:, j])} for j in range(w.n_tables)}

        def provider(j, rr, cache=cache):
            return np.stack([cache[j][int(x)] for x in rr])

        t0 = time.perf_counter()
        O.forward(sub, hsub, lut, w.vocab, w.vocab_compressed, w.orders, w.heads, rows, mult,
                  provider, hid, wk, wv, conv, w.dtype, eps=w.rms_eps)
        elapsed += time.perf_counter() - t0
        done_tokens += n_out
        used += 1
        if elapsed >= seconds:
            break
    return {"value": done_tokens / elapsed, "unit": "tokens/s", "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"{done_tokens} tokens of workload {w.name} ({used} x {desc}); "
                      f"fp64 C loops, OpenMP over tokens; {elapsed:.1f} s of oracle time"}


# ---------------------------------------------------------------------------

def copy_calibration(nbytes: int):
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "launches": 5}), flush=True)


def attainable_gbs(nbytes: int = 1 << 30, reps: int = 10) -> float:
    """HBM bandwidth a plain device copy reaches: bytes read + bytes written
    per second, over a copy much larger than the caches."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def prequeue(seconds: float):
    """Hold the GPU with a spin kernel while the host enqueues the next region,
    so that its steps then run back to back."""
    import torch
    torch.cuda._sleep(int(seconds * 2.5e9))


def prequeue_seconds(steps: int) -> float:
    """Spin long enough for the host to enqueue ``steps`` calls (a call takes
    well under 40 us of host time)."""
    return min(0.25, 40e-6 * steps + 0.005)


def time_region(fn, steps: int, stream, pre: float = 0.0) -> float:
    """Milliseconds per call of fn(i) over ``steps`` calls between two events
    (synchronised on both sides)."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if pre:
        prequeue(pre)
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def stage_timing(setup: Setup, steps: int):
    """Average kernel time of each stage (begin of its first kernel to the end
    of its last, HIP events stamped by the kernels themselves) over ``steps``."""
    import torch
    ns = setup.H.ngram.N_STAGES
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * ns)] for _ in range(steps)]
    torch.cuda.synchronize()
    prequeue(min(0.2, 3e-4 * steps + 0.01))
    mask = 0
    for i in range(steps):
        mask = setup.step_timed(i % setup.pool, evs[i])
    torch.cuda.synchronize()
    names = setup.H.ngram.STAGE_NAMES
    avg = {}
    for k in range(ns):  # 0: absorbed into a later stage's kernel
        avg[names[k]] = (float(np.mean([e[2 * k].elapsed_time(e[2 * k + 1]) for e in evs]))
                         if mask >> k & 1 else 0.0)
    return avg


def roofline(stage_avg, stages_alg, w, attainable: float):
    """Roofline of the dominant kernel (the stage with the largest kernel
    time): its algorithmic bytes or FLOPs per launch over its average launch
    time, against MI355X's published peak."""
    dom = max(stage_avg, key=stage_avg.get)
    sec = stage_avg[dom] * 1e-3
    a = stages_alg[dom]
    t_hbm = a["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = a["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if w.dtype == "bf16" and t_mfma > t_hbm:
        roof = {"bound": "mfma", "achieved": a["flops"] / sec / 1e12,
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": a["bytes"] / sec / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
        roof["frac_of_attainable"] = roof["achieved"] / attainable
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = counter_traffic(dom, w)
    rec = counter_record(dom, w)
    if rec is not None:  # the same figure over the committed rocprofv3 average
        t = rec["rocprof_avg_us"] * 1e-6
        work = a["flops"] / 1e12 if roof["unit"] == "TFLOP/s" else a["bytes"] / 1e9
        roof["avg_ms_rocprof"] = rec["rocprof_avg_us"] * 1e-3
        roof["frac_rocprof"] = work / t / roof["peak"]
    roof.update(kernel=dom, algorithmic_bytes=a["bytes"], algorithmic_flops=a["flops"],
                avg_ms=stage_avg[dom])
    return roof


def gather_op(w, stage_ms):
    """The gather kernel of the materialised route as an operation of its own
    (the ngram_gather entry point): the row ids in, the table rows in and E
    out, over its event-timed average.  Within the fused forward E is an
    intermediate; as an operation it is the output."""
    if route(w) != "materialised" or not stage_ms.get("gather"):
        return None
    tes = {"f32": 4, "bf16": 2, "fp8": 1}[w.tdtype]
    es = 4 if w.dtype == "f32" else 2
    n = w.n_tokens
    nbytes = n * w.n_tables * 4 + n * w.n_tables * w.row_dim * tes + n * w.mem_dim * es
    gbs = nbytes / (stage_ms["gather"] * 1e-3) / 1e9
    return {"bytes": nbytes, "avg_ms": stage_ms["gather"], "achieved_gbs": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS}


def step_fractions(w, total_alg, ms: float):
    """The whole step against each roofline: algorithmic bytes at 8 TB/s,
    FLOPs at 2.5 PFLOP/s, and the binding one (the larger of the two floors
    over the step time)."""
    t = ms * 1e-3
    t_hbm = total_alg["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = total_alg["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    return {"hbm_frac": t_hbm / t, "mfma_frac": t_mfma / t,
            "binding": "hbm" if t_hbm >= t_mfma else "mfma",
            "binding_frac": max(t_hbm, t_mfma) / t}


def other_workload(name: str, steps: int, warmup: int, attainable: float, proj_plan=None):
    """tokens/s, stage times and roofline figures of one more workload over the
    tables already resident (the long prefill, the multi-branch sweep)."""
    import torch
    print(f"[bench] workload {name}", file=sys.stderr, flush=True)
    setup = Setup(name, 1, proj_plan)
    w = setup.w
    stream = torch.cuda.current_stream()
    if w.history_len:  # a decode step: many steps, pre-queued
        steps *= 100
    for i in range(warmup):
        setup.step(0)
    ms = time_region(lambda i: setup.step(0), steps, stream)
    stages_alg, total_alg = algorithmic(w)
    st = stage_timing(setup, max(2, steps // 2))
    res = {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len,
           "tables": f"{w.n_tables} x {w.rows()[0]}.. rows x {w.row_dim} {w.tdtype}",
           "branches": w.n_branches,
           "ids": "uniform" if w.zipf_s is None else f"zipf {w.zipf_s}",
           "tokens_per_step": w.n_tokens, "steps": steps, "ms_per_step": ms,
           "tokens_per_s": w.n_tokens / (ms * 1e-3), "stage_ms": st,
           "algorithmic_bytes_per_step": total_alg["bytes"],
           "algorithmic_flops_per_step": total_alg["flops"],
           "tflops": total_alg["flops"] / (ms * 1e-3) / 1e12,
           "step_roofline": step_fractions(w, total_alg, ms),
           "roofline": roofline(st, stages_alg, w, attainable),
           "gather_op": gather_op(w, st),
           "row_reuse": setup.row_reuse()}
    del setup
    torch.cuda.empty_cache()
    return res


def decode_extras(setup: Setup, steps: int):
    """The headline decode step more ways: with a conv-state ring (the
    realistic long-running decode: three taps read, one row written, residual
    added), replayed from a HIP graph of one pool of steps (no host work per
    step), the host time one ngram_forward call takes to submit, and the
    layer's kernels alone when its lookup was issued ahead."""
    import torch
    w = setup.w
    stream = torch.cuda.current_stream()
    res = {}
    for i in range(20):
        setup.step_ring(i % setup.pool)
    ms_ring = time_region(lambda i: setup.step_ring(i % setup.pool), steps, stream,
                          pre=prequeue_seconds(steps))
    _, tot_ring = algorithmic(w, ring=True)
    res["decode_with_state"] = {
        "ms_per_step": ms_ring, "tokens_per_s": w.n_tokens / (ms_ring * 1e-3),
        "algorithmic_bytes_per_step": tot_ring["bytes"],
        "hbm_pct_of_peak": 100.0 * tot_ring["bytes"] / (ms_ring * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "flags": "NGRAM_UPDATE_STATE | NGRAM_ADD_RESIDUAL"}
    # host cost of one call: enqueue while a spin kernel holds the GPU
    torch.cuda.synchronize()
    prequeue(0.3)
    t0 = time.perf_counter()
    for i in range(200):
        setup.step(i % setup.pool)
    host_us = (time.perf_counter() - t0) / 200 * 1e6
    torch.cuda.synchronize()
    res["host_us_per_call"] = host_us
    # graph replay of one pool of steps
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(setup.pool):
                setup.step(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // setup.pool)
    ms_graph = time_region(lambda i: g.replay(), reps, stream) / setup.pool
    res["graph_replay"] = {"ms_per_step": ms_graph,
                           "tokens_per_s": w.n_tokens / (ms_graph * 1e-3),
                           "steps": reps * setup.pool}
    del g
    # the layer's own kernels when its lookup was issued ahead (by
    # ngram_forward_prefetch, behind a model's earlier layers): the projection
    # and the gate + conv on the rows already in the workspace
    setup.H.ngram_forward_prefetch(setup.cfg, setup.ids[0], setup.lut, setup.tables, setup.ws,
                                   history=setup.hist[0])

    def layer(i):
        s = setup
        s.H.ngram_forward(s.cfg, s.ids[0], s.lut, s.tables, s.hidden[0], s.hbs, s.wk, s.wv,
                          s.conv, s.out, history=s.hist[0], flags=s.H.PREFETCHED,
                          workspace=s.ws)

    for i in range(20):
        layer(i)
    ms_ahead = time_region(layer, steps, stream, pre=prequeue_seconds(steps))
    res["layer_with_lookup_ahead"] = {
        "ms_per_step": ms_ahead, "tokens_per_s": w.n_tokens / (ms_ahead * 1e-3),
        "flags": "NGRAM_PREFETCHED (projection and gate + conv only)"}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures the single-GPU path only: the layer runs on one GPU "
              f"(--gpus {args.gpus} is not supported).", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.pass_ == "backward":
        main_backward(args)
        return
    if args.profile_region:
        profile_region(args)
        return
    args.workload = args.workload or "qwen_decode"
    args.steps = 2000 if args.steps is None else args.steps
    args.warmup = 100 if args.warmup is None else args.warmup
    print("[bench] attainable HBM bandwidth (1 GiB device copy)", file=sys.stderr, flush=True)
    attainable = attainable_gbs()
    print(f"[bench] setting up workload {args.workload}", file=sys.stderr, flush=True)
    setup = Setup(args.workload, args.pool, args.proj_plan)
    w = setup.w
    stages_alg, total_alg = algorithmic(w)
    stream = torch.cuda.current_stream()

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        setup.step(i % setup.pool)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps, no instrumentation
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    # the GPU is held by a spin kernel while the host enqueues the region (as
    # a model's earlier layers would hold it), so the K steps run back to back
    # and the region times the kernels, not the host's first submissions
    pre_s = prequeue_seconds(args.steps)
    t0 = time.perf_counter()
    ms_per_step = time_region(lambda i: setup.step(i % setup.pool), args.steps, stream, pre=pre_s)
    wall = time.perf_counter() - t0
    tokens_per_s = w.n_tokens / (ms_per_step * 1e-3)

    # ---- stage region: each stage's kernels stamp their own begin / end
    # times into a HIP event pair on the stream they run on
    print(f"[bench] stage timing {args.stage_steps} steps", file=sys.stderr, flush=True)
    stage_avg = stage_timing(setup, args.stage_steps)
    # per-step distribution: one plain event pair around each step
    step_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.stage_steps)]
    torch.cuda.synchronize()
    prequeue(min(0.2, 3e-4 * args.stage_steps + 0.01))
    for i in range(args.stage_steps):
        step_evs[i][0].record(stream)
        setup.step(i % setup.pool)
        step_evs[i][1].record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(b) for a, b in step_evs])
    roof = roofline(stage_avg, stages_alg, w, attainable)
    steprf = step_fractions(w, total_alg, ms_per_step)
    roof["step_hbm_frac"] = steprf["hbm_frac"]
    roof["step_hbm_frac_of_attainable"] = steprf["hbm_frac"] * HBM_PEAK_GBS / attainable

    hbm_gbs = total_alg["bytes"] / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.batch, "seq_len": w.seq_len,
            "history": w.history_len, "tokens_per_step": w.n_tokens,
            "tables": f"{w.n_tables} x {w.rows()[0]}.. rows x {w.row_dim} {w.tdtype}",
            "table_gib": sum(w.rows()) * w.row_dim * {"f32": 4, "bf16": 2, "fp8": 1}[w.tdtype] / 2 ** 30,
            "mem_dim": w.mem_dim, "hidden": w.hidden, "branches": w.n_branches,
            "orders": list(w.orders), "heads_per_order": w.heads,
            "distinct_batches": setup.pool, "parallelism": "single GPU",
            "weight_layout": "[d, mem]",
        },
        "hbm_pct_of_peak": 100.0 * hbm_gbs / HBM_PEAK_GBS,
        "algorithmic_gbs": hbm_gbs,
        "algorithmic_bytes_per_step": total_alg["bytes"],
        "attainable_hbm_gbs": attainable,
        "hbm_pct_of_attainable": 100.0 * hbm_gbs / attainable,
        "tflops": total_alg["flops"] / (ms_per_step * 1e-3) / 1e12,
        "step_ms_p50": float(np.percentile(step_ms, 50)),
        "step_ms_p99": float(np.percentile(step_ms, 99)),
        "stage_ms": stage_avg,
        "stage_algorithmic_bytes": {k: v["bytes"] for k, v in stages_alg.items()},
        "wall_s_timed": wall,
        "prequeue_s": pre_s,
        "roofline": roof,
    }
    if gather_op(w, stage_avg):
        result["gather_op"] = gather_op(w, stage_avg)
    if route(w) == "decode" and not args.no_extras:
        print("[bench] decode with a conv-state ring, graph replay, host cost", file=sys.stderr,
              flush=True)
        result.update(decode_extras(setup, min(args.steps, 1000)))
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline (~{1.4 * args.cpu_seconds:.0f} s)", file=sys.stderr,
              flush=True)
        result["cpu_baseline"] = cpu_baseline(setup, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    if not args.no_extras and args.workload == "qwen_decode":
        # the largest single-GPU configuration and the locality sweep, over the
        # same resident tables
        del setup
        torch.cuda.empty_cache()
        result["other_workloads"] = [
            other_workload(n, args.other_steps, 2, attainable, args.proj_plan)
            for n in ("qwen_prefill", "qwen_multibranch_uniform", "qwen_multibranch_zipf13",
                      "qwen_decode_16x160", "qwen_prefill_16x160")]
    print(json.dumps(result), flush=True)


def profile_region(args):
    """The timed region alone (see --profile-region): under a kernel trace the
    host enqueues each call several times more slowly, so the spin that holds
    the GPU is sized at 400 us a step instead of 40, and nothing else runs
    (the stage-event and per-step regions, the extras)."""
    import torch
    w_name = args.workload or "qwen_decode"
    steps = 300 if args.steps is None else args.steps
    warmup = 3 if args.warmup is None else args.warmup
    setup = Setup(w_name, args.pool, args.proj_plan)
    for i in range(warmup):
        setup.step(i % setup.pool)
    torch.cuda.synchronize()
    pre = min(2.0, 400e-6 * steps + 0.02)
    ms = time_region(lambda i: setup.step(i % setup.pool), steps, torch.cuda.current_stream(),
                     pre=pre)
    print(json.dumps({"profile_region": w_name, "steps": steps, "warmup": warmup,
                      "ms_per_step": ms, "prequeue_s": pre}), flush=True)


# ---------------------------------------------------------------------------
# training step: forward + backward
# ---------------------------------------------------------------------------

BWD_STAGES = ("recompute", "rows", "d_e", "d_w_scatter")


def backward_algorithmic(w):
    """Algorithmic flops / bytes of ngram_backward's stages: the recompute of
    K and V, the dE product and the dW products each take 2 n mem d flops per
    projection; the per-row stage reads K, V, the query, d_out and writes dK,
    dV, d_hidden; the scatter reads dE and read-modify-writes one fp32 table
    row per token and table."""
    n, nb, d, mem = w.n_tokens, w.n_branches, w.hidden, w.mem_dim
    nbh = nb if nb > 1 else 1
    g = 2.0 * n * mem * d * (nb + 1)
    rows_b = n * w.n_tables * w.row_dim * 2
    return {
        "recompute": dict(flops=g, bytes=4 * n * (1 + w.n_tables) + rows_b + n * mem * 2
                          + (nb + 1) * mem * d * 2 + n * (nb + 1) * d * 4),
        "rows": dict(flops=0.0, bytes=n * (nb + 1) * d * 4 + n * nbh * d * 2 + n * nb * d * 2
                     + n * (nb + 1) * d * 2 + n * nbh * d * 4),
        "d_e": dict(flops=g, bytes=n * (nb + 1) * d * 2 + (nb + 1) * mem * d * 2 + n * mem * 4),
        "d_w_scatter": dict(flops=g, bytes=n * (nb + 1) * d * 2 + n * mem * 2
                            + (nb + 1) * mem * d * 4 + n * mem * 4 + 2 * n * w.n_tables
                            * w.row_dim * 4),
    }


def cpu_baseline_backward(setup: Setup, d_out_seed: int, seconds: float):
    """The oracle's forward + backward on 256-token slices of the workload's
    sequences, each taken as a sequence of its own (the same shapes and
    tables; the oracle's work per token does not depend on where a slice
    starts)."""
    from oracle import oracle as O

    W, w = setup.W, setup.w
    wk = np.stack([W.weight_values(w, "k", b) for b in range(w.n_branches)])
    wv = W.weight_values(w, "v")
    conv = W.conv_weight_values(w)
    lut = W.make_lut(w)
    mult = W.hash_multipliers(w)
    rows = w.rows()
    L = 256
    rs = np.random.default_rng(d_out_seed)
    O.lib()
    done, elapsed, used = 0, 0.0, 0
    for _ in range(64):
        b = int(rs.integers(0, w.batch))
        start = int(rs.integers(0, w.seq_len - L))
        sub = setup.ids_host[0][b:b + 1, start:start + L]
        toks = b * w.seq_len + np.arange(start, start + L)
        hid = W.hidden_values(w, toks)
        d_out = rs.standard_normal((L, w.n_branches, w.hidden))
        comp, _ = O.compress(sub, lut, w.vocab, w.vocab_compressed)
        r = O.hash_rows(comp, None, w.orders, w.heads, rows, mult)
        cache = {j: {int(x): W.table_row_values(w, j, np.array([x]))[0]
                     for x in np.unique(r[:, j])} for j in range(w.n_tables)}

        def provider(j, rr, cache=cache):
            return np.stack([cache[j][int(x)] for x in rr])

        t0 = time.perf_counter()
        O.backward(sub, None, lut, w.vocab, w.vocab_compressed, w.orders, w.heads, rows, mult,
                   provider, hid, wk, wv, conv, w.dtype, d_out, eps=w.rms_eps)
        elapsed += time.perf_counter() - t0
        done += L
        used += 1
        if elapsed >= seconds:
            break
    return {"value": done / elapsed, "unit": "tokens/s", "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"{done} tokens of workload {w.name} ({used} x 256-token slices taken as "
                      f"sequences); oracle forward + backward, fp64 C loops, OpenMP over tokens; "
                      f"{elapsed:.1f} s of oracle time"}


def main_backward(args):
    import torch
    from synth import device as SD

    name = args.workload or "qwen_train"
    print(f"[bench] setting up training workload {name}", file=sys.stderr, flush=True)
    setup = Setup(name, 1, args.proj_plan)
    H, w = setup.H, setup.w
    if w.dtype != "bf16" or w.seq_len == 1:
        raise SystemExit("--pass backward needs a bf16 prefill-shaped workload")
    n, nb, d = w.n_tokens, w.n_branches, w.hidden
    d_out = torch.empty((w.batch, w.seq_len, nb, d), dtype=torch.bfloat16, device="cuda")
    SD.fill_normal(d_out, w.hidden_seed(977), 1.0)
    # table gradients accumulate over the steps (gradient accumulation); a
    # sparse optimizer would clear only the rows it updates
    d_tabs = [torch.zeros((r, w.row_dim), dtype=torch.float32, device="cuda") for r in w.rows()]
    d_wk = torch.empty((nb, d, w.mem_dim), dtype=torch.float32, device="cuda")
    d_wv = torch.empty((d, w.mem_dim), dtype=torch.float32, device="cuda")
    d_cw = torch.empty((4, d), dtype=torch.float32, device="cuda")
    d_h = torch.empty(tuple(setup.hidden[0].shape), dtype=torch.float32, device="cuda")
    bws = torch.empty(H.ngram_backward_workspace_size(setup.cfg, w.batch, w.seq_len),
                      dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    # the training step: the forward keeps its row ids, E, K and V in the
    # backward's workspace, and the backward uses them (no recompute)
    def fwd():
        H.ngram_forward(setup.cfg, setup.ids[0], setup.lut, setup.tables, setup.hidden[0],
                        setup.hbs, setup.wk, setup.wv, setup.conv, setup.out,
                        history=setup.hist[0], flags=H.KEEP_FOR_BACKWARD, workspace=bws)

    def bwd(flags=H.KEEP_FOR_BACKWARD):
        H.ngram_backward(setup.cfg, setup.ids[0], setup.lut, setup.tables, setup.hidden[0],
                         setup.hbs, setup.wk, setup.wv, setup.conv, d_out, d_tabs, d_wk, d_wv,
                         d_cw, d_hidden=d_h, flags=flags, workspace=bws)

    def train_step():
        fwd()
        bwd()

    def train_step_recompute():  # a plain forward, and a backward that recomputes
        setup.step(0)
        bwd(0)

    def timed(fn, k):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    steps = 100 if args.steps is None else args.steps
    warm = 10 if args.warmup is None else args.warmup
    print(f"[bench] warmup {warm} training steps", file=sys.stderr, flush=True)
    for _ in range(warm):
        train_step()
    torch.cuda.synchronize()
    print(f"[bench] timing {steps} training steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    ms_step = timed(train_step, steps)
    wall = time.perf_counter() - t0
    ms_fwd = timed(fwd, max(10, steps // 4))
    ms_bwd = timed(bwd, max(10, steps // 4))
    for _ in range(3):
        train_step_recompute()
    ms_re = timed(train_step_recompute, max(10, steps // 4))
    fwd()  # the kept intermediates for the stage timing below

    print("[bench] backward stage timing", file=sys.stderr, flush=True)
    k = min(args.stage_steps, 50)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * H.ngram.N_STAGES)]
           for _ in range(k)]
    mask = 0
    for i in range(k):
        mask = H.ngram_backward_timed(evs[i], setup.cfg, setup.ids[0], setup.lut, setup.tables,
                                      setup.hidden[0], setup.hbs, setup.wk, setup.wv, setup.conv,
                                      d_out, d_tabs, d_wk, d_wv, d_cw, d_hidden=d_h,
                                      flags=H.KEEP_FOR_BACKWARD, workspace=bws)
    torch.cuda.synchronize()
    stage_avg = {BWD_STAGES[s]: (float(np.mean([e[2 * s].elapsed_time(e[2 * s + 1])
                                                for e in evs])) if mask >> s & 1 else 0.0)
                 for s in range(len(BWD_STAGES))}
    alg = backward_algorithmic(w)
    dom = max(stage_avg, key=stage_avg.get)
    a = alg[dom]
    sec = stage_avg[dom] * 1e-3
    if a["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12) > a["bytes"] / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": a["flops"] / sec / 1e12,
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": a["bytes"] / sec / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof.update(frac=roof["achieved"] / roof["peak"], traffic=None, kernel=dom,
                algorithmic_bytes=a["bytes"], algorithmic_flops=a["flops"],
                avg_ms=stage_avg[dom])
    fwd_flops = 2.0 * n * w.mem_dim * d * (nb + 1)
    # the backward on the forward's kept intermediates runs no recompute
    bwd_flops = sum(v["flops"] for k, v in alg.items() if k != "recompute")
    result = {
        "metric": "N-gram-embedding training-step tokens/sec (forward + backward), 1 MI355X",
        "value": n / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len,
                   "tokens_per_step": n,
                   "tables": f"{w.n_tables} x {w.rows()[0]}.. rows x {w.row_dim} {w.tdtype}",
                   "table_grads": "fp32, accumulated", "mem_dim": w.mem_dim, "hidden": d,
                   "branches": nb, "parallelism": "single GPU", "weight_layout": "[d, mem]"},
        "ms_forward": ms_fwd, "ms_backward": ms_bwd,
        "tflops_step": (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12,
        "tflops_backward": bwd_flops / (ms_bwd * 1e-3) / 1e12,
        "stage_ms": stage_avg, "wall_s_timed": wall, "roofline": roof,
        "flags": "forward NGRAM_KEEP_FOR_BACKWARD, backward NGRAM_KEEP_FOR_BACKWARD",
        "with_recompute": {"ms_per_step": ms_re, "tokens_per_s": n / (ms_re * 1e-3),
                           "flags": "none: a plain forward, the backward recomputes"},
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline (~{args.cpu_seconds:.0f} s)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline_backward(setup, 977, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
