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
this run), and the CPU oracle timed on this host on a bounded sample.

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
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# workload setup
# ---------------------------------------------------------------------------

class Setup:
    def __init__(self, name: str, pool: int):
        import torch

        import hashed_gram_embedding_amd as H
        from synth import device as SD
        from synth import workloads as W

        self.H, self.W = H, W
        w = W.get(name)
        self.w = w
        # projection weights stored [d, mem] (torch.nn.Linear layout): the
        # library's fast path, where the projection also hashes and gathers
        self.cfg = H.make_config(**W.layer_config(w, "d_mem"))
        self.pool = pool if w.history_len else 1
        dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        self.tables = SD.make_tables(w)
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
        torch.cuda.synchronize()

    def step(self, p: int):
        s = self
        s.H.ngram_forward(s.cfg, s.ids[p], s.lut, s.tables, s.hidden[p], s.hbs, s.wk, s.wv,
                          s.conv, s.out, history=s.hist[p], workspace=s.ws)


# ---------------------------------------------------------------------------
# algorithmic bytes / flops (what the method must move, not the design's
# intermediates): ids in, gathered rows, query in, output out, weights once
# ---------------------------------------------------------------------------

def algorithmic(w):
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
    flops = 2.0 * n * w.mem_dim * w.hidden * (w.n_branches + 1)
    mem_b = n * w.mem_dim * es
    stages = {
        "hash": dict(bytes=ids_b + 4 * n * w.n_tables, flops=0.0),
        "gather": dict(bytes=4 * n * w.n_tables + rows_b + mem_b, flops=0.0),
        "projection": dict(bytes=mem_b + w_b + hid_b, flops=flops),
        "gate_conv": dict(bytes=out_b + conv_b, flops=0.0),
    }
    total = dict(bytes=ids_b + rows_b + hid_b + out_b + w_b + conv_b, flops=flops,
                 per_token=(ids_b + rows_b + hid_b + out_b) / n, weights=w_b + conv_b)
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
    ("projection", "fused"): [_CS + "project_async.hip", _CS + "epilogue.h",
                              _CS + "hashing.h"],
    ("gate_conv", "fused"): [_CS + "finalize.hip"],
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
    sequence); materialised (hash, gather to E, then the projection: the
    default); fused (the projection gathers bf16 rows itself, with
    NGRAM_FUSED_GATHER=1 and 64-wide rows)."""
    if w.dtype == "f32":
        return "f32"
    if w.seq_len == 1:
        return "decode"
    fused = (os.environ.get("NGRAM_FUSED_GATHER") == "1" and w.tdtype == "bf16"
             and w.row_dim % 64 == 0)
    return "fused" if fused else "materialised"


def stage_source_sha(stage: str, w):
    srcs = STAGE_SOURCES.get((stage, route(w)))
    return None if srcs is None else source_sha(srcs)


def counter_traffic(stage: str, w):
    """HBM bytes per launch of the stage's kernel from the committed rocprofv3
    counter runs (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for
    a plain copy of known size), or None when none were taken for this kernel
    source and workload."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        data = json.load(f)
    rec = data.get(f"{stage}:{w.name}")
    sha = stage_source_sha(stage, w)
    if not rec or sha is None or rec.get("source_sha") != sha:
        return None
    return float(rec["traffic_bytes"])


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def cpu_baseline(setup: Setup, seconds: float):
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
    args.workload = args.workload or "qwen_decode"
    args.steps = 2000 if args.steps is None else args.steps
    args.warmup = 100 if args.warmup is None else args.warmup
    print(f"[bench] setting up workload {args.workload}", file=sys.stderr, flush=True)
    setup = Setup(args.workload, args.pool)
    w = setup.w
    stages_alg, total_alg = algorithmic(w)
    stream = torch.cuda.current_stream()

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        setup.step(i % setup.pool)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps, no instrumentation
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        setup.step(i % setup.pool)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1)
    ms_per_step = ms / args.steps
    tokens_per_s = w.n_tokens / (ms_per_step * 1e-3)

    # ---- stage region: each stage's kernels stamp their own begin / end times
    # into a HIP event pair on the stream they run on (hipExtLaunchKernel), and
    # a plain event pair brackets the whole step
    print(f"[bench] stage timing {args.stage_steps} steps", file=sys.stderr, flush=True)
    ns = setup.H.ngram.N_STAGES
    # a spin kernel holds the GPU while the host enqueues the region (the
    # hook costs host time per step), so the steps then run back to back and
    # host submission gaps stay out of the event pairs
    torch.cuda.synchronize()
    torch.cuda._sleep(int(min(0.2, 3e-4 * args.stage_steps) * 2.5e9))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * ns)]
           for _ in range(args.stage_steps)]
    for i in range(args.stage_steps):
        setup.H.ngram.ngram_set_timing_events(evs[i])
        setup.step(i % setup.pool)
    mask = setup.H.ngram.ngram_timing_stage_mask()
    setup.H.ngram.ngram_set_timing_events(None)
    torch.cuda.synchronize()
    # per-step distribution: one plain event pair around each step, no stage hook
    step_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.stage_steps)]
    torch.cuda._sleep(int(min(0.2, 3e-4 * args.stage_steps) * 2.5e9))
    for i in range(args.stage_steps):
        step_evs[i][0].record(stream)
        setup.step(i % setup.pool)
        step_evs[i][1].record(stream)
    torch.cuda.synchronize()
    names = setup.H.ngram.STAGE_NAMES
    stage_avg = {}
    for k in range(ns):
        if mask >> k & 1:
            stage_avg[names[k]] = float(np.mean([e[2 * k].elapsed_time(e[2 * k + 1]) for e in evs]))
        else:
            stage_avg[names[k]] = 0.0  # absorbed into a later stage's kernel
    step_ms = np.array([a.elapsed_time(b) for a, b in step_evs])
    dom = max(stage_avg, key=stage_avg.get)
    dom_s = stage_avg[dom] * 1e-3
    a = stages_alg[dom]
    t_hbm = a["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = a["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if w.dtype == "bf16" and t_mfma > t_hbm:
        roof = {"bound": "mfma", "achieved": a["flops"] / dom_s / 1e12,
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": a["bytes"] / dom_s / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = counter_traffic(dom, w)
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = a["bytes"]
    roof["algorithmic_flops"] = a["flops"]
    roof["avg_ms"] = stage_avg[dom]

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
        "tflops": total_alg["flops"] / (ms_per_step * 1e-3) / 1e12,
        "step_ms_p50": float(np.percentile(step_ms, 50)),
        "step_ms_p99": float(np.percentile(step_ms, 99)),
        "stage_ms": stage_avg,
        "wall_s_timed": wall,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline (~{args.cpu_seconds:.0f} s)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(setup, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


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
    setup = Setup(name, 1)
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

    def bwd():
        H.ngram_backward(setup.cfg, setup.ids[0], setup.lut, setup.tables, setup.hidden[0],
                         setup.hbs, setup.wk, setup.wv, setup.conv, d_out, d_tabs, d_wk, d_wv,
                         d_cw, d_hidden=d_h, workspace=bws)

    def train_step():
        setup.step(0)
        bwd()

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
    ms_fwd = timed(lambda: setup.step(0), max(10, steps // 4))
    ms_bwd = timed(bwd, max(10, steps // 4))

    print("[bench] backward stage timing", file=sys.stderr, flush=True)
    k = min(args.stage_steps, 50)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * H.ngram.N_STAGES)]
           for _ in range(k)]
    for i in range(k):
        H.ngram.ngram_set_timing_events(evs[i])
        bwd()
    mask = H.ngram.ngram_timing_stage_mask()
    H.ngram.ngram_set_timing_events(None)
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
    bwd_flops = sum(v["flops"] for v in alg.values())
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
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline (~{args.cpu_seconds:.0f} s)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline_backward(setup, 977, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
