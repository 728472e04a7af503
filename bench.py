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
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="qwen_decode")
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
    sequence); fused (the projection gathers bf16 rows itself); materialised
    (hash, gather to E, then the projection: fp8 tables, rows not 64-wide)."""
    if w.dtype == "f32":
        return "f32"
    if w.seq_len == 1:
        return "decode"
    return "materialised" if w.tdtype == "fp8" or w.row_dim % 64 else "fused"


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
        print(f"bench.py runs on exactly one GPU: this build measures the single-GPU path "
              f"(--gpus {args.gpus} is not supported).", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
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
    step_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.stage_steps)]
    for i in range(args.stage_steps):
        setup.H.ngram.ngram_set_timing_events(evs[i])
        step_evs[i][0].record(stream)
        setup.step(i % setup.pool)
        step_evs[i][1].record(stream)
    mask = setup.H.ngram.ngram_timing_stage_mask()
    setup.H.ngram.ngram_set_timing_events(None)
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


if __name__ == "__main__":
    main()
