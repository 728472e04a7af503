"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, its config struct matches the binding's layout, and host-side
validation returns the documented status codes before touching the device."""
import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ngram.h")


@pytest.fixture(scope="module")
def H():
    import hashed_gram_embedding_amd as H
    return H


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ngram_[a-z_]+)\s*\(", src)))


def test_header_symbols_exported(H):
    names = _declared_functions()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", H.ngram.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = H.ngram.lib()
    for n in names:
        assert getattr(lib, n) is not None


def test_config_layout_matches_c(H):
    fields = [f for f, _ in H.NgramConfig._fields_]
    prog = "#include <stdio.h>\n#include <stddef.h>\n#include \"ngram.h\"\nint main(void){\n"
    prog += 'printf("%zu\\n", sizeof(ngram_config));\n'
    for f in fields:
        prog += f'printf("%zu\\n", offsetof(ngram_config, {f}));\n'
    prog += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "l.c")
        exe = os.path.join(d, "l")
        open(c, "w").write(prog)
        subprocess.run(["gcc", "-I" + os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                               check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(H.NgramConfig)
    for f, off in zip(fields, vals[1:]):
        assert getattr(H.NgramConfig, f).offset == off, f


def test_status_strings_and_version(H):
    assert H.ngram.abi_version() == 7
    for code in range(-8, 1):
        assert H.ngram.status_str(code).startswith("NGRAM_")


def _cfg(H, name="tiny", **over):
    from synth import workloads as W
    kw = W.layer_config(W.get(name))
    kw.update(over)
    return H.make_config(**kw)


@pytest.mark.parametrize("name", ["tiny", "engram_small", "qwen_decode", "qwen_multibranch_zipf13"])
def test_workload_configs_validate(H, name):
    assert H.ngram_config_validate(_cfg(H, name)) == 0


def test_validation_codes(H):
    ok = _cfg(H)
    assert H.ngram_config_validate(ok) == 0
    E = {"INVAL": -1, "SHAPE": -2, "DTYPE": -3, "ALIGN": -4, "RANGE": -5, "WS": -7}

    def v(**over):
        return H.ngram_config_validate(_cfg(H, **over))

    assert v(rows=[10007, 10009, 10037, 10040]) == E["RANGE"]      # not prime
    assert v(rows=[10007, 10009, 10037, 1]) == E["RANGE"]
    assert v(conv_dilation=2) == E["INVAL"]                        # dilation != max order
    assert v(conv_kernel=3) == E["INVAL"]
    assert v(orders=(3, 2)) == E["INVAL"]                          # not ascending
    assert v(row_dim=3) == E["SHAPE"]                              # 12-byte rows
    assert v(hidden_dim=66) == E["SHAPE"]
    assert v(n_branches=5) == E["INVAL"]
    assert v(pad_id=770) == E["INVAL"]
    assert v(dtype=7) == E["DTYPE"]
    c = _cfg(H)
    c.act_dtype = 1
    assert H.ngram_config_validate(c) == E["DTYPE"]                # mixed dtypes
    c = _cfg(H)
    c.mem_dim = 100
    assert H.ngram_config_validate(c) == E["INVAL"]
    c = _cfg(H, "engram_small")
    c.hidden_dim = 2048 + 16                                       # bf16 needs d % 32
    assert H.ngram_config_validate(c) == E["SHAPE"]
    c = _cfg(H)
    c.w_layout = 2
    assert H.ngram_config_validate(c) == E["INVAL"]
    c = _cfg(H)
    c.rms_eps = float("nan")
    assert H.ngram_config_validate(c) == E["INVAL"]
    # FP8 tables: bf16 activations, rows of whole 16-byte chunks, positive finite scales
    f = _cfg(H, "qwen_decode_fp8")
    assert H.ngram_config_validate(f) == 0
    f.table_scale[3] = 0.0
    assert H.ngram_config_validate(f) == E["INVAL"]
    f = _cfg(H, "qwen_decode_fp8")
    f.table_scale[0] = float("inf")
    assert H.ngram_config_validate(f) == E["INVAL"]
    f = _cfg(H, "qwen_decode_fp8")
    f.act_dtype = 0
    assert H.ngram_config_validate(f) == E["DTYPE"]                # fp8 tables, fp32 activations
    f = _cfg(H, "qwen_decode_fp8")
    f.row_dim, f.mem_dim = 312, 8 * 312
    assert H.ngram_config_validate(f) == E["SHAPE"]                # 312-byte fp8 rows
    c = _cfg(H)
    c.table_dtype = 2                                              # fp8 tables, fp32 activations
    assert H.ngram_config_validate(c) == E["DTYPE"]
    assert H.ngram.lib().ngram_config_validate(None) == E["INVAL"]
    # tile-plan overrides: a prefill plan id 0..12, decode (ni, split) pairs that fit
    assert v(proj_plan=12) == 0 and v(proj_plan=13) == E["INVAL"]
    q = lambda **o: H.ngram_config_validate(_cfg(H, "qwen_decode", **o))  # noqa: E731
    assert q(decode_plan=(5, 4)) == 0 and q(decode_plan=(3, 2)) == 0
    assert q(decode_plan=(7, 4)) == E["INVAL"]                     # ni past 6
    assert q(decode_plan=(5, 3)) == E["INVAL"]                     # 2560 / 3 not whole
    assert q(decode_plan=(6, 2)) == E["INVAL"]                     # 96 x 1280 block > 128 KiB
    c = _cfg(H, "qwen_decode")
    c.tune_decode_ni = 5                                           # one of the pair only
    assert H.ngram_config_validate(c) == E["INVAL"]


def test_primality_proof_only_in_validate(H):
    """ngram_config_validate proves every table size prime; the entry points
    screen for small factors only (the proof costs microseconds per call)."""
    L = H.ngram.lib()
    composite = 10007 * 10009          # no factor up to 61
    c = _cfg(H, rows=[10007, 10009, 10037, composite])
    assert H.ngram_config_validate(c) == -5
    assert L.ngram_forward_workspace_size(ctypes.byref(c), 1, 16) > 0
    c = _cfg(H, rows=[10007, 10009, 10037, 10007 * 61])
    assert L.ngram_forward_workspace_size(ctypes.byref(c), 1, 16) == 0


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


def test_entry_points_reject_before_launch(H):
    """Bad arguments fail on the host (no GPU exists here, so reaching a
    launch would fail differently).  The pointers are fake: on a machine with
    a GPU a validation regression would launch on them, so it is skipped."""
    if _gpu_visible():
        pytest.skip("fake device pointers: run where no GPU is visible")
    L = H.ngram.lib()
    cfg = _cfg(H)
    ref = ctypes.byref(cfg)
    fake = ctypes.c_void_p(0x10000)      # never dereferenced
    odd = ctypes.c_void_p(0x10004)       # 4-byte but not 16-byte aligned
    tabs = (ctypes.c_void_p * 16)(*([0x10000] * 4))
    assert L.ngram_compress_ids(ref, None, 10, fake, fake, None, None) == -1
    assert L.ngram_compress_ids(ref, fake, -1, fake, fake, None, None) == -2
    assert L.ngram_compress_ids(ref, fake, 0, fake, fake, None, None) == 0   # empty: no launch
    assert L.ngram_compress_ids(ref, ctypes.c_void_p(0x10002), 4, fake, fake, None, None) == -4
    assert L.ngram_hash(ref, fake, -1, 4, None, fake, None) == -2
    assert L.ngram_hash(ref, fake, 2, 4, None, None, None) == -1
    assert L.ngram_gather(ref, fake, 4, None, fake, None) == -1
    bad_tabs = (ctypes.c_void_p * 16)(0x10000, 0x10000, 0x10004, 0x10000)
    assert L.ngram_gather(ref, fake, 4, bad_tabs, fake, None) == -4
    assert L.ngram_gather(ref, fake, 4, tabs, odd, None) == -4
    # gate: workspace checks and hidden stride rule
    need = L.ngram_gate_workspace_size(ref, 256)
    assert need > 0
    assert L.ngram_gate(ref, fake, 0, fake, fake, fake, None, None, 256, fake, None, None, 0,
                        None) == -7
    assert L.ngram_gate(ref, fake, 0, fake, fake, fake, None, None, 256, fake, None, fake,
                        need - 1, None) == -7
    assert L.ngram_gate(ref, fake, 5, fake, fake, fake, None, None, 256, fake, None, fake, need,
                        None) == -2
    assert L.ngram_gate(ref, odd, 0, fake, fake, fake, None, None, 256, fake, None, fake, need,
                        None) == -4
    assert L.ngram_causal_conv(ref, fake, 1, 8, None, None, None, None, 0, fake, None) == -1
    assert L.ngram_causal_conv(ref, fake, 1, 8, odd, None, None, None, 0, fake, None) == -4
    assert L.ngram_causal_conv(ref, fake, 1, 8, fake, None, None, None, 2, fake, None) == -1
    assert L.ngram_causal_conv(ref, fake, 1, 8, fake, None, fake, None, 4, fake, None) == -1
    assert L.ngram_causal_conv(ref, fake, 1, 8, fake, None, fake, None, 2, fake, None) == -1
    assert L.ngram_causal_conv(ref, fake, 1, 8, fake, None, fake, ctypes.c_void_p(0x10002), 2,
                               fake, None) == -4
    # forward
    need = L.ngram_forward_workspace_size(ref, 1, 256)
    assert need > L.ngram_gate_workspace_size(ref, 256)
    args = [ref, fake, 1, 256, None, fake, tabs, fake, 0, fake, fake, fake, None, None, None,
            None, None, 0, fake, None, None, fake, need, None]
    bad = list(args)
    bad[17] = 16                                           # unknown flag
    assert L.ngram_forward(*bad) == -1
    bad = list(args)
    bad[17] = 8                                            # keep for backward: bf16 only
    assert L.ngram_forward(*bad) == -3
    bad = list(args)
    bad[17] = 8 | 4                                        # ... and never with a prefetch
    assert L.ngram_forward(*bad) == -1
    ecfg = _cfg(H, "engram_small", w_layout=1)             # W stored [d, mem]
    keep = [ctypes.byref(ecfg)] + args[1:]
    keep[6] = (ctypes.c_void_p * 16)(*([0x10000] * 16))
    keep[17] = 8
    keep[22] = L.ngram_backward_workspace_size(ctypes.byref(ecfg), 1, 256) - 256
    assert keep[22] > L.ngram_forward_workspace_size(ctypes.byref(ecfg), 1, 256)
    assert L.ngram_forward(*keep) == -7                    # it needs a backward workspace
    bad = list(args)
    bad[17] = 2                                            # ring update without a ring
    assert L.ngram_forward(*bad) == -1
    bad = list(args)
    bad[15], bad[17] = fake, 2                             # ... or without its positions
    assert L.ngram_forward(*bad) == -1
    bad = list(args)
    bad[16] = ctypes.c_void_p(0x10002)                     # state_pos misaligned
    assert L.ngram_forward(*bad) == -4
    bad = list(args)
    bad[21] = None                                         # no workspace
    assert L.ngram_forward(*bad) == -7
    bad = list(args)
    bad[22] = need - 256
    assert L.ngram_forward(*bad) == -7
    bad = list(args)
    bad[11] = odd                                          # conv_w misaligned
    assert L.ngram_forward(*bad) == -4
    bad = list(args)
    bad[6] = None
    assert L.ngram_forward(*bad) == -1
    bad = list(args)
    bad[2], bad[3] = 0, 256                                # empty batch
    assert L.ngram_forward(*bad) == 0
    events = (ctypes.c_void_p * 8)(*([0x10000] * 8))
    mask = ctypes.c_int32(-1)
    bad = list(args)
    bad[17] = 16
    assert L.ngram_forward_timed(*bad, events, ctypes.byref(mask)) == -1
    assert L.ngram_forward_timed(*args, None, ctypes.byref(mask)) == -1   # no events
    bad = list(args)
    bad[2], bad[3] = 0, 256
    assert L.ngram_forward_timed(*bad, events, ctypes.byref(mask)) == 0 and mask.value == 0
    # the no-allocation forward: the same checks, then its static scratch's size
    na = args[:21] + [None]
    assert L.ngram_forward_noalloc(*na) != 0                 # no GPU here: the lookup fails
    bad = list(na)
    bad[17] = 16
    assert L.ngram_forward_noalloc(*bad) == -1
    bad = list(na)
    bad[17] = 4                                            # a prefetch needs a workspace
    assert L.ngram_forward_noalloc(*bad) == -1
    bad = list(na)
    bad[17] = 8                                            # so does keeping for a backward
    assert L.ngram_forward_noalloc(*bad) == -1
    bad = list(na)
    bad[2], bad[3] = 0, 256
    assert L.ngram_forward_noalloc(*bad) == 0
    # the lookup ahead of the forward: the forward's checks of its arguments
    pf = [ref, fake, 1, 256, None, fake, tabs, None, fake, need, None]
    bad = list(pf)
    bad[1] = None
    assert L.ngram_forward_prefetch(*bad) == -1
    bad = list(pf)
    bad[2] = -1
    assert L.ngram_forward_prefetch(*bad) == -2
    bad = list(pf)
    bad[6] = None
    assert L.ngram_forward_prefetch(*bad) == -1
    bad = list(pf)
    bad[8] = None
    assert L.ngram_forward_prefetch(*bad) == -7
    bad = list(pf)
    bad[9] = need - 256                                    # too small for the whole forward
    assert L.ngram_forward_prefetch(*bad) == -7
    bad = list(pf)
    bad[8] = odd
    assert L.ngram_forward_prefetch(*bad) == -4
    bad = list(pf)
    bad[4] = ctypes.c_void_p(0x10002)                      # history misaligned
    assert L.ngram_forward_prefetch(*bad) == -4
    bad = list(pf)
    bad[2], bad[3] = 0, 256
    assert L.ngram_forward_prefetch(*bad) == 0             # empty: no launch
    q = _cfg(H, "qwen_prefill")
    big = [ctypes.byref(q)] + na[1:]
    big[2], big[3] = 1, 8192                                 # ~16 KB per token > 64 MiB
    big[6] = (ctypes.c_void_p * 16)(*([0x10000] * 8))
    assert L.ngram_forward_workspace_size(ctypes.byref(q), 1, 8192) > H.ngram.NOALLOC_SCRATCH_BYTES
    assert L.ngram_forward_noalloc(*big) == -8


def test_workspace_sizes_scale(H):
    L = H.ngram.lib()
    cfg = _cfg(H, "qwen_prefill")
    ref = ctypes.byref(cfg)
    a = L.ngram_forward_workspace_size(ref, 1, 1024)
    b = L.ngram_forward_workspace_size(ref, 1, 262144)
    per_tok = 8 * 4 + 2560 * 2 + 2560 * 4
    assert b >= 262144 * per_tok and b < 262144 * (per_tok + 4 * 4 * 64) + 4096
    assert a < b
    assert L.ngram_forward_workspace_size(None, 1, 1) == 0


@pytest.mark.parametrize("name,B,T", [("qwen_decode", 256, 1), ("qwen_decode", 3000, 1),
                                      ("qwen_prefill", 1, 1000), ("tiny", 2, 77)])
def test_workspace_view(H, name, B, T):
    """Row ids and E sit inside the workspace, without overlap; decode (one
    token per sequence, up to 2,048 of them, W stored [d, mem]) keeps E in
    16-token MFMA tiles, every other shape row-major."""
    from synth import workloads as W
    w = W.get(name)
    cfg = H.make_config(**W.layer_config(w, "d_mem" if w.dtype == "bf16" else "mem_d"))
    total = H.ngram_forward_workspace_size(cfg, B, T)
    v = H.ngram_forward_workspace_view(cfg, B, T)
    n = B * T
    es = 4 if w.dtype == "f32" else 2
    e_rows = (n + 15) // 16 * 16 if v.mem_layout == H.MEM_TILES16 else n
    spans = sorted([(v.row_idx_offset, v.row_idx_offset + 4 * n * w.n_tables),
                    (v.mem_offset, v.mem_offset + e_rows * w.mem_dim * es)])
    assert spans[0][0] >= 0 and spans[0][1] <= spans[1][0] and spans[1][1] <= total
    assert v.row_idx_offset % 16 == 0 and v.mem_offset % 16 == 0
    want_tiles = name == "qwen_decode" and B <= 2048
    assert v.mem_layout == (H.MEM_TILES16 if want_tiles else H.MEM_ROWS)


HOST_PATH_C = r'''
#include <stdio.h>
#include <stdint.h>
#include <time.h>
#include <dlfcn.h>
#include "ngram.h"
typedef int (*fwd_t)(const ngram_config*, const int32_t*, int32_t, int32_t, const int32_t*,
                     const int32_t*, const void* const*, const void*, int64_t, const void*,
                     const void*, const void*, const void*, const void*, const void*, float*,
                     const int32_t*, int32_t, void*, float*, int32_t*, void*, size_t, void*);
typedef size_t (*wss_t)(const ngram_config*, int32_t, int32_t);
int main(int argc, char** argv) {
  void* h = dlopen(argv[1], RTLD_NOW);
  if (!h) { printf("dlopen failed\n"); return 1; }
  fwd_t fwd = (fwd_t)dlsym(h, "ngram_forward");
  wss_t wss = (wss_t)dlsym(h, "ngram_forward_workspace_size");
  ngram_config c;
  FILE* f = fopen(argv[2], "rb");
  if (!f || fread(&c, sizeof c, 1, f) != 1) { printf("config read failed\n"); return 1; }
  fclose(f);
  const size_t need = wss(&c, 256, 1);
  void* fake = (void*)0x10000;
  const void* tabs[16];
  for (int j = 0; j < 16; ++j) tabs[j] = fake;
  int st = 0;
  struct timespec a, b;
  const int iters = 200000;
  clock_gettime(CLOCK_MONOTONIC, &a);
  for (int i = 0; i < iters; ++i)  /* every check runs; the short workspace stops it */
    st |= fwd(&c, fake, 256, 1, fake, fake, tabs, fake, 0, fake, fake, fake, NULL, NULL, NULL,
              NULL, NULL, 0, fake, NULL, NULL, fake, need - 1, NULL);
  clock_gettime(CLOCK_MONOTONIC, &b);
  printf("%d %.4f\n", st, ((b.tv_sec - a.tv_sec) * 1e9 + (b.tv_nsec - a.tv_nsec)) / iters / 1e3);
  return 0;
}
'''


def test_forward_host_path_is_cheap(H):
    """The host work of one ngram_forward at the Qwen decode configuration
    (every argument check and the workspace layout; the call stops at the
    workspace check, before any launch) takes at most 3 us, well below the
    GPU step it submits."""
    from synth import workloads as W
    cfg = H.make_config(**W.layer_config(W.get("qwen_decode"), "d_mem"))
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "hp.c")
        exe = os.path.join(d, "hp")
        blob = os.path.join(d, "cfg.bin")
        open(c, "w").write(HOST_PATH_C)
        open(blob, "wb").write(bytes(cfg))
        subprocess.run(["gcc", "-O2", "-I" + os.path.join(ROOT, "include"), c, "-o", exe, "-ldl"],
                       check=True)
        out = subprocess.run([exe, H.ngram.LIB_PATH, blob], capture_output=True, text=True,
                             check=True).stdout.split()
    status, us = int(out[0]), float(out[1])
    print(f"host path of ngram_forward: {us:.3f} us per call")
    assert status == -7                                    # NGRAM_EWORKSPACE on every call
    assert us <= 3.0
