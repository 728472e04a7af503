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
    assert H.ngram.abi_version() == 3
    for code in range(-7, 1):
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


def test_entry_points_reject_before_launch(H):
    """Bad arguments fail on the host (no GPU exists here, so reaching a
    launch would fail differently)."""
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
    assert L.ngram_causal_conv(ref, fake, 1, 8, None, None, None, fake, None) == -1
    assert L.ngram_causal_conv(ref, fake, 1, 8, odd, None, None, fake, None) == -4
    # forward
    need = L.ngram_forward_workspace_size(ref, 1, 256)
    assert need > L.ngram_gate_workspace_size(ref, 256)
    args = [ref, fake, 1, 256, None, fake, tabs, fake, 0, fake, fake, fake, None, None, None,
            None, 0, fake, None, None, fake, need, None]
    bad = list(args)
    bad[16] = 2                                            # unknown flag
    assert L.ngram_forward(*bad) == -1
    bad = list(args)
    bad[20] = None                                         # no workspace
    assert L.ngram_forward(*bad) == -7
    bad = list(args)
    bad[21] = need - 256
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
