"""Host-side checks of the benchmark (no GPU): the multi-GPU refusal and the
algorithmic byte and FLOP counts its roofline figures divide by, pinned to
values worked out by hand from the workload shapes."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single-GPU path only" in r.stderr
    assert r.stdout == ""


def test_decode_stage_bytes_and_flops():
    """256 tokens, mem = d = 2,560, one branch, bf16.  Each stage is charged
    the method's bytes its kernel moves: the hash + gather kernel the ids (the
    token and its 2-token history) and 8 rows of 320 bf16 per token; the
    projection both weight matrices once (2 x 2,560 x 2,560 x 2 B) and
    2 x 256 x 2,560 x 5,120 FLOPs; the gate + conv kernel the query row in,
    the output row out and the conv taps.  E, V and the partial sums are this
    design's intermediates, not algorithmic bytes; the stages add up to the
    step."""
    stages, total = bench.algorithmic(W.get("qwen_decode"))
    w = 2 * 2560 * 2560 * 2
    assert stages["projection"]["bytes"] == w == 26_214_400
    assert stages["projection"]["flops"] == 2.0 * 256 * 2560 * 5120 == 6_710_886_400
    assert stages["hash"]["bytes"] == 0
    assert stages["gather"]["bytes"] == 256 * (4 * 3 + 8 * 320 * 2)
    assert stages["gate_conv"]["bytes"] == 256 * 2560 * 2 * 2 + 4 * 2560 * 2
    assert sum(v["bytes"] for v in stages.values()) == total["bytes"]
    # per token: ids of the token and its 2-token history, 8 rows of 320
    # bf16, the query row in, the output row out
    assert total["per_token"] == 4 * 3 + 8 * 320 * 2 + 2560 * 2 + 2560 * 2
    assert total["weights"] == w + 4 * 2560 * 2


def test_decode_ring_bytes():
    """A conv-state ring adds, per token and branch, three fp32 rows read (the
    taps at t - 3, t - 6, t - 9) and one written."""
    w = W.get("qwen_decode")
    _, plain = bench.algorithmic(w)
    stages, ring = bench.algorithmic(w, ring=True)
    assert ring["bytes"] - plain["bytes"] == 256 * 4 * 2560 * 4
    assert sum(v["bytes"] for v in stages.values()) == ring["bytes"]


@pytest.mark.parametrize("name,tes", [("qwen_prefill", 2), ("qwen_prefill_fp8", 1)])
def test_gather_bytes_follow_the_table_format(name, tes):
    """Prefill: the hash kernel is charged each token's id, the gather each
    token's 8 rows of 320 values in the table format."""
    w = W.get(name)
    stages, total = bench.algorithmic(w)
    n = w.n_tokens
    assert stages["hash"]["bytes"] == 4 * n
    assert stages["gather"]["bytes"] == n * 8 * 320 * tes
    assert sum(v["bytes"] for v in stages.values()) == total["bytes"]


def test_gather_operation_bytes():
    """The gather as an operation at Qwen prefill (262,144 tokens): 8 row ids
    of 4 bytes in, 8 rows of 320 bf16 values in, E of 2,560 bf16 values out
    per token -- 2,692,743,168 bytes, so 1 ms is 2.69 TB/s; decode has no
    separate gather kernel to report."""
    w = W.get("qwen_prefill")
    g = bench.gather_op(w, {"gather": 1.0})
    assert g["bytes"] == 262144 * (32 + 5120 + 5120) == 2692743168
    assert abs(g["achieved_gbs"] - 2692.743168) < 1e-6
    assert abs(g["hbm_frac"] - 2692.743168 / 8000) < 1e-9
    assert bench.gather_op(W.get("qwen_decode"), {"gather": 1.0}) is None


def test_multibranch_counts_every_key_projection():
    """Four branches with their own W_K and a shared W_V: five d x mem
    products per token and five weight matrices."""
    w = W.get("qwen_multibranch_zipf13")
    stages, total = bench.algorithmic(w)
    assert stages["projection"]["flops"] == 2.0 * w.n_tokens * 2560 * 2560 * 5
    assert total["weights"] == 5 * 2560 * 2560 * 2 + 4 * 2560 * 2


def test_training_step_products():
    """qwen_train: 65,536 tokens; the recompute, dE and dW products each do
    2 x n x mem x d x (nb + 1) FLOPs."""
    w = W.get("qwen_train")
    b = bench.backward_algorithmic(w)
    g = 2.0 * 65536 * 2560 * 2560 * 2
    assert w.n_tokens == 65536
    for stage in ("recompute", "d_e", "d_w_scatter"):
        assert b[stage]["flops"] == g
    assert b["rows"]["flops"] == 0.0
