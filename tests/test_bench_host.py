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


def test_decode_projection_roofline_bytes_and_flops():
    """256 tokens, mem = d = 2,560, one branch, bf16: the projection reads E
    (256 x 2,560 x 2 B), both weight matrices once (2 x 2,560 x 2,560 x 2 B)
    and the query rows (256 x 2,560 x 2 B), and does 2 x 256 x 2,560 x 5,120
    FLOPs."""
    stages, total = bench.algorithmic(W.get("qwen_decode"))
    e = 256 * 2560 * 2
    w = 2 * 2560 * 2560 * 2
    assert stages["projection"]["bytes"] == e + w + e == 28_835_840
    assert stages["projection"]["flops"] == 2.0 * 256 * 2560 * 5120 == 6_710_886_400
    # per token: ids of the token and its 2-token history, 8 rows of 320
    # bf16, the query row in, the output row out
    assert total["per_token"] == 4 * 3 + 8 * 320 * 2 + 2560 * 2 + 2560 * 2
    assert total["weights"] == w + 4 * 2560 * 2


@pytest.mark.parametrize("name,tes", [("qwen_prefill", 2), ("qwen_prefill_fp8", 1)])
def test_gather_bytes_follow_the_table_format(name, tes):
    """The gather reads each token's 8 rows of 320 values in the table format
    and writes 2,560 bf16 values of E, plus 4-byte row ids."""
    w = W.get(name)
    stages, _ = bench.algorithmic(w)
    n = w.n_tokens
    assert stages["gather"]["bytes"] == n * (4 * 8 + 8 * 320 * tes + 2560 * 2)


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
