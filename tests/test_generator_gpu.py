"""The device fill of synthetic tensors reproduces the host generator bit for
bit (both sides of the parity tests draw inputs from the same definition)."""
import numpy as np
import pytest
import torch

from synth import device as SD
from synth import rng
from synth import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 7, 8, 1000, 4099])
def test_fill_matches_host(dtype, n):
    t = torch.empty(n, dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")
    SD.fill_normal(t, 12345, 0.02, offset=17)
    host = rng.normal_values(12345, np.arange(17, 17 + n), 0.02, dtype)
    dev = t.cpu().numpy() if dtype == "f32" else t.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(dev, host)


def test_tiny_tables_full():
    w = W.get("tiny")
    tabs = SD.make_tables(w)
    for j in range(w.n_tables):
        assert np.array_equal(tabs[j].cpu().numpy(), W.table_values(w, j))


def test_weights_and_hidden_sampled():
    w = W.get("engram_small")
    wk, wv = SD.make_weights(w)
    assert np.array_equal(wk[0].view(torch.int16).cpu().numpy().view(np.uint16),
                          W.weight_values(w, "k", 0))
    assert np.array_equal(wv.view(torch.int16).cpu().numpy().view(np.uint16),
                          W.weight_values(w, "v"))
    hid = SD.make_hidden(w, 4096)
    toks = np.array([0, 1, 2047, 4095])
    dev = hid[toks].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(dev, W.hidden_values(w, toks))


def test_large_table_rows_sampled():
    import gpu_support as G
    w = W.get("qwen_decode")
    tabs = G.tables(w)
    rs = np.random.default_rng(9)
    for j in range(w.n_tables):
        rows = np.concatenate([[0, w.rows()[j] - 1], rs.integers(0, w.rows()[j], 30)])
        dev = tabs[j][torch.from_numpy(rows).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(dev, W.table_row_values(w, j, rows))


@pytest.mark.parametrize("n", [1, 7, 16, 1000, 4099])
def test_fill_fp8_matches_host(n):
    """E4M3 codes of the draws over a table scale: the device encoder against
    the host's (torch's float8_e4m3fn conversion)."""
    t = torch.empty(n, dtype=torch.uint8, device="cuda")
    SD.fill_normal_fp8(t, 777, 0.02, 4096.0, offset=33)
    host = rng.normal_values(777, np.arange(33, 33 + n), 0.02, "fp8", 4096.0)
    assert np.array_equal(t.cpu().numpy(), host)


def test_fill_fp8_every_code_path():
    """Wide draws (sigma 100, scale 1: |x| <= 346) reach subnormal and normal
    codes of every exponent; device and host agree on all of them."""
    n = 1 << 16
    t = torch.empty(n, dtype=torch.uint8, device="cuda")
    SD.fill_normal_fp8(t, 99, 100.0, 1.0)
    host = rng.normal_values(99, np.arange(n), 100.0, "fp8", 1.0)
    assert np.array_equal(t.cpu().numpy(), host)
    assert len(np.unique(host)) > 200


def test_large_fp8_table_rows_sampled():
    import gpu_support as G
    w = W.get("qwen_decode_fp8")
    tabs = G.tables(w)
    rs = np.random.default_rng(10)
    for j in range(w.n_tables):
        rows = np.concatenate([[0, w.rows()[j] - 1], rs.integers(0, w.rows()[j], 30)])
        dev = tabs[j][torch.from_numpy(rows).cuda()].cpu().numpy()
        assert np.array_equal(dev, W.table_row_values(w, j, rows))
