"""Pins for the oracle: each check ties a step to something other than the
oracle itself -- a published test vector, a fact the pages state, brute force
over explicit n-grams, a library routine the step reduces to, a closed form,
or an invariant -- so that a dropped term, a wrong sign or index or a
transposed operand in the oracle fails at least one of them."""
import json
import math
import os

import numpy as np
import pytest
import torch

from synth import rng
from synth import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# the input generator (shared by both sides) against published definitions
# --------------------------------------------------------------------------

def test_splitmix64_published_vector():
    g = _golden("splitmix64_vector.json")
    want = [int(x) for x in g["outputs"]]
    assert [rng.splitmix64_int(g["seed"], i) for i in range(5)] == want
    assert [int(x) for x in rng.splitmix64(g["seed"], np.arange(5))] == want


def test_bf16_rounding_matches_torch():
    x = rng.normal_f32(7, np.arange(100000), 3.0)
    specials = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0,
                         65504.0, 1e-30], dtype=np.float32)
    x = np.concatenate([x, specials])
    ours = rng.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_normal_generator_moments():
    x = rng.normal_f32(11, np.arange(1 << 20), 0.02).astype(np.float64)
    assert abs(x.mean()) < 0.02 * 5 / math.sqrt(x.size)
    assert abs(x.std() / 0.02 - 1.0) < 0.01
    # Irwin-Hall of 4 terms: bounded support at sqrt(12)*sigma
    assert np.abs(x).max() <= 0.02 * math.sqrt(12) * (1 + 1e-6)


# --------------------------------------------------------------------------
# fixed facts the pages state
# --------------------------------------------------------------------------

def test_fixed_facts_geometry():
    f = _golden("fixed_facts.json")
    # the pages' own layout: 16 row ids x 160 values = 2560
    assert f["row_ids_per_token"]["value"] * f["values_per_row"]["value"] == f["memory_dim"]["value"]
    # the Qwen-scale workload: 8 tables x 320 = 2560 as well
    w = W.get("qwen_decode")
    assert w.mem_dim == f["memory_dim"]["value"] == w.hidden == f["hidden_dim"]["value"]
    rows = w.rows()
    assert all(W.is_prime(r) for r in rows) and rows[0] == 20000003 and rows == sorted(rows)
    params = sum(rows) * w.row_dim
    assert abs(params / f["ngram_params"]["value"] - 1) < 1e-3
    gib = params * 2 / 2 ** 30
    assert abs(gib - f["ngram_bf16_gib"]["value"]) < 0.1
    # conv: kernel 4, dilation = max order = 3
    assert w.conv_kernel == f["conv_kernel"]["value"]
    assert w.max_order == max(f["orders"]["value"]) == 3


def test_fixed_facts_tiny_primes():
    assert W.get("tiny").rows() == W.primes_from(10007, 4) == [10007, 10009, 10037, 10039]
    assert W.primes_from(499979, 16)[0] == 499979 and len(set(W.primes_from(499979, 16))) == 16


@pytest.mark.parametrize("name", ["tiny", "engram_small", "qwen_decode"])
def test_lut_compression_fact(name, orc):
    w = W.get(name)
    lut = W.make_lut(w)
    f = _golden("fixed_facts.json")
    C = w.vocab_compressed
    assert C == round(0.77 * w.vocab)
    assert abs((1 - C / w.vocab) - f["compression_ratio"]["value"]) < 1e-3
    assert lut[0] == 0
    img = np.unique(lut)
    assert img[0] == 0 and img[-1] == C - 1 and img.size == C  # surjective onto [0, C)
    # the oracle's compression is exactly a table lookup (numpy fancy indexing)
    ids, _ = W.make_ids(w.replace(batch=1, seq_len=min(w.seq_len, 4096)))
    comp, bad = orc.compress(ids, lut, w.vocab, C)
    assert bad == 0 and np.array_equal(comp, lut[ids])


def test_compress_invalid_ids_become_pad(orc):
    lut = np.array([0, 2, 1, 2, 5], dtype=np.int32)  # entry 4 maps outside [0, 3)
    raw = np.array([1, 2, 3, -1, 5, 4, 0], dtype=np.int32)
    comp, bad = orc.compress(raw, lut, 5, 3, pad_id=0)
    assert comp.tolist() == [2, 1, 2, 0, 0, 0, 0] and bad == 3


# --------------------------------------------------------------------------
# hashing: brute force over explicit n-grams, reductions, statistics
# --------------------------------------------------------------------------

def _tiny_setup(batch=3, T=200, seed_shift=0):
    w = W.get("tiny")
    w = w.replace(batch=batch, seq_len=T, index=w.index + seed_shift) if seed_shift else \
        w.replace(batch=batch, seq_len=T)
    ids, _ = W.make_ids(w)
    return w, ids


def test_hash_brute_force_dict(orc):
    """Every position's row ids equal those of a dict keyed by the explicit
    n-gram tuple (left-padded per sequence), built by independent code."""
    w, ids = _tiny_setup()
    lut = W.make_lut(w)
    comp = lut[ids]
    mult = W.hash_multipliers(w)
    rows = w.rows()
    r = orc.hash_rows(comp, None, w.orders, w.heads, rows, mult)
    table_of = {}
    for o, n in enumerate(w.orders):
        for k in range(w.heads):
            table_of[(n, k)] = o * w.heads + k

    def row_for(tup, n, k):  # tup is (x_{t-n+1}, ..., x_t)
        j = table_of[(n, k)]
        key = 0
        for slot, c in enumerate(reversed(tup)):  # slot 0 is the current token
            key ^= (c * int(mult[j, slot])) % (1 << 64)
        return key % rows[j]

    cache = {}
    B, T = comp.shape
    for b in range(B):
        padded = [0] * (w.max_order - 1) + comp[b].tolist()
        for t in range(T):
            for n in w.orders:
                tup = tuple(padded[t + w.max_order - n: t + w.max_order])
                for k in range(w.heads):
                    want = cache.setdefault((tup, n, k), row_for(tup, n, k))
                    assert r[b * T + t, table_of[(n, k)]] == want
    # identical n-gram tuples anywhere in the batch -> identical ids (per table)
    assert len(cache) < B * T * w.n_tables


def test_hash_order1_reduces_to_embedding(orc):
    """orders=(1,), one head, multiplier 1, rows > vocab_c: the lookup is a
    plain embedding lookup of the compressed id (torch.nn.functional.embedding)."""
    w, ids = _tiny_setup(batch=2, T=100)
    lut = W.make_lut(w)
    comp = lut[ids]
    mult = np.zeros((16, 4), dtype=np.uint64)
    mult[0, 0] = 1
    rows = [10007]
    r = orc.hash_rows(comp, None, (1,), 1, rows, mult)
    table = W.table_values(w, 0)
    e = orc.gather(r, [table], "f32")
    ref = torch.nn.functional.embedding(torch.from_numpy(comp.astype(np.int64)),
                                        torch.from_numpy(table)).reshape(-1, w.row_dim)
    assert np.array_equal(e, ref.double().numpy())


@pytest.mark.parametrize("slot", [1, 2])
def test_hash_context_slots_are_earlier_tokens(orc, slot):
    """A multiplier only in slot i makes the row the id i positions back (pad
    id 0 before the sequence start, per sequence), i.e. an embedding of the
    shifted sequence -- pins the direction and padding of the n-gram window."""
    w, ids = _tiny_setup(batch=3, T=50)
    comp = W.make_lut(w)[ids]
    mult = np.zeros((16, 4), dtype=np.uint64)
    mult[0, slot] = 1
    r = orc.hash_rows(comp, None, (3,), 1, [10007], mult).reshape(3, 50)
    shifted = np.zeros_like(comp)
    shifted[:, slot:] = comp[:, :-slot]
    assert np.array_equal(r, shifted)


def test_hash_history_supplies_context(orc):
    """With history ids the missing positions come from them (decode), and the
    result equals hashing the concatenated sequence."""
    w, ids = _tiny_setup(batch=4, T=30)
    comp = W.make_lut(w)[ids]
    mult, rows = W.hash_multipliers(w), w.rows()
    full = orc.hash_rows(comp, None, w.orders, w.heads, rows, mult).reshape(4, 30, -1)
    tail = orc.hash_rows(comp[:, 2:], comp[:, :2], w.orders, w.heads, rows, mult)
    assert np.array_equal(tail.reshape(4, 28, -1), full[:, 2:])
    one = orc.hash_rows(comp[:, 2:3], comp[:, :2], w.orders, w.heads, rows, mult)
    assert np.array_equal(one.reshape(4, -1), full[:, 2])


def test_hash_range_uniformity_and_collisions(orc):
    """Rows lie in [0, p_j); over many distinct n-grams each table's rows pass a
    chi-square uniformity test and collide about as often as birthday odds."""
    w = W.get("tiny")
    rs = np.random.default_rng(0)
    n = 60000
    comp = rs.integers(1, w.vocab_compressed, size=(1, n), dtype=np.int32)
    mult, rows = W.hash_multipliers(w), w.rows()
    r = orc.hash_rows(comp, None, w.orders, w.heads, rows, mult)
    for j, p in enumerate(rows):
        col = r[:, j].astype(np.int64)
        assert col.min() >= 0 and col.max() < p
        bins = np.bincount(col * 50 // p, minlength=50)
        expect = n / 50
        chi2 = ((bins - expect) ** 2 / expect).sum()
        assert chi2 < 100, (j, chi2)  # 49 dof: p(chi2 > 100) < 1e-4
    # distinct trigrams -> rows of a 3-gram table: collisions near m^2 / (2p)
    order3 = [j for j in range(w.n_tables) if w.orders[j // w.heads] == 3][0]
    tri = {}
    pad = np.concatenate([[0, 0], comp[0]])
    for t in range(n):
        tri.setdefault((pad[t], pad[t + 1], pad[t + 2]), r[t, order3])
    vals = np.array(list(tri.values()))
    m, p = vals.size, rows[order3]
    collisions = m - np.unique(vals).size
    expected = m - p * (1 - (1 - 1 / p) ** m)
    assert abs(collisions - expected) < 6 * math.sqrt(expected) + 5


# --------------------------------------------------------------------------
# gather / concatenation
# --------------------------------------------------------------------------

def test_gather_is_concatenation_in_table_order(orc):
    w, ids = _tiny_setup(batch=2, T=64)
    comp = W.make_lut(w)[ids]
    r = orc.hash_rows(comp, None, w.orders, w.heads, w.rows(), W.hash_multipliers(w))
    tabs = [W.table_values(w, j) for j in range(w.n_tables)]
    e = orc.gather(r, tabs, "f32")
    ref = np.concatenate([tabs[j][r[:, j]] for j in range(w.n_tables)], axis=1)
    assert np.array_equal(e, ref.astype(np.float64))
    # the compact-copy path used for tables too large to hold gives the same bits
    e2 = orc.gather_from_rows(r, lambda j, rows: W.table_row_values(w, j, rows), "f32")
    assert np.array_equal(e, e2)


def test_gather_bf16_conversion_exact(orc):
    w = W.get("engram_small")
    r = np.array([[0, 1, 2, 3] * 4, [499978, 7, 100, 5] * 4], dtype=np.int32)
    e = orc.gather_from_rows(r, lambda j, rows: W.table_row_values(w, j, rows), "bf16")
    for t in range(2):
        for j in range(16):
            bits = W.table_row_values(w, j, np.array([r[t, j]]))[0]
            ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
            assert np.array_equal(e[t, j * 64:(j + 1) * 64], ref)


# Values of OCP FP8 E4M3 codes fixed by the format's definition (bias 7, 3
# mantissa bits, subnormals m * 2^-9, S.1111.111 NaN, no infinities).
FP8_CODES = [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
             (0x0F, 1.875 * 2.0 ** -6), (0x38, 1.0), (0x39, 1.125), (0x40, 2.0),
             (0x57, 15.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9))]


def test_fp8_decode_definition_and_library(orc):
    for code, value in FP8_CODES:
        assert orc.fp8_e4m3_value(code) == value, hex(code)
    assert np.isnan(orc.fp8_e4m3_value(0x7F)) and np.isnan(orc.fp8_e4m3_value(0xFF))
    assert math.copysign(1.0, orc.fp8_e4m3_value(0x80)) == -1.0  # negative zero
    # every code against torch's float8_e4m3fn
    codes = np.arange(256, dtype=np.uint8)
    mine = np.array([orc.fp8_e4m3_value(c) for c in codes])
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(mine), ~fin) and np.array_equal(mine[fin], ref[fin])


def test_gather_fp8_scaled_bf16(orc):
    """E of an FP8 table: code value times the table's scale, rounded to fp32,
    then to bf16 (torch's conversions as the reference); distinct scales per
    table, each applied to its own table only."""
    rs = np.random.default_rng(5)
    codes = rs.integers(0, 256, (3, 50, 32)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    scales = [2.0 ** -12, 0.3, 1.7e-3]
    r = rs.integers(0, 50, (9, 3)).astype(np.int32)
    e = orc.gather(r, [codes[j] for j in range(3)], "fp8", scales)
    for j in range(3):
        v = torch.from_numpy(codes[j][r[:, j]]).view(torch.float8_e4m3fn).float()
        ref = (v * torch.tensor(scales[j], dtype=torch.float32)).bfloat16().double().numpy()
        assert np.array_equal(e[:, j * 32:(j + 1) * 32], ref), j
    with pytest.raises(ValueError):
        orc.gather(r, [codes[j] for j in range(3)], "fp8")


def test_fp8_tables_generator(orc):
    """The FP8 tables' codes are the bf16 tables' draws over the scale, rounded
    to E4M3: decoding them lands within half an E4M3 step of the draw."""
    w = W.get("qwen_decode_fp8")
    rows = np.array([0, 1, 12345, w.rows()[0] - 1])
    codes = W.table_row_values(w, 0, rows)
    draws = rng.normal_f32(w.table_seed(0), (rows[:, None] * w.row_dim +
                                            np.arange(w.row_dim)[None, :]).ravel(), w.table_sigma)
    vals = np.array([orc.fp8_e4m3_value(c) for c in codes.ravel()]) * w.table_scale
    rel = np.abs(vals - draws) / np.maximum(np.abs(draws), 2.0 ** -6 * w.table_scale)
    assert rel.max() <= 2.0 ** -4 + 1e-12


# --------------------------------------------------------------------------
# projections, gate, gated value
# --------------------------------------------------------------------------

def test_project_matches_library_matmul(orc):
    rs = np.random.default_rng(1)
    e = rs.standard_normal((37, 96))
    wmat = rs.standard_normal((96, 40)).astype(np.float32)
    out = orc.project(e, wmat, "f32")
    assert np.allclose(out, e @ wmat.astype(np.float64), rtol=1e-12, atol=1e-12)
    # orientation: W is [mem, d] (a transposed operand would not even fit)
    wsq = rs.standard_normal((96, 96)).astype(np.float32)
    e2 = rs.standard_normal((5, 96))
    assert np.allclose(orc.project(e2, wsq, "f32"), e2 @ wsq.astype(np.float64))
    assert not np.allclose(orc.project(e2, wsq, "f32"), e2 @ wsq.T.astype(np.float64))


def test_identity_projections_give_memory(orc):
    d = 64
    e = np.random.default_rng(2).standard_normal((9, d))
    eye = np.eye(d, dtype=np.float32)
    assert np.array_equal(orc.project(e, eye, "f32"), e)


def test_gate_orthogonal_is_half(orc):
    d = 64
    h = np.zeros((1, 1, d), dtype=np.float32)
    k = np.zeros((1, 1, d))
    h[0, 0, :32] = 1.0
    k[0, 0, 32:] = 3.0
    assert orc.gate(h, "f32", k)[0, 0] == 0.5


def test_gate_equal_query_key_closed_form(orc):
    d, eps = 64, 1e-6
    rs = np.random.default_rng(3)
    for scale in [1e-3, 0.3, 5.0]:
        h = (rs.standard_normal((1, 1, d)) * scale).astype(np.float32)
        k = h.astype(np.float64)
        m = float((k ** 2).mean())
        z = math.sqrt(d) * m / (m + eps)
        got = orc.gate(h, "f32", k, eps=eps)[0, 0]
        assert abs(got - 1 / (1 + math.exp(-z))) < 1e-15
        # opposite key: sigmoid symmetry, gate < 1/2
        neg = orc.gate(h, "f32", -k, eps=eps)[0, 0]
        assert abs(got + neg - 1) < 1e-15 and neg < 0.5 < got


def test_gate_scale_invariance_and_range(orc):
    rs = np.random.default_rng(4)
    n, nb, d = 50, 4, 128
    h = rs.standard_normal((n, nb, d)).astype(np.float32)
    k = rs.standard_normal((n, nb, d))
    g = orc.gate(h, "f32", k)
    assert np.all((g > 0) & (g < 1))
    zmax = math.sqrt(d)
    assert np.all(g >= 1 / (1 + math.exp(zmax))) and np.all(g <= 1 / (1 + math.exp(-zmax)))
    # RMSNorm makes the gate blind to the scale of query and key (eps aside)
    g2 = orc.gate((h * 4).astype(np.float32), "f32", k * 0.25, eps=0.0)
    g1 = orc.gate(h, "f32", k, eps=0.0)
    assert np.allclose(g1, g2, rtol=1e-13, atol=1e-15)
    # per-branch queries: branch b's gate uses hidden row b only
    g_b = orc.gate(h[:, 2:3], "f32", k[:, 2:3])
    assert np.array_equal(g_b[:, 0], g[:, 2])
    # shared query (one hidden row) equals repeating it per branch
    g_sh = orc.gate(h[:, :1], "f32", k)
    g_rep = orc.gate(np.repeat(h[:, :1], nb, axis=1), "f32", k)
    assert np.array_equal(g_sh, g_rep)


def test_gate_gammas_enter_the_dot(orc):
    d = 8
    h = np.ones((1, 1, d), dtype=np.float32)
    k = np.ones((1, 1, d))
    gq = np.zeros(d, dtype=np.float32)
    gq[0] = 1.0
    # only one coordinate survives: q.k^ = 1*1 (both rms = 1 with eps 0) -> z = 1/sqrt(d)
    got = orc.gate(h, "f32", k, gamma_q=gq, eps=0.0)[0, 0]
    assert abs(got - 1 / (1 + math.exp(-1 / math.sqrt(d)))) < 1e-15
    # the same through the key's gain
    got = orc.gate(h, "f32", k, gamma_k=gq, eps=0.0)[0, 0]
    assert abs(got - 1 / (1 + math.exp(-1 / math.sqrt(d)))) < 1e-15
    # both gains 2: q^ = k^ = 2 (all ones, rms 1) -> dot = 4d -> z = 4 sqrt(d)
    two = np.full(d, 2.0, dtype=np.float32)
    got = orc.gate(h, "f32", k, gamma_q=two, gamma_k=two, eps=0.0)[0, 0]
    assert abs(got - 1 / (1 + math.exp(-4 * math.sqrt(d)))) < 1e-15


def test_gated_value(orc):
    rs = np.random.default_rng(5)
    v = rs.standard_normal((6, 16))
    g = np.array([[1.0, 0.5], [0.0, 0.25]] * 3)
    u = orc.gated_value(g, v)
    assert np.array_equal(u[:, 0], v * g[:, :1]) and np.array_equal(u[:, 1], v * g[:, 1:])


# --------------------------------------------------------------------------
# convolution block
# --------------------------------------------------------------------------

def _silu(x):
    return x / (1 + np.exp(-x))


def _rmsnorm(u, eps=1e-6):
    return u / np.sqrt((u ** 2).mean(axis=-1, keepdims=True) + eps)


def _u(B=2, T=40, nb=2, d=32, seed=6):
    return np.random.default_rng(seed).standard_normal((B, T, nb, d)) * 0.01


def test_conv_zero_taps_is_identity(orc):
    u = _u()
    w = np.zeros((4, 32), dtype=np.float32)
    assert np.array_equal(orc.conv_block(u, w, "f32", 3), u)


@pytest.mark.parametrize("tap", [0, 1, 2, 3])
def test_conv_single_tap_alignment(orc, tap):
    """Only tap i set to 1: Delta_t = U_t + SiLU(RMSNorm(U)_{t-3i}), zero
    (SiLU(0) = 0) for t < 3i -- pins tap order, dilation and causal padding."""
    u = _u()
    w = np.zeros((4, 32), dtype=np.float32)
    w[tap] = 1.0
    out = orc.conv_block(u, w, "f32", 3)
    n = _rmsnorm(u)
    ref = u.copy()
    s = 3 * tap
    ref[:, s:] += _silu(n[:, :u.shape[1] - s]) if s else _silu(n)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_conv_causal_and_state_streaming(orc):
    u = _u(B=1, T=60, nb=1, d=32)
    w = np.random.default_rng(7).standard_normal((4, 32)).astype(np.float32)
    full = orc.conv_block(u, w, "f32", 3)
    # causality: changing U_s leaves every t < s unchanged, bit for bit
    u2 = u.copy()
    u2[0, 30] += 1.0
    out2 = orc.conv_block(u2, w, "f32", 3)
    assert np.array_equal(out2[0, :30], full[0, :30]) and not np.array_equal(out2[0, 30], full[0, 30])
    assert np.array_equal(out2[0, 40:], full[0, 40:])  # beyond t = s + 9 again unchanged
    # streaming: the second half with the first half's last 9 normalised rows as
    # state equals the full-sequence result
    state = _rmsnorm(u[:, 21:30])
    half = orc.conv_block(u[:, 30:], w, "f32", 3, state=state)
    assert np.allclose(half, full[:, 30:], rtol=1e-12, atol=1e-14)


def test_normalised_rows(orc):
    """The rows a conv state holds: RMSNorm(U) with gain gamma_u.  Pinned by
    its closed forms -- mean(N^2) = m / (m + eps) with m = mean(U^2) when
    gamma = 1, invariance under scaling U when eps = 0, N parallel to
    gamma (.) U -- and by the conv it feeds: with taps (1, 0, 0, 0),
    Delta - U = SiLU(N) exactly."""
    u = _u()
    eps = 1e-6
    n = orc.normalised_rows(u, eps=eps)
    m = (u ** 2).mean(axis=-1)
    assert np.allclose((n ** 2).mean(axis=-1), m / (m + eps), rtol=1e-13, atol=0)
    n0 = orc.normalised_rows(u, eps=0.0)
    assert np.allclose(orc.normalised_rows(37.5 * u, eps=0.0), n0, rtol=1e-13, atol=1e-15)
    g = np.random.default_rng(9).standard_normal(32).astype(np.float32)
    ng = orc.normalised_rows(u, g, "f32", eps)
    x = (g.astype(np.float64) * u).reshape(-1, 32)
    y = ng.reshape(-1, 32)
    cos = (x * y).sum(1) / np.linalg.norm(x, axis=1) / np.linalg.norm(y, axis=1)
    assert np.allclose(cos, 1.0, rtol=0, atol=1e-13)
    assert np.all((x * y).sum(1) > 0)
    w = np.zeros((4, 32), dtype=np.float32)
    w[0] = 1.0
    delta = orc.conv_block(u, w, "f32", 3, eps=eps)
    assert np.allclose(delta - u, _silu(n), rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------------
# the composed forward pass
# --------------------------------------------------------------------------

def _tiny_forward(orc, ids, hist=None, w=None, **kw):
    w = w or W.get("tiny")
    B, T = ids.shape
    lut = W.make_lut(w)
    tabs = [W.table_values(w, j) for j in range(w.n_tables)]
    hid = kw.pop("hidden", None)
    if hid is None:
        hid = W.hidden_values(w, np.arange(B * T))
    wk = np.stack([W.weight_values(w, "k", b) for b in range(w.n_branches)])
    return orc.forward(ids, hist, lut, w.vocab, w.vocab_compressed, w.orders, w.heads,
                       w.rows(), W.hash_multipliers(w), tabs, hid, wk, W.weight_values(w, "v"),
                       W.conv_weight_values(w), w.dtype, **kw)


def test_forward_receptive_field_is_twelve_tokens(orc):
    """Changing x_s changes Delta_t exactly for t in [s, s+11] (the conv's
    trigram windows at t, t-3, t-6, t-9 tile [t-11, t])."""
    w = W.get("tiny")
    ids, _ = W.make_ids(w)
    base = _tiny_forward(orc, ids)["delta"]
    s = 100
    ids2 = ids.copy()
    ids2[0, s] = ids[0, s] % (w.vocab - 1) + 1 if ids[0, s] != ids[0, s + 1] else 5
    if W.make_lut(w)[ids2[0, s]] == W.make_lut(w)[ids[0, s]]:
        ids2[0, s] = next(x for x in range(1, w.vocab)
                          if W.make_lut(w)[x] != W.make_lut(w)[ids[0, s]])
    out = _tiny_forward(orc, ids2)["delta"]
    changed = np.array([not np.array_equal(out[t], base[t]) for t in range(w.seq_len)])
    assert not changed[:s].any()
    assert changed[s] and changed[s + 11]
    assert not changed[s + 12:].any()


def test_forward_sequences_independent_and_context_invariant(orc):
    """Batch rows never leak into each other, and the same token context in
    another batch slot gives identical row ids, memory vector and gate."""
    w = W.get("tiny").replace(batch=2, seq_len=64)
    ids, _ = W.make_ids(w)
    ids[1] = ids[0]
    hid = W.hidden_values(w, np.arange(64))
    hid = np.concatenate([hid, hid])
    out = _tiny_forward(orc, ids, w=w, hidden=hid)
    for key in ["row_idx", "e", "gate", "delta"]:
        a = out[key].reshape(2, 64, -1)
        assert np.array_equal(a[0], a[1]), key
    # and a changed sequence 0 leaves sequence 1 untouched
    ids2 = ids.copy()
    ids2[0, 10:20] = 7
    out2 = _tiny_forward(orc, ids2, w=w, hidden=hid)
    assert np.array_equal(out2["delta"].reshape(2, 64, -1)[1], out["delta"].reshape(2, 64, -1)[1])


def test_forward_repeated_span_gives_identical_memory(orc):
    w = W.get("tiny")
    ids, _ = W.make_ids(w)
    ids[0, 150:170] = ids[0, 40:60]
    out = _tiny_forward(orc, ids)
    # positions whose whole trigram lies in the copy see identical memory vectors
    assert np.array_equal(out["e"][152:170], out["e"][42:60])
    assert np.array_equal(out["row_idx"][152:170], out["row_idx"][42:60])


def test_forward_decode_with_history_equals_prefill(orc):
    """One new token with a 2-token history gives the prefill result at
    position 2 (no conv taps reach before the history)."""
    w = W.get("tiny").replace(batch=5, seq_len=3)
    ids, _ = W.make_ids(w)
    hid = W.hidden_values(w, np.arange(15))
    full = _tiny_forward(orc, ids, w=w, hidden=hid)
    step = _tiny_forward(orc, ids[:, 2:3], ids[:, :2], w=w, hidden=hid.reshape(5, 3, 1, -1)[:, 2])
    for key in ["row_idx", "e", "gate", "u"]:
        assert np.array_equal(step[key].reshape(5, -1), full[key].reshape(5, 3, -1)[:, 2]), key
    # Delta at position 2 uses only tap 0 (positions -1, -4, -7 are outside)
    assert np.array_equal(step["delta"].reshape(5, -1), full["delta"].reshape(5, 3, -1)[:, 2])


def test_hash_hand_worked_examples(orc):
    g = _golden("hash_worked_example.json")
    for case in g["cases"]:
        mult = np.zeros((16, 4), dtype=np.uint64)
        mult[0, 0] = np.uint64(int(case["A"][0]))
        mult[0, 1] = np.uint64(int(case["A"][1]))
        comp = np.array([case["ids"]], dtype=np.int32)
        r = orc.hash_rows(comp, None, (2,), 1, [case["p"]], mult)
        assert r[:, 0].tolist() == case["rows"], case["work"]
