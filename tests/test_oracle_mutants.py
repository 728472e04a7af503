"""The oracle's pins have teeth: each case plants one plausible mistake in a
copy of the oracle's C source (on the CPU), builds it, routes the oracle
through it and checks that at least one pin of tests/test_oracle_pins.py
fails.  The real oracle is untouched."""
import os
import subprocess
import tempfile

import pytest

import test_oracle_backward as BW
import test_oracle_pins as P
from oracle import oracle as O

SRC = os.path.join(os.path.dirname(O.__file__), "ngram_oracle.c")

# (name, text in the source, replacement)
MUTANTS = [
    ("hash combines by add, not xor", "key ^= c * mult", "key += c * mult"),
    ("n-gram window shifted one back", "(int64_t)t - i, hist", "(int64_t)t - i - 1, hist"),
    ("hash ignores the modulus", "out[j] = (int32_t)(key % (uint64_t)rows[j]);",
     "out[j] = (int32_t)(key % (uint64_t)(rows[j] + 2));"),
    ("tables concatenated in reverse", "e[t * mem + (int64_t)j * row_dim + c]",
     "e[t * mem + (int64_t)(n_tables - 1 - j) * row_dim + c]"),
    ("compression bypasses the LUT", "      c = lut[x];", "      c = x % vocab_c;"),
    ("projection uses W transposed", "load_value(w, dtype, (int64_t)m * d + n)",
     "load_value(w, dtype, (int64_t)n * mem + m)"),
    ("gate drops epsilon", "double inv_h = 1.0 / sqrt(hh / d + eps);",
     "double inv_h = 1.0 / sqrt(hh / d);"),
    ("gate scales by d, not sqrt(d)", "double z = dot / sqrt((double)d);",
     "double z = dot / (double)d;"),
    ("gate sigmoid sign flipped", "gate[t * nb + b] = 1.0 / (1.0 + exp(-z));",
     "gate[t * nb + b] = 1.0 / (1.0 + exp(z));"),
    ("gate drops gamma_k", "double kn = gk * kr[n] * inv_k;", "double kn = kr[n] * inv_k;"),
    ("gated value uses branch 0 gate", "u[(t * nb + b) * (int64_t)d + n] = gate[t * nb + b]",
     "u[(t * nb + b) * (int64_t)d + n] = gate[t * nb]"),
    ("conv norm uses sum, not mean", "double inv = 1.0 / sqrt(ss / d + eps);",
     "double inv = 1.0 / sqrt(ss + eps);"),
    ("conv taps spaced by dil-1", "int64_t p = (int64_t)t - (int64_t)i * dil;",
     "int64_t p = (int64_t)t - (int64_t)i * (dil - 1);"),
    ("conv drops SiLU gate", "delta[off + n] = u[off + n] + c / (1.0 + exp(-c));",
     "delta[off + n] = u[off + n] + c;"),
    ("conv drops the residual U", "delta[off + n] = u[off + n] + c / (1.0 + exp(-c));",
     "delta[off + n] = c / (1.0 + exp(-c));"),
    ("conv state row off by one", "int64_t s = (int64_t)span + p;", "int64_t s = (int64_t)span + p - 1;"),
    ("fp8 exponent bias 8", "v = ldexp(1.0 + m / 8.0, ex - 7);", "v = ldexp(1.0 + m / 8.0, ex - 8);"),
    ("fp8 subnormal step 2^-10", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    ("fp8 table scale dropped", "* (double)scales[j]);", "* 1.0);"),
    ("fp8 E rounded to bf16 by truncation", "if (low > 0x8000u || (low == 0x8000u && (high & 1u))) high += 1;",
     "(void)low;"),
    ("SiLU derivative drops c(1-s)", "dc[off + n] = d_delta[off + n] * s * (1.0 + c * (1.0 - s));",
     "dc[off + n] = d_delta[off + n] * s;"),
    ("conv backward taps run backwards", "const int64_t t = (int64_t)p + (int64_t)i * dil;",
     "const int64_t t = (int64_t)p - (int64_t)i * dil;"),
    ("RMSNorm backward drops the norm term", "dx[n] = g * dy[n] / r - x[n] * s / (d * r * r * r);",
     "dx[n] = g * dy[n] / r;"),
    ("sigmoid derivative is g", "const double dz = d_gate[t * nb + b] * g * (1.0 - g);",
     "const double dz = d_gate[t * nb + b] * g;"),
    ("projection backward uses W transposed",
     "acc += d_out[t * d + n] * load_value(w, dtype, (int64_t)m * d + n);",
     "acc += d_out[t * d + n] * load_value(w, dtype, (int64_t)n * mem + m);"),
    ("normalised rows drop gamma_u", "out[r * d + n] = g * x[n] * inv;",
     "out[r * d + n] = x[n] * inv;"),
    ("normalised rows drop epsilon", "const double inv = 1.0 / sqrt(ss / d + eps);\n    for (int32_t n = 0; n < d; ++n) {\n      const double g",
     "const double inv = 1.0 / sqrt(ss / d);\n    for (int32_t n = 0; n < d; ++n) {\n      const double g"),
]

# the pins run against each mutant (test function, keyword arguments)
PINS = [
    (P.test_lut_compression_fact, {"name": "tiny"}),
    (P.test_compress_invalid_ids_become_pad, {}),
    (P.test_hash_brute_force_dict, {}),
    (P.test_hash_order1_reduces_to_embedding, {}),
    (P.test_hash_context_slots_are_earlier_tokens, {"slot": 1}),
    (P.test_hash_context_slots_are_earlier_tokens, {"slot": 2}),
    (P.test_hash_hand_worked_examples, {}),
    (P.test_hash_range_uniformity_and_collisions, {}),
    (P.test_gather_is_concatenation_in_table_order, {}),
    (P.test_project_matches_library_matmul, {}),
    (P.test_identity_projections_give_memory, {}),
    (P.test_gate_orthogonal_is_half, {}),
    (P.test_gate_equal_query_key_closed_form, {}),
    (P.test_gate_scale_invariance_and_range, {}),
    (P.test_gate_gammas_enter_the_dot, {}),
    (P.test_gated_value, {}),
    (P.test_conv_zero_taps_is_identity, {}),
    (P.test_conv_single_tap_alignment, {"tap": 1}),
    (P.test_conv_single_tap_alignment, {"tap": 2}),
    (P.test_conv_causal_and_state_streaming, {}),
    (P.test_normalised_rows, {}),
    (P.test_fp8_decode_definition_and_library, {}),
    (P.test_gather_fp8_scaled_bf16, {}),
    (BW.test_backward_matches_finite_differences, dict(nb=2, nbh=2, with_state=True, residual=False)),
    (BW.test_backward_matches_finite_differences, dict(nb=1, nbh=1, with_state=False, residual=True)),
    (BW.test_scatter_is_the_gathers_adjoint, {}),
]


@pytest.fixture(scope="module")
def builddir():
    with tempfile.TemporaryDirectory() as d:
        yield d


def _build_mutant(src_text, path):
    c = path + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-shared", "-fPIC", c, "-o", path, "-lm"],
                   check=True, capture_output=True)


def test_unmutated_source_passes_every_pin(orc):
    for fn, kw in PINS:
        fn(orc=orc, **kw)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(orc, builddir, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    path = os.path.join(builddir, "m_%d.so" % MUTANTS.index((name, old, new)))
    _build_mutant(src.replace(old, new), path)
    caught = []
    with O.use_library(path):
        for fn, kw in PINS:
            try:
                fn(orc=orc, **kw)
            except AssertionError:
                caught.append(fn.__name__)
    assert caught, f"no pin fails for the planted mistake: {name}"
