"""The five synthetic workloads and their seeded input recipes.

Each workload is a frozen description (sizes, orders, heads, dtypes, value
scales, id distribution) plus functions that regenerate every input from
``seed = 1000 + index`` split into named sub-streams.  Large tensors (tables,
hidden states, projection weights) are never materialised on the host whole:
``*_values`` functions regenerate any slice on demand and the device fill
kernel produces the same bits on the GPU.

Input recipe (what the generator draws; none of it is the method itself):

* ids: bounded Zipf(s) over ranks 1..V-1 mapped to raw ids by a seeded
  permutation of [1, V); uniform over [1, V) when ``zipf_s`` is None; the long
  prefill workload builds its stream span by span (length U{8..64}; with
  probability 0.2 a span repeats the tokens at a uniformly chosen earlier
  start, otherwise it is fresh Zipf).
* LUT: seeded surjective map, raw 0 -> 0 (pad); raw [1, V) onto [1, C).
* hash multipliers: SplitMix64 draws forced odd, one per (table, n-gram slot).
* tables N(0, 0.02) (FP8 tables: the same draws divided by the table scale,
  rounded to E4M3); hidden N(0, 1); W_K, W_V N(0, 1/sqrt(mem));
  conv taps N(0, 0.5); RMSNorm gains 1 unless a test asks for random gains.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import rng

# sub-stream identifiers
S_LUT, S_IDS, S_TABLE, S_HIDDEN, S_WK, S_WV, S_CONV, S_HASH = 1, 2, 3, 4, 5, 6, 7, 8
S_GQ, S_GK, S_GU, S_PERM, S_STATE, S_HIST = 9, 10, 11, 12, 13, 14

MAX_TABLES = 16
MAX_ORDER_SLOTS = 4


def is_prime(n: int) -> bool:
    if n < 2:
        return False
    if n % 2 == 0:
        return n == 2
    f = 3
    while f * f <= n:
        if n % f == 0:
            return False
        f += 2
    return True


def primes_from(start: int, count: int) -> list:
    """The first ``count`` primes >= ``start`` (ascending)."""
    out, n = [], start
    while len(out) < count:
        if is_prime(n):
            out.append(n)
        n += 1
    return out


def compressed_vocab(vocab: int, keep: float = 0.77) -> int:
    """Size of the compressed vocabulary for a 23 % reduction (pad id included)."""
    return int(math.floor(vocab * keep + 0.5))


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # seed = 1000 + index
    vocab: int
    batch: int
    seq_len: int               # tokens per sequence in one call
    history_len: int           # ids known before position 0 (decode), else 0
    orders: tuple
    heads: int                 # hash heads per order
    row_start: int             # first candidate prime for table rows
    row_dim: int
    hidden: int
    n_branches: int
    dtype: str                 # 'f32' or 'bf16' (tables and activations)
    zipf_s: Optional[float]    # None: uniform ids
    copy_prob: float = 0.0     # repeated-span probability (long prefill)
    table_sigma: float = 0.02
    hidden_sigma: float = 1.0
    conv_kernel: int = 4
    rms_eps: float = 1e-6
    explicit_rows: tuple = ()  # table sizes given outright
    param_index: int = 0       # workloads that share tables/weights share this (0: own)
    table_dtype: Optional[str] = None  # tables' storage if not ``dtype``: 'fp8' (E4M3)
    table_scale: float = 2.0 ** -12    # fp8 tables: value = table_scale * code

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def param_seed(self) -> int:
        """Seed of the parameters (tables, W, conv, gains, hash constants)."""
        return 1000 + (self.param_index or self.index)

    @property
    def vocab_compressed(self) -> int:
        return compressed_vocab(self.vocab)

    @property
    def tdtype(self) -> str:
        """Storage dtype of the tables."""
        return self.table_dtype or self.dtype

    def table_scales(self) -> list:
        """Per-table scales (fp8 tables; 1 otherwise)."""
        s = self.table_scale if self.tdtype == "fp8" else 1.0
        return [s] * self.n_tables

    @property
    def n_tables(self) -> int:
        return len(self.orders) * self.heads

    @property
    def mem_dim(self) -> int:
        return self.n_tables * self.row_dim

    @property
    def max_order(self) -> int:
        return max(self.orders)

    @property
    def n_tokens(self) -> int:
        return self.batch * self.seq_len

    @property
    def w_sigma(self) -> float:
        return 1.0 / math.sqrt(self.mem_dim)

    @property
    def conv_sigma(self) -> float:
        return 1.0 / math.sqrt(self.conv_kernel)

    def rows(self) -> list:
        if self.explicit_rows:
            return list(self.explicit_rows)
        return primes_from(self.row_start, self.n_tables)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    # ---- per-tensor stream seeds -------------------------------------
    def table_seed(self, j: int) -> int:
        return rng.sub_seed(self.param_seed, S_TABLE, j)

    def hidden_seed(self, batch_id: int = 0) -> int:
        return rng.sub_seed(self.seed, S_HIDDEN, batch_id)

    def wk_seed(self, branch: int) -> int:
        return rng.sub_seed(self.param_seed, S_WK, branch)

    def wv_seed(self) -> int:
        return rng.sub_seed(self.param_seed, S_WV)


WORKLOADS = {
    "tiny": Workload("tiny", 1, vocab=1000, batch=1, seq_len=256, history_len=0,
                     orders=(2, 3), heads=2, row_start=10007, row_dim=32, hidden=64,
                     n_branches=1, dtype="f32", zipf_s=1.1,
                     explicit_rows=(10007, 10009, 10037, 10039)),
    "engram_small": Workload("engram_small", 2, vocab=128000, batch=8, seq_len=4096,
                             history_len=0, orders=(2, 3), heads=8, row_start=499979,
                             row_dim=64, hidden=2048, n_branches=1, dtype="bf16",
                             zipf_s=1.1),
    "qwen_decode": Workload("qwen_decode", 3, vocab=248320, batch=256, seq_len=1,
                            history_len=2, orders=(2, 3), heads=4, row_start=20000003,
                            row_dim=320, hidden=2560, n_branches=1, dtype="bf16",
                            zipf_s=1.1),
    "qwen_prefill": Workload("qwen_prefill", 4, vocab=248320, batch=1, seq_len=262144,
                             history_len=0, orders=(2, 3), heads=4, row_start=20000003,
                             row_dim=320, hidden=2560, n_branches=1, dtype="bf16",
                             zipf_s=1.1, copy_prob=0.2, param_index=3),
    "qwen_multibranch_uniform": Workload("qwen_multibranch_uniform", 5, vocab=248320,
                                         batch=16, seq_len=8192, history_len=0,
                                         orders=(2, 3), heads=4, row_start=20000003,
                                         row_dim=320, hidden=2560, n_branches=4,
                                         dtype="bf16", zipf_s=None, param_index=3),
    "qwen_multibranch_zipf13": Workload("qwen_multibranch_zipf13", 5, vocab=248320,
                                        batch=16, seq_len=8192, history_len=0,
                                        orders=(2, 3), heads=4, row_start=20000003,
                                        row_dim=320, hidden=2560, n_branches=4,
                                        dtype="bf16", zipf_s=1.3, param_index=3),
    # the same decode and prefill steps over the tables stored as FP8 E4M3
    # (scale 2^-12: the draws of N(0, 0.02) span at most +-0.07 -> codes +-283)
    "qwen_decode_fp8": Workload("qwen_decode_fp8", 3, vocab=248320, batch=256, seq_len=1,
                                history_len=2, orders=(2, 3), heads=4, row_start=20000003,
                                row_dim=320, hidden=2560, n_branches=1, dtype="bf16",
                                zipf_s=1.1, param_index=3, table_dtype="fp8"),
    # a training step of the layer at the Qwen dimensions: 16 x 4,096 tokens;
    # tables of ~2M rows so that their fp32 gradients (8 x 2M x 320 x 4 B) fit
    "qwen_train": Workload("qwen_train", 7, vocab=248320, batch=16, seq_len=4096,
                           history_len=0, orders=(2, 3), heads=4, row_start=2000003,
                           row_dim=320, hidden=2560, n_branches=1, dtype="bf16",
                           zipf_s=1.1),
    "qwen_prefill_fp8": Workload("qwen_prefill_fp8", 4, vocab=248320, batch=1, seq_len=262144,
                                 history_len=0, orders=(2, 3), heads=4, row_start=20000003,
                                 row_dim=320, hidden=2560, n_branches=1, dtype="bf16",
                                 zipf_s=1.1, copy_prob=0.2, param_index=3, table_dtype="fp8"),
    # the page's own table geometry: 16 tables (8 heads per order) of ~20M rows
    # x 160 bf16 values -- the same 2,560-wide E and 51.2B parameters, but
    # 320-byte rows that straddle 128-byte lines
    "qwen_decode_16x160": Workload("qwen_decode_16x160", 8, vocab=248320, batch=256, seq_len=1,
                                   history_len=2, orders=(2, 3), heads=8, row_start=20000003,
                                   row_dim=160, hidden=2560, n_branches=1, dtype="bf16",
                                   zipf_s=1.1),
    "qwen_prefill_16x160": Workload("qwen_prefill_16x160", 9, vocab=248320, batch=1,
                                    seq_len=262144, history_len=0, orders=(2, 3), heads=8,
                                    row_start=20000003, row_dim=160, hidden=2560, n_branches=1,
                                    dtype="bf16", zipf_s=1.1, copy_prob=0.2, param_index=8),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


# ---------------------------------------------------------------------------
# ids, LUT, hash multipliers
# ---------------------------------------------------------------------------

def raw_id_permutation(w: Workload) -> np.ndarray:
    """Seeded permutation of [1, V): Zipf rank r (1-based) -> raw id perm[r-1]."""
    keys = rng.splitmix64(rng.sub_seed(w.param_seed, S_PERM), np.arange(w.vocab - 1))
    return (np.argsort(keys, kind="stable") + 1).astype(np.int32)


def make_lut(w: Workload) -> np.ndarray:
    """Seeded surjective compression LUT: int32[V], LUT[0] = 0, image = [0, C)."""
    V, C = w.vocab, w.vocab_compressed
    seed = rng.sub_seed(w.param_seed, S_LUT)
    order = np.argsort(rng.splitmix64(seed, np.arange(V - 1)), kind="stable") + 1
    lut = np.zeros(V, dtype=np.int32)
    lut[order[: C - 1]] = np.arange(1, C, dtype=np.int32)
    rest = order[C - 1:]
    if rest.size:
        draws = rng.splitmix64(rng.sub_seed(seed, 1), np.arange(rest.size))
        lut[rest] = (1 + (draws % np.uint64(C - 1))).astype(np.int32)
    return lut


def hash_multipliers(w: Workload) -> np.ndarray:
    """uint64[MAX_TABLES, MAX_ORDER_SLOTS] odd multipliers (unused slots zero)."""
    seed = rng.sub_seed(w.param_seed, S_HASH)
    out = np.zeros((MAX_TABLES, MAX_ORDER_SLOTS), dtype=np.uint64)
    for o, n in enumerate(w.orders):
        for k in range(w.heads):
            j = o * w.heads + k
            for i in range(n):
                out[j, i] = np.uint64(rng.splitmix64_int(seed, MAX_ORDER_SLOTS * j + i) | 1)
    return out


def zipf_ids(seed: int, n: int, vocab: int, s: float, perm: np.ndarray) -> np.ndarray:
    ranks = np.arange(1, vocab, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-s))
    u = rng.uniform01(seed, np.arange(n)) * cdf[-1]
    r = np.searchsorted(cdf, u, side="right")
    r = np.minimum(r, vocab - 2)
    return perm[r].astype(np.int32)


def uniform_ids(seed: int, n: int, vocab: int) -> np.ndarray:
    u = rng.uniform01(seed, np.arange(n))
    return (1 + np.floor(u * (vocab - 1))).astype(np.int32)


def _draw_ids(w: Workload, seed: int, n: int, perm: Optional[np.ndarray]) -> np.ndarray:
    if w.zipf_s is None:
        return uniform_ids(seed, n, w.vocab)
    return zipf_ids(seed, n, w.vocab, w.zipf_s, perm)


def copy_span_stream(w: Workload, seed: int, n: int, perm: np.ndarray) -> np.ndarray:
    """Span-by-span stream: U{8..64} lengths, repeated spans with ``copy_prob``."""
    out = np.empty(n, dtype=np.int32)
    fresh = _draw_ids(w, rng.sub_seed(seed, 1), n, perm)
    ctl = rng.uniform01(rng.sub_seed(seed, 2), np.arange(3 * (n // 8 + 1)))
    pos, c = 0, 0
    while pos < n:
        length = min(8 + int(ctl[c] * 57), n - pos)
        copy = ctl[c + 1] < w.copy_prob and pos >= length
        if copy:
            start = int(ctl[c + 2] * (pos - length + 1))
            out[pos:pos + length] = out[start:start + length]
        else:
            out[pos:pos + length] = fresh[pos:pos + length]
        pos += length
        c += 3
    return out


def make_ids(w: Workload, batch_id: int = 0):
    """Raw ids int32[B, T] and history int32[B, history_len] (or None)."""
    perm = raw_id_permutation(w) if w.zipf_s is not None else None
    seed = rng.sub_seed(w.seed, S_IDS, batch_id)
    B, T = w.batch, w.seq_len
    if w.copy_prob > 0:
        ids = np.stack([copy_span_stream(w, rng.sub_seed(seed, b), T, perm) for b in range(B)])
    else:
        ids = _draw_ids(w, seed, B * T, perm).reshape(B, T)
    hist = None
    if w.history_len:
        hseed = rng.sub_seed(w.seed, S_HIST, batch_id)
        hist = _draw_ids(w, hseed, B * w.history_len, perm).reshape(B, w.history_len)
    return np.ascontiguousarray(ids), hist


# ---------------------------------------------------------------------------
# dense parameters and on-demand slices of the large tensors
# ---------------------------------------------------------------------------

def table_row_values(w: Workload, j: int, rows: np.ndarray) -> np.ndarray:
    """Rows ``rows`` of table ``j``: [len(rows), row_dim] (f32 or bf16 bits)."""
    rows = np.asarray(rows, dtype=np.int64)
    idx = rows[:, None] * w.row_dim + np.arange(w.row_dim, dtype=np.int64)[None, :]
    return rng.normal_values(w.table_seed(j), idx, w.table_sigma, w.tdtype, 1.0 / w.table_scale)


def table_values(w: Workload, j: int) -> np.ndarray:
    """Whole table ``j`` (only sensible for the small workloads)."""
    n = w.rows()[j] * w.row_dim
    return rng.normal_values(w.table_seed(j), np.arange(n), w.table_sigma, w.tdtype,
                             1.0 / w.table_scale).reshape(
        -1, w.row_dim)


def hidden_rows_per_token(w: Workload) -> int:
    return w.n_branches if w.n_branches > 1 else 1


def hidden_values(w: Workload, tokens: np.ndarray, batch_id: int = 0) -> np.ndarray:
    """Hidden rows of flat token indices ``tokens``: [len, nb_h, d]."""
    tokens = np.asarray(tokens, dtype=np.int64)
    per = hidden_rows_per_token(w) * w.hidden
    idx = tokens[:, None] * per + np.arange(per, dtype=np.int64)[None, :]
    v = rng.normal_values(w.hidden_seed(batch_id), idx, w.hidden_sigma, w.dtype)
    return v.reshape(len(tokens), hidden_rows_per_token(w), w.hidden)


def weight_values(w: Workload, which: str, branch: int = 0) -> np.ndarray:
    """W_K[branch] or W_V as [mem, d] (row-major, k = e @ W)."""
    seed = w.wk_seed(branch) if which == "k" else w.wv_seed()
    n = w.mem_dim * w.hidden
    return rng.normal_values(seed, np.arange(n), w.w_sigma, w.dtype).reshape(w.mem_dim, w.hidden)


def conv_weight_values(w: Workload) -> np.ndarray:
    """Depthwise conv taps [kernel, d]; tap i multiplies position t - i*dilation."""
    n = w.conv_kernel * w.hidden
    return rng.normal_values(rng.sub_seed(w.param_seed, S_CONV), np.arange(n), w.conv_sigma,
                             w.dtype).reshape(w.conv_kernel, w.hidden)


def gamma_values(w: Workload, which: str, random: bool = False) -> np.ndarray:
    """RMSNorm gain [d]: ones by default, else 1 + N(0, 0.1) (stored in w.dtype)."""
    if not random:
        one = np.ones(w.hidden, dtype=np.float32)
        return one if w.dtype == "f32" else rng.f32_to_bf16_bits(one)
    sid = {"q": S_GQ, "k": S_GK, "u": S_GU}[which]
    x = rng.normal_f32(rng.sub_seed(w.param_seed, sid), np.arange(w.hidden), 0.1) + np.float32(1.0)
    return x if w.dtype == "f32" else rng.f32_to_bf16_bits(x)


def to_f64(values: np.ndarray, dtype: str) -> np.ndarray:
    """Storage (f32 array or bf16 bits) -> exact float64."""
    if dtype == "f32":
        return np.asarray(values, dtype=np.float32).astype(np.float64)
    return rng.bf16_bits_to_f32(values).astype(np.float64)


def layer_config(w: Workload, w_layout: str = "mem_d") -> dict:
    """Keyword arguments describing the layer for a workload (plain data);
    ``w_layout`` says how the projection matrices are stored."""
    return dict(orders=tuple(w.orders), heads=w.heads, rows=w.rows(),
                hash_mult=hash_multipliers(w), row_dim=w.row_dim, hidden_dim=w.hidden,
                n_branches=w.n_branches, vocab=w.vocab, vocab_compressed=w.vocab_compressed,
                dtype=0 if w.dtype == "f32" else 1, pad_id=0, rms_eps=w.rms_eps,
                w_layout={"mem_d": 0, "d_mem": 1}[w_layout],
                table_dtype={"f32": 0, "bf16": 1, "fp8": 2}[w.tdtype],
                table_scales=w.table_scales())
