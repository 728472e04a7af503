// Per-token compression and multi-head hashing, shared by the standalone
// hash kernel and the fused projection kernel's prologue.  Compression is
// Engram's first component and multi-head hashing its second ("Qwen 4用上
// DeepSeek的Engram", section "DeepSeek Engram 更复杂，Qwen 更精简"); the n-gram
// windows follow "Qwen3.8-Flash-Next 深度研究" §2.3 (2-gram heads read
// x_{t-1}, x_t; 3-gram heads x_{t-2}, x_{t-1}, x_t).  The hash itself is the
// multiply-xor-mod-prime reading documented in ngram.h.
#pragma once

#include "epilogue.h"

namespace ngram {

__device__ __forceinline__ int32_t compress_one(int32_t x, const int32_t* __restrict__ lut,
                                                int32_t vocab, int32_t vocab_c, int32_t pad,
                                                int32_t* __restrict__ err) {
  if (x >= 0 && x < vocab) {
    const int32_t c = lut[x];
    if (c >= 0 && c < vocab_c) return c;
  }
  if (err) *err = 1;
  return pad;
}

// The raw ids of a token's context, positions t - i (i < max_order): inside
// the sequence from ids, before it from the history (oldest first).  Every id
// is loaded unconditionally -- a position without one reads the token's own id
// as a stand-in and is marked absent -- so the loads go out at once instead of
// one round trip per position behind a branch.
struct CtxIds {
  int32_t x[NGRAM_MAX_ORDER];
  bool have[NGRAM_MAX_ORDER];
};

__device__ __forceinline__ CtxIds load_context(const int32_t* __restrict__ ids, int64_t tok,
                                               int32_t b, int32_t t,
                                               const int32_t* __restrict__ hist,
                                               const HashArgs& a) {
  CtxIds r;
#pragma unroll
  for (int i = 0; i < NGRAM_MAX_ORDER; ++i) {
    const int32_t p = t - i;
    const bool in_seq = p >= 0;
    const bool in_hist = !in_seq && hist != nullptr && a.hist_len + p >= 0;
    r.have[i] = i < a.max_order && (in_seq || in_hist);
    const int32_t* src = in_seq    ? ids + (tok - i)
                         : in_hist ? hist + ((int64_t)b * a.hist_len + a.hist_len + p)
                                   : ids + tok;
    r.x[i] = *src;
  }
  return r;
}

// Compressed ids c[i] of the context (pad where absent).  RAW: the ids are
// raw and go through the LUT (every entry loaded at once).  Returns true when
// an id it used was out of the vocabulary or mapped out of the compressed
// range (the caller raises the error flag; the store is left to it so that no
// branch sits between these loads and the caller's next ones).
template <bool RAW>
__device__ __forceinline__ bool compress_context(const CtxIds& r, const int32_t* __restrict__ lut,
                                                 const HashArgs& a, uint64_t (&c)[NGRAM_MAX_ORDER]) {
  if (RAW) {
    int32_t cx[NGRAM_MAX_ORDER];
    bool in_vocab[NGRAM_MAX_ORDER];
#pragma unroll
    for (int i = 0; i < NGRAM_MAX_ORDER; ++i) {
      in_vocab[i] = r.x[i] >= 0 && r.x[i] < a.vocab;
      cx[i] = lut[in_vocab[i] ? r.x[i] : 0];
    }
    bool bad = false;
#pragma unroll
    for (int i = 0; i < NGRAM_MAX_ORDER; ++i) {
      const bool ok = in_vocab[i] && cx[i] >= 0 && cx[i] < a.vocab_c;
      bad = bad || (r.have[i] && !ok);
      c[i] = (uint64_t)(uint32_t)(r.have[i] && ok ? cx[i] : a.pad_id);
    }
    return bad;
  } else {
#pragma unroll
    for (int i = 0; i < NGRAM_MAX_ORDER; ++i)
      c[i] = (uint64_t)(uint32_t)(r.have[i] ? r.x[i] : a.pad_id);
    return false;
  }
}

// Both steps for token (b, t).
template <bool RAW>
__device__ __forceinline__ bool context_ids(const int32_t* __restrict__ ids, int64_t tok, int32_t b,
                                            int32_t t, const int32_t* __restrict__ hist,
                                            const int32_t* __restrict__ lut, const HashArgs& a,
                                            uint64_t (&c)[NGRAM_MAX_ORDER]) {
  return compress_context<RAW>(load_context(ids, tok, b, t, hist, a), lut, a, c);
}

// Hash constants of one table: its multipliers, prime and Barrett constant.
struct RowHash {
  uint64_t m[NGRAM_MAX_ORDER];
  uint64_t p, magic;
  int order;
};

__device__ __forceinline__ RowHash row_hash_of(const HashArgs& a, int j, int order) {
  RowHash r;
#pragma unroll
  for (int i = 0; i < NGRAM_MAX_ORDER; ++i) r.m[i] = a.mult[j][i];
  r.p = a.rows[j];
  r.magic = a.magic[j];
  r.order = order;
  return r;
}

// Row of the table for the context c.
__device__ __forceinline__ uint32_t table_row(const RowHash& r, const uint64_t (&c)[NGRAM_MAX_ORDER]) {
  // every multiplier is used, none behind a branch: the empty asm makes the
  // values opaque, so the compiler cannot sink a multiplier's load into the
  // i < order case (which made each load wait for the one before); a kernel
  // that loads the constants before its token loop finds them there already
  uint64_t m[NGRAM_MAX_ORDER];
#pragma unroll
  for (int i = 0; i < NGRAM_MAX_ORDER; ++i) m[i] = r.m[i];
  static_assert(NGRAM_MAX_ORDER == 4, "one operand per order below");
  asm volatile("" : "+v"(m[0]), "+v"(m[1]), "+v"(m[2]), "+v"(m[3]));
  uint64_t key = 0;
#pragma unroll
  for (int i = 0; i < NGRAM_MAX_ORDER; ++i) key ^= i < r.order ? c[i] * m[i] : 0;
  return mod_prime(key, r.p, r.magic);
}

// Row of table j for the context c.
__device__ __forceinline__ uint32_t table_row(const HashArgs& a, int j, int order,
                                              const uint64_t (&c)[NGRAM_MAX_ORDER]) {
  return table_row(row_hash_of(a, j, order), c);
}

}  // namespace ngram
