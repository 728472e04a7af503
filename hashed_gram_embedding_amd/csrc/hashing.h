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

// Compressed ids c[i] of positions t - i (i < max_order) for token (b, t):
// inside the sequence from ids, before it from the history (oldest first),
// else pad.  RAW: ids/history are raw ids, compressed through the LUT.
template <bool RAW>
__device__ __forceinline__ void context_ids(const int32_t* __restrict__ ids, int64_t tok, int32_t b,
                                            int32_t t, const int32_t* __restrict__ hist,
                                            const int32_t* __restrict__ lut, const HashArgs& a,
                                            int32_t* __restrict__ err,
                                            uint64_t (&c)[NGRAM_MAX_ORDER]) {
#pragma unroll
  for (int i = 0; i < NGRAM_MAX_ORDER; ++i) {
    int32_t id = a.pad_id;
    bool have = false;
    if (i < a.max_order) {
      const int32_t p = t - i;
      if (p >= 0) {
        id = ids[tok - i];
        have = true;
      } else if (hist != nullptr && a.hist_len + p >= 0) {
        id = hist[(int64_t)b * a.hist_len + a.hist_len + p];
        have = true;
      }
    }
    if (RAW && have) id = compress_one(id, lut, a.vocab, a.vocab_c, a.pad_id, err);
    c[i] = (uint64_t)(uint32_t)id;
  }
}

// Row of table j for the context c.
__device__ __forceinline__ uint32_t table_row(const HashArgs& a, int j, int order,
                                              const uint64_t (&c)[NGRAM_MAX_ORDER]) {
  uint64_t key = 0;
#pragma unroll
  for (int i = 0; i < NGRAM_MAX_ORDER; ++i)
    if (i < order) key ^= c[i] * a.mult[j][i];
  return mod_prime(key, a.rows[j], a.magic[j]);
}

}  // namespace ngram
