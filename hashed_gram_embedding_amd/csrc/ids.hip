// Tokenizer compression and multi-head n-gram hashing.
//
// Compression is Engram's first component and hashing its second ("Qwen 4用上
// DeepSeek的Engram", section "DeepSeek Engram 更复杂，Qwen 更精简"); the n-gram
// windows are those of "Qwen3.8-Flash-Next 深度研究" §2.3 (2-gram heads on
// (x_{t-1}, x_t), 3-gram heads on (x_{t-2}, x_{t-1}, x_t)).  The hash is the
// multiply-xor-mod-prime reading documented in ngram.h.
//
// One thread per token: the token's ids (and up to max_order-1 predecessors)
// are a handful of 4-byte loads that stay in L2, the LUT (<= 1 MB) is
// L2-resident, and the n_tables 64-bit products and remainders are plain ALU
// work.  The kernel is tiny next to the gather and the projections.
#include "hashing.h"

namespace ngram {
namespace {

__global__ void compress_kernel(const int32_t* __restrict__ raw, int64_t n,
                                const int32_t* __restrict__ lut, int32_t vocab, int32_t vocab_c,
                                int32_t pad, int32_t* __restrict__ comp, int32_t* __restrict__ err) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    comp[i] = compress_one(raw[i], lut, vocab, vocab_c, pad, err);
}

// RAW: ids and history are raw token ids (compressed here with the LUT);
// otherwise they are already compressed.
template <bool RAW>
__global__ void hash_kernel(const int32_t* __restrict__ ids, int32_t B, int32_t T,
                            const int32_t* __restrict__ hist, const int32_t* __restrict__ lut,
                            HashArgs a, int32_t* __restrict__ row_idx, int32_t* __restrict__ err) {
  const int64_t n = (int64_t)B * T;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t tok = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; tok < n; tok += stride) {
    const int32_t b = (int32_t)(tok / T);
    const int32_t t = (int32_t)(tok - (int64_t)b * T);
    uint64_t c[NGRAM_MAX_ORDER];
    const bool bad = context_ids<RAW>(ids, tok, b, t, hist, lut, a, c);
    int32_t* out = row_idx + tok * a.n_tables;
    for (int o = 0; o < a.n_orders; ++o) {
      const int n_o = a.orders[o];
      for (int k = 0; k < a.heads; ++k) {
        const int j = o * a.heads + k;
        out[j] = (int32_t)table_row(a, j, n_o, c);
      }
    }
    if (bad && err) *err = 1;
  }
}

int grid_for(int64_t n, int threads) {
  int64_t b = (n + threads - 1) / threads;
  if (b < 1) b = 1;
  if (b > 65536) b = 65536;
  return (int)b;
}

}  // namespace

hipError_t launch_compress(const int32_t* raw, int64_t n, const int32_t* lut, int32_t vocab,
                           int32_t vocab_c, int32_t pad_id, int32_t* comp, int32_t* err,
                           hipStream_t s) {
  return launch(compress_kernel, grid_for(n, 256), 256, 0, s, raw, n, lut, vocab, vocab_c, pad_id,
                comp, err);
}

hipError_t launch_hash(bool raw_input, const int32_t* ids, int32_t B, int32_t T,
                       const int32_t* hist, const int32_t* lut, const HashArgs& a,
                       int32_t* row_idx, int32_t* err, hipStream_t s) {
  const int64_t n = (int64_t)B * T;
  if (raw_input)
    return launch(hash_kernel<true>, grid_for(n, 256), 256, 0, s, ids, B, T, hist, lut, a, row_idx,
                  err);
  return launch(hash_kernel<false>, grid_for(n, 256), 256, 0, s, ids, B, T, hist, lut, a, row_idx,
                err);
}

}  // namespace ngram
