// Gather + concatenation of the hashed rows into the memory vector E_t
// ("Qwen3.8-Flash-Next 深度研究" §2.3: the row ids' rows are concatenated into
// E_t; Engram's second component in "Qwen 4用上DeepSeek的Engram").  FP8 E4M3
// tables (the same page, §9.3: FP8 storage with a per-tensor scale) are
// widened to bf16 E on the way, each value times its table's scale.
//
// HBM-bound random reads.  One wavefront owns one token: its n_tables rows
// are split into 16-byte chunks, lane l takes chunks l, l+64, ..., so a
// 640-byte row (320 bf16) is read as five aligned 128-byte lines by 40
// consecutive lanes, and the concatenated E_t row is written with fully
// coalesced 16-byte stores.  All of a token's loads are issued before its
// stores (up to 8 chunks per lane in flight) to keep enough random row
// fetches outstanding; the table base pointers sit in LDS because the lanes
// of one wave touch different tables.
#include <type_traits>

#include "hashing.h"

namespace ngram {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Table rows as global-address-space chunks.  The table pointers are kept in
// LDS; a plain pointer read back from LDS would be a flat one, and flat loads
// also count against the LDS wait counter, so each chunk's pointer read would
// wait for the previous chunk's table load.
typedef const __attribute__((address_space(1))) u32x4 gchunk;

// Wait for every vector-memory load in flight (vmcnt 0; the LDS and export
// counters untouched).  Issued once between a batch of loads and the stores
// that use them, so the compiler does not wait before each store behind its
// per-lane guard (stores count against the same counter, so those waits
// would serialise the stores).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0xF70); }

// E is written once and read by the next kernel: streamed past the caches
__device__ __forceinline__ void nt_store16(uint4* p, const uint4& v) {
  u32x4 x;
  x[0] = v.x;
  x[1] = v.y;
  x[2] = v.z;
  x[3] = v.w;
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
}

constexpr int kGatherUnroll = 8;

// FP8 tables: a source chunk holds 16 values and becomes two bf16 chunks of E
// (fp8x16_to_bf16 applies the table's scale); otherwise chunks are copied.
// row_chunks counts the 16-byte chunks of one table row in the table.
template <bool FP8>
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ row_idx,
                                                     int64_t n_tok, int32_t n_tables,
                                                     int32_t row_chunks, TablePtrs tabs,
                                                     uint4* __restrict__ mem) {
  // FP8: global-space table pointers (see gchunk); bf16: plain ones
  __shared__ std::conditional_t<FP8, gchunk*, const u32x4*> s_tab[NGRAM_MAX_TABLES];
  __shared__ float s_scale[NGRAM_MAX_TABLES];
  if (threadIdx.x < NGRAM_MAX_TABLES) {
    const int j = threadIdx.x < n_tables ? threadIdx.x : 0;
    s_tab[threadIdx.x] = (std::conditional_t<FP8, gchunk*, const u32x4*>)tabs.p[j];
    s_scale[threadIdx.x] = tabs.scale[j];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int waves_per_block = blockDim.x >> 6;
  const int64_t wave0 = (int64_t)blockIdx.x * waves_per_block + (threadIdx.x >> 6);
  const int64_t wstride = (int64_t)gridDim.x * waves_per_block;
  const int32_t chunks = n_tables * row_chunks;  // table chunks per token

  for (int64_t tok = wave0; tok < n_tok; tok += wstride) {
    const int32_t* rix = row_idx + tok * n_tables;
    // FP8: the token's row ids, one per lane, loaded once; the chunk loads
    // take theirs by shuffle and go out together (a lane past the last chunk
    // re-reads the last one, unused), through global-space pointers, and the
    // stores follow one wait (FP8 gather 0.63 -> 0.50 ms at Qwen prefill).
    // bf16 keeps one row-id load per chunk and flat table pointers, which
    // measured 6 % faster there for its twice as many chunks per token.
    const int32_t my_r = FP8 ? rix[lane < n_tables ? lane : 0] : 0;
    uint4* dst = mem + tok * chunks * (FP8 ? 2 : 1);
    for (int base = 0; base < chunks; base += 64 * kGatherUnroll) {
      uint4 v[kGatherUnroll];
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        if (FP8) {
          if (base + u * 64 < chunks) {  // the same for every lane
            int q = base + u * 64 + lane;
            q = q < chunks ? q : chunks - 1;
            const int j = q / row_chunks;
            const int c = q - j * row_chunks;
            const int64_t r = __shfl(my_r, j);
            const u32x4 x = __builtin_nontemporal_load(s_tab[j] + r * row_chunks + c);
            v[u] = make_uint4(x[0], x[1], x[2], x[3]);
          }
        } else {
          const int q = base + u * 64 + lane;
          if (q < chunks) {
            const int j = q / row_chunks;
            const int c = q - j * row_chunks;
            const int64_t r = rix[j];
            const u32x4 x = __builtin_nontemporal_load(s_tab[j] + r * row_chunks + c);
            v[u] = make_uint4(x[0], x[1], x[2], x[3]);
          }
        }
      }
      if (FP8) wait_loads();
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        const int q = base + u * 64 + lane;
        if (q < chunks) {
          if (FP8) {
            uint4 lo, hi;
            fp8x16_to_bf16(v[u], s_scale[q / row_chunks], lo, hi);
            nt_store16(dst + 2 * q, lo);
            nt_store16(dst + 2 * q + 1, hi);
          } else {
            nt_store16(dst + q, v[u]);
          }
        }
      }
    }
  }
}

// Hash + gather in one pass for the decode step, one wavefront per token:
// every lane reads the token's context ids (the same few words, served by the
// cache), lane j hashes table j, and each 16-byte chunk's lane fetches its
// table's row id from lane j with a cross-lane read before the loads above.
// E is written in the decode projection's operand order (internal.h,
// "decode E tiles"), so that kernel reads each 16-row x 32-k operand of
// v_mfma_f32_16x16x32_bf16 as one contiguous kilobyte.  The row ids go to
// row_idx as well (32 bytes a token), when it is given.
//
// WPT waves share one token (a few hundred tokens cannot otherwise occupy
// every CU): each hashes all of the token's tables and fetches 1 / WPT of its
// chunks.
template <bool FP8, int WPT>
__global__ __launch_bounds__(256) void hash_gather_kernel(const int32_t* __restrict__ ids,
                                                          int32_t B, int32_t T,
                                                          const int32_t* __restrict__ hist,
                                                          const int32_t* __restrict__ lut, HashArgs h,
                                                          int32_t row_chunks, TablePtrs tabs,
                                                          uint4* __restrict__ mem,
                                                          int32_t* __restrict__ row_idx,
                                                          int32_t* __restrict__ err) {
  __shared__ gchunk* s_tab[NGRAM_MAX_TABLES];
  __shared__ float s_scale[NGRAM_MAX_TABLES];
  const int lane = threadIdx.x & 63;
  // this lane's table hash constants, loaded once and first, so that their
  // round trip overlaps the table pointers' below
  const int jl = lane < h.n_tables ? lane : 0;
  const RowHash rh = row_hash_of(h, jl, h.orders[jl / h.heads]);
  constexpr int tok_per_block = 4 / WPT;
  const int64_t n_tok = (int64_t)B * T;
  const int64_t tstride = (int64_t)gridDim.x * tok_per_block;
  const int64_t tok0 = (int64_t)blockIdx.x * tok_per_block + (threadIdx.x >> 6) / WPT;
  // the first token's context ids also go out before the barrier (a token
  // past the end reads token 0's, unused)
  auto ctx_of = [&](int64_t tok) {
    const int64_t tk = tok < n_tok ? tok : 0;
    const int32_t b = (int32_t)(tk / T);
    return load_context(ids, tk, b, (int32_t)(tk - (int64_t)b * T), hist, h);
  };
  CtxIds ctx = ctx_of(tok0);
  if (threadIdx.x < NGRAM_MAX_TABLES) {
    const int j = threadIdx.x < h.n_tables ? threadIdx.x : 0;
    s_tab[threadIdx.x] = (gchunk*)tabs.p[j];
    s_scale[threadIdx.x] = tabs.scale[j];
  }
  __syncthreads();
  const int part = (threadIdx.x >> 6) % WPT;
  const int32_t chunks = h.n_tables * row_chunks;  // table chunks per token
  const int32_t per = (chunks + WPT - 1) / WPT;
  const int32_t q0 = part * per, q1 = q0 + per < chunks ? q0 + per : chunks;
  const int32_t n_kk = chunks * (FP8 ? 2 : 1) >> 2;  // 32-wide K steps per token
  for (int64_t tok = tok0; tok < n_tok; tok += tstride) {
    uint64_t c[NGRAM_MAX_ORDER];
    const bool bad = compress_context<true>(ctx, lut, h, c);
    ctx = ctx_of(tok + tstride);  // the next token's ids, in flight during this one
    const int32_t my_row = (int32_t)table_row(rh, c);
    if (row_idx && part == 0 && lane < h.n_tables) row_idx[tok * h.n_tables + lane] = my_row;
    uint4* dst = mem + (tok >> 4) * n_kk * 64 + (tok & 15);
    // E chunk e (16 bytes, 8 bf16): K step e/4, quarter e%4
    auto put = [&](int e, const uint4& x) { dst[(e >> 2) * 64 + (e & 3) * 16] = x; };
    for (int base = q0; base < q1; base += 64 * kGatherUnroll) {
      uint4 v[kGatherUnroll];
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        const int q = base + u * 64 + lane;
        const int j = q / row_chunks;
        const int64_t r = __shfl(my_row, j < h.n_tables ? j : 0);
        if (q < q1) {  // random rows, read once: streamed past the caches
          const u32x4 x = __builtin_nontemporal_load(s_tab[j] + r * row_chunks + (q - j * row_chunks));
          v[u] = make_uint4(x[0], x[1], x[2], x[3]);
        }
      }
      wait_loads();
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        const int q = base + u * 64 + lane;
        if (q < q1) {
          if (FP8) {
            uint4 lo, hi;
            fp8x16_to_bf16(v[u], s_scale[q / row_chunks], lo, hi);
            put(2 * q, lo);
            put(2 * q + 1, hi);
          } else {
            put(q, v[u]);
          }
        }
      }
    }
    if (bad && err) *err = 1;
  }
}

}  // namespace

hipError_t launch_hash_gather(int dtype, const int32_t* ids, int32_t B, int32_t T,
                              const int32_t* hist, const int32_t* lut, const HashArgs& h,
                              int32_t n_tables, int32_t row_dim, const TablePtrs& t, void* mem,
                              int32_t* row_idx, int32_t* err, hipStream_t s) {
  // the tiled E layout is defined for bf16 E of whole 32-wide K steps
  if ((dtype != NGRAM_BF16 && dtype != NGRAM_FP8_E4M3) || (n_tables * row_dim) % 32 != 0)
    return hipErrorInvalidValue;
  const bool fp8 = dtype == NGRAM_FP8_E4M3;
  const int32_t row_chunks = row_dim * (fp8 ? 1 : 2) / 16;
  const int64_t n_tok = (int64_t)B * T;
  // waves per token: enough to put work on every CU for the decode batch
  // (one wave per token left three quarters of the CUs idle at 256 tokens;
  // 5 or 8 waves per token measured no better than 4)
  const int wpt = n_tok <= 1024 ? 4 : n_tok <= 2048 ? 2 : 1;
  int64_t blocks = (n_tok * wpt + 3) / 4;
  if (blocks > 262144) blocks = 262144;
  if (blocks < 1) blocks = 1;
  uint4* m = static_cast<uint4*>(mem);
#define NGRAM_HG(F, W)                                                                     \
  return launch(hash_gather_kernel<F, W>, (unsigned)blocks, 256, 0, s, ids, B, T, hist, lut, h, \
                row_chunks, t, m, row_idx, err)
#define NGRAM_HG_W(F)       \
  switch (wpt) {            \
    case 4: NGRAM_HG(F, 4); \
    case 2: NGRAM_HG(F, 2); \
    default: NGRAM_HG(F, 1); \
  }
  if (fp8) NGRAM_HG_W(true);
  NGRAM_HG_W(false);
#undef NGRAM_HG_W
#undef NGRAM_HG
}

hipError_t launch_gather(int dtype, const int32_t* row_idx, int64_t n_tok, int32_t n_tables,
                         int32_t row_dim, const TablePtrs& t, void* mem, hipStream_t s) {
  const int esize = dtype == NGRAM_BF16 ? 2 : dtype == NGRAM_FP8_E4M3 ? 1 : 4;
  const int32_t row_chunks = row_dim * esize / 16;
  const int threads = 256;
  int64_t blocks = (n_tok + 3) / 4;
  if (blocks > 262144) blocks = 262144;
  if (blocks < 1) blocks = 1;
  if (dtype == NGRAM_FP8_E4M3)
    return launch(gather_kernel<true>, (unsigned)blocks, threads, 0, s, row_idx, n_tok, n_tables,
                  row_chunks, t, static_cast<uint4*>(mem));
  return launch(gather_kernel<false>, (unsigned)blocks, threads, 0, s, row_idx, n_tok, n_tables,
                row_chunks, t, static_cast<uint4*>(mem));
}

}  // namespace ngram
