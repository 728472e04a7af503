// Internal declarations shared by the kernel sources of libngram.so.
// Not installed; the public interface is include/ngram.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ngram.h"

namespace ngram {

// ---------------------------------------------------------------------------
// storage types
// ---------------------------------------------------------------------------
typedef uint16_t bf16_bits;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  uint32_t b = __float_as_uint(x);
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return (b >> 16) | 0x40u;
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static float4 load4(const float* p, int64_t i) {
    return *reinterpret_cast<const float4*>(p + i);
  }
  __device__ __forceinline__ static void store4(float* p, int64_t i, float4 v) {
    *reinterpret_cast<float4*>(p + i) = v;
  }
  __device__ __forceinline__ static void store4_stream(float* p, int64_t i, float4 v) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    f4v x;
    x[0] = v.x;
    x[1] = v.y;
    x[2] = v.z;
    x[3] = v.w;
    __builtin_nontemporal_store(x, reinterpret_cast<f4v*>(p + i));
  }
};
template <>
struct Elem<bf16_bits> {
  __device__ __forceinline__ static float load(const bf16_bits* p, int64_t i) {
    return bf16_to_f32(p[i]);
  }
  __device__ __forceinline__ static float4 load4(const bf16_bits* p, int64_t i) {
    uint2 r = *reinterpret_cast<const uint2*>(p + i);
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xFFFF0000u));
  }
  __device__ __forceinline__ static void store4(bf16_bits* p, int64_t i, float4 v) {
    uint2 r;
    r.x = f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16);
    r.y = f32_to_bf16(v.z) | (f32_to_bf16(v.w) << 16);
    *reinterpret_cast<uint2*>(p + i) = r;
  }
  __device__ __forceinline__ static void store4_stream(bf16_bits* p, int64_t i, float4 v) {
    typedef uint32_t u2v __attribute__((ext_vector_type(2)));
    u2v r;
    r[0] = f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16);
    r[1] = f32_to_bf16(v.z) | (f32_to_bf16(v.w) << 16);
    __builtin_nontemporal_store(r, reinterpret_cast<u2v*>(p + i));
  }
};

// ---------------------------------------------------------------------------
// kernel argument blocks (passed by value)
// ---------------------------------------------------------------------------
struct HashArgs {
  int32_t n_orders, heads, n_tables, max_order;
  int32_t pad_id, vocab, vocab_c, hist_len;
  int32_t orders[NGRAM_MAX_ORDER];
  uint64_t rows[NGRAM_MAX_TABLES];
  uint64_t magic[NGRAM_MAX_TABLES];  // floor(2^64 / rows[j]) for mod_prime
  uint64_t mult[NGRAM_MAX_TABLES][NGRAM_MAX_ORDER];
};

struct TablePtrs {
  const void* p[NGRAM_MAX_TABLES];
  float scale[NGRAM_MAX_TABLES];  // fp8 tables: value = scale * decode(byte)
};

// OCP FP8 E4M3 -> fp32 (exact): sign, 4 exponent bits with bias 7, 3 mantissa
// bits; exponent field 0 holds the subnormals m * 2^-9, S.1111.111 is NaN.
__device__ __forceinline__ float fp8_e4m3_to_f32(uint32_t b) {
  const uint32_t sign = (b & 0x80u) << 24;
  const uint32_t ex = (b >> 3) & 0xFu, m = b & 7u;
  const float sub = __uint_as_float(sign | __float_as_uint((float)m * 0x1p-9f));
  const float nor = __uint_as_float(sign | ((ex + 120u) << 23) | (m << 20));
  const float v = ex == 0 ? sub : nor;
  return (ex == 15u && m == 7u) ? __uint_as_float(sign | 0x7FC00000u) : v;
}

// 16 fp8 table values (one 16-byte chunk) -> 16 bf16 of E: each value times
// the table's scale in fp32, then rounded to bf16 (both to nearest even).
__device__ __forceinline__ void fp8x16_to_bf16(const uint4& q, float scale, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float a = fp8_e4m3_to_f32((w[i] >> (16 * h)) & 0xFFu) * scale;
      const float b = fp8_e4m3_to_f32((w[i] >> (16 * h + 8)) & 0xFFu) * scale;
      o[2 * i + h] = f32_to_bf16(a) | (f32_to_bf16(b) << 16);
    }
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// Projection + gate-partials problem (one launch covers all segments: the
// n_branches key projections, then the value projection).
struct ProjArgs {
  const void* e;          // [M, K] table dtype
  const void* wk;         // [nb, K, d]
  const void* wv;         // [K, d]
  const void* hidden;     // act dtype
  int64_t h_tok_stride;   // elements
  int64_t h_branch_stride;
  const void* gamma_q;    // [d] nullable
  const void* gamma_k;    // [d] nullable
  float* v;               // [M, d] fp32 (bf16 path) / [M, nb+1, d] (fp32 path)
  float* parts;           // [M, 3*nb+1, np] fp32
  int64_t M;
  int32_t K, d, nb, np;
  int32_t w_dk;           // fp32 path: W stored [d, K] instead of [K, d]
  int64_t v_ld;           // bf16 path: fp32 elements between V rows (d, or (nb+1) d when kept)
  float* k_keep;          // bf16 path, nullable: K of branch s written at k_keep + s d, rows v_ld apart
};

// Epilogue of the projections: gate row partials for key segments, fp32 V
// and sum(v^2) for the value segment.
struct EpiArgs {
  const bf16_bits* hidden;
  int64_t h_tok_stride, h_branch_stride;
  const bf16_bits* gamma_q;  // nullable
  const bf16_bits* gamma_k;  // nullable
  float* v;                  // [M, v_ld]: row m's values at v + m v_ld
  float* parts;              // [M, 3*nb+1, np]
  int64_t M;
  int32_t d, nb, np;
  int64_t v_ld;
  float* k_keep;             // nullable: key segment s also stored at k_keep + m v_ld + s d
};

// Projection with operands copied global -> LDS (W stored [d, mem]); the A
// operand is E [M, K].
struct AsyncProjArgs {
  const bf16_bits* e;
  const bf16_bits* wk;       // [nb, d, K]
  const bf16_bits* wv;       // [d, K]
  EpiArgs epi;
  int32_t K, tiles_m, tiles_n, group_m;
  // launch_projection_raw: C[M, (nb+1)*d] = A B^T written in fp32 to
  // raw_out[row * raw_ld + seg * d + col] instead of the gate epilogue.
  // raw_split > 1 splits the K steps over that many workgroups per tile
  // (split-major block order, ragged), split s writing its partial product
  // at raw_out + s * raw_split_stride.
  float* raw_out;
  int64_t raw_ld;
  int32_t raw_split;
  int64_t raw_split_stride;
  // launch_projection_raw_tn: A = e [K][M] and B = wv [K][N] with these row
  // strides (elements); M = epi.M, N = epi.d
  int64_t tn_lda, tn_ldb;
};

// Gate + gated value + conv block over a [B, T] token grid.
struct ConvArgs {
  // value source: fused path reads fp32 V and gate partials; the op path
  // reads U rows of the act dtype.
  const float* v;         // fused: [M, v_stride]
  int64_t v_stride;
  const float* parts;     // fused: [M, 3*nb+1, np]
  int32_t np;
  const void* u;          // op: [M, nb, d] act dtype
  const void* conv_w;     // [4, d] act dtype
  const void* gamma_u;    // [d] nullable
  // conv-state ring [B, 3*dil, nb, d] (nullable): the normalised row of
  // absolute position p in slot p mod 3*dil; state_pos[b] (nullable = 3*dil)
  // positions of sequence b precede this call's first token; update_state:
  // the call writes its last rows into the ring and advances state_pos by T
  float* state;
  int32_t* state_pos;
  int32_t update_state;
  const void* hidden;     // residual source (flag)
  int64_t h_tok_stride, h_branch_stride;
  void* out;              // [M, nb, d] act dtype
  float* gates;           // [M, nb] nullable
  int32_t B, T, nb, d, tile;
  float eps;
  int32_t add_residual;
  int32_t dil;                // conv dilation (decode finalize)
  const void* gamma_q;        // decode finalize: the gate's gains
  const void* gamma_k;
};

// Ring slot of the row at position q (< 0, relative to the call's first
// token) of a sequence whose ring position is pos (state_pos, >= 0), or -1
// when that position lies before the start of the sequence.
__device__ __forceinline__ int ring_slot(int pos, int q, int ring) {
  const int p = pos + q;
  return p < 0 ? -1 : p % ring;
}
__device__ __forceinline__ int ring_pos(const int32_t* state_pos, int64_t b, int ring) {
  if (state_pos == nullptr) return ring;
  const int p = state_pos[b];
  return p < 0 ? 0 : p;
}

// ---------------------------------------------------------------------------
// kernel launch
// ---------------------------------------------------------------------------
// Every kernel goes through launch(): a plain launch unless the calling
// thread is inside an instrumented entry point (ngram_forward_timed /
// ngram_backward_timed) with a stage open, in which case the stage's first
// kernel stamps its begin time into the stage's start event and each of its
// kernels stamps its end time into the stop event, so the event pair spans
// exactly the stage's kernels.  The open stage is thread-local and set only
// for the duration of such a call.
struct StageClock {
  hipEvent_t start, stop;
  int launches;
};
extern thread_local StageClock* t_open_stage;

template <typename T>
struct same_type {
  using type = T;
};

template <typename... P>
inline hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, uint32_t shmem,
                         hipStream_t s, typename same_type<P>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (StageClock* c = t_open_stage) {
    e0 = c->launches == 0 ? c->start : nullptr;
    e1 = c->stop;
    ++c->launches;
  }
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, shmem, s,
                            e0, e1, 0);
}

// ---------------------------------------------------------------------------
// backward pass (backward.hip)
// ---------------------------------------------------------------------------
struct GradTablePtrs {
  float* p[NGRAM_MAX_TABLES];  // fp32 [rows_j, row_dim] gradient accumulators
};

struct BwdArgs {
  int64_t n;                        // tokens
  int32_t T, nb, d, dil;
  float eps;
  const bf16_bits* hidden;          // query rows: token t, branch b at t*h_tok + b*h_br
  int64_t h_tok, h_br;
  const float* kv;                  // recomputed [n, kv_ld]: K of each branch, then V (fp32)
  int64_t kv_ld;
  float* stats;                     // [n, nb, kStatsStride]: g, 1/rho_h, 1/rho_k, 1/r, P
  float* dc;                        // [n, nb, d]: dC
  const bf16_bits* d_out;           // [n, nb, d]
  const bf16_bits* conv_w;          // [4, d]
  const bf16_bits* gamma_q;         // nullable (= 1)
  const bf16_bits* gamma_k;
  const bf16_bits* gamma_u;
  const float* state;               // conv-state ring [B, 3*dil, nb, d], or nullptr
  const int32_t* state_pos;         // ring positions [B] (nullptr = 3*dil)
  int32_t add_residual;
  bf16_bits* dkv;                   // [n, dkv_ld]: dK of each branch, then dV (bf16)
  int64_t dkv_ld;
  float* d_hidden;                  // hidden's layout, fp32, nullable
  float* part_conv;                 // [kBwdBlocks, 4, d]: per-block partial d_conv_w
  float* part_gain;                 // [kBwdBlocks, 3, d]: per-block partial d_gammas, nullable
};

constexpr int kStatsStride = 8;     // floats per (token, branch) stats row
constexpr int kBwdBlocks = 1024;    // grid cap of the per-row backward kernels

// stats, dC, then dK / dV / d_hidden; d_conv_w [4, d] and d_gammas [3, d]
// (nullable) written from the per-block partials by a two-pass column sum
// through reduce_tmp [32, 4 d] (d <= 4096)
hipError_t launch_bwd_rows(const BwdArgs& a, float* d_conv_w, float* d_gammas,
                           float* reduce_tmp, hipStream_t s);
// The gather's adjoint: dE slices added into the fp32 gradient rows of the
// tables the tokens named, every row's contributions in ascending token order
// (bit-identical run to run), through table_grad_bytes() of scratch;
// table_rows: the host's row count of each table.
size_t table_grad_bytes(int64_t n_tok, int32_t n_tables, int32_t row_dim);
hipError_t launch_table_grad(const int32_t* row_idx, int64_t n_tok, int32_t n_tables,
                             int32_t row_dim, const int64_t* table_rows, const float* d_e,
                             const GradTablePtrs& g, void* scratch, hipStream_t s);
// out[i] = sum_{s < split} part[s * stride + i], i < n (fp32, in split order)
hipError_t launch_sum_splits(const float* part, int32_t split, int64_t stride, int64_t n,
                             float* out, hipStream_t s);
hipError_t launch_transpose_bf16(const bf16_bits* src, int64_t rows, int64_t cols, int64_t ld_src,
                                 bf16_bits* dst, int64_t rows_pad, int64_t ld_dst, hipStream_t s);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);

// ---------------------------------------------------------------------------
// launchers (return hipError_t of the launch)
// ---------------------------------------------------------------------------
hipError_t launch_compress(const int32_t* raw, int64_t n, const int32_t* lut, int32_t vocab,
                           int32_t vocab_c, int32_t pad_id, int32_t* comp, int32_t* err,
                           hipStream_t s);
hipError_t launch_hash(bool raw_input, const int32_t* ids, int32_t B, int32_t T,
                       const int32_t* hist, const int32_t* lut, const HashArgs& a,
                       int32_t* row_idx, int32_t* err, hipStream_t s);
hipError_t launch_gather(int dtype, const int32_t* row_idx, int64_t n_tok, int32_t n_tables,
                         int32_t row_dim, const TablePtrs& t, void* mem, hipStream_t s);

// Projection tile shape picked for M tokens (bf16 path); np = partials per row.
struct ProjPlan {
  int bm, bn, np;
};
ProjPlan plan_projection(int dtype, int64_t M, int32_t d);
hipError_t launch_projection(int dtype, const ProjPlan& plan, const ProjArgs& a, hipStream_t s);

// Tile plan for M rows (override: a plan id >= 0); wave_cols = partial width.
constexpr int kAsyncPlans = 13;
int async_plan(int64_t M, int override_plan);
int async_wave_cols(int plan);
hipError_t launch_projection_async(int plan, const AsyncProjArgs& a, hipStream_t s);
hipError_t launch_projection_raw(int plan, const AsyncProjArgs& a, hipStream_t s);
hipError_t launch_projection_raw_tn(const AsyncProjArgs& a, hipStream_t s);
// split-K raw-tile variant for small M (decode); E given densely
// Decode E tiles: the decode step's E [M, K] bf16 is stored as 1 KB tiles of
// 16 tokens x 32 K values, tile (mb, kk) at element ((mb * K/32) + kk) * 512,
// and inside a tile the 8 values k = 32*kk + 8*q .. +8 of token 16*mb + r at
// element (16*q + r) * 8: lane 16*q + r's A operand of
// v_mfma_f32_16x16x32_bf16.  The buffer holds whole 16-token blocks.
//
// Weight-stationary decode projection (project_decode.hip): workgroup
// (n-tile of 16*ni columns, K slice) holds its weight block in LDS and writes
// the fp32 partial of its slice to split_out[slice][M][(nb+1)*d].  The grid is
// sized for kWstatCus compute units (MI355X).
constexpr int kWstatLdsBytes = 128 * 1024;
constexpr int kWstatCus = 256;
struct WstatPlan {
  int ni;     // 16-column MFMA blocks per workgroup (0: no plan fits)
  int split;  // K slices
  int ring;   // K steps of E loads in flight per wave
};
struct WstatArgs {
  const bf16_bits* e;   // [M, K]
  const bf16_bits* wk;  // [nb*d, K]
  const bf16_bits* wv;  // [d, K]
  int64_t M;
  int32_t K, nb, d;
  int32_t kt, tiles_n;  // set by the launcher
  float* split_out;
};
WstatPlan wstat_plan(int64_t M, int32_t N, int32_t K);
// whether the kernel can run a plan (LDS block, K slices, ring steps)
bool wstat_plan_fits(const WstatPlan& plan, int32_t K);
hipError_t launch_projection_wstat(const WstatPlan& plan, const WstatArgs& a, hipStream_t s);
// row_idx (nullable): the token's row ids, [n_tok, n_tables]
hipError_t launch_hash_gather(int dtype, const int32_t* ids, int32_t B, int32_t T,
                              const int32_t* hist, const int32_t* lut, const HashArgs& h,
                              int32_t n_tables, int32_t row_dim, const TablePtrs& t, void* mem,
                              int32_t* row_idx, int32_t* err, hipStream_t s);
hipError_t launch_decode_finalize(int dtype, int32_t k_split, const float* split, const ConvArgs& a,
                                  hipStream_t s);

hipError_t launch_gate_values(int dtype, const ConvArgs& a, int64_t M, hipStream_t s);
hipError_t launch_fused_conv(int dtype, int32_t dil, const ConvArgs& a, hipStream_t s);
hipError_t launch_op_conv(int dtype, int32_t dil, const ConvArgs& a, hipStream_t s);
// The ring update after a conv over a [B, T] grid (update_state): the last
// min(T, 3*dil) normalised rows of each sequence and branch into their slots,
// recomputed from V and the partials (fused) or from U (op); launched after
// the conv, whose reads of the ring it must follow.
hipError_t launch_state_update(int dtype, bool fused, int32_t dil, const ConvArgs& a,
                               hipStream_t s);
int conv_tile_for(int32_t T);

}  // namespace ngram
