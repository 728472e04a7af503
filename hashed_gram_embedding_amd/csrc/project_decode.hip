// Key / value projections for the decode step (one new token per sequence).
//
// Same product as the other projection kernels ("Qwen3.8-Flash-Next 深度研究"
// §2.3: E_t -> K_t, V_t; the multi-branch remark of "Qwen 4用上DeepSeek的
// Engram" gives one W_K per branch and a shared W_V): C = E [W_K^(0) .. W_V]^T,
// bf16 in, fp32 accumulate, W stored [d, mem].
//
// At decode M (the batch) is a few hundred rows, so the weights -- 2*mem*d*2
// bytes per matrix, 26 MB at Qwen scale -- are the only large operand and the
// one stream that has to be fast.  The kernel is weight-stationary: workgroup
// (n-tile, k-slice) copies its W block [NT columns x KT] into LDS once
// (global_load_lds, rows XOR-swizzled by 16-byte chunk so the MFMA operand
// reads are bank-conflict free), then streams E[:, k-slice] for every token
// straight from global memory (E is a few MB and stays in L2) into the A
// operands of v_mfma_f32_16x16x32_bf16, RING K steps ahead, and writes its
// fp32 partial C[M, NT].  The finalize kernel sums the k-slices.  Every weight
// byte crosses HBM once per call, and the host sizes the grid to about one
// workgroup per CU (one block fills most of a CU's LDS).
//
// Wave w of the sixteen handles token rows [16*MI*w, 16*MI*(w+1)) of each
// pass of 256*MI rows; lane l reads row l%16 of a 16-row block and the 8 k
// values (l/16)*8.. of a 32-wide K step -- E arrives in that order (decode E
// tiles, internal.h), one contiguous kilobyte per operand -- and holds C rows
// 4*(l/16)+r, column l%16.  Sixteen waves of one 16-row block each (four per
// SIMD) hide the E loads' L2 latency far better than four waves of four
// blocks: at Qwen decode the kernel went from 14.3 to 10.7 us, although
// every wave now reads the whole W block from LDS.
#include "internal.h"

namespace ngram {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWstatWaves = 16;  // one 16-row block per wave (MI = 1)

__device__ __forceinline__ void copy16_to_lds(const void* src, bf16_bits* wave_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)wave_dst, 16, 0, 0);
}

template <int NI, int MI, int RING>
__global__ __launch_bounds__(64 * kWstatWaves, 1) void proj_wstat_kernel(WstatArgs a) {
  static_assert(RING % 2 == 0, "the B operands alternate between two register sets");
  constexpr int NT = 16 * NI;
  __shared__ __attribute__((aligned(16))) bf16_bits s_w[kWstatLdsBytes / 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroup b runs on XCD b % 8: give each XCD a contiguous range of
  // (k-slice, n-tile) blocks, so that its workgroups share one or two E
  // slices instead of all of them.  An XCD's L2 then holds its weight blocks
  // (3.3 MB at Qwen scale, kept from the previous step) beside a 0.3 MB E
  // slice, where all four slices (1.3 MB) pushed part of the weights out.
  int bid = (int)blockIdx.x;
  if ((gridDim.x & 7) == 0) bid = (bid & 7) * (int)(gridDim.x >> 3) + (bid >> 3);
  const int n_tile = bid % a.tiles_n, ks = bid / a.tiles_n;
  const int nkd = a.nb * a.d;        // key columns
  const int N = nkd + a.d;           // key columns of every branch, then value columns
  const int n0 = n_tile * NT;
  const int K = a.K, KT = a.kt, k0 = ks * KT;
  const int rch = KT / 8;            // 16-byte chunks per LDS row (a multiple of 16)
  const int nk = KT / 32;            // K steps of the slice (a multiple of RING)
  const int64_t M = a.M;
  const int64_t last_blk = (M - 1) >> 4;
  const int64_t tiles_per_blk = K / 32;

  // A operands: E tile (16-row block, K step) is one contiguous kilobyte and
  // lane l's 16 bytes sit at l * 16; blocks past the last are clamped to it
  // (their rows are computed, never stored)
  const bf16_bits* ep[MI];
  bf16x8 ring[RING][MI];
  auto point = [&](int64_t rbase) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      int64_t blk = (rbase >> 4) + mi;
      if (blk > last_blk) blk = last_blk;
      ep[mi] = a.e + ((blk * tiles_per_blk + k0 / 32) * 64 + lane) * 8;
    }
  };
  auto load = [&](int kk, bf16x8 (&dst)[MI]) {  // a step past the last re-reads it
    const int k = (kk < nk ? kk : nk - 1) * 512;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) dst[mi] = *reinterpret_cast<const bf16x8*>(ep[mi] + k);
  };

  // the first pass's look-ahead goes out with the weight copies
  int64_t rbase = (int64_t)wave * 16 * MI;
  point(rbase);
#pragma unroll
  for (int u = 0; u < RING; ++u) load(u, ring[u]);

  // the W block: LDS position p = row * rch + pc holds chunk pc ^ (row & 15)
  // of weight row n0 + row (k from k0); rows past N repeat the last row
  const int total = NT * rch;        // a multiple of 64 * waves
  for (int base = wave * 64; base < total; base += 64 * kWstatWaves) {
    const int p = base + lane;
    const int row = p / rch, pc = p - row * rch;
    int n = n0 + row;
    if (n > N - 1) n = N - 1;
    const bf16_bits* wrow =
        n < nkd ? a.wk + (int64_t)n * K : a.wv + (int64_t)(n - nkd) * K;
    copy16_to_lds(wrow + k0 + ((pc ^ (row & 15)) << 3), s_w + (int64_t)base * 8);
  }
  __syncthreads();  // drains this wave's copies and loads, then waits for the others

  const int r16 = lane & 15, q = lane >> 4;
  // B operand of block ni at K step kk: row ni*16 + r16, logical chunk kk*4 + q
  const char* sw = reinterpret_cast<const char*>(s_w) + r16 * rch * 16;
  auto bload = [&](int kk, bf16x8 (&dst)[NI]) {
    const int c = (((kk < nk ? kk : nk - 1) * 4 + q) ^ r16);  // physical chunk
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      dst[ni] = *reinterpret_cast<const bf16x8*>(sw + ni * 16 * rch * 16 + c * 16);
  };
  float* __restrict__ P = a.split_out + (int64_t)ks * M * N;

  constexpr int kPassRows = 16 * MI * kWstatWaves;
  for (; rbase < M; rbase += kPassRows) {
    floatx4 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    auto mma = [&](const bf16x8 (&af)[MI], const bf16x8 (&bf)[NI]) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
    };
    bf16x8 b0[NI], b1[NI];
    bload(0, b0);
    for (int kb = 0; kb < nk; kb += RING) {
#pragma unroll
      for (int u = 0; u < RING; ++u) {
        // the barriers pin the schedule: step kk's MFMAs wait only for their
        // own operands (E loads issued RING steps earlier, B reads one step
        // earlier), and each slot is refilled as soon as it is consumed
        const int kk = kb + u;
        if (u & 1) {
          bload(kk + 1, b0);
          __builtin_amdgcn_sched_barrier(0);
          mma(ring[u], b1);
        } else {
          bload(kk + 1, b1);
          __builtin_amdgcn_sched_barrier(0);
          mma(ring[u], b0);
        }
        __builtin_amdgcn_sched_barrier(0);
        load(kk + RING, ring[u]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = rbase + mi * 16 + q * 4 + r;
        if (row < M) {
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const int col = n0 + ni * 16 + r16;
            // streamed: the partials are read once, by the finalize, and
            // should not evict the weights, which the next step reads again
            if (col < N) __builtin_nontemporal_store(acc[mi][ni][r], &P[row * N + col]);
          }
        }
      }
    }
    // the next pass's look-ahead
    if (rbase + kPassRows < M) {
      point(rbase + kPassRows);
#pragma unroll
      for (int u = 0; u < RING; ++u) load(u, ring[u]);
    }
  }
}

template <int NI>
hipError_t launch_ni(int ring, unsigned blocks, const WstatArgs& a, hipStream_t s) {
  constexpr unsigned T = 64 * kWstatWaves;
  // four waves per SIMD leave 128 registers a lane: a four-step ring fits
  // every tile width without spills (a ten-step ring or an unrolled K loop
  // does not, and measured slower)
  if (ring == 4) return launch(proj_wstat_kernel<NI, 1, 4>, blocks, T, 0, s, a);
  return hipErrorInvalidValue;
}

}  // namespace

// Tile choice: NT = 16*ni columns by KT = K/split of the reduction per
// workgroup, over the candidates whose W block fits the LDS block and whose
// KT is a multiple of 128, minimising the bytes the busiest CU moves: its
// workgroups' E slices, W blocks and partial writes, plus its share of the
// partial sums the finalize kernel reads back.
WstatPlan wstat_plan(int64_t M, int32_t N, int32_t K) {
  WstatPlan best{0, 0, 0};
  double best_cost = 0.0;
  const int nis[] = {5, 4, 6, 3, 2};  // wider tiles spill at 128 registers a lane
  for (int ni : nis) {
    const int nt = 16 * ni;
    for (int split = 1; split <= 16; ++split) {
      if (K % split != 0 || (K / split) % 128 != 0) continue;
      const int kt = K / split;
      if ((int64_t)nt * kt * 2 > kWstatLdsBytes) continue;
      const int64_t groups = (int64_t)((N + nt - 1) / nt) * split;
      const int64_t rounds = (groups + kWstatCus - 1) / kWstatCus;
      const double per_wg = 2.0 * M * kt + 2.0 * nt * kt + 4.0 * M * nt;
      const double cost = rounds * per_wg + (double)split * M * N * 4.0 / kWstatCus;
      if (best.ni == 0 || cost < best_cost) {
        best = WstatPlan{ni, split, 0};
        best_cost = cost;
      }
    }
  }
  if (best.ni) best.ring = 4;  // nk = KT / 32 is a multiple of 4
  return best;
}

// The kernel's copy loop and K-step ring assume these.
bool wstat_plan_fits(const WstatPlan& plan, int32_t K) {
  if (plan.ni < 2 || plan.ni > 6 || plan.ring != 4) return false;
  if (plan.split < 1 || K % plan.split != 0) return false;
  const int kt = K / plan.split;
  return kt % 128 == 0 && (int64_t)16 * plan.ni * kt * 2 <= kWstatLdsBytes &&
         (kt / 32) % plan.ring == 0;
}

hipError_t launch_projection_wstat(const WstatPlan& plan, const WstatArgs& a0, hipStream_t s) {
  WstatArgs a = a0;
  const int N = (a.nb + 1) * a.d;
  const int nt = 16 * plan.ni;
  if (!wstat_plan_fits(plan, a.K)) return hipErrorInvalidValue;
  a.kt = a.K / plan.split;
  a.tiles_n = (N + nt - 1) / nt;
  const int64_t blocks = (int64_t)a.tiles_n * plan.split;
  if (a.M == 0) return hipSuccess;
  switch (plan.ni) {
    case 2: return launch_ni<2>(plan.ring, (unsigned)blocks, a, s);
    case 3: return launch_ni<3>(plan.ring, (unsigned)blocks, a, s);
    case 4: return launch_ni<4>(plan.ring, (unsigned)blocks, a, s);
    case 5: return launch_ni<5>(plan.ring, (unsigned)blocks, a, s);
    case 6: return launch_ni<6>(plan.ring, (unsigned)blocks, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ngram
