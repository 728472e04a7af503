// Epilogue of the projection kernels: turns a wave's 32x32-MFMA accumulator
// tile into the gate's row partials (key segments) or fp32 V plus sum(v^2)
// (value segment).  See project.hip for the layer context.
#pragma once

#include <type_traits>

#include "internal.h"

namespace ngram {

// Sum 16 per-row values over the 32 lanes of a half-wave by recursive
// halving: each exchange sends half of the remaining values, so 16 shuffles
// replace 80.  Lane l ends up owning row index owner16(l) (lanes l and l^1
// hold the same value).
__device__ __forceinline__ float xsum16(float (&x)[16], int lane) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const bool up = lane & 16;
    const float keep = up ? x[8 + q] : x[q];
    const float send = up ? x[q] : x[8 + q];
    x[q] = keep + __shfl_xor(send, 16);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool up = lane & 8;
    const float keep = up ? x[4 + q] : x[q];
    const float send = up ? x[q] : x[4 + q];
    x[q] = keep + __shfl_xor(send, 8);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const bool up = lane & 4;
    const float keep = up ? x[2 + q] : x[q];
    const float send = up ? x[q] : x[2 + q];
    x[q] = keep + __shfl_xor(send, 4);
  }
  {
    const bool up = lane & 2;
    const float keep = up ? x[1] : x[0];
    const float send = up ? x[0] : x[1];
    x[0] = keep + __shfl_xor(send, 2);
  }
  return x[0] + __shfl_xor(x[0], 1);
}

__device__ __forceinline__ int owner16(int lane) {
  return ((lane >> 4) & 1) * 8 + ((lane >> 3) & 1) * 4 + ((lane >> 2) & 1) * 2 + ((lane >> 1) & 1);
}

// Row (within a 32x32 block) held by accumulator register r of this lane.
__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// seg < nb: key projection of branch seg; seg == nb: value projection.
// The wave owns rows [wrow0, wrow0 + 32*MI) and columns [wcol0, wcol0 + 32*NI),
// its partial index is pidx.  hread(row, col) returns the query element of
// branch seg (a copy staged in LDS, or the hidden state itself).
template <int MI, int NI, class HRead>
__device__ __forceinline__ void gate_epilogue(const floatx16 (&acc)[MI][NI], const EpiArgs& a,
                                              int seg, int64_t wrow0, int wcol0, int pidx,
                                              int lane, HRead&& hread) {
  const int d = a.d;
  const int64_t M = a.M;
  const int nq = 3 * a.nb + 1;
  if (seg < a.nb) {
    // K itself is kept only for a later backward pass (fp32, streamed)
    float* __restrict__ K = a.k_keep ? a.k_keep + (int64_t)seg * d : nullptr;
    float g[NI];
    bool cv[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int col = wcol0 + ni * 32 + (lane & 31);
      cv[ni] = col < d;
      const int cc = cv[ni] ? col : 0;
      g[ni] = (a.gamma_q ? bf16_to_f32(a.gamma_q[cc]) : 1.0f) *
              (a.gamma_k ? bf16_to_f32(a.gamma_k[cc]) : 1.0f);
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      float xd[16], xk[16], xh[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) xd[r] = xk[r] = xh[r] = 0.0f;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int col = wcol0 + ni * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = wrow0 + mi * 32 + acc_row(r, lane);
          if (cv[ni] && row < M) {
            const float h = hread(row, col);
            const float k = acc[mi][ni][r];
            if (K) __builtin_nontemporal_store(k, &K[row * a.v_ld + col]);
            xd[r] += g[ni] * h * k;
            xk[r] += k * k;
            xh[r] += h * h;
          }
        }
      }
      const float sd = xsum16(xd, lane);
      const float sk = xsum16(xk, lane);
      const float sh = xsum16(xh, lane);
      const int64_t row = wrow0 + mi * 32 + acc_row(owner16(lane), lane);
      if (!(lane & 1) && row < M) {
        float* p = a.parts + (row * nq + 3 * seg) * a.np + pidx;
        p[0] = sd;
        p[a.np] = sk;
        p[2 * a.np] = sh;
      }
    }
  } else {
    float* __restrict__ V = a.v;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      float xv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) xv[r] = 0.0f;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int col = wcol0 + ni * 32 + (lane & 31);
        if (col < d) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t row = wrow0 + mi * 32 + acc_row(r, lane);
            if (row < M) {
              const float v = acc[mi][ni][r];
              __builtin_nontemporal_store(v, &V[row * a.v_ld + col]);  // read once, by the conv
              xv[r] += v * v;
            }
          }
        }
      }
      const float sv = xsum16(xv, lane);
      const int64_t row = wrow0 + mi * 32 + acc_row(owner16(lane), lane);
      if (!(lane & 1) && row < M) a.parts[(row * nq + 3 * a.nb) * a.np + pidx] = sv;
    }
  }
}

template <int MI, int NI>
__device__ __forceinline__ void gate_epilogue(const floatx16 (&acc)[MI][NI], const EpiArgs& a,
                                              int seg, int64_t wrow0, int wcol0, int pidx,
                                              int lane) {
  const bf16_bits* __restrict__ H = a.hidden + seg * a.h_branch_stride;
  const int64_t ht = a.h_tok_stride;
  gate_epilogue<MI, NI>(acc, a, seg, wrow0, wcol0, pidx, lane,
                        [&](int64_t row, int col) { return bf16_to_f32(H[row * ht + col]); });
}

// 64-bit key mod a prime p < 2^31 with magic = floor(2^64 / p): the quotient
// estimate is exact or one short (Barrett), so one correction suffices.
__device__ __forceinline__ uint32_t mod_prime(uint64_t key, uint64_t p, uint64_t magic) {
  const uint64_t q = __umul64hi(key, magic);
  uint64_t r = key - q * p;
  if (r >= p) r -= p;
  return (uint32_t)r;
}

// The same for a wave tile of 16x16-MFMA blocks (v_mfma_f32_16x16x32_bf16):
// accumulator register j of lane l holds row 4 * (l / 16) + j, column l % 16
// of its block, so a row's columns are spread over the 16 lanes of one
// quarter-wave.  Each lane sums its columns of the tile's blocks first, then
// the quarter-wave sums its four rows by recursive halving (5 shuffles a
// quantity instead of 16); lane l ends up with row owner4(l) of its quarter
// (the four lanes l & ~3 .. l | 3 hold the same value).
__device__ __forceinline__ float xsum4_16(float (&x)[4], int lane) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const bool up = lane & 8;
    const float keep = up ? x[2 + q] : x[q];
    const float send = up ? x[q] : x[2 + q];
    x[q] = keep + __shfl_xor(send, 8);
  }
  {
    const bool up = lane & 4;
    const float keep = up ? x[1] : x[0];
    const float send = up ? x[0] : x[1];
    x[0] = keep + __shfl_xor(send, 4);
  }
  x[0] += __shfl_xor(x[0], 2);
  return x[0] + __shfl_xor(x[0], 1);
}

__device__ __forceinline__ int owner4(int lane) { return ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1); }

template <int MI, int NI, class HRead>
__device__ __forceinline__ void gate_epilogue16(const floatx4 (&acc)[MI][NI], const EpiArgs& a,
                                                int seg, int64_t wrow0, int wcol0, int pidx,
                                                int lane, HRead&& hread) {
  const int d = a.d;
  const int64_t M = a.M;
  const int nq = 3 * a.nb + 1;
  const int rq = 4 * (lane >> 4);  // first of the lane's four rows in a block
  if (seg < a.nb) {
    float* __restrict__ K = a.k_keep ? a.k_keep + (int64_t)seg * d : nullptr;
    float g[NI];
    bool cv[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int col = wcol0 + ni * 16 + (lane & 15);
      cv[ni] = col < d;
      const int cc = cv[ni] ? col : 0;
      g[ni] = (a.gamma_q ? bf16_to_f32(a.gamma_q[cc]) : 1.0f) *
              (a.gamma_k ? bf16_to_f32(a.gamma_k[cc]) : 1.0f);
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      float xd[4], xk[4], xh[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) xd[j] = xk[j] = xh[j] = 0.0f;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int col = wcol0 + ni * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t row = wrow0 + mi * 16 + rq + j;
          if (cv[ni] && row < M) {
            const float h = hread(row, col);
            const float k = acc[mi][ni][j];
            if (K) __builtin_nontemporal_store(k, &K[row * a.v_ld + col]);
            xd[j] += g[ni] * h * k;
            xk[j] += k * k;
            xh[j] += h * h;
          }
        }
      }
      const float sd = xsum4_16(xd, lane);
      const float sk = xsum4_16(xk, lane);
      const float sh = xsum4_16(xh, lane);
      const int64_t row = wrow0 + mi * 16 + rq + owner4(lane);
      if (!(lane & 3) && row < M) {
        float* p = a.parts + (row * nq + 3 * seg) * a.np + pidx;
        p[0] = sd;
        p[a.np] = sk;
        p[2 * a.np] = sh;
      }
    }
  } else {
    float* __restrict__ V = a.v;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      float xv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[j] = 0.0f;
      if constexpr (NI % 2 == 0) {
        // Column blocks in pairs: quarter-waves 2p and 2p+1 swap halves
        // (lane l and l ^ 16), so that each store writes 32 consecutive
        // columns (128 bytes) of two rows instead of 16 columns of four --
        // the even quarter's rows from block ni then ni + 1, the odd
        // quarter's likewise, one row in each store.
        const bool qodd = (lane >> 4) & 1;
#pragma unroll
        for (int ni = 0; ni < NI; ni += 2) {
          const int c0 = wcol0 + ni * 16 + (lane & 15);
          const int cs = c0 + (qodd ? 16 : 0);  // the column this lane stores
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x0 = acc[mi][ni][j], x1 = acc[mi][ni + 1][j];
            const int64_t row = wrow0 + mi * 16 + rq + j;
            if (row < M) {
              if (c0 < d) xv[j] += x0 * x0;
              if (c0 + 16 < d) xv[j] += x1 * x1;
            }
            const float got = __shfl_xor(qodd ? x0 : x1, 16);
            const int64_t re = wrow0 + mi * 16 + 4 * ((lane >> 4) & ~1) + j;  // even quarter's row
            if (cs < d) {  // read once, by the conv
              if (re < M) __builtin_nontemporal_store(qodd ? got : x0, &V[re * a.v_ld + cs]);
              if (re + 4 < M)
                __builtin_nontemporal_store(qodd ? x1 : got, &V[(re + 4) * a.v_ld + cs]);
            }
          }
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int col = wcol0 + ni * 16 + (lane & 15);
          if (col < d) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int64_t row = wrow0 + mi * 16 + rq + j;
              if (row < M) {
                const float v = acc[mi][ni][j];
                __builtin_nontemporal_store(v, &V[row * a.v_ld + col]);  // read once, by the conv
                xv[j] += v * v;
              }
            }
          }
        }
      }
      const float sv = xsum4_16(xv, lane);
      const int64_t row = wrow0 + mi * 16 + rq + owner4(lane);
      if (!(lane & 3) && row < M) a.parts[(row * nq + 3 * a.nb) * a.np + pidx] = sv;
    }
  }
}

template <int MI, int NI>
__device__ __forceinline__ void gate_epilogue16(const floatx4 (&acc)[MI][NI], const EpiArgs& a,
                                                int seg, int64_t wrow0, int wcol0, int pidx,
                                                int lane) {
  const bf16_bits* __restrict__ H = a.hidden + seg * a.h_branch_stride;
  const int64_t ht = a.h_tok_stride;
  gate_epilogue16<MI, NI>(acc, a, seg, wrow0, wcol0, pidx, lane,
                          [&](int64_t row, int col) { return bf16_to_f32(H[row * ht + col]); });
}

}  // namespace ngram
