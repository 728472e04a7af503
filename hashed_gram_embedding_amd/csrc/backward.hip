// Backward pass of the layer: the gradients a training step needs, for the
// tables, W_K, W_V, the conv taps, the query rows and the RMSNorm gains.
//
// Each kernel is the chain rule of one forward step ("Qwen3.8-Flash-Next
// 深度研究" §2.3: E_t -> K_t, V_t; g_t = Gate(Norm(Q_t), Norm(K_t));
// U_t = g_t V_t; Delta_t = U_t + SiLU(DWConv(RMSNorm(U_t))); Engram's third
// and fourth components in "Qwen 4用上DeepSeek的Engram").  The table gradient,
// the gather's adjoint (a scatter-add of dE into the rows the tokens named),
// is in table_grad.hip.  The dense products (K/V recompute, dE = dKV W, dW = dKV^T E) run on
// the MFMA projection kernel with a raw fp32 epilogue; the kernels here do the
// per-row work between them and the layout transposes that feed them.
//
// RMSNorm y = gamma (.) x / r, r = sqrt(mean(x^2) + eps) has the backward
// dx = gamma (.) dy / r - x * sum(gamma dy x) / (d r^3), dgamma += dy x / r;
// SiLU'(c) = s (1 + c (1 - s)) with s = sigmoid(c).
#include <type_traits>

#include "internal.h"

namespace ngram {
namespace {

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ float4 mk4(float x) { return make_float4(x, x, x, x); }
__device__ __forceinline__ float4 add(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 mul(float4 a, float4 b) {
  return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}
__device__ __forceinline__ float4 fma4(float4 a, float4 b, float4 c) {
  return make_float4(fmaf(a.x, b.x, c.x), fmaf(a.y, b.y, c.y), fmaf(a.z, b.z, c.z),
                     fmaf(a.w, b.w, c.w));
}
__device__ __forceinline__ float dot(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
__device__ __forceinline__ float4 gain4(const bf16_bits* g, int c) {
  return g ? Elem<bf16_bits>::load4(g, c) : mk4(1.0f);
}
// The same without a branch around the load: an absent gain reads the
// always-present `any` and is replaced by 1 as 1 + (x - 1) * 0, so the load
// goes out with the others instead of waiting behind a branch.
__device__ __forceinline__ float4 gain4_nb(const bf16_bits* g, const bf16_bits* any, int c) {
  const float4 x = Elem<bf16_bits>::load4(g ? g : any, c);
  const float on = g ? 1.0f : 0.0f;
  return make_float4(fmaf(x.x - 1.0f, on, 1.0f), fmaf(x.y - 1.0f, on, 1.0f),
                     fmaf(x.z - 1.0f, on, 1.0f), fmaf(x.w - 1.0f, on, 1.0f));
}
__device__ __forceinline__ float silu_grad(float c) {
  const float s = 1.0f / (1.0f + expf(-c));
  return s * (1.0f + c * (1.0f - s));
}

// Sum of NV values over the 256-thread block; every thread gets the totals.
template <int NV>
__device__ __forceinline__ void block_sum(float (&v)[NV], float (*red)[NV]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < NV; ++q) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v[q] += __shfl_xor(v[q], off);
  }
  __syncthreads();  // red may still be read from the previous call
  if (lane == 0)
#pragma unroll
    for (int q = 0; q < NV; ++q) red[wave][q] = v[q];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NV; ++q) v[q] = red[0][q] + red[1][q] + red[2][q] + red[3][q];
}

// Columns of a thread: the 4-column groups c = 4 * (x + 256 * i), i < ITEMS.
template <int ITEMS>
struct Cols {
  int c[ITEMS];
  bool ok[ITEMS];
  __device__ Cols(int d) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int v = 4 * ((int)threadIdx.x + 256 * i);
      ok[i] = v < d;
      c[i] = ok[i] ? v : d - 4;
    }
  }
};

// 1. Per token and branch: g = sigmoid(q^ . k^ / sqrt(d)), the three
// reciprocal norms 1/rho_h, 1/rho_k, 1/r (r: the norm of U = g V) and the
// gate's raw product P = sum (gamma_q h)(gamma_k K), from the query rows and
// the recomputed fp32 K/V.  stats row: g, 1/rho_h, 1/rho_k, 1/r, P, 0, 0, 0.
template <int ITEMS>
__global__ __launch_bounds__(256) void bwd_stats_kernel(BwdArgs a) {
  __shared__ float red[4][4];
  const int nb = a.nb, d = a.d;
  const Cols<ITEMS> cl(d);
  for (int64_t t = blockIdx.x; t < a.n; t += gridDim.x) {
    const float* kv = a.kv + t * a.kv_ld;
    float vv[1] = {0.0f};
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      if (cl.ok[i]) {
        const float4 v = ld4(kv + nb * d + cl.c[i]);
        vv[0] += dot(v, v);
      }
    block_sum<1>(vv, reinterpret_cast<float(*)[1]>(red));
    for (int br = 0; br < nb; ++br) {
      float s[3] = {0.0f, 0.0f, 0.0f};  // sum h^2, sum K^2, sum (gq h)(gk K)
#pragma unroll
      for (int i = 0; i < ITEMS; ++i)
        if (cl.ok[i]) {
          const float4 h = Elem<bf16_bits>::load4(a.hidden, t * a.h_tok + br * a.h_br + cl.c[i]);
          const float4 k = ld4(kv + br * d + cl.c[i]);
          s[0] += dot(h, h);
          s[1] += dot(k, k);
          s[2] += dot(mul(gain4(a.gamma_q, cl.c[i]), h), mul(gain4(a.gamma_k, cl.c[i]), k));
        }
      block_sum<3>(s, reinterpret_cast<float(*)[3]>(red));
      if (threadIdx.x == 0) {
        const float ih = 1.0f / sqrtf(s[0] / d + a.eps), ik = 1.0f / sqrtf(s[1] / d + a.eps);
        const float g = 1.0f / (1.0f + expf(-s[2] * ih * ik / sqrtf((float)d)));
        const float ir = 1.0f / sqrtf(g * g * vv[0] / d + a.eps);
        float* o = a.stats + (t * nb + br) * kStatsStride;
        st4(o, make_float4(g, ih, ik, ir));
        st4(o + 4, make_float4(s[2], 0.0f, 0.0f, 0.0f));
      }
    }
  }
}

// 2. dC = dOut (.) SiLU'(C) per token and branch, C = sum_i w_i (.) N_{t-i*dil}
// with N = gamma_u g V / r inside the sequence, the caller's ring rows before
// it (zeros without a ring, or before the sequence's start), and the taps' gradient d_w[i] = sum dC (.)
// N_{t-i*dil}.  A workgroup walks a tile of kBwdTile positions of one sequence
// and branch (plus the 3*dil positions before it) with each thread owning
// four columns, as the forward conv does: every V row is read once into a
// ring of the last 3*dil+1 positions, each group of positions loads its rows
// together, and the taps' gradient sums in registers and then into the
// workgroup's partial row [4 d] of a.part_conv (its first tile writes it, the
// others add to it; the column sum over workgroups runs afterwards).
constexpr int kBwdTile = 64;

template <int DIL>
__global__ __launch_bounds__(256) void bwd_conv_kernel(BwdArgs a) {
  constexpr int HALO = 3 * DIL, R = HALO + 1;
  __shared__ float s_sc[kBwdTile + HALO];  // g / r of each position (0 before the sequence)
  const int nb = a.nb, d = a.d;
  const int tiles = (a.T + kBwdTile - 1) / kBwdTile;
  const int64_t total = a.n / a.T * tiles * nb;
  float* __restrict__ part = a.part_conv + (int64_t)blockIdx.x * 4 * d;
  bool first = true;
  for (int64_t wi = blockIdx.x; wi < total; wi += gridDim.x) {
    const int br = (int)(wi % nb);
    const int64_t bt = wi / nb;
    const int64_t b = bt / tiles;
    const int p0 = (int)(bt - b * tiles) * kBwdTile;
    const int p1 = min(p0 + kBwdTile, a.T);
    const int qs = p0 - HALO, L = p1 - qs;
    const int64_t seq0 = b * a.T;
    __syncthreads();  // the previous tile's walk is done with s_sc
    for (int i = threadIdx.x; i < L; i += blockDim.x) {
      const int q = qs + i;
      const float* st = a.stats + ((seq0 + (q < 0 ? 0 : q)) * nb + br) * kStatsStride;
      s_sc[i] = q < 0 ? 0.0f : st[0] * st[3];
    }
    __syncthreads();
    for (int c0 = threadIdx.x * 4; c0 < d; c0 += blockDim.x * 4) {
      const float4 gu = gain4_nb(a.gamma_u, a.conv_w, c0);
      const float4 w0 = Elem<bf16_bits>::load4(a.conv_w, c0);
      const float4 w1 = Elem<bf16_bits>::load4(a.conv_w, (int64_t)d + c0);
      const float4 w2 = Elem<bf16_bits>::load4(a.conv_w, 2 * (int64_t)d + c0);
      const float4 w3 = Elem<bf16_bits>::load4(a.conv_w, 3 * (int64_t)d + c0);
      // positions before the sequence (a sequence's first tile, i < HALO of
      // the first group): the ring starts with the state rows there
      float4 ring[R];
#pragma unroll
      for (int u = 0; u < R; ++u) ring[u] = mk4(0.0f);
      if (qs < 0 && a.state) {
        const int pos = ring_pos(a.state_pos, b, HALO);
#pragma unroll
        for (int u = 0; u < HALO; ++u) {
          int q = qs + u;
          q = q < -HALO ? -HALO : (q > -1 ? -1 : q);
          const int slot = ring_slot(pos, q, HALO);
          const float4 sv =
              ld4(a.state + ((b * HALO + (slot < 0 ? 0 : slot)) * nb + br) * (int64_t)d + c0);
          if (qs + u < 0 && slot >= 0) ring[u] = sv;
        }
      }
      float4 dw0 = mk4(0.0f), dw1 = mk4(0.0f), dw2 = mk4(0.0f), dw3 = mk4(0.0f);
      for (int base = 0; base < L; base += R) {
        // the group's V rows and output-gradient rows, loaded together from
        // clamped positions (positions outside the tile's range are unused)
        float4 raw[R], go[R];
#pragma unroll
        for (int u = 0; u < R; ++u) {
          int q = qs + base + u;
          q = q < 0 ? 0 : (q > p1 - 1 ? p1 - 1 : q);
          raw[u] = ld4(a.kv + (seq0 + q) * a.kv_ld + (int64_t)nb * d + c0);
          int qo = qs + base + u;
          qo = qo < p0 ? p0 : (qo > p1 - 1 ? p1 - 1 : qo);
          go[u] = Elem<bf16_bits>::load4(a.d_out, ((seq0 + qo) * nb + br) * (int64_t)d + c0);
        }
#pragma unroll
        for (int u = 0; u < R; ++u) {
          const int i = base + u;
          if (i < L) {
            const int q = qs + i;
            if (q >= 0) ring[u] = mul(gu, mul(raw[u], mk4(s_sc[i])));
            if (q >= p0) {
              const float4 n1 = ring[(u - DIL + R) % R], n2 = ring[(u - 2 * DIL + R) % R],
                           n3 = ring[(u - 3 * DIL + R) % R];
              float4 cc = mul(w0, ring[u]);
              cc = fma4(w1, n1, cc);
              cc = fma4(w2, n2, cc);
              cc = fma4(w3, n3, cc);
              const float4 dc = make_float4(go[u].x * silu_grad(cc.x), go[u].y * silu_grad(cc.y),
                                            go[u].z * silu_grad(cc.z), go[u].w * silu_grad(cc.w));
              st4(a.dc + ((seq0 + q) * nb + br) * (int64_t)d + c0, dc);
              dw0 = fma4(dc, ring[u], dw0);
              dw1 = fma4(dc, n1, dw1);
              dw2 = fma4(dc, n2, dw2);
              dw3 = fma4(dc, n3, dw3);
            }
          }
        }
      }
      float* pc = part + c0;
      if (!first) {
        dw0 = add(dw0, ld4(pc));
        dw1 = add(dw1, ld4(pc + d));
        dw2 = add(dw2, ld4(pc + 2 * d));
        dw3 = add(dw3, ld4(pc + 3 * d));
      }
      st4(pc, dw0);
      st4(pc + d, dw1);
      st4(pc + 2 * d, dw2);
      st4(pc + 3 * d, dw3);
    }
    first = false;
  }
  if (first)  // a workgroup without a tile leaves a zero partial row
    for (int c = threadIdx.x * 4; c < 4 * d; c += blockDim.x * 4) st4(part + c, mk4(0.0f));
}

// 3. Per token, all branches: dN -> dU (residual + RMSNorm), dg and dV (U = g V),
// dz -> dK and the query's gradient (both RMSNorms), the gains' gradients.
// dK and dV are written in bf16 as the operands of the dE and dW products.
//
// One block reduction per row suffices.  With A = sum gamma_u dN V and
// B = sum dOut V (both from rows already loaded):
//   dg = sum dU V = B + A r^-1 (1 - g^2 sum(V^2) / (d r^2)) = B + A eps r^-3,
// since r^2 = g^2 sum(V^2) / d + eps (the norm's scale invariance leaves only
// the eps term; this form also avoids the cancellation).  The two RMSNorm
// backward sums of the gate are multiples of the gate's raw product P:
//   sum gamma_k dk^ K = (dz / sqrt d) rho_h^-1 P,  sum gamma_q dq^ h = (dz / sqrt d) rho_k^-1 P.
// The gains' gradients accumulate per thread in LDS (each thread owns its
// columns) and leave as the block's partial row [3 d] of a.part_gain.
template <int ITEMS, bool ONE_BRANCH>
__global__ __launch_bounds__(256) void bwd_main_kernel(BwdArgs a) {
  __shared__ float red[4][2];
  __shared__ float4 gacc[3][ITEMS][256];
  const int nb = ONE_BRANCH ? 1 : a.nb, d = a.d, dil = a.dil;
  const float fd = (float)d, rsd = 1.0f / sqrtf(fd);
  const Cols<ITEMS> cl(d);
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) gacc[q][j][tid] = mk4(0.0f);
  for (int64_t t = blockIdx.x; t < a.n; t += gridDim.x) {
    const int pos = (int)(t % a.T);
    const float* kv = a.kv + t * a.kv_ld;
    float4 v[ITEMS], dv[ITEMS], dhs[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      v[j] = ld4(kv + nb * d + cl.c[j]);
      dv[j] = dhs[j] = mk4(0.0f);
    }
    for (int br = 0; br < nb; ++br) {
      const int64_t row = t * nb + br;
      const float4 st = ld4(a.stats + row * kStatsStride);  // g, 1/rho_h, 1/rho_k, 1/r
      const float P = a.stats[row * kStatsStride + 4];
      const float g = st.x, ih = st.y, ik = st.z, ir = st.w;
      // dN = sum_i w_i (.) dC_{t + i*dil} inside the sequence.  Every load is
      // unconditional (taps past the sequence end read the row itself and are
      // weighted by 0, columns past d read a clamped valid column and are
      // dropped), so they all go out before the first wait.
      float4 dn[ITEMS], go[ITEMS], h[ITEMS], k[ITEMS], gu[ITEMS], w[4][ITEMS], dcv[4][ITEMS];
      float s[2] = {0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        const int c = cl.c[j];
        go[j] = Elem<bf16_bits>::load4(a.d_out, row * d + c);
        h[j] = Elem<bf16_bits>::load4(a.hidden, t * a.h_tok + br * a.h_br + c);
        k[j] = ld4(kv + br * d + c);
        gu[j] = gain4_nb(a.gamma_u, a.conv_w, c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool in = pos + i * dil < a.T;
          w[i][j] = Elem<bf16_bits>::load4(a.conv_w, (int64_t)i * d + c);
          dcv[i][j] = ld4(a.dc + (row + (in ? (int64_t)i * dil * nb : 0)) * d + c);
        }
      }
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        dn[j] = mk4(0.0f);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (pos + i * dil < a.T) dn[j] = fma4(w[i][j], dcv[i][j], dn[j]);
        if (cl.ok[j]) {
          s[0] += dot(mul(gu[j], dn[j]), v[j]);
          s[1] += dot(go[j], v[j]);
        }
      }
      block_sum<2>(s, red);
      const float A = s[0];
      const float dz = (s[1] + A * a.eps * ir * ir * ir) * g * (1.0f - g);
      const float cu = -g * g * A * ir * ir * ir / fd;  // dU's term along V
      const float cz = dz * rsd;
      const float sk = cz * ih * P * ik * ik * ik / fd, sq = cz * ik * P * ih * ih * ih / fd;
      float4 gqs[ITEMS], gks[ITEMS];  // both gains of every column group, loaded together
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        gqs[j] = gain4_nb(a.gamma_q, a.conv_w, cl.c[j]);
        gks[j] = gain4_nb(a.gamma_k, a.conv_w, cl.c[j]);
      }
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        if (!cl.ok[j]) continue;
        const int c = cl.c[j];
        const float4 gq = gqs[j], gk = gks[j];
        // dU = dOut + gamma_u dN / r - U sum(gamma_u dN U) / (d r^3), U = g V
        const float4 du = fma4(v[j], mk4(cu), fma4(mul(gu[j], dn[j]), mk4(ir), go[j]));
        // q^ = gamma_q h / rho_h, k^ = gamma_k K / rho_k; dq^ = dz k^ / sqrt d, dk^ = dz q^ / sqrt d
        const float4 dqh = mul(mk4(cz * ik), mul(gk, k[j]));
        const float4 dkh = mul(mk4(cz * ih), mul(gq, h[j]));
        const float4 dkk = fma4(k[j], mk4(-sk), mul(mul(gk, dkh), mk4(ik)));
        float4 dh = fma4(h[j], mk4(-sq), mul(mul(gq, dqh), mk4(ih)));
        if (a.add_residual) dh = add(dh, go[j]);
        Elem<bf16_bits>::store4(a.dkv, t * a.dkv_ld + br * d + c, dkk);
        gacc[0][j][tid] = fma4(mul(dqh, h[j]), mk4(ih), gacc[0][j][tid]);
        gacc[1][j][tid] = fma4(mul(dkh, k[j]), mk4(ik), gacc[1][j][tid]);
        gacc[2][j][tid] = fma4(mul(dn[j], v[j]), mk4(g * ir), gacc[2][j][tid]);
        if (ONE_BRANCH) {
          Elem<bf16_bits>::store4(a.dkv, t * a.dkv_ld + d + c, mul(mk4(g), du));
          if (a.d_hidden) st4(a.d_hidden + t * a.h_tok + c, dh);
        } else {
          dv[j] = fma4(mk4(g), du, dv[j]);
          if (a.d_hidden) {
            if (a.h_br == 0)
              dhs[j] = add(dhs[j], dh);
            else
              st4(a.d_hidden + t * a.h_tok + br * a.h_br + c, dh);
          }
        }
      }
    }
    if (!ONE_BRANCH) {
#pragma unroll
      for (int j = 0; j < ITEMS; ++j)
        if (cl.ok[j]) {
          Elem<bf16_bits>::store4(a.dkv, t * a.dkv_ld + nb * d + cl.c[j], dv[j]);
          if (a.d_hidden && a.h_br == 0) st4(a.d_hidden + t * a.h_tok + cl.c[j], dhs[j]);
        }
    }
  }
  if (a.part_gain) {
    float* part = a.part_gain + (int64_t)blockIdx.x * 3 * d;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      if (cl.ok[j])
#pragma unroll
        for (int q = 0; q < 3; ++q) st4(part + (int64_t)q * d + cl.c[j], gacc[q][j][tid]);
  }
}

// Column sums of a row-major [rows, cols] fp32 matrix: block row y of the
// grid sums rows [y*per, min((y+1)*per, rows)) into dst[y, :].
__global__ __launch_bounds__(256) void sum_rows_kernel(const float* __restrict__ src,
                                                       int64_t rows, int64_t cols, int per,
                                                       float* __restrict__ dst) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * per;
  const int64_t r1 = r0 + per < rows ? r0 + per : rows;
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  int64_t r = r0;
  for (; r + 8 <= r1; r += 8)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += src[(r + u) * cols + col];
  for (; r < r1; ++r) acc[0] += src[r * cols + col];
  dst[(int64_t)blockIdx.y * cols + col] =
      ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

// out[i] = sum_s part[s * stride + i] over the split-K partial products,
// four floats per thread, the splits added in order.
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part,
                                                         int32_t split, int64_t stride, int64_t n4,
                                                         float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * 256) {
    float4 x = ld4(part + 4 * i);
    for (int sp = 1; sp < split; ++sp) x = add(x, ld4(part + sp * stride + 4 * i));
    st4(out + 4 * i, x);
  }
}

// bf16 [rows, cols] (row stride ld_src) -> [cols, rows_pad] (row stride
// ld_dst), rows rows..rows_pad-1 of the result zero; 64 x 64 tiles via LDS.
// A thread reads 8 consecutive columns of a source row and writes 8
// consecutive entries of a result row (8 source rows of one column, gathered
// from the tile), both as 16-byte accesses: rows 16-byte aligned on both
// sides, rows_pad a multiple of 64; columns may be ragged.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16_bits* __restrict__ src,
                                                                 int64_t rows, int64_t cols,
                                                                 int64_t ld_src,
                                                                 bf16_bits* __restrict__ dst,
                                                                 int64_t ld_dst) {
  __shared__ __attribute__((aligned(16))) bf16_bits tile[64][72];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int r = i >> 3, cc = (i & 7) * 8;
    const int64_t gr = r0 + r, gc = c0 + cc;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (gr < rows) {
      const bf16_bits* sp = src + gr * ld_src + gc;
      if (gc + 8 <= cols) {
        v = *reinterpret_cast<const uint4*>(sp);
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        for (int e = 0; e < 8 && gc + e < cols; ++e) w[e >> 1] |= (uint32_t)sp[e] << (16 * (e & 1));
        v = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    *reinterpret_cast<uint4*>(&tile[r][cc]) = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int c = i >> 3, rr = (i & 7) * 8;
    const int64_t gc = c0 + c;
    if (gc >= cols) continue;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (uint32_t)tile[rr + 2 * k][c] | ((uint32_t)tile[rr + 2 * k + 1][c] << 16);
    *reinterpret_cast<uint4*>(dst + gc * ld_dst + r0 + rr) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__global__ void zero_f32_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

unsigned grid_of(int64_t work, int64_t cap) {
  int64_t g = work < cap ? work : cap;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_bwd_rows(const BwdArgs& a, float* d_conv_w, float* d_gammas,
                           float* reduce_tmp, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const int items = (a.d + 1023) / 1024;
  hipError_t e;
  if (a.T <= 0 || a.n % a.T != 0 || a.dil < 1 || a.dil > 4 || a.d % 4 != 0)
    return hipErrorInvalidValue;
  const int64_t conv_work = a.n / a.T * ((a.T + kBwdTile - 1) / kBwdTile) * a.nb;
  const unsigned g1 = grid_of(a.n, 4096), g2 = grid_of(conv_work, kBwdBlocks),
                 g3 = grid_of(a.n, kBwdBlocks);
  auto conv = [&]() -> hipError_t {
    switch (a.dil) {
      case 1: return launch(bwd_conv_kernel<1>, g2, 256, 0, s, a);
      case 2: return launch(bwd_conv_kernel<2>, g2, 256, 0, s, a);
      case 3: return launch(bwd_conv_kernel<3>, g2, 256, 0, s, a);
      default: return launch(bwd_conv_kernel<4>, g2, 256, 0, s, a);
    }
  };
#define NGRAM_BWD_ITEMS(I)                                                        \
  case I:                                                                         \
    e = launch(bwd_stats_kernel<I>, g1, 256, 0, s, a);                            \
    if (e != hipSuccess) return e;                                                \
    e = conv();                                                                   \
    if (e != hipSuccess) return e;                                                \
    e = a.nb == 1 ? launch(bwd_main_kernel<I, true>, g3, 256, 0, s, a)            \
                  : launch(bwd_main_kernel<I, false>, g3, 256, 0, s, a);          \
    break;
  switch (items) {
    NGRAM_BWD_ITEMS(1)
    NGRAM_BWD_ITEMS(2)
    NGRAM_BWD_ITEMS(3)
    NGRAM_BWD_ITEMS(4)
    default: return hipErrorInvalidValue;
  }
#undef NGRAM_BWD_ITEMS
  if (e != hipSuccess) return e;
  // column sums of the per-block partial rows, in two passes of <= 32 rows
  auto col_sum = [&](const float* part, int64_t rows, int64_t cols, float* out) {
    const unsigned gx = (unsigned)((cols + 255) / 256);
    const int64_t mid = (rows + 31) / 32;
    hipError_t r = launch(sum_rows_kernel, dim3(gx, (unsigned)mid), 256, 0, s, part, rows, cols,
                          32, reduce_tmp);
    if (r != hipSuccess) return r;
    return launch(sum_rows_kernel, dim3(gx, 1), 256, 0, s, (const float*)reduce_tmp, mid, cols,
                  (int)mid, out);
  };
  e = col_sum(a.part_conv, g2, 4 * (int64_t)a.d, d_conv_w);
  if (e != hipSuccess || d_gammas == nullptr) return e;
  return col_sum(a.part_gain, g3, 3 * (int64_t)a.d, d_gammas);
}

hipError_t launch_sum_splits(const float* part, int32_t split, int64_t stride, int64_t n,
                             float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (n % 4 != 0 || stride % 4 != 0 || split < 1) return hipErrorInvalidValue;
  return launch(sum_splits_kernel, grid_of((n / 4 + 255) / 256, 8192), 256, 0, s, part, split,
                stride, n / 4, out);
}

hipError_t launch_transpose_bf16(const bf16_bits* src, int64_t rows, int64_t cols, int64_t ld_src,
                                 bf16_bits* dst, int64_t rows_pad, int64_t ld_dst, hipStream_t s) {
  if (rows_pad == 0 || cols == 0) return hipSuccess;
  const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows_pad + 63) / 64));
  if (ld_src % 8 != 0 || ld_dst % 8 != 0 || rows_pad % 64 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return hipErrorInvalidValue;
  return launch(transpose_bf16_kernel, grid, 256, 0, s, src, rows, cols, ld_src, dst, ld_dst);
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  return launch(zero_f32_kernel, grid_of((n + 255) / 256, 16384), 256, 0, s, p, n);
}

}  // namespace ngram
