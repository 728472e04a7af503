// Gate, gated value and the convolution block.
//
// "Qwen3.8-Flash-Next 深度研究" §2.3: g_t = Gate(Norm(Q_t), Norm(K_t)),
// U_t = g_t (.) V_t, Delta_t = U_t + SiLU(DWConv(RMSNorm(U_t))); Engram's third
// and fourth components ("Qwen 4用上DeepSeek的Engram", section "DeepSeek Engram
// 更复杂，Qwen 更精简"): a scalar sigmoid gate per token and branch from an
// RMSNorm'd scaled dot product, and a depthwise causal conv of kernel 4 whose
// dilation is the largest n-gram order.
//
// Streaming, HBM-bound work.  One workgroup takes a tile of consecutive
// positions of one sequence and one branch:
//   1. per position of the tile and its 3*dil-position halo it folds the
//      projection's row partials into the gate g and the RMSNorm scale of
//      U = g V (|U|^2 = g^2 |V|^2, so U itself is never reduced again), kept
//      in LDS;
//   2. each thread owns 4 columns and walks the positions in order, holding
//      the normalised values of the last 3*dil+1 positions in registers, so
//      every V element is read once per tile (plus the halo) and each output
//      element is written once as a 16/8-byte vector.
// The op-level ngram_causal_conv takes U itself and computes the row norms in
// step 1 instead.
#include "internal.h"

namespace ngram {
namespace {

constexpr int kMaxTile = 64;
constexpr int kMaxHalo = 3 * NGRAM_MAX_ORDER;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 f4(float x) { return make_float4(x, x, x, x); }
__device__ __forceinline__ float4 mul4(float4 a, float4 b) {
  return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}
__device__ __forceinline__ float4 fma4(float4 a, float4 b, float4 c) {
  return make_float4(fmaf(a.x, b.x, c.x), fmaf(a.y, b.y, c.y), fmaf(a.z, b.z, c.z), fmaf(a.w, b.w, c.w));
}
__device__ __forceinline__ float silu(float c) { return c / (1.0f + expf(-c)); }
__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// Row partials of one position folded by a 16-lane group (lane sub of 16):
// the gate's dot product, sum k^2, sum h^2 of branch br and sum v^2, summed
// over the np partials in a fixed order and combined across the group.
struct RowSums {
  float dot, kk, hh, vv;
};
__device__ __forceinline__ RowSums fold_partials16(const float* pr, int np, int br, int nb,
                                                   int sub) {
  RowSums r{0.0f, 0.0f, 0.0f, 0.0f};
  for (int p = sub; p < np; p += 16) {
    r.dot += pr[(3 * br) * np + p];
    r.kk += pr[(3 * br + 1) * np + p];
    r.hh += pr[(3 * br + 2) * np + p];
    r.vv += pr[(3 * nb) * np + p];
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) {
    r.dot += __shfl_xor(r.dot, off);
    r.kk += __shfl_xor(r.kk, off);
    r.hh += __shfl_xor(r.hh, off);
    r.vv += __shfl_xor(r.vv, off);
  }
  return r;
}

// Gate of a position and the factor that turns its V row into the
// normalised row N = gamma_u (.) U / rms(U) (with U = g V, rms(U)^2 =
// g^2 mean(v^2) + eps, so N = gamma_u (.) V * g / sqrt(g^2 mean(v^2) + eps)).
__device__ __forceinline__ void gate_and_scale(const RowSums& r, float fd, float eps, float& al,
                                               float& sc) {
  const float z = r.dot / (sqrtf(r.hh / fd + eps) * sqrtf(r.kk / fd + eps) * sqrtf(fd));
  al = 1.0f / (1.0f + expf(-z));
  sc = al / sqrtf(al * al * (r.vv / fd) + eps);
}

// 1 / rms of a U row, one wave (lane of 64) over d columns.
template <typename T>
__device__ __forceinline__ float inv_rms_row(const T* row, int d, float eps, int lane) {
  float ss = 0.0f;
  for (int c = lane * 4; c < d; c += 256) {
    const float4 x = Elem<T>::load4(row, c);
    ss += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  return 1.0f / sqrtf(ss / (float)d + eps);
}

// With a ring update, sequence b's ring position moves on by the call's
// positions.  Every thread of the workgroup read the position from memory and
// used it (in the addresses of ring reads or writes issued before this
// point), so after the barrier no read of it can still see the new value.
__device__ __forceinline__ void advance_ring(const ConvArgs& a, int64_t b, int pos, int T) {
  if (!a.update_state) return;
  __syncthreads();
  if (threadIdx.x == 0) a.state_pos[b] = pos + T;
}

// ngram_gate: gates and U = g V in the activation dtype.
template <typename T>
__global__ __launch_bounds__(256) void gate_values_kernel(ConvArgs a, int64_t M) {
  __shared__ float s_alpha[NGRAM_MAX_BRANCHES];
  const int64_t tok = blockIdx.x;
  if (tok >= M) return;
  const int nq = 3 * a.nb + 1;
  const float* pr = a.parts + tok * nq * a.np;
  {
    // one wave per branch; lanes split the row partials
    const int lane = threadIdx.x & 63, br = threadIdx.x >> 6;
    if (br < a.nb) {
      float dot = 0.0f, kk = 0.0f, hh = 0.0f;
      for (int p = lane; p < a.np; p += 64) {
        dot += pr[(3 * br) * a.np + p];
        kk += pr[(3 * br + 1) * a.np + p];
        hh += pr[(3 * br + 2) * a.np + p];
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        dot += __shfl_xor(dot, off);
        kk += __shfl_xor(kk, off);
        hh += __shfl_xor(hh, off);
      }
      if (lane == 0) {
        const float fd = (float)a.d;
        const float z = dot / (sqrtf(hh / fd + a.eps) * sqrtf(kk / fd + a.eps) * sqrtf(fd));
        const float al = 1.0f / (1.0f + expf(-z));
        s_alpha[br] = al;
        if (a.gates) a.gates[tok * a.nb + br] = al;
      }
    }
  }
  __syncthreads();
  T* out = static_cast<T*>(a.out);
  if (out == nullptr) return;
  const float* v = a.v + tok * a.v_stride;
  for (int c = threadIdx.x * 4; c < a.d; c += blockDim.x * 4) {
    const float4 vv = *reinterpret_cast<const float4*>(v + c);
    for (int br = 0; br < a.nb; ++br)
      Elem<T>::store4(out, (tok * a.nb + br) * a.d + c, mul4(f4(s_alpha[br]), vv));
  }
}

// FUSED: source is fp32 V + partials (U = g V); else the act-dtype U rows.
// RES: the hidden state is added to the output (FUSED only).
template <int DIL, typename T, bool FUSED, bool RES>
__global__ __launch_bounds__(512) void conv_kernel(ConvArgs a) {
  constexpr int HALO = 3 * DIL;
  constexpr int R = HALO + 1;
  __shared__ float s_alpha[kMaxTile + kMaxHalo];
  __shared__ float s_scale[kMaxTile + kMaxHalo];

  const int tiles = (a.T + a.tile - 1) / a.tile;
  // Block -> (sequence tile, branch), branch innermost: the branches of one
  // tile read the same V rows, so their workgroups run together, and on one
  // XCD (workgroup w runs on XCD w % 8) when the tile count allows it, where
  // one L2 then serves the later ones.  One branch: block = tile.
  const int nbr = a.nb, blk = (int)blockIdx.x;
  int tl, br;
  if (((int64_t)a.B * tiles) % 8 == 0) {
    const int slot = blk >> 3;
    tl = (slot / nbr) * 8 + (blk & 7);
    br = slot % nbr;
  } else {
    tl = blk / nbr;
    br = blk % nbr;
  }
  const int b = tl / tiles;
  const int p0 = (tl - b * tiles) * a.tile;
  const int p1 = min(p0 + a.tile, a.T);
  const int qs = p0 - HALO;
  const int L = p1 - qs;
  const int nb = a.nb, d = a.d;
  const int64_t seq0 = (int64_t)b * a.T;

  // ---- step 1: per-position scalars, four positions per wave at a time:
  // each 16-lane group splits the np row partials of one position and
  // combines them with shuffles (the four positions' loads go out together)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (FUSED) {
    const int nq = 3 * nb + 1;
    const float fd = (float)d;
    const int sub = lane & 15, grp = lane >> 4;
    for (int i0 = wave * 4; i0 < L; i0 += nw * 4) {
      const int i = i0 + grp;
      const int q = qs + i;
      const bool live = i < L && q >= 0;
      const int64_t tok = seq0 + (live ? q : 0);  // any valid row when not live
      const RowSums r = fold_partials16(a.parts + tok * nq * a.np, a.np, br, nb, sub);
      if (sub == 0 && i < L) {
        if (q < 0) {
          s_alpha[i] = 0.0f;
          s_scale[i] = 0.0f;
        } else {
          float al, sc;
          gate_and_scale(r, fd, a.eps, al, sc);
          s_alpha[i] = al;
          s_scale[i] = sc;
          if (a.gates && q >= p0) a.gates[tok * nb + br] = al;
        }
      }
    }
  } else {
    const T* U = static_cast<const T*>(a.u);
    for (int i = wave; i < L; i += nw) {
      const int q = qs + i;
      float sc = 0.0f;
      if (q >= 0) sc = inv_rms_row(U + ((seq0 + q) * nb + br) * d, d, a.eps, lane);
      if (lane == 0) {
        s_alpha[i] = 1.0f;
        s_scale[i] = sc;
      }
    }
  }
  __syncthreads();

  // ---- step 2: walk the positions, 4 columns per thread
  const T* __restrict__ CW = static_cast<const T*>(a.conv_w);
  const T* __restrict__ GU = static_cast<const T*>(a.gamma_u);
  T* __restrict__ OUT = static_cast<T*>(a.out);
  const T* __restrict__ H = static_cast<const T*>(a.hidden);
  const int pos = qs < 0 && a.state ? ring_pos(a.state_pos, b, HALO) : 0;
  for (int c0 = threadIdx.x * 4; c0 < d; c0 += blockDim.x * 4) {
    const float4 w0 = Elem<T>::load4(CW, c0);
    const float4 w1 = Elem<T>::load4(CW, d + c0);
    const float4 w2 = Elem<T>::load4(CW, 2 * d + c0);
    const float4 w3 = Elem<T>::load4(CW, 3 * d + c0);
    const float4 gu = GU ? Elem<T>::load4(GU, c0) : f4(1.0f);
    // Positions before the sequence occur only in its first tile (qs < 0,
    // p0 == 0), at i < HALO of the first group: the ring starts with the
    // caller's state rows there (zeros without a state, or for positions
    // before the sequence's start), and the walk assigns positions q >= 0
    // only.  No load then sits behind a branch of the walk, which would make
    // the compiler wait for every load in flight.
    float4 ring[R];
#pragma unroll
    for (int u = 0; u < R; ++u) ring[u] = f4(0.0f);
    if (qs < 0 && a.state) {
#pragma unroll
      for (int u = 0; u < HALO; ++u) {
        int q = qs + u;
        q = q < -HALO ? -HALO : (q > -1 ? -1 : q);
        const int slot = ring_slot(pos, q, HALO);
        const float4 st = *reinterpret_cast<const float4*>(
            a.state + (((int64_t)b * HALO + (slot < 0 ? 0 : slot)) * nb + br) * d + c0);
        if (qs + u < 0 && slot >= 0) ring[u] = st;
      }
    }
    for (int base = 0; base < L; base += R) {
      // the group's R source rows (and residual rows) are loaded first, from
      // clamped row indices, so that all of them are in flight together; rows
      // outside [0, p1) are never used
      float4 raw[R], hres[RES ? R : 1];
#pragma unroll
      for (int u = 0; u < R; ++u) {
        int q = qs + base + u;
        q = q < 0 ? 0 : (q > p1 - 1 ? p1 - 1 : q);
        if (FUSED) {
          const f32x4 x = __builtin_nontemporal_load(
              reinterpret_cast<const f32x4*>(a.v + (seq0 + q) * a.v_stride + c0));
          raw[u] = make_float4(x[0], x[1], x[2], x[3]);
        } else {
          raw[u] = Elem<T>::load4(static_cast<const T*>(a.u), ((seq0 + q) * nb + br) * d + c0);
        }
      }
      if (RES) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
          int q = qs + base + u;
          q = q < p0 ? p0 : (q > p1 - 1 ? p1 - 1 : q);
          hres[u] = Elem<T>::load4(H, (seq0 + q) * a.h_tok_stride + br * a.h_branch_stride + c0);
        }
      }
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int i = base + u;
        if (i < L) {
          const int q = qs + i;
          const float4 src = raw[u];
          if (q >= 0) ring[u] = mul4(mul4(gu, src), f4(s_scale[i]));
          if (q >= p0) {
            float4 C = mul4(w0, ring[u]);
            C = fma4(w1, ring[(u - DIL + R) % R], C);
            C = fma4(w2, ring[(u - 2 * DIL + R) % R], C);
            C = fma4(w3, ring[(u - 3 * DIL + R) % R], C);
            const float g = FUSED ? s_alpha[i] : 1.0f;
            float4 D = make_float4(fmaf(g, src.x, silu(C.x)), fmaf(g, src.y, silu(C.y)),
                                   fmaf(g, src.z, silu(C.z)), fmaf(g, src.w, silu(C.w)));
            const int64_t tok = seq0 + q;
            if (RES) D = add4(D, hres[u]);
            Elem<T>::store4_stream(OUT, (tok * nb + br) * d + c0, D);
          }
        }
      }
    }
  }
}

// Decode (one new token per sequence): sum the K splits of the projection,
// then gate, U, RMSNorm(U), the conv taps (the current position's and the
// caller's state rows, or zeros, for the earlier ones) and the output.  One
// workgroup per token; the token's (nb+1)*d columns are read twice from L2,
// once for the row reductions and once for the outputs.
template <typename T>
__global__ __launch_bounds__(256) void decode_finalize_kernel(ConvArgs a, const float* __restrict__ split,
                                                              int32_t k_split, int32_t dil) {
  __shared__ float s_red[4][3 * NGRAM_MAX_BRANCHES + 1];
  __shared__ float s_tot[3 * NGRAM_MAX_BRANCHES + 1];
  const int64_t tok = blockIdx.x;  // T == 1: token = sequence
  const int nb = a.nb, d = a.d;
  const int64_t ntot = (int64_t)(nb + 1) * d;
  const int64_t sstride = (int64_t)a.B * ntot;
  const float* __restrict__ P = split + tok * ntot;
  const T* __restrict__ H = static_cast<const T*>(a.hidden);
  const T* __restrict__ GQ = static_cast<const T*>(a.gamma_q);
  const T* __restrict__ GK = static_cast<const T*>(a.gamma_k);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int halo = 3 * dil;
  const int pos = a.state ? ring_pos(a.state_pos, tok, halo) : 0;

  auto col4 = [&](int64_t off, int c) {  // sum of the splits, 4 columns
    float4 x = *reinterpret_cast<const float4*>(P + off + c);
    for (int s = 1; s < k_split; ++s) {
      const float4 y = *reinterpret_cast<const float4*>(P + s * sstride + off + c);
      x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
    }
    return x;
  };

  // pass 1: row reductions (dot, sum k^2, sum h^2 per branch; sum v^2)
  float acc[3 * NGRAM_MAX_BRANCHES + 1];
#pragma unroll
  for (int q = 0; q < 3 * NGRAM_MAX_BRANCHES + 1; ++q) acc[q] = 0.0f;
  for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4) {
    const float4 gq = GQ ? Elem<T>::load4(GQ, c) : f4(1.0f);
    const float4 gk = GK ? Elem<T>::load4(GK, c) : f4(1.0f);
#pragma unroll
    for (int br = 0; br < NGRAM_MAX_BRANCHES; ++br) {
      if (br < nb) {
        const float4 k = col4((int64_t)br * d, c);
        const float4 h = Elem<T>::load4(H, tok * a.h_tok_stride + br * a.h_branch_stride + c);
        acc[3 * br] += gq.x * gk.x * h.x * k.x + gq.y * gk.y * h.y * k.y + gq.z * gk.z * h.z * k.z +
                       gq.w * gk.w * h.w * k.w;
        acc[3 * br + 1] += k.x * k.x + k.y * k.y + k.z * k.z + k.w * k.w;
        acc[3 * br + 2] += h.x * h.x + h.y * h.y + h.z * h.z + h.w * h.w;
      }
    }
    const float4 v = col4((int64_t)nb * d, c);
    acc[3 * NGRAM_MAX_BRANCHES] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
#pragma unroll
  for (int q = 0; q < 3 * NGRAM_MAX_BRANCHES + 1; ++q) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc[q] += __shfl_xor(acc[q], off);
    if (lane == 0) s_red[wave][q] = acc[q];
  }
  __syncthreads();
  if (threadIdx.x < 3 * NGRAM_MAX_BRANCHES + 1)
    s_tot[threadIdx.x] = s_red[0][threadIdx.x] + s_red[1][threadIdx.x] + s_red[2][threadIdx.x] +
                         s_red[3][threadIdx.x];
  __syncthreads();

  const float fd = (float)d;
  const T* __restrict__ CW = static_cast<const T*>(a.conv_w);
  const T* __restrict__ GU = static_cast<const T*>(a.gamma_u);
  T* __restrict__ OUT = static_cast<T*>(a.out);
  for (int br = 0; br < nb; ++br) {
    RowSums r{s_tot[3 * br], s_tot[3 * br + 1], s_tot[3 * br + 2], s_tot[3 * NGRAM_MAX_BRANCHES]};
    float al, sc;
    gate_and_scale(r, fd, a.eps, al, sc);
    if (a.gates && threadIdx.x == 0) a.gates[tok * nb + br] = al;
    // pass 2: outputs
    for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4) {
      const float4 v = col4((int64_t)nb * d, c);
      const float4 gu = GU ? Elem<T>::load4(GU, c) : f4(1.0f);
      const float4 nrm = mul4(mul4(gu, v), f4(sc));  // this position's normalised row
      float4 C = mul4(Elem<T>::load4(CW, c), nrm);
      if (a.state) {
        // taps at positions -dil, -2 dil, -3 dil from the ring, zero before
        // the sequence's start; every read precedes the write below
        for (int i = 1; i < 4; ++i) {
          const int slot = ring_slot(pos, -i * dil, halo);
          if (slot >= 0) {
            const float4 st = *reinterpret_cast<const float4*>(
                a.state + ((tok * halo + slot) * nb + br) * d + c);
            C = fma4(Elem<T>::load4(CW, (int64_t)i * d + c), st, C);
          }
        }
        if (a.update_state)
          *reinterpret_cast<float4*>(a.state + ((tok * halo + pos % halo) * nb + br) * d + c) = nrm;
      }
      float4 D = make_float4(fmaf(al, v.x, silu(C.x)), fmaf(al, v.y, silu(C.y)),
                             fmaf(al, v.z, silu(C.z)), fmaf(al, v.w, silu(C.w)));
      if (a.add_residual) {
        const float4 h = Elem<T>::load4(H, tok * a.h_tok_stride + br * a.h_branch_stride + c);
        D = make_float4(D.x + h.x, D.y + h.y, D.z + h.z, D.w + h.w);
      }
      Elem<T>::store4(OUT, (tok * nb + br) * d + c, D);
    }
  }
  advance_ring(a, tok, pos, 1);
}

// The same for d <= 4 * BS * ITEMS and NB branches, in registers: thread x of
// the BS owns the 4-column groups c = 4 * (x + BS * i), i < ITEMS.  Every load the token
// needs before its row reductions is issued up front (addresses past d are
// clamped to a valid column and their contribution dropped, so the code is
// branch-free and the loads go out together), V and h stay in registers for
// the outputs, and one block reduction separates the two memory round trips.
// KS > 0: exactly KS K slices, summed with every load issued up front;
// KS == 0: k_split slices in a loop.
template <typename T, int NB, int ITEMS, int KS, int BS>
__global__ __launch_bounds__(BS) void decode_finalize_reg_kernel(ConvArgs a,
                                                                  const float* __restrict__ split,
                                                                  int32_t k_split, int32_t dil) {
  constexpr int NQ = 3 * NB + 1;
  static_assert(BS % 64 == 0 && BS >= 64 * 2 && BS <= 1024, "whole waves, enough for NQ sums");
  constexpr int NW = BS / 64;
  __shared__ float s_red[NW][NQ];
  __shared__ float s_tot[NQ];
  const int64_t tok = blockIdx.x;  // T == 1: token = sequence
  const int d = a.d;
  const int64_t ntot = (int64_t)(NB + 1) * d;
  const int64_t sstride = (int64_t)a.B * ntot;
  const float* __restrict__ P = split + tok * ntot;
  const T* __restrict__ H = static_cast<const T*>(a.hidden);
  const T* __restrict__ GQ = static_cast<const T*>(a.gamma_q);
  const T* __restrict__ GK = static_cast<const T*>(a.gamma_k);
  const T* __restrict__ GU = static_cast<const T*>(a.gamma_u);
  const T* __restrict__ CW = static_cast<const T*>(a.conv_w);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  int col[ITEMS];
  bool ok[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int c = 4 * ((int)threadIdx.x + BS * i);
    ok[i] = c < d;
    col[i] = ok[i] ? c : d - 4;
  }
  // the partials are read once: streamed, so that they do not evict the
  // weights the next decode step's projection reads from L2
  auto ld_stream = [](const float* p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
  };
  auto splits = [&](int64_t off) {  // sum of the K slices, 4 columns, in slice order
    float4 x = ld_stream(P + off);
    if (KS > 0) {
#pragma unroll
      for (int s = 1; s < KS; ++s) x = add4(x, ld_stream(P + s * sstride + off));
    } else {
      for (int s = 1; s < k_split; ++s) x = add4(x, ld_stream(P + s * sstride + off));
    }
    return x;
  };
  // absent gains read the conv taps (always there) and are replaced by 1 as
  // 1 + (x - 1) * 0, so every load is unconditional and none sits behind a
  // branch (a select would let the compiler move the load under one)
  const bool has_gq = GQ != nullptr, has_gk = GK != nullptr, has_gu = GU != nullptr;
  auto gain = [](float4 x, bool on) {
    const float s = on ? 1.0f : 0.0f;
    return make_float4(fmaf(x.x - 1.0f, s, 1.0f), fmaf(x.y - 1.0f, s, 1.0f),
                       fmaf(x.z - 1.0f, s, 1.0f), fmaf(x.w - 1.0f, s, 1.0f));
  };
  const T* __restrict__ gq_p = has_gq ? GQ : CW;
  const T* __restrict__ gk_p = has_gk ? GK : CW;
  const T* __restrict__ gu_p = has_gu ? GU : CW;

  // the ring position first: the taps' addresses wait for it alone
  const int halo = 3 * dil;
  const int pos = a.state ? ring_pos(a.state_pos, tok, halo) : 0;
  float4 v[ITEMS], h[NB][ITEMS], k[NB][ITEMS], gq[ITEMS], gk[ITEMS], cw0[ITEMS], gu[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
#pragma unroll
    for (int br = 0; br < NB; ++br) {
      k[br][i] = splits((int64_t)br * d + col[i]);
      h[br][i] = Elem<T>::load4(H, tok * a.h_tok_stride + br * a.h_branch_stride + col[i]);
    }
    v[i] = splits((int64_t)NB * d + col[i]);
    gq[i] = Elem<T>::load4(gq_p, col[i]);
    gk[i] = Elem<T>::load4(gk_p, col[i]);
    cw0[i] = Elem<T>::load4(CW, col[i]);
    gu[i] = Elem<T>::load4(gu_p, col[i]);
  }
  // the ring's taps at positions -dil, -2 dil, -3 dil (dropped before the
  // sequence's start), loaded with the rest when they fit in registers; every
  // read of the ring precedes this call's write to it
  constexpr bool kPreTaps = NB * ITEMS <= 4;
  float4 tap[kPreTaps ? NB : 1][3][kPreTaps ? ITEMS : 1];
  float tw[3];
  int tslot[3];
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int sl = ring_slot(pos, -(t + 1) * dil, halo);
    tw[t] = sl >= 0 ? 1.0f : 0.0f;
    tslot[t] = sl >= 0 ? sl : 0;
  }
  if (kPreTaps && a.state) {
#pragma unroll
    for (int br = 0; br < (kPreTaps ? NB : 1); ++br)
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int i = 0; i < (kPreTaps ? ITEMS : 1); ++i)
          tap[br][t][i] = *reinterpret_cast<const float4*>(
              a.state + ((tok * halo + tslot[t]) * NB + br) * d + col[i]);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load above issued before the first wait
  float acc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] = 0.0f;
  float4 g[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    g[i] = mul4(gain(gq[i], has_gq), gain(gk[i], has_gk));
    const float m = ok[i] ? 1.0f : 0.0f;
    acc[3 * NB] += m * dot4(v[i], v[i]);
#pragma unroll
    for (int br = 0; br < NB; ++br) {
      acc[3 * br] += m * dot4(mul4(g[i], h[br][i]), k[br][i]);
      acc[3 * br + 1] += m * dot4(k[br][i], k[br][i]);
      acc[3 * br + 2] += m * dot4(h[br][i], h[br][i]);
    }
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc[q] += __shfl_xor(acc[q], off);
    if (lane == 0) s_red[wave][q] = acc[q];
  }
  __syncthreads();
  if (threadIdx.x < NQ) {
    float t = s_red[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < NW; ++w) t += s_red[w][threadIdx.x];
    s_tot[threadIdx.x] = t;
  }
  __syncthreads();

  const float fd = (float)d;
  T* __restrict__ OUT = static_cast<T*>(a.out);
  float4 gun[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) gun[i] = gain(gu[i], has_gu);
#pragma unroll
  for (int br = 0; br < NB; ++br) {
    RowSums r{s_tot[3 * br], s_tot[3 * br + 1], s_tot[3 * br + 2], s_tot[3 * NB]};
    float al, sc;
    gate_and_scale(r, fd, a.eps, al, sc);
    if (a.gates && threadIdx.x == 0) a.gates[tok * NB + br] = al;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const float4 nrm = mul4(mul4(gun[i], v[i]), f4(sc));  // this position's normalised row
      float4 C = mul4(cw0[i], nrm);
      if (a.state) {
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          const float4 st = kPreTaps ? tap[kPreTaps ? br : 0][t][kPreTaps ? i : 0]
                                     : *reinterpret_cast<const float4*>(
                                           a.state + ((tok * halo + tslot[t]) * NB + br) * d + col[i]);
          // a position before the sequence's start contributes zero, whatever
          // its slot holds (selected, not weighted: the slot may hold NaN)
          C = fma4(Elem<T>::load4(CW, (int64_t)(t + 1) * d + col[i]), tw[t] != 0.0f ? st : f4(0.0f),
                   C);
        }
        if (a.update_state && ok[i])
          *reinterpret_cast<float4*>(a.state + ((tok * halo + pos % halo) * NB + br) * d + col[i]) =
              nrm;
      }
      float4 D = make_float4(fmaf(al, v[i].x, silu(C.x)), fmaf(al, v[i].y, silu(C.y)),
                             fmaf(al, v[i].z, silu(C.z)), fmaf(al, v[i].w, silu(C.w)));
      if (a.add_residual) D = add4(D, h[br][i]);
      if (ok[i]) Elem<T>::store4(OUT, (tok * NB + br) * d + col[i], D);
    }
  }
  advance_ring(a, tok, pos, 1);
}

// Ring update after a conv over a [B, T] grid: the normalised rows of the last
// min(T, 3*DIL) positions of sequence blockIdx.x, every branch, into their
// slots, and the sequence's ring position advanced by T.  The scalars come
// from the same folds as the conv's (so the rows equal the ones the conv
// used): from V and the partials (FUSED) or from the U rows.
template <int DIL, typename T, bool FUSED>
__global__ __launch_bounds__(256) void state_update_kernel(ConvArgs a) {
  constexpr int HALO = 3 * DIL;
  __shared__ float s_scale[NGRAM_MAX_BRANCHES][HALO];
  const int64_t b = blockIdx.x;
  const int nb = a.nb, d = a.d;
  const int n = a.T < HALO ? a.T : HALO;  // rows written per branch
  const int q0 = a.T - n;                  // first position written
  const int64_t seq0 = b * a.T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int pos = ring_pos(a.state_pos, b, HALO);
  if (FUSED) {
    const int sub = lane & 15, grp = lane >> 4;
    for (int i0 = wave * 4; i0 < n * nb; i0 += nw * 4) {
      const int k = i0 + grp;             // (branch, row) pair k = br * n + i
      const int kk = k < n * nb ? k : 0;
      const int br = kk / n, i = kk - br * n;
      const int64_t tok = seq0 + q0 + i;
      const RowSums r = fold_partials16(a.parts + tok * (3 * nb + 1) * a.np, a.np, br, nb, sub);
      if (sub == 0 && k < n * nb) {
        float al, sc;
        gate_and_scale(r, (float)d, a.eps, al, sc);
        s_scale[br][i] = sc;
      }
    }
  } else {
    const T* U = static_cast<const T*>(a.u);
    for (int k = wave; k < n * nb; k += nw) {
      const int br = k / n, i = k - br * n;
      const float sc = inv_rms_row(U + ((seq0 + q0 + i) * nb + br) * d, d, a.eps, lane);
      if (lane == 0) s_scale[br][i] = sc;
    }
  }
  __syncthreads();
  const T* __restrict__ GU = static_cast<const T*>(a.gamma_u);
  for (int c0 = threadIdx.x * 4; c0 < d; c0 += blockDim.x * 4) {
    const float4 gu = GU ? Elem<T>::load4(GU, c0) : f4(1.0f);
    for (int br = 0; br < nb; ++br) {
      for (int i = 0; i < n; ++i) {
        const int64_t tok = seq0 + q0 + i;
        float4 src;
        if (FUSED) {
          src = *reinterpret_cast<const float4*>(a.v + tok * a.v_stride + c0);
        } else {
          src = Elem<T>::load4(static_cast<const T*>(a.u), (tok * nb + br) * d + c0);
        }
        const int slot = (pos + q0 + i) % HALO;
        *reinterpret_cast<float4*>(a.state + ((b * HALO + slot) * nb + br) * d + c0) =
            mul4(mul4(gu, src), f4(s_scale[br][i]));
      }
    }
  }
  advance_ring(a, b, pos, a.T);
}

template <typename T, bool FUSED>
hipError_t launch_conv_t(int32_t dil, const ConvArgs& a, hipStream_t s) {
  const int tiles = (a.T + a.tile - 1) / a.tile;
  const int64_t blocks = (int64_t)a.B * tiles * a.nb;  // (tile, branch) pairs, see conv_kernel
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  // Few tiles (fewer than 4 per CU): one 4-column group per thread, so each
  // tile brings more waves (engram_small's 512 tiles: 0.20 -> 0.12 ms).  Many
  // tiles: 256 threads, which keeps more tiles resident per CU (at Qwen
  // prefill's 4,096 tiles, larger blocks measured 25-35 % slower).
  int threads = 256;
  if (blocks < 4 * 256) {
    threads = (a.d / 4 + 63) / 64 * 64;
    if (threads > 512) threads = 512;
    if (threads < 256) threads = 256;
  }
  if (FUSED && a.add_residual) {
    switch (dil) {
      case 1: return launch(conv_kernel<1, T, FUSED, FUSED>, grid, threads, 0, s, a);
      case 2: return launch(conv_kernel<2, T, FUSED, FUSED>, grid, threads, 0, s, a);
      case 3: return launch(conv_kernel<3, T, FUSED, FUSED>, grid, threads, 0, s, a);
      case 4: return launch(conv_kernel<4, T, FUSED, FUSED>, grid, threads, 0, s, a);
      default: return hipErrorInvalidValue;
    }
  }
  switch (dil) {
    case 1: return launch(conv_kernel<1, T, FUSED, false>, grid, threads, 0, s, a);
    case 2: return launch(conv_kernel<2, T, FUSED, false>, grid, threads, 0, s, a);
    case 3: return launch(conv_kernel<3, T, FUSED, false>, grid, threads, 0, s, a);
    case 4: return launch(conv_kernel<4, T, FUSED, false>, grid, threads, 0, s, a);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int NB, int ITEMS, int BS>
hipError_t launch_finalize_reg_items(int32_t k_split, const float* split, const ConvArgs& a,
                                     hipStream_t s) {
  const unsigned g = (unsigned)a.B;
  switch (k_split) {
    case 1: return launch(decode_finalize_reg_kernel<T, NB, ITEMS, 1, BS>, g, BS, 0, s, a, split, k_split, a.dil);
    case 2: return launch(decode_finalize_reg_kernel<T, NB, ITEMS, 2, BS>, g, BS, 0, s, a, split, k_split, a.dil);
    case 4: return launch(decode_finalize_reg_kernel<T, NB, ITEMS, 4, BS>, g, BS, 0, s, a, split, k_split, a.dil);
    default: return launch(decode_finalize_reg_kernel<T, NB, ITEMS, 0, BS>, g, BS, 0, s, a, split, k_split, a.dil);
  }
}

// items 4-column groups per thread of a 256-thread block, or (wide) of a
// 320-thread block, which covers d = 1,280 * items with no clamped group
template <typename T, int NB>
hipError_t launch_finalize_reg_nb(int items, bool wide, int32_t k_split, const float* split,
                                  const ConvArgs& a, hipStream_t s) {
  if (wide) {
    switch (items) {
      case 1: return launch_finalize_reg_items<T, NB, 1, 320>(k_split, split, a, s);
      case 2: return launch_finalize_reg_items<T, NB, 2, 320>(k_split, split, a, s);
      case 3: return launch_finalize_reg_items<T, NB, 3, 320>(k_split, split, a, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (items) {
    case 1: return launch_finalize_reg_items<T, NB, 1, 256>(k_split, split, a, s);
    case 2: return launch_finalize_reg_items<T, NB, 2, 256>(k_split, split, a, s);
    case 3: return launch_finalize_reg_items<T, NB, 3, 256>(k_split, split, a, s);
    case 4: return launch_finalize_reg_items<T, NB, 4, 256>(k_split, split, a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_finalize_reg(int nb, int items, bool wide, int32_t k_split, const float* split,
                               const ConvArgs& a, hipStream_t s) {
  switch (nb) {
    case 1: return launch_finalize_reg_nb<T, 1>(items, wide, k_split, split, a, s);
    case 2: return launch_finalize_reg_nb<T, 2>(items, wide, k_split, split, a, s);
    case 3: return launch_finalize_reg_nb<T, 3>(items, wide, k_split, split, a, s);
    case 4: return launch_finalize_reg_nb<T, 4>(items, wide, k_split, split, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gate_values(int dtype, const ConvArgs& a, int64_t M, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (dtype == NGRAM_BF16) return launch(gate_values_kernel<bf16_bits>, (unsigned)M, 256, 0, s, a, M);
  return launch(gate_values_kernel<float>, (unsigned)M, 256, 0, s, a, M);
}

hipError_t launch_fused_conv(int dtype, int32_t dil, const ConvArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0) return hipSuccess;
  return dtype == NGRAM_BF16 ? launch_conv_t<bf16_bits, true>(dil, a, s)
                             : launch_conv_t<float, true>(dil, a, s);
}

hipError_t launch_op_conv(int dtype, int32_t dil, const ConvArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0) return hipSuccess;
  return dtype == NGRAM_BF16 ? launch_conv_t<bf16_bits, false>(dil, a, s)
                             : launch_conv_t<float, false>(dil, a, s);
}

hipError_t launch_decode_finalize(int dtype, int32_t k_split, const float* split, const ConvArgs& a,
                                  hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  int items = (a.d + 1023) / 1024;  // 4-column groups per thread of 256
  // one fewer group per thread on 320 threads when that still covers d (at
  // d = 2,560: two groups each instead of three, the third half clamped)
  const bool wide = items >= 2 && items <= 4 && a.d <= 1280 * (items - 1);
  if (wide) --items;
  if (items <= 4) {
    return dtype == NGRAM_BF16
               ? launch_finalize_reg<bf16_bits>(a.nb, items, wide, k_split, split, a, s)
               : launch_finalize_reg<float>(a.nb, items, wide, k_split, split, a, s);
  }
  if (dtype == NGRAM_BF16)
    return launch(decode_finalize_kernel<bf16_bits>, (unsigned)a.B, 256, 0, s, a, split, k_split,
                  a.dil);
  return launch(decode_finalize_kernel<float>, (unsigned)a.B, 256, 0, s, a, split, k_split, a.dil);
}

hipError_t launch_state_update(int dtype, bool fused, int32_t dil, const ConvArgs& a,
                               hipStream_t s) {
  if (a.B == 0 || a.T == 0 || a.state == nullptr || a.state_pos == nullptr) return hipSuccess;
  const dim3 grid((unsigned)a.B);
#define NGRAM_SU(D)                                                                         \
  if (dtype == NGRAM_BF16)                                                                  \
    return fused ? launch(state_update_kernel<D, bf16_bits, true>, grid, 256, 0, s, a)      \
                 : launch(state_update_kernel<D, bf16_bits, false>, grid, 256, 0, s, a);    \
  return fused ? launch(state_update_kernel<D, float, true>, grid, 256, 0, s, a)            \
               : launch(state_update_kernel<D, float, false>, grid, 256, 0, s, a)
  switch (dil) {
    case 1: NGRAM_SU(1);
    case 2: NGRAM_SU(2);
    case 3: NGRAM_SU(3);
    case 4: NGRAM_SU(4);
    default: return hipErrorInvalidValue;
  }
#undef NGRAM_SU
}

int conv_tile_for(int32_t T) { return T < kMaxTile ? T : kMaxTile; }

}  // namespace ngram
