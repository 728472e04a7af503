// Key / value projections with the gate's row reductions fused into the
// epilogue.  "Qwen3.8-Flash-Next 深度研究" §2.3 gives E_t -> K_t, V_t and
// g_t = Gate(Norm(Q_t), Norm(K_t)); Engram's third component ("Qwen 4用上
// DeepSeek的Engram", section "DeepSeek Engram 更复杂，Qwen 更精简") makes the
// hidden state the query and RMSNorms both sides.
//
// The only dense contraction of the layer, so it runs on the matrix cores:
// C[M, (nb+1)*d] = E[M, K] x [W_K^(0) | ... | W_K^(nb-1) | W_V], bf16 in, fp32
// accumulate, v_mfma_f32_32x32x16_bf16.  K never leaves the chip: for a key
// column tile the epilogue reduces, per token row, sum(gq*gk*h*k), sum(k^2)
// and sum(h^2) over the wave's columns and writes only those three partials;
// a value tile writes V in fp32 plus sum(v^2).  The gate needs full-row sums
// over d, which spans several workgroups, so the partials are combined by
// the next kernel.
//
// Tiling (gfx950, wave64): 256 threads = 2x2 waves, workgroup tile BM x BN,
// wave tile (BM/2) x (BN/2) of 32x32 MFMA blocks, K step 64.  Both operands
// are staged through LDS with double buffering (one barrier per K step):
// E rows are copied as 16-byte chunks; W ([K, d], n contiguous) is loaded as
// 8x8 blocks, transposed in registers and stored n-major so each lane reads
// its 8 consecutive k values with one 16-byte LDS load.  The LDS k pitch is
// padded by 16 bytes so the 32 rows read by a half-wave hit distinct banks.
#include "epilogue.h"

namespace ngram {
namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // bf16 elements per LDS row (144 bytes)

template <int BM, int BN>
struct Tile {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MI = WM / 32, NI = WN / 32;
  static constexpr int A_CHUNKS = BM * (BK / 8) / 256;
  static constexpr int B_THREADS = (BK / 8) * (BN / 8);
  static constexpr int LDS_A = BM * LDK, LDS_B = BN * LDK;
  static constexpr int LDS_BUF = LDS_A + LDS_B;
};

// A tile rows row0 + 32*i (clamped to the last valid row: values of rows
// past M are computed but never written), 16 bytes at element column kcol.
template <int N>
__device__ __forceinline__ void load_a_chunks(uint32_t (&ra)[N][4], const bf16_bits* __restrict__ E,
                                              int64_t row0, int64_t M, int K, int kcol) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    int64_t row = row0 + 32 * i;
    row = row < M ? row : M - 1;
    const uint4 v = *reinterpret_cast<const uint4*>(E + row * K + kcol);
    ra[i][0] = v.x;
    ra[i][1] = v.y;
    ra[i][2] = v.z;
    ra[i][3] = v.w;
  }
}

template <int N>
__device__ __forceinline__ void store_a_chunks(const uint32_t (&ra)[N][4], bf16_bits* As, int a_row,
                                               int a_chunk) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    *reinterpret_cast<uint4*>(As + (a_row + 32 * i) * LDK + a_chunk * 8) =
        make_uint4(ra[i][0], ra[i][1], ra[i][2], ra[i][3]);
}

// 8 consecutive k rows of W, 8 columns each (zeros past the last column).
__device__ __forceinline__ void load_b_block(uint32_t (&rb)[8][4], const bf16_bits* __restrict__ src,
                                             int d, bool active, bool valid) {
  if (!active) return;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (valid) v = *reinterpret_cast<const uint4*>(src + (int64_t)r * d);
    rb[r][0] = v.x;
    rb[r][1] = v.y;
    rb[r][2] = v.z;
    rb[r][3] = v.w;
  }
}

// Transpose the 8x8 block in registers: rb[r][q] holds columns (2q, 2q+1)
// of k row r; LDS row n = 8*b_nb + c receives k = 8*b_kb .. +7 of column c.
__device__ __forceinline__ void store_b_block(const uint32_t (&rb)[8][4], bf16_bits* Bs, int b_nb,
                                              int b_kb) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int q = c >> 1;
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t x0 = rb[2 * p][q];
      const uint32_t x1 = rb[2 * p + 1][q];
      w[p] = (c & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (x1 << 16));
    }
    *reinterpret_cast<uint4*>(Bs + (b_nb * 8 + c) * LDK + b_kb * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int BM, int BN>
__global__ __launch_bounds__(256, 1) void proj_bf16_kernel(ProjArgs a, int tiles_m, int tiles_n) {
  using TL = Tile<BM, BN>;
  __shared__ __attribute__((aligned(16))) bf16_bits lds[2 * TL::LDS_BUF];

  const int n_seg = a.nb + 1;
  const int per_m = n_seg * tiles_n;
  const int bid = blockIdx.x;
  const int m_tile = bid / per_m;
  const int rem = bid - m_tile * per_m;
  const int seg = rem / tiles_n;
  const int n_tile = rem - seg * tiles_n;
  (void)tiles_m;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)m_tile * BM;
  const int n0 = n_tile * BN;
  const int K = a.K, d = a.d;
  const int64_t M = a.M;

  const bf16_bits* __restrict__ E = static_cast<const bf16_bits*>(a.e);
  const bf16_bits* __restrict__ W =
      seg < a.nb ? static_cast<const bf16_bits*>(a.wk) + (int64_t)seg * K * d
                 : static_cast<const bf16_bits*>(a.wv);

  // global -> register assignment: A as 16-byte chunks (8 lanes per 128-byte
  // row), W as one 8x8 block per thread (8 lanes cover 8 rows x 128 bytes).
  const int a_row = tid >> 3, a_chunk = tid & 7;
  const bool b_active = tid < TL::B_THREADS;
  const int b_kb = tid & 7, b_nb = tid >> 3;
  const int b_col = n0 + b_nb * 8;
  const bool b_valid = b_active && b_col < d;
  const bf16_bits* b_src = W + (int64_t)(b_kb * 8) * d + (b_valid ? b_col : 0);

  uint32_t ra[TL::A_CHUNKS][4];
  uint32_t rb[8][4];
  load_a_chunks<TL::A_CHUNKS>(ra, E, m0 + a_row, M, K, a_chunk * 8);
  load_b_block(rb, b_src, d, b_active, b_valid);
  store_a_chunks<TL::A_CHUNKS>(ra, lds, a_row, a_chunk);
  if (b_active) store_b_block(rb, lds + TL::LDS_A, b_nb, b_kb);
  __syncthreads();

  floatx16 acc[TL::MI][TL::NI];
#pragma unroll
  for (int mi = 0; mi < TL::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < TL::NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  const int nk = K / BK;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      load_a_chunks<TL::A_CHUNKS>(ra, E, m0 + a_row, M, K, (kt + 1) * BK + a_chunk * 8);
      load_b_block(rb, b_src + (int64_t)(kt + 1) * BK * d, d, b_active, b_valid);
    }
    const bf16_bits* As = lds + buf * TL::LDS_BUF;
    const bf16_bits* Bs = As + TL::LDS_A;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[TL::MI], bfr[TL::NI];
      const int koff = kk * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int mi = 0; mi < TL::MI; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8*>(As + (wm * TL::WM + mi * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
      for (int ni = 0; ni < TL::NI; ++ni)
        bfr[ni] = *reinterpret_cast<const bf16x8*>(Bs + (wn * TL::WN + ni * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
      for (int mi = 0; mi < TL::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < TL::NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      bf16_bits* nxt = lds + (buf ^ 1) * TL::LDS_BUF;
      store_a_chunks<TL::A_CHUNKS>(ra, nxt, a_row, a_chunk);
      if (b_active) store_b_block(rb, nxt + TL::LDS_A, b_nb, b_kb);
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  const int wcol0 = n0 + wn * TL::WN;  // first column of this wave
  if (wcol0 >= d) return;
  EpiArgs ea;
  ea.hidden = static_cast<const bf16_bits*>(a.hidden);
  ea.h_tok_stride = a.h_tok_stride;
  ea.h_branch_stride = a.h_branch_stride;
  ea.gamma_q = static_cast<const bf16_bits*>(a.gamma_q);
  ea.gamma_k = static_cast<const bf16_bits*>(a.gamma_k);
  ea.v = a.v;
  ea.parts = a.parts;
  ea.M = M;
  ea.d = d;
  ea.nb = a.nb;
  ea.np = a.np;
  ea.v_ld = d;
  ea.k_keep = nullptr;
  gate_epilogue<TL::MI, TL::NI>(acc, ea, seg, m0 + wm * TL::WM, wcol0, wcol0 / TL::WN, lane);
}

// ---------------------------------------------------------------------------
// fp32 storage (small configurations): plain LDS-tiled FMA GEMM writing K and
// V in full, then a row-reduction kernel producing one partial per row.
// ---------------------------------------------------------------------------
constexpr int FT = 16;

__global__ __launch_bounds__(256) void proj_f32_kernel(ProjArgs a) {
  __shared__ float As[FT][FT + 1];
  __shared__ float Bs[FT][FT + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int n_seg = a.nb + 1;
  const int64_t row = (int64_t)blockIdx.y * FT + ty;
  const int seg = blockIdx.z;
  const int col = blockIdx.x * FT + tx;
  const float* E = static_cast<const float*>(a.e);
  const float* W = seg < a.nb ? static_cast<const float*>(a.wk) + (int64_t)seg * a.K * a.d
                              : static_cast<const float*>(a.wv);
  // W[k][col] is at k*d + col ([K, d]) or col*K + k ([d, K])
  const int64_t sk = a.w_dk ? 1 : a.d, sc = a.w_dk ? a.K : 1;
  float acc = 0.0f;
  for (int k0 = 0; k0 < a.K; k0 += FT) {
    const int64_t arow = (int64_t)blockIdx.y * FT + ty;
    As[ty][tx] = (arow < a.M && k0 + tx < a.K) ? E[arow * a.K + k0 + tx] : 0.0f;
    Bs[ty][tx] = (k0 + ty < a.K && col < a.d) ? W[(int64_t)(k0 + ty) * sk + col * sc] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FT; ++k) acc = fmaf(As[ty][k], Bs[k][tx], acc);
    __syncthreads();
  }
  if (row < a.M && col < a.d) a.v[(row * n_seg + seg) * a.d + col] = acc;
}

__global__ __launch_bounds__(256) void partials_f32_kernel(ProjArgs a) {
  // one wave per (row, segment)
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n_seg = a.nb + 1;
  if (item >= a.M * n_seg) return;
  const int64_t row = item / n_seg;
  const int seg = (int)(item - row * n_seg);
  const float* x = a.v + (row * n_seg + seg) * a.d;
  const float* H = static_cast<const float*>(a.hidden);
  const float* GQ = static_cast<const float*>(a.gamma_q);
  const float* GK = static_cast<const float*>(a.gamma_k);
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f;
  for (int c = lane; c < a.d; c += 64) {
    const float k = x[c];
    if (seg < a.nb) {
      const float h = H[row * a.h_tok_stride + seg * a.h_branch_stride + c];
      const float g = (GQ ? GQ[c] : 1.0f) * (GK ? GK[c] : 1.0f);
      s0 += g * h * k;
      s1 += k * k;
      s2 += h * h;
    } else {
      s0 += k * k;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    s0 += __shfl_xor(s0, off);
    s1 += __shfl_xor(s1, off);
    s2 += __shfl_xor(s2, off);
  }
  if (lane == 0) {
    const int nq = 3 * a.nb + 1;
    float* p = a.parts + row * nq;  // np == 1
    if (seg < a.nb) {
      p[3 * seg] = s0;
      p[3 * seg + 1] = s1;
      p[3 * seg + 2] = s2;
    } else {
      p[3 * a.nb] = s0;
    }
  }
}

template <int BM, int BN>
hipError_t launch_bf16(const ProjArgs& a, hipStream_t s) {
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  const int tiles_n = (a.d + BN - 1) / BN;
  const int64_t blocks = (int64_t)tiles_m * (a.nb + 1) * tiles_n;
  return launch(proj_bf16_kernel<BM, BN>, (unsigned)blocks, 256, 0, s, a, tiles_m, tiles_n);
}

}  // namespace

ProjPlan plan_projection(int dtype, int64_t M, int32_t d) {
  ProjPlan p;
  if (dtype != NGRAM_BF16) {
    p.bm = FT;
    p.bn = FT;
    p.np = 1;
    return p;
  }
  if (M >= 1024) {
    p.bm = 128;
    p.bn = 128;
  } else {
    p.bm = 64;
    p.bn = 64;
  }
  const int wn = p.bn / 2;
  p.np = (d + wn - 1) / wn;
  return p;
}

hipError_t launch_projection(int dtype, const ProjPlan& plan, const ProjArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (dtype != NGRAM_BF16) {
    dim3 grid((a.d + FT - 1) / FT, (unsigned)((a.M + FT - 1) / FT), a.nb + 1);
    const hipError_t e = launch(proj_f32_kernel, grid, 256, 0, s, a);
    if (e != hipSuccess) return e;
    const int64_t items = a.M * (a.nb + 1);
    return launch(partials_f32_kernel, (unsigned)((items + 3) / 4), 256, 0, s, a);
  }
  if (plan.bm == 128) return launch_bf16<128, 128>(a, s);
  return launch_bf16<64, 64>(a, s);
}

}  // namespace ngram
