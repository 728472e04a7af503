// Key / value projections, bf16 MFMA, operands streamed straight from global
// memory into LDS -- the fast path for W stored [d, mem] (NGRAM_W_D_MEM).
//
// Same contract as project.hip ("Qwen3.8-Flash-Next 深度研究" §2.3:
// E_t -> K_t, V_t, then g_t from RMSNorm'd query and key; Engram's third
// component in "Qwen 4用上DeepSeek的Engram"): C = E [W_K^(0) .. W_K^(nb-1) W_V]^T
// with the gate's row partials in the epilogue, K never written.  With W
// stored [d, mem] both operands are contiguous along the reduction axis, so
// every 16-byte chunk is copied global -> LDS by global_load_lds_dwordx4
// (no register staging, no transposes) and a STAGES-deep ring of LDS buffers
// keeps up to STAGES-1 K steps of copies in flight while the matrix cores
// work on the current one.
//
// The A operand is the memory vector E, materialised by the gather kernel.
// A variant that hashed and gathered its own A operand straight from the
// tables (E never written) measured slower at every prefill size: the
// gathered copies lengthen the ring's load latency by more than the E round
// trip costs.
//
// Each ring slot is its own __shared__ array and the K loop is unrolled by
// the ring depth, so every copy and every operand read names its slot at
// compile time: the compiler's wait-count insertion then sees that a read of
// slot s does not depend on copies still in flight into the other slots and
// keeps only the explicit partial vmcnt waits below (with one shared array it
// would drain all copies before every LDS read, serialising the ring).
//
// LDS layout per stage: A [BM][BK], B [BN][BK] bf16, rows of BK*2 bytes whose
// 16-byte chunks are XOR-swizzled by row (chunk ^ f(row)); a copy writes the
// lanes' chunks contiguously, so the swizzle is applied to the source address,
// and the MFMA operand reads hit distinct banks: a 16-byte-per-lane LDS read
// is served 16 lanes (256 bytes, all 64 banks) at a time, and those 16 lanes
// read rows r..r+15 of one logical chunk.  Tile order is XCD-aware: workgroup b runs on XCD b % 8, so each XCD
// gets a contiguous range of tiles, walked in groups of group_m M-tiles with
// the M index fastest -- concurrently running workgroups of one XCD share A
// and B slabs in its L2.
#include "epilogue.h"

namespace ngram {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt: at most N vector-memory ops outstanding, all LDS ops done
// (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4]<<14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Workgroup barrier that leaves global->LDS copies of later stages in flight
// (__syncthreads() would drain vmcnt); the memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void barrier_keep_copies() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ void copy16_to_lds(const void* src, bf16_bits* wave_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)wave_dst, 16, 0, 0);
}

template <int BK>
__device__ __forceinline__ int swz(int row);
// 64-wide K: 128-byte rows, two per 256-byte bank window, so the 16 rows of
// one read pass must spread over 8 chunk slots per row parity: the low three
// row bits, flipped by row bit 3, do that.
template <>
__device__ __forceinline__ int swz<64>(int row) {
  return (row & 7) ^ ((row >> 3) & 1);
}
// 32-wide K: four 64-byte rows per bank window.
template <>
__device__ __forceinline__ int swz<32>(int row) {
  return (row >> 2) & 3;
}

// Part of swz(rblk + lrow) that depends on the copy's first row rblk (a
// multiple of the 64 / (BK / 8) rows one wave-wide copy covers).
template <int BK>
__device__ __forceinline__ int swz_block(int rblk) {
  return BK == 64 ? (rblk >> 3) & 1 : 0;
}

__device__ __forceinline__ void map_tile(int bid, int tiles_m, int n_seg, int tiles_n, int gm,
                                         int& m, int& seg, int& n) {
  const int total = tiles_m * n_seg * tiles_n;
  int logical = bid;
  if ((total & 7) == 0) logical = (bid & 7) * (total >> 3) + (bid >> 3);
  const int per_m = n_seg * tiles_n;
  const int group = logical / (gm * per_m);
  const int first_m = group * gm;
  const int gsize = min(gm, tiles_m - first_m);
  const int idx = logical - group * gm * per_m;
  m = first_m + idx % gsize;
  const int sn = idx / gsize;
  seg = sn / tiles_n;
  n = sn - seg * tiles_n;
}

// MF: the MFMA shape, v_mfma_f32_32x32x16_bf16 (32) or v_mfma_f32_16x16x32_bf16
// (16).  Both read their operands as 16 lanes x 16 bytes of 16 consecutive
// rows per pass, so the ring, the copies and the swizzle are the same.
template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, bool RAW = false, int MF = 32>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void proj_async_kernel(AsyncProjArgs a) {
  constexpr int NW = WGM * WGN;          // waves per workgroup
  constexpr int CH = BK / 8;            // 16-byte chunks per LDS row
  constexpr int RPI = 64 / CH;          // rows covered by one wave-wide copy
  constexpr int A_INS = BM / (RPI * NW);  // copies per wave per stage
  constexpr int B_INS = BN / (RPI * NW);
  constexpr int PER_STAGE = A_INS + B_INS;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MI = WTM / MF, NI = WTN / MF;
  constexpr int AR = MF == 32 ? 16 : 4;   // accumulator registers per MFMA block
  typedef std::conditional_t<MF == 32, floatx16, floatx4> acc_t;
  constexpr int A_ELEMS = BM * BK;
  constexpr int STAGE_ELEMS = (BM + BN) * BK;
  static_assert(A_INS * RPI * NW == BM && B_INS * RPI * NW == BN, "tile / copy shape");
  static_assert(MI * MF == WTM && NI * MF == WTN, "wave tile");
  static_assert(MF == 32 || (MF == 16 && BK % 32 == 0 && NI % 2 == 0), "MFMA shape");
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");

  __shared__ __attribute__((aligned(16))) bf16_bits ring0[STAGE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_bits ring1[STAGE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_bits ring2[STAGES > 2 ? STAGE_ELEMS : 8];
  __shared__ __attribute__((aligned(16))) bf16_bits ring3[STAGES > 3 ? STAGE_ELEMS : 8];
  // slot index is a compile-time constant at every use (unrolled loops)
  auto slot = [&](int sl) -> bf16_bits* {
    // (the placeholder arrays of absent slots stay unreferenced)
    if (STAGES > 3 && sl == 3) return ring3;
    if (STAGES > 2 && sl == 2) return ring2;
    return sl == 1 ? ring1 : ring0;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const EpiArgs& ep = a.epi;
  const int n_seg = ep.nb + 1;
  // RAW split-K: blocks [s * tiles, (s + 1) * tiles) take K split s
  const int split = RAW && a.raw_split > 1 ? a.raw_split : 1;
  const int tiles = a.tiles_m * n_seg * a.tiles_n;
  const int ksl = split > 1 ? (int)blockIdx.x / tiles : 0;
  const int bid = split > 1 ? (int)blockIdx.x - ksl * tiles : (int)blockIdx.x;
  int m_tile, seg, n_tile;
  map_tile(bid, a.tiles_m, n_seg, a.tiles_n, a.group_m, m_tile, seg, n_tile);
  const int64_t M = ep.M;
  const int64_t m0 = (int64_t)m_tile * BM;
  const int n0 = n_tile * BN;
  const int K = a.K, d = ep.d;
  const bf16_bits* __restrict__ W = seg < ep.nb ? a.wk + (int64_t)seg * d * K : a.wv;

  const int kt_first = split > 1 ? ksl * (K / BK) / split : 0;

  // Copy lanes: lane -> (row lrow of the copy's RPI-row block, 16-byte chunk
  // pch of the LDS row).  A block starts at a multiple of RPI rows, so the
  // row's swizzle is that of lrow, XOR the block's part (swz_block).
  const int lrow = lane / CH, pch = lane - (lane / CH) * CH;
  const int lch8 = (pch ^ swz<BK>(lrow)) * 8;  // element offset of the fetched chunk
  // Operand-read lanes: LDS byte offset of this lane's A and B rows for
  // mi = ni = 0; the other blocks are +MF rows (immediate offsets), and the
  // swizzle of all of them equals that of the lane's row (rows differ by
  // multiples of 16, which leaves row bits 0..3 alone).
  const int frow = lane & (MF - 1);
  const uint32_t a_row_b = (uint32_t)((wm * WTM + frow) * BK * 2);
  const uint32_t b_row_b = (uint32_t)((wn * WTN + frow) * BK * 2);
  const int fsw = swz<BK>(frow);

  // Copy K step kt into ring slot sl: A rows then B rows, one 16-byte chunk
  // per lane, RPI rows per wave-wide copy.
  auto issue = [&](int kt, int sl) {
    bf16_bits* As = slot(sl);
    bf16_bits* Bs = As + A_ELEMS;
    const int k0 = (kt_first + kt) * BK;
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int rblk = (wave * A_INS + i) * RPI;
      const int ch8 = lch8 ^ (swz_block<BK>(rblk) << 3);
      int64_t grow = m0 + rblk + lrow;
      if (grow > M - 1) grow = M - 1;
      copy16_to_lds(a.e + grow * K + k0 + ch8, As + rblk * BK);
    }
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
      const int rblk = (wave * B_INS + i) * RPI;
      const int ch8 = lch8 ^ (swz_block<BK>(rblk) << 3);
      int n = n0 + rblk + lrow;
      if (n > d - 1) n = d - 1;  // columns past d are computed, never stored
      copy16_to_lds(W + (uint32_t)(n * K + k0 + ch8), Bs + rblk * BK);
    }
  };

  acc_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < AR; ++r) acc[mi][ni][r] = 0.0f;

  // MFMAs over the K step held in ring slot sl: BK / (512 / MF) sub-steps,
  // lane l reading row l % MF of each block and the 16-byte chunk
  // l / MF of the sub-step (MF = 32: 2 chunks of 16 K; 16: 4 chunks of 32 K)
  auto compute = [&](int sl) {
    const char* As = reinterpret_cast<const char*>(slot(sl));
    const char* Bs = As + A_ELEMS * 2;
    constexpr int CPS = 64 / MF;  // chunks per sub-step
#pragma unroll
    for (int kk = 0; kk < BK / (8 * CPS); ++kk) {
      const uint32_t co = (uint32_t)(((kk * CPS + lane / MF) ^ fsw) * 16);
      bf16x8 af[MI], bfr[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8*>(As + a_row_b + co + mi * MF * BK * 2);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        bfr[ni] = *reinterpret_cast<const bf16x8*>(Bs + b_row_b + co + ni * MF * BK * 2);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          if constexpr (MF == 32)
            acc[mi][ni] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
          else
            acc[mi][ni] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
        }
    }
  };

  // this block's K steps: [kt_first, kt_first + nk) of K / BK
  const int nk = split > 1 ? (ksl + 1) * (K / BK) / split - kt_first : K / BK;
  // The last slot first receives a throw-away copy of step 0 (overwritten
  // before it is read), so that on entry to the loop every slot has one copy
  // outstanding in the same order as at the loop's back edge; the compiler's
  // wait-count state then merges exactly at the loop header instead of
  // falling back to draining every copy before the first read.
  issue(0, STAGES - 1);
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < nk) issue(st, st);

  for (int base = 0; base < nk; base += STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) {
      const int kt = base + u;
      if (kt < nk) {
        // this wave's copies of step kt have landed; later steps may be in flight
        if (kt + STAGES - 2 < nk)
          wait_vmcnt<(STAGES - 2) * PER_STAGE>();
        else
          wait_vmcnt<0>();
        barrier_keep_copies();  // ... and every other wave's; slot of step kt-1 is free
        if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (u + STAGES - 1) % STAGES);
        compute(u);
      }
    }
  }

  // Key tiles: the tile's query rows [m0, m0 + BM) x [n0, n0 + BN) go to LDS
  // (the ring is free now) with one 16-byte copy per lane, so the epilogue
  // reads them there instead of with one 2-byte global load per element.
  // Rows are split over the ring slots, RPS rows per slot.
  constexpr int RPS = (BM + BN) * BK / BN;      // query rows per ring slot
  constexpr int HCH = BN / 8;                   // 16-byte chunks per query row
  constexpr int HRPI = 64 / HCH;                // rows per wave-wide copy
  constexpr int HINS = BM / HRPI / NW;          // copies per wave
  constexpr bool HSTAGE = !RAW && HCH <= 64 && HRPI * HCH == 64 && RPS % 32 == 0 &&
                          RPS % HRPI == 0 && (BM + RPS - 1) / RPS <= STAGES &&
                          HINS * HRPI * NW == BM;
  if (HSTAGE && seg < ep.nb) {
    __syncthreads();  // every wave is done reading the ring
    const bf16_bits* __restrict__ Hs = ep.hidden + seg * ep.h_branch_stride;
    const int hr = lane / HCH;
    int hc = n0 + (lane - hr * HCH) * 8;
    if (hc > d - 8) hc = d - 8;                 // columns past d: never read
#pragma unroll
    for (int i = 0; i < HINS; ++i) {
      const int r0 = (wave * HINS + i) * HRPI;  // first row of the copy
      int64_t grow = m0 + r0 + hr;
      if (grow > M - 1) grow = M - 1;           // rows past M: never read
      copy16_to_lds(Hs + grow * ep.h_tok_stride + hc, slot(r0 / RPS) + (r0 % RPS) * BN);
    }
    wait_vmcnt<0>();
    __syncthreads();
  }

  const int wcol0 = n0 + wn * WTN;
  if (wcol0 >= d) return;
  if constexpr (RAW) {
    // plain product in fp32: a half-wave stores 32 consecutive columns (128
    // bytes) of one row per register, streamed (the products are larger than
    // the caches and read by a later kernel)
    float* __restrict__ C = a.raw_out + ksl * a.raw_split_stride + (int64_t)seg * d;
    if constexpr (MF == 32) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int col = wcol0 + ni * 32 + (lane & 31);
          if (col < d) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int64_t row = m0 + wm * WTM + mi * 32 + acc_row(r, lane);
              if (row < M) __builtin_nontemporal_store(acc[mi][ni][r], &C[row * a.raw_ld + col]);
            }
          }
        }
    } else {
      // 16x16 blocks in column pairs, quarter-waves 2p and 2p + 1 swapping
      // halves, so that each store writes 128 contiguous bytes of two rows
      // (as the value epilogue of gate_epilogue16 does)
      const bool qodd = (lane >> 4) & 1;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ni += 2) {
          const int cs = wcol0 + ni * 16 + (lane & 15) + (qodd ? 16 : 0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x0 = acc[mi][ni][j], x1 = acc[mi][ni + 1][j];
            const float got = __shfl_xor(qodd ? x0 : x1, 16);
            const int64_t re = m0 + wm * WTM + mi * 16 + 4 * ((lane >> 4) & ~1) + j;
            if (cs < d) {
              if (re < M) __builtin_nontemporal_store(qodd ? got : x0, &C[re * a.raw_ld + cs]);
              if (re + 4 < M)
                __builtin_nontemporal_store(qodd ? x1 : got, &C[(re + 4) * a.raw_ld + cs]);
            }
          }
        }
    }
  } else {
    auto staged = [&](int64_t row, int col) {
      const int rl = (int)(row - m0), cl = col - n0;
      return bf16_to_f32(slot(rl / RPS)[(rl % RPS) * BN + cl]);
    };
    if constexpr (MF == 32) {
      if (HSTAGE)
        gate_epilogue<MI, NI>(acc, ep, seg, m0 + wm * WTM, wcol0, wcol0 / WTN, lane, staged);
      else
        gate_epilogue<MI, NI>(acc, ep, seg, m0 + wm * WTM, wcol0, wcol0 / WTN, lane);
    } else {
      if (HSTAGE)
        gate_epilogue16<MI, NI>(acc, ep, seg, m0 + wm * WTM, wcol0, wcol0 / WTN, lane, staged);
      else
        gate_epilogue16<MI, NI>(acc, ep, seg, m0 + wm * WTM, wcol0, wcol0 / WTN, lane);
    }
  }
}

// The raw product with both operands stored K-outer ("TN"): C[M, N] =
// A^T B over K, A [K][M] (row stride tn_lda) and B [K][N] (row stride
// tn_ldb), both bf16 -- the backward's dW = [dK dV]^T E, whose operands are
// row-per-token, without transposing them first.  The tiles are copied
// global -> LDS as they lie (a K row of the tile is BM contiguous elements,
// its 16-byte chunks XOR-swizzled by (row & 3) << 2), and the MFMA operands,
// which hold 8 consecutive K per lane, come out of LDS through gfx950's
// transposing read ds_read_b64_tr_b16: within a group of 16 lanes, lane j
// names 4 elements of K row j / 4; lane i receives element i % 4 of rows
// 4r + i / 4's lane, r = 0..3 -- so lanes naming rows k0..k0+3 at columns
// c + 4 (j % 4) hand lane i the 4 K values of column c + i.  A 16-lane group
// thus reads a 4 x 16 block; two reads give an operand's 8 K values.  The
// swizzle puts the 4 rows x 64 bytes that lanes 0-31 read on distinct banks.
// Rows of K past the product's K are the caller's zeros; columns past M or N
// are clamped to the last chunk, computed and never stored.
template <int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void proj_raw_tn_kernel(AsyncProjArgs a) {
  constexpr int BM = 256, BN = 256, BK = 64, STAGES = 2;
  constexpr int NW = WGM * WGN;
  constexpr int RPC = 2;                    // K rows per wave-wide copy (512-byte rows)
  constexpr int A_INS = BK / (RPC * NW);    // copies per wave per stage and operand
  constexpr int PER_STAGE = 2 * A_INS;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  constexpr int A_ELEMS = BK * BM;
  constexpr int STAGE_ELEMS = BK * (BM + BN);
  static_assert(A_INS * RPC * NW == BK, "copy shape");
  static_assert(MI * 32 == WTM && NI * 32 == WTN, "wave tile");

  __shared__ __attribute__((aligned(16))) bf16_bits ring0[STAGE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_bits ring1[STAGE_ELEMS];
  auto slot = [&](int sl) -> bf16_bits* { return sl ? ring1 : ring0; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int split = a.raw_split > 1 ? a.raw_split : 1;
  const int tiles = a.tiles_m * a.tiles_n;
  const int ksl = split > 1 ? (int)blockIdx.x / tiles : 0;
  const int bid = split > 1 ? (int)blockIdx.x - ksl * tiles : (int)blockIdx.x;
  int m_tile, seg, n_tile;
  map_tile(bid, a.tiles_m, 1, a.tiles_n, a.group_m, m_tile, seg, n_tile);
  const int64_t M = a.epi.M;
  const int N = a.epi.d;
  const int m0 = m_tile * BM, n0 = n_tile * BN;
  const int K = a.K;
  const int kt_first = split > 1 ? ksl * (K / BK) / split : 0;
  const int nk = split > 1 ? (ksl + 1) * (K / BK) / split - kt_first : K / BK;

  // copy lanes: K row 2 i + lane / 32 of the copy, physical chunk lane % 32
  // holding logical chunk (lane % 32) ^ ((row & 3) << 2); the copy's first
  // row is even, so row & 3 = 2 (i & 1) + lane / 32
  const int cpc = lane & 31, crow = lane >> 5;
  auto issue = [&](int kt, int sl) {
    bf16_bits* As = slot(sl);
    bf16_bits* Bs = As + A_ELEMS;
    const int64_t k0 = (int64_t)(kt_first + kt) * BK;
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int r = (wave * A_INS + i) * RPC + crow;  // K row within the tile
      const int lch = cpc ^ ((r & 3) << 2);
      int ma = m0 + lch * 8;
      if (ma > M - 8) ma = (int)M - 8;
      int nb_ = n0 + lch * 8;
      if (nb_ > N - 8) nb_ = N - 8;
      copy16_to_lds(a.e + (k0 + r) * a.tn_lda + ma, As + (wave * A_INS + i) * RPC * BM);
      copy16_to_lds(a.wv + (k0 + r) * a.tn_ldb + nb_, Bs + (wave * A_INS + i) * RPC * BN);
    }
  };

  floatx16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  // operand lanes: group g = lane / 16 takes columns 16 (g & 1) + 4 (j & 3)
  // of a 32-column block and K rows 8 (g >> 1) + j / 4 (+4 for the second
  // read) of a 16-wide K step; row & 3 = j / 4 for every read, so the
  // swizzle is fixed per lane
  const int j = lane & 15, g = lane >> 4, q = j >> 2;
  const uint32_t lane_row_b = (uint32_t)((8 * (g >> 1) + q) * (BM * 2));  // BM == BN
  const int lane_cin = 2 * (g & 1) + ((j & 3) >> 1);   // chunk within a 32-column block
  const uint32_t lane_half_b = (uint32_t)(8 * (j & 1));
  auto frag_off = [&](int blk32) -> uint32_t {          // byte offset within a K row
    return (uint32_t)((((blk32 ^ q) << 2) | lane_cin) * 16) + lane_half_b;
  };
  uint32_t a_off[MI], b_off[NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) a_off[mi] = frag_off((wm * WTM) / 32 + mi);
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) b_off[ni] = frag_off((wn * WTN) / 32 + ni);

  typedef short s4v __attribute__((ext_vector_type(4)));
  typedef short s8v __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) s4v lds_s4v;
  auto tr8 = [&](const char* base, uint32_t off) -> bf16x8 {
    const lds_s4v* p0 = (const lds_s4v*)(const __attribute__((address_space(3))) char*)(base + off);
    const lds_s4v* p1 = (const lds_s4v*)(const __attribute__((address_space(3))) char*)(
        base + off + 4 * BM * 2);
    const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)p0);
    const s4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)p1);
    const s8v x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, x);
  };
  auto compute = [&](int sl) {
    const char* As = reinterpret_cast<const char*>(slot(sl));
    const char* Bs = As + A_ELEMS * 2;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const uint32_t rb = lane_row_b + (uint32_t)(kk * 16 * BM * 2);
      bf16x8 af[MI], bfr[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) af[mi] = tr8(As, rb + a_off[mi]);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) bfr[ni] = tr8(Bs, rb + b_off[ni]);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
  };

  // the same two-slot ring as proj_async_kernel (its loop-header argument
  // applies unchanged)
  issue(0, 1);
  if (nk > 0) issue(0, 0);
  for (int base = 0; base < nk; base += STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) {
      const int kt = base + u;
      if (kt < nk) {
        if (kt + STAGES - 2 < nk)
          wait_vmcnt<(STAGES - 2) * PER_STAGE>();
        else
          wait_vmcnt<0>();
        barrier_keep_copies();
        if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (u + STAGES - 1) % STAGES);
        compute(u);
      }
    }
  }

  // fp32 out, as the raw epilogue of proj_async_kernel
  const int wcol0 = n0 + wn * WTN;
  if (wcol0 >= N) return;
  float* __restrict__ C = a.raw_out + ksl * a.raw_split_stride;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int col = wcol0 + ni * 32 + (lane & 31);
      if (col < N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * WTM + mi * 32 + acc_row(r, lane);
          if (row < M) __builtin_nontemporal_store(acc[mi][ni][r], &C[row * a.raw_ld + col]);
        }
      }
    }
}

template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, int MF = 32>
hipError_t launch_raw_t(const AsyncProjArgs& a0, hipStream_t s) {
  AsyncProjArgs a = a0;
  if (a.raw_out == nullptr || a.K % BK != 0) return hipErrorInvalidValue;
  a.tiles_m = (int)((a.epi.M + BM - 1) / BM);
  a.tiles_n = (a.epi.d + BN - 1) / BN;
  const int split = a.raw_split > 1 ? a.raw_split : 1;
  if (split > a.K / BK) return hipErrorInvalidValue;  // every split needs a K step
  const int64_t blocks = (int64_t)a.tiles_m * (a.epi.nb + 1) * a.tiles_n * split;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  return launch(proj_async_kernel<BM, BN, BK, STAGES, WGM, WGN, true, MF>, (unsigned)blocks,
                64 * WGM * WGN, 0, s, a);
}

template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, int MF>
hipError_t launch_async_t(const AsyncProjArgs& a0, hipStream_t s) {
  constexpr int WTN = BN / WGN;  // columns per wave = width of one row partial
  AsyncProjArgs a = a0;
  // the host sized the partials for this tile's wave width; refuse to launch
  // (instead of writing past the workspace) if the two ever disagree
  if (a.epi.np != (a.epi.d + WTN - 1) / WTN) return hipErrorInvalidValue;
  a.tiles_m = (int)((a.epi.M + BM - 1) / BM);
  a.tiles_n = (a.epi.d + BN - 1) / BN;
  const int64_t blocks = (int64_t)a.tiles_m * (a.epi.nb + 1) * a.tiles_n;
  return launch(proj_async_kernel<BM, BN, BK, STAGES, WGM, WGN, false, MF>, (unsigned)blocks,
                64 * WGM * WGN, 0, s, a);
}

// One table of tile plans serves both the launch and the host's partial
// count, so the two cannot drift apart.
#define NGRAM_ASYNC_PLANS(X)      \
  X(0, 256, 128, 32, 4, 2, 2, 32)  \
  X(1, 128, 128, 64, 4, 2, 2, 32)  \
  X(2, 64, 64, 64, 4, 2, 2, 32)    \
  X(3, 256, 128, 64, 3, 2, 2, 32)  \
  X(4, 128, 64, 64, 4, 2, 2, 32)   \
  X(5, 64, 128, 64, 4, 2, 2, 32)   \
  X(6, 256, 256, 32, 2, 2, 4, 32)  \
  X(7, 256, 256, 64, 2, 2, 4, 32)  \
  X(8, 128, 128, 64, 2, 2, 2, 32)  \
  X(9, 256, 128, 32, 2, 2, 2, 32)  \
  X(10, 256, 256, 32, 4, 2, 4, 32) \
  X(11, 256, 256, 64, 2, 4, 2, 32) \
  X(12, 256, 256, 64, 2, 4, 2, 16)

}  // namespace

// Tile plans (id, BM, BN, K step, ring depth, wave rows, wave columns): see
// NGRAM_ASYNC_PLANS.  A plan id in [0, kAsyncPlans) overrides the choice (the
// configuration's tuning field).
int async_plan(int64_t M, int override_plan) {
  if (override_plan >= 0 && override_plan < kAsyncPlans) return override_plan;
  // 256 x 256 tiles from 8,192 rows: waves as 4 x 2 (64 x 128 each; 1 %
  // faster than 2 x 4 at Qwen prefill, multibranch and engram sizes), on
  // 16x16x32 MFMAs (projection 4 % faster than on 32x32x16 at Qwen prefill,
  // 2-4 % at multibranch, the same at engram_small)
  if (M >= 8192) return 12;
  if (M >= 1024) return 8;
  return 2;
}

int async_wave_cols(int plan) {
#define NGRAM_WAVE_COLS(id, bm, bn, bk, st, wgm, wgn, mf) \
  if (plan == id) return bn / wgn;
  NGRAM_ASYNC_PLANS(NGRAM_WAVE_COLS)
#undef NGRAM_WAVE_COLS
  return -1;
}

// The raw product of two K-outer operands (proj_raw_tn_kernel): K a
// multiple of 64 whose rows past the true K are zero, M and N multiples of 8,
// the operands' rows 16-byte aligned.
hipError_t launch_projection_raw_tn(const AsyncProjArgs& a0, hipStream_t s) {
  AsyncProjArgs a = a0;
  if (a.epi.M == 0 || a.epi.d == 0) return hipSuccess;
  if (a.raw_out == nullptr || a.K % 64 != 0 || a.epi.M % 8 != 0 || a.epi.d % 8 != 0 ||
      a.tn_lda % 8 != 0 || a.tn_ldb % 8 != 0 || a.tn_lda < a.epi.M || a.tn_ldb < a.epi.d)
    return hipErrorInvalidValue;
  a.tiles_m = (int)((a.epi.M + 255) / 256);
  a.tiles_n = (a.epi.d + 255) / 256;
  const int split = a.raw_split > 1 ? a.raw_split : 1;
  if (split > a.K / 64) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n * split;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  return launch(proj_raw_tn_kernel<2, 4>, (unsigned)blocks, 512, 0, s, a);
}

// The raw product serves the backward pass; it is built for the default
// plans only (async_plan without an override).
hipError_t launch_projection_raw(int plan, const AsyncProjArgs& a, hipStream_t s) {
  if (a.epi.M == 0) return hipSuccess;
  switch (plan) {
    case 2: return launch_raw_t<64, 64, 64, 4, 2, 2>(a, s);
    case 7: return launch_raw_t<256, 256, 64, 2, 2, 4>(a, s);
    case 8: return launch_raw_t<128, 128, 64, 2, 2, 2>(a, s);
    case 12: return launch_raw_t<256, 256, 64, 2, 4, 2, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_projection_async(int plan, const AsyncProjArgs& a, hipStream_t s) {
  if (a.epi.M == 0) return hipSuccess;
#define NGRAM_LAUNCH_PLAN(id, bm, bn, bk, st, wgm, wgn, mf) \
  if (plan == id) return launch_async_t<bm, bn, bk, st, wgm, wgn, mf>(a, s);
  NGRAM_ASYNC_PLANS(NGRAM_LAUNCH_PLAN)
#undef NGRAM_LAUNCH_PLAN
  return hipErrorInvalidValue;
}

}  // namespace ngram
