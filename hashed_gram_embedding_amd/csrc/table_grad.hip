// The table gradient of the backward pass with a fixed summation order.
//
// The lookup reads row r_j(t) of table j for every token t, so the table's
// gradient is the adjoint of that gather: row r of table j receives the sum
// of dE[t, j-th slice] over the tokens t that named it ("Qwen3.8-Flash-Next
// 深度研究" §2.3 for the lookup; the same page's §9.4 lists this scatter beside
// the gather among the layer's operators).  Rows named by several tokens (a
// frequent n-gram) take many terms; here every row's terms are added in
// ascending token order, whatever the schedule, so the gradients are
// bit-identical from run to run:
//
//  1. per table, the (row, token) pairs are sorted by row with a stable LSD
//     radix sort (8-bit digits, as many passes as the largest table's row
//     count needs), so each row's tokens end up contiguous and ascending;
//  2. one wavefront per 64 sorted positions adds up the dE slices of each run
//     of equal rows in position order (the slices' columns across the lanes)
//     and adds the sum into the row (plain load and store: the row has no
//     other writer) -- or, for a run that crosses the wavefront's range, leaves
//     the piece in a carry slot;
//  3. one wavefront per run that continues past its range adds the carried
//     pieces in range order and adds the sum into the row.
//
// Scratch (table_grad_bytes): the keys and tokens twice over (the sort's ping
// and pong), the digit counts, and a carry pair of row_dim floats per range.
#include "internal.h"

namespace ngram {
namespace {

constexpr int kSortItems = 16;                 // keys per thread of a sort block
constexpr int kSortTile = 256 * kSortItems;    // keys per sort block
constexpr int kRange = 64;                     // sorted positions per wavefront
constexpr int kColsPerPass = 64 * 8;           // columns a wavefront holds at once

// flags of a range: it holds the tail of the run continuing from the range
// before (HEAD), the start of a run continuing into the next (TAIL), or a run
// that covers the whole range and continues both ways (MIDDLE, with HEAD)
constexpr int32_t kHead = 1, kTail = 2, kMiddle = 4;

struct RowCounts {
  int32_t r[NGRAM_MAX_TABLES];  // rows of each table
};

// keys[j n + t] = row of table j named by token t, toks[j n + t] = t
__global__ __launch_bounds__(256) void pairs_kernel(const int32_t* __restrict__ row_idx, int64_t n,
                                                    int32_t nt, int32_t* __restrict__ keys,
                                                    int32_t* __restrict__ toks) {
  const int64_t total = n * nt;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t j = i / n, t = i - j * n;
    keys[i] = row_idx[t * nt + j];
    toks[i] = (int32_t)t;
  }
}

// Digit counts of block b of table j: hist[(j * 256 + digit) * nblk + b].
__global__ __launch_bounds__(256) void digit_count_kernel(const int32_t* __restrict__ keys,
                                                          int64_t n, int shift, int32_t nblk,
                                                          int32_t* __restrict__ hist) {
  __shared__ int32_t cnt[256];
  const int j = blockIdx.y, b = blockIdx.x;
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int32_t* __restrict__ kj = keys + (int64_t)j * n;
  const int64_t t0 = (int64_t)b * kSortTile;
#pragma unroll 4
  for (int k = 0; k < kSortItems; ++k) {
    const int64_t i = t0 + k * 256 + threadIdx.x;
    if (i < n) atomicAdd(&cnt[((uint32_t)kj[i] >> shift) & 255u], 1);
  }
  __syncthreads();
  hist[((int64_t)j * 256 + threadIdx.x) * nblk + b] = cnt[threadIdx.x];
}

// Exclusive prefix sum, in place, of table blockIdx.x's 256 * nblk counts in
// (digit, block) order: the position where block b's keys of that digit start.
__global__ __launch_bounds__(1024) void digit_scan_kernel(int32_t* __restrict__ hist,
                                                          int32_t nblk) {
  __shared__ int32_t part[1024];
  const int64_t len = (int64_t)256 * nblk;
  int32_t* __restrict__ h = hist + (int64_t)blockIdx.x * len;
  const int64_t per = (len + 1023) / 1024;
  const int64_t a = (int64_t)threadIdx.x * per;
  const int64_t e = a + per < len ? a + per : len;
  int32_t s = 0;
  for (int64_t i = a; i < e; ++i) s += h[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = threadIdx.x >= (unsigned)off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t run = threadIdx.x ? part[threadIdx.x - 1] : 0;
  for (int64_t i = a; i < e; ++i) {
    const int32_t c = h[i];
    h[i] = run;
    run += c;
  }
}

// One stable pass: block b of table j moves its keys, in their order, to the
// positions its digit offsets give.  The block takes its tile 256 keys at a
// time; a key's rank among the equal digits before it is found with eight
// ballots within its wavefront, plus the counts of the wavefronts before it
// and of the earlier groups.
__global__ __launch_bounds__(256) void digit_move_kernel(const int32_t* __restrict__ kin,
                                                         const int32_t* __restrict__ tin, int64_t n,
                                                         int shift, int32_t nblk,
                                                         const int32_t* __restrict__ offs,
                                                         int32_t* __restrict__ kout,
                                                         int32_t* __restrict__ tout) {
  __shared__ int32_t base[256];
  __shared__ int32_t wcnt[4][256];
  const int j = blockIdx.y, b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  base[tid] = offs[((int64_t)j * 256 + tid) * nblk + b];
  const int64_t jo = (int64_t)j * n;
  const int64_t t0 = (int64_t)b * kSortTile;
  const uint64_t below = (uint64_t(1) << lane) - 1;  // the lanes before this one
  for (int k = 0; k < kSortItems; ++k) {
#pragma unroll
    for (int w = 0; w < 4; ++w) wcnt[w][tid] = 0;
    __syncthreads();  // the counts are clear; base[] holds the earlier groups
    const int64_t i = t0 + k * 256 + tid;
    const bool act = i < n;
    const uint32_t key = act ? (uint32_t)kin[jo + i] : 0u;
    const int32_t tok = act ? tin[jo + i] : 0;
    const uint32_t dg = (key >> shift) & 255u;
    uint64_t peers = __ballot(act);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (dg >> bit) & 1u;
      const uint64_t m = __ballot(on);
      peers &= on ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    if (act && rank == 0) wcnt[wave][dg] = __popcll(peers);
    __syncthreads();
    if (act) {
      int64_t pos = base[dg] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][dg];
      if (pos >= 0 && pos < n) {
        kout[jo + pos] = (int32_t)key;
        tout[jo + pos] = tok;
      }
    }
    __syncthreads();  // every read of base[] and wcnt[] for this group is done
    base[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
  }
}

// Step 2: range w = (table j, range c) of the sorted pairs, one wavefront.
// Lane l holds the key and token of position p0 + l.  A row's columns are
// spread over the lanes four at a time (16-byte accesses), kColsPerPass per
// pass; the positions are taken eight at a time, their dE slices -- and the
// table rows of the runs that end among them -- loaded before any is added,
// so that a run's read-modify-write costs no round trip of its own.  The
// slices are added in position order.
__global__ __launch_bounds__(64) void run_sum_kernel(const int32_t* __restrict__ keys,
                                                     const int32_t* __restrict__ toks, int64_t n,
                                                     int32_t nt, int32_t row_dim, int64_t n_range,
                                                     const float* __restrict__ d_e,
                                                     GradTablePtrs g, RowCounts rows,
                                                     float* __restrict__ carry,
                                                     int32_t* __restrict__ flags) {
  constexpr int UQ = kColsPerPass / 256;  // 16-byte column groups per lane and pass
  const int lane = threadIdx.x;
  const int64_t w = blockIdx.x;
  const int j = (int)(w / n_range);
  const int64_t c = w - (int64_t)j * n_range;
  const int64_t p0 = c * kRange;
  const int cnt = (int)(n - p0 < kRange ? n - p0 : kRange);
  const int32_t* __restrict__ kj = keys + (int64_t)j * n;
  const int32_t* __restrict__ tj = toks + (int64_t)j * n;
  // (every position holds a token index below n and a row of table j; the
  // clamps only keep the accesses inside their arrays whatever they hold)
  const int32_t n_rows = rows.r[j];
  int32_t my_key = lane < cnt ? kj[p0 + lane] : -1;
  my_key = my_key >= n_rows ? -1 : my_key;
  int32_t my_tok = lane < cnt ? tj[p0 + lane] : 0;
  my_tok = my_tok < 0 ? 0 : (my_tok >= n ? (int32_t)(n - 1) : my_tok);
  const int32_t prev = p0 > 0 ? kj[p0 - 1] : -1;          // rows are >= 0
  const int32_t next = p0 + cnt < n ? kj[p0 + cnt] : -1;
  const bool cont_in = prev == __builtin_amdgcn_readlane(my_key, 0);
  const bool cont_out = next == __builtin_amdgcn_readlane(my_key, cnt - 1);
  // bit i: a run ends at position i; rmw: ... and its sum goes into the row
  // (all but a run begun in an earlier range, whose piece is carried)
  const int32_t key_after = __shfl_down(my_key, 1);
  const uint64_t ends =
      __ballot(lane < cnt && (lane + 1 < cnt ? key_after != my_key : !cont_out));
  uint64_t rmw = ends;
  if (cont_in && ends) rmw &= rmw - 1;  // the first end closes the carried-in run
  const float* __restrict__ dej = d_e + (int64_t)j * row_dim;
  const int64_t dstride = (int64_t)nt * row_dim;
  float* __restrict__ head = carry + (w * 2) * row_dim;
  float* __restrict__ tail = head + row_dim;
  float* __restrict__ tab = g.p[j];
  int32_t flag = 0;
  for (int cb = 0; cb < row_dim; cb += kColsPerPass) {
    // this lane's column groups of the pass (row_dim is a multiple of 4);
    // groups past the row load column 0 and are never stored
    int col[UQ];
    bool ok[UQ];
#pragma unroll
    for (int u = 0; u < UQ; ++u) {
      const int cc = cb + 4 * lane + 256 * u;
      ok[u] = cc < row_dim;
      col[u] = ok[u] ? cc : 0;
    }
    float4 acc[UQ];
#pragma unroll
    for (int u = 0; u < UQ; ++u) acc[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    auto emit = [&](float* dst) {
#pragma unroll
      for (int u = 0; u < UQ; ++u)
        if (ok[u]) *reinterpret_cast<float4*>(dst + col[u]) = acc[u];
    };
    for (int i0 = 0; i0 < cnt; i0 += 8) {
      float4 v[8][UQ], r[8][UQ];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = i0 + q < cnt ? i0 + q : cnt - 1;
        const int32_t t = __builtin_amdgcn_readlane(my_tok, i);
        const float* __restrict__ src = dej + (int64_t)t * dstride;
#pragma unroll
        for (int u = 0; u < UQ; ++u) v[q][u] = *reinterpret_cast<const float4*>(src + col[u]);
        const int32_t kp = __builtin_amdgcn_readlane(my_key, i);
        if (i0 + q < cnt && ((rmw >> (i0 + q)) & 1) && kp >= 0) {
          const float* row = tab + (int64_t)kp * row_dim;
#pragma unroll
          for (int u = 0; u < UQ; ++u) r[q][u] = *reinterpret_cast<const float4*>(row + col[u]);
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = i0 + q;
        if (i < cnt) {
#pragma unroll
          for (int u = 0; u < UQ; ++u) {
            acc[u].x += v[q][u].x;
            acc[u].y += v[q][u].y;
            acc[u].z += v[q][u].z;
            acc[u].w += v[q][u].w;
          }
          if ((ends >> i) & 1) {
            if ((rmw >> i) & 1) {
              const int32_t kp = __builtin_amdgcn_readlane(my_key, i);
              if (kp >= 0) {
                float* row = tab + (int64_t)kp * row_dim;
#pragma unroll
                for (int u = 0; u < UQ; ++u)
                  if (ok[u])
                    *reinterpret_cast<float4*>(row + col[u]) =
                        make_float4(r[q][u].x + acc[u].x, r[q][u].y + acc[u].y,
                                    r[q][u].z + acc[u].z, r[q][u].w + acc[u].w);
              }
            } else {
              emit(head);  // the end of a run begun in an earlier range
              flag |= kHead;
            }
#pragma unroll
            for (int u = 0; u < UQ; ++u) acc[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          }
        }
      }
    }
    if (cont_out) {  // the open piece continues into the next range
      if (cont_in && !ends) {
        emit(head);
        flag |= kHead | kMiddle;
      } else {
        emit(tail);
        flag |= kTail;
      }
    }
  }
  if (lane == 0) flags[w] = flag;
}

// Step 3: a run that starts in range w and continues: its piece there, then
// the following ranges' head pieces in order, until a range where the run
// ends.  The flags of eight ranges are read at a time, then their pieces.
__global__ __launch_bounds__(64) void run_join_kernel(const int32_t* __restrict__ keys, int64_t n,
                                                      int32_t row_dim, int64_t n_range,
                                                      GradTablePtrs g, RowCounts rows,
                                                      const float* __restrict__ carry,
                                                      const int32_t* __restrict__ flags) {
  const int64_t w = blockIdx.x;
  if (!(flags[w] & kTail)) return;
  const int lane = threadIdx.x;
  const int j = (int)(w / n_range);
  const int64_t c = w - (int64_t)j * n_range;
  const int64_t last = (c + 1) * kRange < n ? (c + 1) * kRange - 1 : n - 1;
  const int32_t key = keys[(int64_t)j * n + last];
  if (key < 0 || key >= rows.r[j]) return;
  float* __restrict__ row = g.p[j] + (int64_t)key * row_dim;
  const float* __restrict__ cj = carry + (int64_t)j * n_range * 2 * row_dim;
  for (int cb = 0; cb < row_dim; cb += 256) {
    const int col = cb + 4 * lane;
    const bool ok = col < row_dim;
    const int cl = ok ? col : 0;
    float4 acc = *reinterpret_cast<const float4*>(carry + (w * 2 + 1) * row_dim + cl);
    bool done = false;
    for (int64_t c2 = c + 1; !done && c2 < n_range;) {
      int32_t f[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) f[q] = c2 + q < n_range ? flags[(int64_t)j * n_range + c2 + q] : 0;
      int take = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (!done && c2 + q < n_range) {
          take = q + 1;
          done = !(f[q] & kMiddle);
        }
      }
      float4 h[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < take) h[q] = *reinterpret_cast<const float4*>(cj + ((c2 + q) * 2) * row_dim + cl);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < take) {
          acc.x += h[q].x;
          acc.y += h[q].y;
          acc.z += h[q].z;
          acc.w += h[q].w;
        }
      c2 += take;
    }
    if (ok) {
      float4 x = *reinterpret_cast<const float4*>(row + col);
      x.x += acc.x;
      x.y += acc.y;
      x.z += acc.z;
      x.w += acc.w;
      *reinterpret_cast<float4*>(row + col) = x;
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct TgLayout {
  size_t keys[2], toks[2], hist, flags, carry, total;
  int64_t nblk, n_range;
};

TgLayout tg_layout(int64_t n, int32_t nt, int32_t row_dim) {
  TgLayout L;
  const size_t m = (size_t)n * nt * 4;
  L.nblk = (n + kSortTile - 1) / kSortTile;
  L.n_range = (n + kRange - 1) / kRange;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L.keys[0] = take(m);
  L.toks[0] = take(m);
  L.keys[1] = take(m);
  L.toks[1] = take(m);
  L.hist = take((size_t)nt * 256 * L.nblk * 4);
  L.flags = take((size_t)nt * L.n_range * 4);
  L.carry = take((size_t)nt * L.n_range * 2 * row_dim * 4);
  L.total = off;
  return L;
}

unsigned blocks_for(int64_t work, int64_t cap) {
  const int64_t g = work < cap ? work : cap;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

size_t table_grad_bytes(int64_t n_tok, int32_t n_tables, int32_t row_dim) {
  return tg_layout(n_tok, n_tables, row_dim).total;
}

hipError_t launch_table_grad(const int32_t* row_idx, int64_t n_tok, int32_t n_tables,
                             int32_t row_dim, const int64_t* table_rows, const float* d_e,
                             const GradTablePtrs& g, void* scratch, hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  if (n_tables < 1 || n_tables > NGRAM_MAX_TABLES || row_dim < 1 ||
      n_tok >= (int64_t(1) << 31) || scratch == nullptr)
    return hipErrorInvalidValue;
  RowCounts rows;
  int64_t max_rows = 1;
  for (int j = 0; j < NGRAM_MAX_TABLES; ++j) rows.r[j] = 0;
  for (int j = 0; j < n_tables; ++j) {
    if (table_rows[j] < 1 || table_rows[j] > 0x7FFFFFFF) return hipErrorInvalidValue;
    rows.r[j] = (int32_t)table_rows[j];
    max_rows = table_rows[j] > max_rows ? table_rows[j] : max_rows;
  }
  const TgLayout L = tg_layout(n_tok, n_tables, row_dim);
  if ((int64_t)n_tables * L.n_range > 0x7FFFFFFF) return hipErrorInvalidValue;
  char* ws = static_cast<char*>(scratch);
  int32_t* keys[2] = {reinterpret_cast<int32_t*>(ws + L.keys[0]),
                      reinterpret_cast<int32_t*>(ws + L.keys[1])};
  int32_t* toks[2] = {reinterpret_cast<int32_t*>(ws + L.toks[0]),
                      reinterpret_cast<int32_t*>(ws + L.toks[1])};
  int32_t* hist = reinterpret_cast<int32_t*>(ws + L.hist);
  int32_t* flags = reinterpret_cast<int32_t*>(ws + L.flags);
  float* carry = reinterpret_cast<float*>(ws + L.carry);

  hipError_t e = launch(pairs_kernel, blocks_for((n_tok * n_tables + 255) / 256, 16384), 256, 0,
                        s, row_idx, n_tok, n_tables, keys[0], toks[0]);
  if (e != hipSuccess) return e;
  // digits of the largest row index
  int bits = 1;
  while (bits < 31 && (int64_t(1) << bits) < max_rows) ++bits;
  const dim3 grid((unsigned)L.nblk, (unsigned)n_tables);
  int cur = 0;
  for (int shift = 0; shift < bits; shift += 8) {
    e = launch(digit_count_kernel, grid, 256, 0, s, keys[cur], n_tok, shift, (int32_t)L.nblk,
               hist);
    if (e != hipSuccess) return e;
    e = launch(digit_scan_kernel, dim3((unsigned)n_tables), 1024, 0, s, hist, (int32_t)L.nblk);
    if (e != hipSuccess) return e;
    e = launch(digit_move_kernel, grid, 256, 0, s, keys[cur], toks[cur], n_tok, shift,
               (int32_t)L.nblk, (const int32_t*)hist, keys[cur ^ 1], toks[cur ^ 1]);
    if (e != hipSuccess) return e;
    cur ^= 1;
  }
  const unsigned waves = (unsigned)((int64_t)n_tables * L.n_range);
  e = launch(run_sum_kernel, waves, 64, 0, s, (const int32_t*)keys[cur], (const int32_t*)toks[cur],
             n_tok, n_tables, row_dim, L.n_range, d_e, g, rows, carry, flags);
  if (e != hipSuccess) return e;
  return launch(run_join_kernel, waves, 64, 0, s, (const int32_t*)keys[cur], n_tok, row_dim,
                L.n_range, g, rows, (const float*)carry, (const int32_t*)flags);
}

}  // namespace ngram
