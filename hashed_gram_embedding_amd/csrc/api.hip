// extern "C" entry points of libngram.so: argument validation on the host,
// workspace layout, and the launch sequence of each operation.  Every step
// of the layer runs in the kernels of ids.hip, gather.hip, project.hip,
// project_async.hip, project_decode.hip, finalize.hip, backward.hip and
// table_grad.hip (each cites the passages it implements); this file launches
// them on the caller's stream.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "internal.h"

using namespace ngram;

thread_local ngram::StageClock* ngram::t_open_stage = nullptr;

// The scratch of ngram_forward_noalloc: one copy per GPU, reserved with the
// library's code object.  Host code never names it directly (the name is a
// host-side stand-in there): it uses the device address that
// hipGetSymbolAddress returns for the current device, kept per device.
static __device__ __align__(256) unsigned char scratch[NGRAM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kAbiVersion = 7;
constexpr int64_t kMaxTokens = int64_t(1) << 28;

int esize_of(int dtype) { return dtype == NGRAM_BF16 ? 2 : dtype == NGRAM_FP8_E4M3 ? 1 : 4; }

// dtype of the memory vector E: the tables', except that fp8 tables are
// widened to bf16 while they are gathered
int mem_dtype(const ngram_config* c) {
  return c->table_dtype == NGRAM_FP8_E4M3 ? NGRAM_BF16 : c->table_dtype;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

uint64_t mulmod(uint64_t a, uint64_t b, uint64_t m) {
  return (uint64_t)((unsigned __int128)a * b % m);
}
uint64_t powmod(uint64_t a, uint64_t e, uint64_t m) {
  uint64_t r = 1;
  a %= m;
  while (e) {
    if (e & 1) r = mulmod(r, a, m);
    a = mulmod(a, a, m);
    e >>= 1;
  }
  return r;
}

// Deterministic Miller-Rabin for n < 2^32 (bases 2, 7, 61 suffice: Jaeschke,
// "On strong pseudoprimes to several bases", Math. Comp. 1993).
bool is_prime_u32(uint64_t n) {
  if (n < 2) return false;
  static const uint64_t small[] = {2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37, 61};
  for (uint64_t p : small) {
    if (n == p) return true;
    if (n % p == 0) return false;
  }
  uint64_t d = n - 1;
  int s = 0;
  while (!(d & 1)) {
    d >>= 1;
    ++s;
  }
  for (uint64_t a : {2ull, 7ull, 61ull}) {
    uint64_t x = powmod(a, d, n);
    if (x == 1 || x == n - 1) continue;
    bool comp = true;
    for (int i = 1; i < s; ++i) {
      x = mulmod(x, x, n);
      if (x == n - 1) {
        comp = false;
        break;
      }
    }
    if (comp) return false;
  }
  return true;
}

// Every rows[j] has no prime factor up to 61 (or is one of them): the screen
// each entry point runs; the proof is is_prime_u32, run by
// ngram_config_validate.
bool passes_small_prime_screen(uint64_t n) {
  static const uint64_t small[] = {2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37, 41, 43, 47, 53, 59, 61};
  for (uint64_t p : small) {
    if (n == p) return true;
    if (n % p == 0) return false;
  }
  return true;
}

// prove_primes: run the Miller-Rabin proof on every table size (otherwise
// only the small-factor screen).  Everything else is checked either way.
int validate(const ngram_config* c, bool prove_primes) {
  if (c == nullptr) return NGRAM_EINVAL;
  if (c->table_dtype != NGRAM_F32 && c->table_dtype != NGRAM_BF16 &&
      c->table_dtype != NGRAM_FP8_E4M3)
    return NGRAM_EDTYPE;
  if (c->act_dtype != NGRAM_F32 && c->act_dtype != NGRAM_BF16) return NGRAM_EDTYPE;
  if (mem_dtype(c) != c->act_dtype) return NGRAM_EDTYPE;
  if (c->n_orders < 1 || c->n_orders > NGRAM_MAX_ORDER) return NGRAM_EINVAL;
  for (int o = 0; o < c->n_orders; ++o) {
    if (c->orders[o] < 1 || c->orders[o] > NGRAM_MAX_ORDER) return NGRAM_EINVAL;
    if (o > 0 && c->orders[o] <= c->orders[o - 1]) return NGRAM_EINVAL;
  }
  if (c->heads_per_order < 1) return NGRAM_EINVAL;
  if ((int64_t)c->n_orders * c->heads_per_order > NGRAM_MAX_TABLES) return NGRAM_ESHAPE;
  if (c->n_tables != c->n_orders * c->heads_per_order) return NGRAM_EINVAL;
  for (int j = 0; j < c->n_tables; ++j) {
    if (c->rows[j] < 2 || c->rows[j] > INT32_MAX) return NGRAM_ERANGE;
    const uint64_t n = (uint64_t)c->rows[j];
    if (!(prove_primes ? is_prime_u32(n) : passes_small_prime_screen(n))) return NGRAM_ERANGE;
  }
  const int es = esize_of(c->table_dtype);
  if (c->row_dim < 1 || ((int64_t)c->row_dim * es) % 16 != 0) return NGRAM_ESHAPE;
  if ((int64_t)c->mem_dim != (int64_t)c->n_tables * c->row_dim) return NGRAM_EINVAL;
  if (c->hidden_dim < 4 || c->hidden_dim % 4 != 0) return NGRAM_ESHAPE;
  if (c->act_dtype == NGRAM_BF16 && (c->mem_dim % 64 != 0 || c->hidden_dim % 32 != 0))
    return NGRAM_ESHAPE;
  if (c->table_dtype == NGRAM_FP8_E4M3)
    for (int j = 0; j < c->n_tables; ++j)
      if (!(c->table_scale[j] > 0.0f) || !isfinite(c->table_scale[j])) return NGRAM_EINVAL;
  if (c->n_branches < 1 || c->n_branches > NGRAM_MAX_BRANCHES) return NGRAM_EINVAL;
  if (c->conv_kernel != 4) return NGRAM_EINVAL;
  if (c->conv_dilation != c->orders[c->n_orders - 1]) return NGRAM_EINVAL;
  if (c->vocab < 1 || c->vocab_compressed < 1) return NGRAM_EINVAL;
  if (c->pad_id < 0 || c->pad_id >= c->vocab_compressed) return NGRAM_EINVAL;
  if (!(c->rms_eps >= 0.0f) || !isfinite(c->rms_eps)) return NGRAM_EINVAL;
  if (c->w_layout != NGRAM_W_MEM_D && c->w_layout != NGRAM_W_D_MEM) return NGRAM_EINVAL;
  if ((int64_t)c->hidden_dim * c->mem_dim >= (int64_t(1) << 31)) return NGRAM_ESHAPE;
  // tuning overrides
  if (c->tune_proj_plan < 0 || c->tune_proj_plan > kAsyncPlans) return NGRAM_EINVAL;
  if ((c->tune_decode_ni == 0) != (c->tune_decode_split == 0)) return NGRAM_EINVAL;
  if (c->tune_decode_ni != 0) {
    if (c->tune_decode_ni < 2 || c->tune_decode_ni > 6 || c->tune_decode_split < 1)
      return NGRAM_EINVAL;
    if (!wstat_plan_fits(WstatPlan{c->tune_decode_ni, c->tune_decode_split, 4}, c->mem_dim))
      return NGRAM_EINVAL;
  }
  return NGRAM_OK;
}

// bf16 with W stored [d, mem]: operands copied global -> LDS (project_async).
bool async_path(const ngram_config* c) {
  return mem_dtype(c) == NGRAM_BF16 && c->w_layout == NGRAM_W_D_MEM;
}

// Decode (one new token per sequence, up to kDecodeMaxRows sequences): E is
// materialised once by the hash + gather kernel, the weight-stationary
// projection writes one fp32 partial per K slice, and the decode finalize
// sums them.  Larger batches take the prefill route, where the weights are
// reused across many more rows.
constexpr int64_t kDecodeMaxRows = 2048;

// Tile plan of the decode projection: the configuration's override (checked
// by validate) or the library's choice; ni == 0 when none fits.
WstatPlan decode_plan(const ngram_config* c, int64_t n_tok) {
  if (c->tune_decode_ni != 0) return WstatPlan{c->tune_decode_ni, c->tune_decode_split, 4};
  return wstat_plan(n_tok, (c->n_branches + 1) * c->hidden_dim, c->mem_dim);
}

HashArgs hash_args(const ngram_config* c, int32_t hist_len) {
  HashArgs a;
  memset(&a, 0, sizeof a);
  a.n_orders = c->n_orders;
  a.heads = c->heads_per_order;
  a.n_tables = c->n_tables;
  a.max_order = c->orders[c->n_orders - 1];
  a.pad_id = c->pad_id;
  a.vocab = c->vocab;
  a.vocab_c = c->vocab_compressed;
  a.hist_len = hist_len;
  for (int o = 0; o < c->n_orders; ++o) a.orders[o] = c->orders[o];
  for (int j = 0; j < c->n_tables; ++j) {
    a.rows[j] = (uint64_t)c->rows[j];
    a.magic[j] = (uint64_t)(((unsigned __int128)1 << 64) / (uint64_t)c->rows[j]);
    for (int i = 0; i < NGRAM_MAX_ORDER; ++i) a.mult[j][i] = c->hash_mult[j][i];
  }
  return a;
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t row_idx = 0, e = 0, v = 0, parts = 0, split = 0, total = 0;
  ProjPlan plan;       // plan.np is the number of partials per row on every path
  int async = -1;      // async projection tile plan, -1 when not used
  int k_split = 0;     // decode path: K slices (0: not the decode path)
  WstatPlan wplan{0, 0, 0};  // decode path: projection plan
  int64_t v_stride = 0;  // fp32 elements between V rows
  int64_t v_offset = 0;  // fp32 elements from the V buffer to row 0's values
};

// forward: the forward pass (row ids and E live in the workspace).  T:
// tokens per sequence (the decode route when 1).
Layout layout_for(const ngram_config* c, int64_t n_tok, bool forward, int32_t T = 0) {
  Layout L;
  if (forward && async_path(c) && T == 1 && n_tok <= kDecodeMaxRows) {
    const WstatPlan wp = decode_plan(c, n_tok);
    if (wp.ni > 0) {
      L.wplan = wp;
      L.k_split = wp.split;
      L.plan.np = 1;
      size_t off = 0;
      L.e = off;  // decode E tiles: whole 16-token blocks
      off = align_up(off + (size_t)((n_tok + 15) / 16 * 16) * c->mem_dim *
                               esize_of(mem_dtype(c)));
      L.row_idx = off;
      off = align_up(off + (size_t)n_tok * c->n_tables * sizeof(int32_t));
      L.split = off;
      off = align_up(off + (size_t)L.k_split * n_tok * (c->n_branches + 1) * c->hidden_dim *
                               sizeof(float));
      L.total = off;
      return L;
    }
  }
  const int dt = mem_dtype(c);
  const int nb = c->n_branches, d = c->hidden_dim;
  L.plan = plan_projection(dt, n_tok, d);
  if (async_path(c)) {
    L.async = async_plan(n_tok, c->tune_proj_plan - 1);
    const int wc = async_wave_cols(L.async);
    L.plan.np = (d + wc - 1) / wc;
  }
  size_t off = 0;
  if (forward) {
    L.row_idx = off;
    off = align_up(off + (size_t)n_tok * c->n_tables * sizeof(int32_t));
    L.e = off;
    off = align_up(off + (size_t)n_tok * c->mem_dim * esize_of(dt));
  }
  L.v = off;
  if (dt == NGRAM_BF16) {
    off = align_up(off + (size_t)n_tok * d * sizeof(float));
    L.v_stride = d;
    L.v_offset = 0;
  } else {  // the fp32 path keeps K and V: [n_tok, nb+1, d]
    off = align_up(off + (size_t)n_tok * (nb + 1) * d * sizeof(float));
    L.v_stride = (int64_t)(nb + 1) * d;
    L.v_offset = (int64_t)nb * d;
  }
  L.parts = off;
  off = align_up(off + (size_t)n_tok * (3 * nb + 1) * L.plan.np * sizeof(float));
  L.total = off;
  return L;
}

int hip_status(hipError_t e) { return e == hipSuccess ? NGRAM_OK : NGRAM_EHIP; }

// Backward workspace: row ids, E, K / V (fp32), per-row stats, dC, dK / dV
// (bf16), the weights transposed, dE (fp32), and dK / dV and E transposed
// over tokens padded to a multiple of 64.
struct BwdLayout {
  size_t row_idx, e, kv, stats, dc, dkv, wt, de, part, rtmp, dw, tgrad, fparts, total;
  int64_t n_pad;
  int32_t dw_split;  // K splits of the dW product
};

// K splits of the dW product [(nb+1) d, mem] over n_pad tokens on the
// 256 x 256 tile plan (one workgroup per CU): the count in 1..8 that
// minimises the launch's rounds of 256 workgroups per unit of work, the
// smaller count on ties, keeping at least 16 K steps per split.
int32_t dw_split_for(int64_t rows, int64_t cols, int64_t n_pad) {
  const int64_t tiles = ((rows + 255) / 256) * ((cols + 255) / 256);
  int32_t best = 1;
  double best_cost = 0.0;
  for (int32_t sp = 1; sp <= 8; ++sp) {
    if (n_pad / 64 / sp < 16) break;
    const double cost = (double)((tiles * sp + kWstatCus - 1) / kWstatCus) / sp;
    if (sp == 1 || cost < best_cost - 1e-9) {
      best = sp;
      best_cost = cost;
    }
  }
  return best;
}

BwdLayout bwd_layout(const ngram_config* c, int64_t n) {
  BwdLayout L;
  const int64_t nb = c->n_branches, d = c->hidden_dim, mem = c->mem_dim, N = (nb + 1) * d;
  L.n_pad = (n + 63) / 64 * 64;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.row_idx = take((size_t)n * c->n_tables * 4);
  // E and [dK dV] hold n_pad rows: the dW product reads both K-outer over
  // n_pad tokens, the rows past n zero
  L.e = take((size_t)L.n_pad * mem * 2);
  L.kv = take((size_t)n * N * 4);
  L.stats = take((size_t)n * nb * kStatsStride * 4);
  L.dc = take((size_t)n * nb * d * 4);
  L.dkv = take((size_t)L.n_pad * N * 2);
  L.wt = take((size_t)mem * N * 2);
  L.de = take((size_t)n * mem * 4);
  L.part = take((size_t)kBwdBlocks * 7 * d * 4);
  L.rtmp = take((size_t)32 * 4 * d * 4);
  L.dw_split = dw_split_for(N, mem, L.n_pad);
  L.dw = take((size_t)L.dw_split * N * mem * 4);
  // the table gradient's sort and carries run last, when dC is no longer
  // read: they reuse that region when it is large enough (row ids, E and
  // K / V stay intact, so a forward's kept intermediates serve any number of
  // backward calls)
  const size_t tg = table_grad_bytes(n, c->n_tables, c->row_dim);
  L.tgrad = tg <= (size_t)n * nb * d * 4 ? L.dc : take(tg);
  // a forward that keeps its intermediates for this pass puts its gate
  // partials where dE goes later
  const size_t fp = (size_t)n * (3 * nb + 1) * layout_for(c, n, true, 0).plan.np * 4;
  L.fparts = fp <= (size_t)n * mem * 4 ? L.de : take(fp);
  L.total = off;
  return L;
}

// The backward's products index some operands with 32-bit offsets: the dE
// product's weights transposed to [mem, (nb+1) d] (whose split sums also
// take (nb+1) d mem as a 32-bit stride); (nb+1) d n_pad and mem n_pad are
// held to the same bound, conservatively.  Also the supported set of the
// backward pass.
int backward_shape_ok(const ngram_config* cfg, int64_t n) {
  if (cfg->act_dtype != NGRAM_BF16 || cfg->w_layout != NGRAM_W_D_MEM || !async_path(cfg))
    return NGRAM_EDTYPE;
  if (cfg->hidden_dim % 64 != 0 || cfg->hidden_dim > 4096) return NGRAM_ESHAPE;
  const int64_t n_pad = (n + 63) / 64 * 64;
  const int64_t N64 = (int64_t)(cfg->n_branches + 1) * cfg->hidden_dim;
  if (N64 * n_pad >= (int64_t(1) << 31) || (int64_t)cfg->mem_dim * n_pad >= (int64_t(1) << 31) ||
      N64 * cfg->mem_dim >= (int64_t(1) << 31))
    return NGRAM_ESHAPE;
  return NGRAM_OK;
}

// C[M, (nb+1)*dd] = A[M, K] B^T in fp32 (B: nb key blocks of dd rows from wk,
// then dd rows from wv, all [., K] bf16) on the MFMA projection kernel.
hipError_t raw_gemm(const bf16_bits* A, int64_t M, int32_t K, const bf16_bits* wk,
                    const bf16_bits* wv, int32_t nb, int32_t dd, float* C, int64_t ldc,
                    hipStream_t s, int32_t split = 1) {
  AsyncProjArgs a;
  memset(&a, 0, sizeof a);
  a.e = A;
  a.wk = wk;
  a.wv = wv;
  a.epi.M = M;
  a.epi.d = dd;
  a.epi.nb = nb;
  a.K = K;
  a.group_m = 4;
  a.raw_out = C;
  a.raw_ld = ldc;
  a.raw_split = split;
  a.raw_split_stride = M * ldc;
  // split-K products run on the 256 x 256 plan, whose tile count the split was
  // chosen for; from 8,192 rows on its 16x16x32 form
  return launch_projection_raw(split > 1 ? 7 : M >= 8192 ? 12 : M >= 1024 ? 8 : 2, a, s);
}

// Stage timing of one instrumented call (ngram_forward_timed /
// ngram_backward_timed): stage(i) closes the open stage and opens stage i,
// whose kernels then stamp the stage's event pair (launch() in internal.h
// reads the calling thread's open stage).  Untimed calls carry a Timer
// without events, which opens nothing.
struct Timer {
  const hipEvent_t* ev = nullptr;
  int mask = 0;
  int index = -1;
  StageClock clock{};
  void close() {
    if (index >= 0) {
      if (clock.launches > 0) mask |= 1 << index;
      t_open_stage = nullptr;
      index = -1;
    }
  }
  void stage(int i) {
    close();
    if (ev == nullptr) return;
    clock = StageClock{ev[2 * i], ev[2 * i + 1], 0};
    index = i;
    t_open_stage = &clock;
  }
  ~Timer() { close(); }
};

int check_tables(const ngram_config* c, const void* const* tables, TablePtrs* out) {
  if (tables == nullptr) return NGRAM_EINVAL;
  memset(out, 0, sizeof *out);
  for (int j = 0; j < c->n_tables; ++j) {
    if (tables[j] == nullptr) return NGRAM_EINVAL;
    if (!aligned16(tables[j])) return NGRAM_EALIGN;
    out->p[j] = tables[j];
    out->scale[j] = c->table_dtype == NGRAM_FP8_E4M3 ? c->table_scale[j] : 1.0f;
  }
  return NGRAM_OK;
}

int check_hidden_stride(const ngram_config* c, int64_t hbs, int64_t* tok_stride) {
  if (hbs != 0 && hbs != c->hidden_dim) return NGRAM_ESHAPE;
  *tok_stride = hbs == 0 ? c->hidden_dim : (int64_t)c->n_branches * c->hidden_dim;
  return NGRAM_OK;
}

ProjArgs proj_args(const ngram_config* c, const void* e, const void* w_k, const void* w_v,
                   const void* hidden, int64_t h_tok, int64_t h_br, const void* gq,
                   const void* gk, char* ws, const Layout& L, int64_t M) {
  ProjArgs a;
  a.e = e;
  a.wk = w_k;
  a.wv = w_v;
  a.hidden = hidden;
  a.h_tok_stride = h_tok;
  a.h_branch_stride = h_br;
  a.gamma_q = gq;
  a.gamma_k = gk;
  a.v = reinterpret_cast<float*>(ws + L.v);
  a.parts = reinterpret_cast<float*>(ws + L.parts);
  a.M = M;
  a.K = c->mem_dim;
  a.d = c->hidden_dim;
  a.nb = c->n_branches;
  a.np = L.plan.np;
  a.w_dk = c->w_layout == NGRAM_W_D_MEM;
  a.v_ld = c->hidden_dim;
  a.k_keep = nullptr;
  return a;
}

AsyncProjArgs async_args(const ProjArgs& p) {
  AsyncProjArgs a;
  memset(&a, 0, sizeof a);
  a.e = static_cast<const bf16_bits*>(p.e);
  a.wk = static_cast<const bf16_bits*>(p.wk);
  a.wv = static_cast<const bf16_bits*>(p.wv);
  a.epi.hidden = static_cast<const bf16_bits*>(p.hidden);
  a.epi.h_tok_stride = p.h_tok_stride;
  a.epi.h_branch_stride = p.h_branch_stride;
  a.epi.gamma_q = static_cast<const bf16_bits*>(p.gamma_q);
  a.epi.gamma_k = static_cast<const bf16_bits*>(p.gamma_k);
  a.epi.v = p.v;
  a.epi.parts = p.parts;
  a.epi.M = p.M;
  a.epi.d = p.d;
  a.epi.nb = p.nb;
  a.epi.np = p.np;
  a.epi.v_ld = p.v_ld;
  a.epi.k_keep = p.k_keep;
  a.K = p.K;
  a.group_m = 4;
  return a;
}

// Launch the projection for E (or, with gather, for raw ids hashed in-kernel).
hipError_t run_projection(const ngram_config* c, const Layout& L, const ProjArgs& p,
                          hipStream_t s) {
  if (L.async < 0) return launch_projection(mem_dtype(c), L.plan, p, s);
  return launch_projection_async(L.async, async_args(p), s);
}

ConvArgs conv_args_base(const ngram_config* c) {
  ConvArgs a;
  memset(&a, 0, sizeof a);
  a.nb = c->n_branches;
  a.d = c->hidden_dim;
  a.eps = c->rms_eps;
  return a;
}


constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch, looked up once per device
// (nullptr if the device or the lookup fails).
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

// Steps 1-4 of the forward into the workspace of layout L: row ids and E
// (the decode route's one hash + gather kernel, else hash then gather).
int launch_lookup(const ngram_config* cfg, const Layout& L, const int32_t* raw_ids, int32_t B,
                  int32_t T, const int32_t* history, const int32_t* lut, const TablePtrs& tp,
                  int32_t* err_flag, char* ws, hipStream_t s, Timer& tm) {
  const int64_t n_tok = (int64_t)B * T;
  int32_t* row_idx = reinterpret_cast<int32_t*>(ws + L.row_idx);
  void* e = ws + L.e;
  const HashArgs ha = hash_args(cfg, cfg->orders[cfg->n_orders - 1] - 1);
  if (L.k_split > 0) {
    tm.stage(1);
    return hip_status(launch_hash_gather(cfg->table_dtype, raw_ids, B, T, history, lut, ha,
                                         cfg->n_tables, cfg->row_dim, tp, e, row_idx, err_flag, s));
  }
  tm.stage(0);
  int st = hip_status(launch_hash(true, raw_ids, B, T, history, lut, ha, row_idx, err_flag, s));
  if (st) return st;
  tm.stage(1);
  return hip_status(launch_gather(cfg->table_dtype, row_idx, n_tok, cfg->n_tables,
                                  cfg->row_dim, tp, e, s));
}

// Shared by ngram_forward, ngram_forward_timed and ngram_forward_noalloc
// (static_scratch: the current device's static scratch replaces the
// workspace, taken once every argument has passed its checks).
int forward_impl(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                 const int32_t* history, const int32_t* lut, const void* const* tables,
                 const void* hidden, int64_t hidden_branch_stride, const void* w_k,
                 const void* w_v, const void* conv_w, const void* gamma_q, const void* gamma_k,
                 const void* gamma_u, float* conv_state, int32_t* state_pos,
                 int32_t flags, void* out, float* gates, int32_t* err_flag, void* workspace,
                 size_t workspace_bytes, hipStream_t s, Timer& tm, bool static_scratch = false) {
  int st = validate(cfg, false);
  if (st) return st;
  if (B < 0 || T < 0 || (int64_t)B * T > kMaxTokens) return NGRAM_ESHAPE;
  if (flags & ~(NGRAM_ADD_RESIDUAL | NGRAM_UPDATE_STATE | NGRAM_PREFETCHED | NGRAM_KEEP_FOR_BACKWARD))
    return NGRAM_EINVAL;
  if ((flags & NGRAM_PREFETCHED) && static_scratch) return NGRAM_EINVAL;
  const bool keep = flags & NGRAM_KEEP_FOR_BACKWARD;
  if (keep && (static_scratch || (flags & NGRAM_PREFETCHED))) return NGRAM_EINVAL;
  if (keep) {
    st = backward_shape_ok(cfg, (int64_t)B * T);
    if (st) return st;
  }
  if ((flags & NGRAM_UPDATE_STATE) && (conv_state == nullptr || state_pos == nullptr))
    return NGRAM_EINVAL;
  int64_t h_tok = 0;
  st = check_hidden_stride(cfg, hidden_branch_stride, &h_tok);
  if (st) return st;
  const int64_t n_tok = (int64_t)B * T;
  if (n_tok == 0) return NGRAM_OK;
  if (!raw_ids || !lut || !hidden || !w_k || !w_v || !conv_w || !out) return NGRAM_EINVAL;
  TablePtrs tp;
  st = check_tables(cfg, tables, &tp);
  if (st) return st;
  if (!aligned4(raw_ids) || !aligned4(history) || !aligned4(lut) || !aligned4(err_flag) ||
      !aligned4(state_pos))
    return NGRAM_EALIGN;
  for (const void* p : {hidden, w_k, w_v, conv_w, gamma_q, gamma_k, gamma_u,
                        (const void*)conv_state, (const void*)out, (const void*)gates})
    if (!aligned16(p)) return NGRAM_EALIGN;
  // keeping: the prefill route, its row ids, E, K and V where the backward
  // pass reads them (K / V fp32 [n, (nb+1) d]), its partials in a region the
  // backward fills only later
  Layout L = layout_for(cfg, n_tok, true, keep ? 0 : T);
  BwdLayout BL{};
  if (keep) {
    BL = bwd_layout(cfg, n_tok);
    L.row_idx = BL.row_idx;
    L.e = BL.e;
    L.v = BL.kv;
    L.v_stride = (int64_t)(cfg->n_branches + 1) * cfg->hidden_dim;
    L.v_offset = (int64_t)cfg->n_branches * cfg->hidden_dim;
    L.parts = BL.fparts;
    L.total = BL.total;
  }
  if (static_scratch) {  // ngram_forward_noalloc, after every other check
    if (L.total > NGRAM_NOALLOC_SCRATCH_BYTES) return NGRAM_ESCRATCH;
    workspace = device_scratch();
    if (workspace == nullptr) return NGRAM_EHIP;
    workspace_bytes = NGRAM_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace) return NGRAM_EWORKSPACE;
  if (workspace_bytes < L.total) return NGRAM_EWORKSPACE;
  if (!aligned16(workspace)) return NGRAM_EALIGN;

  char* ws = static_cast<char*>(workspace);
  void* e = ws + L.e;
  ConvArgs ca = conv_args_base(cfg);
  ca.conv_w = conv_w;
  ca.gamma_u = gamma_u;
  ca.state = conv_state;
  ca.state_pos = state_pos;
  ca.update_state = (flags & NGRAM_UPDATE_STATE) ? 1 : 0;
  ca.hidden = hidden;
  ca.h_tok_stride = h_tok;
  ca.h_branch_stride = hidden_branch_stride;
  ca.out = out;
  ca.gates = gates;
  ca.B = B;
  ca.T = T;
  ca.dil = cfg->conv_dilation;
  ca.add_residual = (flags & NGRAM_ADD_RESIDUAL) ? 1 : 0;
  if (L.k_split > 0) {
    // decode: hash + gather -> E, weight-stationary projection, decode finalize
    // (which reads the ring's taps and writes this position's row)
    float* split = reinterpret_cast<float*>(ws + L.split);
    if (!(flags & NGRAM_PREFETCHED)) {
      st = launch_lookup(cfg, L, raw_ids, B, T, history, lut, tp, err_flag, ws, s, tm);
      if (st) return st;
    }
    tm.stage(2);
    WstatArgs wa{};
    wa.e = static_cast<const bf16_bits*>(e);
    wa.wk = static_cast<const bf16_bits*>(w_k);
    wa.wv = static_cast<const bf16_bits*>(w_v);
    wa.M = n_tok;
    wa.K = cfg->mem_dim;
    wa.nb = cfg->n_branches;
    wa.d = cfg->hidden_dim;
    wa.split_out = split;
    st = hip_status(launch_projection_wstat(L.wplan, wa, s));
    if (st) return st;
    tm.stage(3);
    ca.gamma_q = gamma_q;
    ca.gamma_k = gamma_k;
    return hip_status(launch_decode_finalize(cfg->act_dtype, L.k_split, split, ca, s));
  }
  ProjArgs pa = proj_args(cfg, e, w_k, w_v, hidden, h_tok, hidden_branch_stride, gamma_q,
                          gamma_k, ws, L, n_tok);
  if (keep) {
    pa.k_keep = reinterpret_cast<float*>(ws + L.v);
    pa.v = pa.k_keep + L.v_offset;
    pa.v_ld = L.v_stride;
  }
  if (!(flags & NGRAM_PREFETCHED)) {
    st = launch_lookup(cfg, L, raw_ids, B, T, history, lut, tp, err_flag, ws, s, tm);
    if (st) return st;
  }
  tm.stage(2);
  st = hip_status(run_projection(cfg, L, pa, s));
  if (st) return st;
  tm.stage(3);
  ca.v = reinterpret_cast<const float*>(ws + L.v) + L.v_offset;
  ca.v_stride = L.v_stride;
  ca.parts = reinterpret_cast<const float*>(ws + L.parts);
  ca.np = L.plan.np;
  ca.tile = conv_tile_for(T);
  st = hip_status(launch_fused_conv(cfg->act_dtype, cfg->conv_dilation, ca, s));
  if (st) return st;
  // the ring's new rows, after every read of it by the conv
  if (ca.update_state)
    return hip_status(launch_state_update(cfg->act_dtype, true, cfg->conv_dilation, ca, s));
  return NGRAM_OK;
}

int backward_impl(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                  const int32_t* history, const int32_t* lut, const void* const* tables,
                  const void* hidden, int64_t hidden_branch_stride, const void* w_k,
                  const void* w_v, const void* conv_w, const void* gamma_q, const void* gamma_k,
                  const void* gamma_u, const float* conv_state, const int32_t* state_pos,
                  int32_t flags, const void* d_out, float* const* d_tables, float* d_w_k,
                  float* d_w_v, float* d_conv_w, float* d_hidden, float* d_gammas,
                  void* workspace, size_t workspace_bytes, hipStream_t s, Timer& tm) {
  int st = validate(cfg, false);
  if (st) return st;
  if (B < 0 || T < 0 || (int64_t)B * T > kMaxTokens) return NGRAM_ESHAPE;
  st = backward_shape_ok(cfg, (int64_t)B * T);
  if (st) return st;
  if (flags & ~(NGRAM_ADD_RESIDUAL | NGRAM_KEEP_FOR_BACKWARD)) return NGRAM_EINVAL;
  const bool kept = flags & NGRAM_KEEP_FOR_BACKWARD;
  int64_t h_tok = 0;
  st = check_hidden_stride(cfg, hidden_branch_stride, &h_tok);
  if (st) return st;
  const int64_t n = (int64_t)B * T;
  if (n == 0) return NGRAM_OK;
  if (!raw_ids || !lut || !hidden || !w_k || !w_v || !conv_w || !d_out || !d_tables || !d_w_k ||
      !d_w_v || !d_conv_w)
    return NGRAM_EINVAL;
  TablePtrs tp;
  st = check_tables(cfg, tables, &tp);
  if (st) return st;
  GradTablePtrs gp;
  memset(&gp, 0, sizeof gp);
  for (int j = 0; j < cfg->n_tables; ++j) {
    if (d_tables[j] == nullptr) return NGRAM_EINVAL;
    if (!aligned16(d_tables[j])) return NGRAM_EALIGN;
    gp.p[j] = d_tables[j];
  }
  if (!aligned4(raw_ids) || !aligned4(history) || !aligned4(lut) || !aligned4(state_pos))
    return NGRAM_EALIGN;
  for (const void* p : {hidden, w_k, w_v, conv_w, gamma_q, gamma_k, gamma_u, d_out,
                        (const void*)conv_state, (const void*)d_w_k, (const void*)d_w_v,
                        (const void*)d_conv_w, (const void*)d_hidden, (const void*)d_gammas})
    if (!aligned16(p)) return NGRAM_EALIGN;
  const BwdLayout L = bwd_layout(cfg, n);
  const int nb = cfg->n_branches, d = cfg->hidden_dim, mem = cfg->mem_dim;
  const int64_t N64 = (int64_t)(nb + 1) * d;
  if (!workspace || workspace_bytes < L.total) return NGRAM_EWORKSPACE;
  if (!aligned16(workspace)) return NGRAM_EALIGN;

  char* ws = static_cast<char*>(workspace);
  const int32_t N = (int32_t)N64;
  int32_t* row_idx = reinterpret_cast<int32_t*>(ws + L.row_idx);
  bf16_bits* e = reinterpret_cast<bf16_bits*>(ws + L.e);
  float* kv = reinterpret_cast<float*>(ws + L.kv);
  bf16_bits* dkv = reinterpret_cast<bf16_bits*>(ws + L.dkv);
  bf16_bits* wt = reinterpret_cast<bf16_bits*>(ws + L.wt);
  float* de = reinterpret_cast<float*>(ws + L.de);
  const bf16_bits* wk = static_cast<const bf16_bits*>(w_k);
  const bf16_bits* wv = static_cast<const bf16_bits*>(w_v);

  // recompute: row ids, E, and K / V in fp32 (unless a forward kept them here)
  if (!kept) {
    tm.stage(0);
    const HashArgs ha = hash_args(cfg, cfg->orders[cfg->n_orders - 1] - 1);
    st = hip_status(launch_hash(true, raw_ids, B, T, history, lut, ha, row_idx, nullptr, s));
    if (st) return st;
    st = hip_status(
        launch_gather(cfg->table_dtype, row_idx, n, cfg->n_tables, cfg->row_dim, tp, e, s));
    if (st) return st;
    st = hip_status(raw_gemm(e, n, mem, wk, wv, nb, d, kv, N, s));
    if (st) return st;
  }
  // the per-row backward: gates, conv, RMSNorms -> dK, dV (bf16), d_hidden, d_conv_w, d_gammas
  tm.stage(1);
  BwdArgs ba;
  memset(&ba, 0, sizeof ba);
  ba.n = n;
  ba.T = T;
  ba.nb = nb;
  ba.d = d;
  ba.dil = cfg->conv_dilation;
  ba.eps = cfg->rms_eps;
  ba.hidden = static_cast<const bf16_bits*>(hidden);
  ba.h_tok = h_tok;
  ba.h_br = hidden_branch_stride;
  ba.kv = kv;
  ba.kv_ld = N;
  ba.stats = reinterpret_cast<float*>(ws + L.stats);
  ba.dc = reinterpret_cast<float*>(ws + L.dc);
  ba.d_out = static_cast<const bf16_bits*>(d_out);
  ba.conv_w = static_cast<const bf16_bits*>(conv_w);
  ba.gamma_q = static_cast<const bf16_bits*>(gamma_q);
  ba.gamma_k = static_cast<const bf16_bits*>(gamma_k);
  ba.gamma_u = static_cast<const bf16_bits*>(gamma_u);
  ba.state = conv_state;
  ba.state_pos = state_pos;
  ba.add_residual = (flags & NGRAM_ADD_RESIDUAL) ? 1 : 0;
  ba.dkv = dkv;
  ba.dkv_ld = N;
  ba.d_hidden = d_hidden;
  ba.part_conv = reinterpret_cast<float*>(ws + L.part);
  ba.part_gain = d_gammas ? ba.part_conv + (size_t)kBwdBlocks * 4 * d : nullptr;
  st = hip_status(launch_bwd_rows(ba, d_conv_w, d_gammas, reinterpret_cast<float*>(ws + L.rtmp),
                                  s));
  if (st) return st;
  // dE = [dK dV] [W_K; W_V]: the weights transposed to [mem, N] feed the product
  tm.stage(2);
  st = hip_status(launch_transpose_bf16(wk, (int64_t)nb * d, mem, mem, wt, (int64_t)nb * d, N, s));
  if (st) return st;
  st = hip_status(launch_transpose_bf16(wv, d, mem, mem, wt + (int64_t)nb * d, d, N, s));
  if (st) return st;
  st = hip_status(raw_gemm(dkv, n, N, nullptr, wt, 0, mem, de, mem, s));
  if (st) return st;
  // dW = [dK dV]^T E over n_pad tokens, both operands read as they lie (a row
  // per token) by the K-outer product
  tm.stage(3);
  // the tokens past n contribute nothing: zero rows of both operands
  if (L.n_pad > n) {
    st = hip_status(launch_zero_f32(reinterpret_cast<float*>(dkv + n * N), (L.n_pad - n) * N / 2, s));
    if (st) return st;
    st = hip_status(launch_zero_f32(reinterpret_cast<float*>(e + n * mem), (L.n_pad - n) * mem / 2, s));
    if (st) return st;
  }
  // one split-K product for every row of [dK dV]^T, the splits summed into d_w_k and d_w_v
  float* dw = reinterpret_cast<float*>(ws + L.dw);
  {
    AsyncProjArgs a;
    memset(&a, 0, sizeof a);
    a.e = dkv;
    a.wv = e;
    a.tn_lda = N;
    a.tn_ldb = mem;
    a.epi.M = N;
    a.epi.d = mem;
    a.K = (int32_t)L.n_pad;
    a.group_m = 4;
    a.raw_out = dw;
    a.raw_ld = mem;
    a.raw_split = L.dw_split;
    a.raw_split_stride = N64 * mem;
    st = hip_status(launch_projection_raw_tn(a, s));
  }
  if (st) return st;
  const int64_t kw = (int64_t)nb * d * mem;
  st = hip_status(launch_sum_splits(dw, L.dw_split, N64 * mem, kw, d_w_k, s));
  if (st) return st;
  st = hip_status(launch_sum_splits(dw + kw, L.dw_split, N64 * mem, (int64_t)d * mem, d_w_v, s));
  if (st) return st;
  // the gather's adjoint, each row's contributions added in token order
  return hip_status(launch_table_grad(row_idx, n, cfg->n_tables, cfg->row_dim, cfg->rows, de, gp,
                                      ws + L.tgrad, s));
}

}  // namespace

extern "C" {

const char* ngram_status_str(int status) {
  switch (status) {
    case NGRAM_OK: return "NGRAM_OK";
    case NGRAM_EINVAL: return "NGRAM_EINVAL: null pointer or inconsistent configuration";
    case NGRAM_ESHAPE: return "NGRAM_ESHAPE: size out of range or not a supported multiple";
    case NGRAM_EDTYPE: return "NGRAM_EDTYPE: unsupported dtype or dtype combination";
    case NGRAM_EALIGN: return "NGRAM_EALIGN: device pointer not aligned";
    case NGRAM_ERANGE: return "NGRAM_ERANGE: table rows not prime or out of range";
    case NGRAM_EHIP: return "NGRAM_EHIP: HIP launch failed";
    case NGRAM_EWORKSPACE: return "NGRAM_EWORKSPACE: workspace missing or too small";
    case NGRAM_ESCRATCH:
      return "NGRAM_ESCRATCH: the call needs more scratch than ngram_forward_noalloc holds "
             "(NGRAM_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown ngram status";
  }
}

int ngram_abi_version(void) { return kAbiVersion; }

int ngram_config_validate(const ngram_config* cfg) { return validate(cfg, true); }

int ngram_compress_ids(const ngram_config* cfg, const int32_t* raw_ids, int64_t n,
                       const int32_t* lut, int32_t* comp_ids, int32_t* err_flag, void* stream) {
  int st = validate(cfg, false);
  if (st) return st;
  if (n < 0) return NGRAM_ESHAPE;
  if (n == 0) return NGRAM_OK;
  if (!raw_ids || !lut || !comp_ids) return NGRAM_EINVAL;
  if (!aligned4(raw_ids) || !aligned4(lut) || !aligned4(comp_ids) || !aligned4(err_flag))
    return NGRAM_EALIGN;
  return hip_status(launch_compress(raw_ids, n, lut, cfg->vocab, cfg->vocab_compressed,
                                    cfg->pad_id, comp_ids, err_flag,
                                    static_cast<hipStream_t>(stream)));
}

int ngram_hash(const ngram_config* cfg, const int32_t* comp_ids, int32_t B, int32_t T,
               const int32_t* history, int32_t* row_idx, void* stream) {
  int st = validate(cfg, false);
  if (st) return st;
  if (B < 0 || T < 0 || (int64_t)B * T > kMaxTokens) return NGRAM_ESHAPE;
  if ((int64_t)B * T == 0) return NGRAM_OK;
  if (!comp_ids || !row_idx) return NGRAM_EINVAL;
  if (!aligned4(comp_ids) || !aligned4(row_idx) || !aligned4(history)) return NGRAM_EALIGN;
  const HashArgs a = hash_args(cfg, cfg->orders[cfg->n_orders - 1] - 1);
  return hip_status(launch_hash(false, comp_ids, B, T, history, nullptr, a, row_idx, nullptr,
                                static_cast<hipStream_t>(stream)));
}

int ngram_gather(const ngram_config* cfg, const int32_t* row_idx, int64_t n_tok,
                 const void* const* tables, void* mem, void* stream) {
  int st = validate(cfg, false);
  if (st) return st;
  if (n_tok < 0 || n_tok > kMaxTokens) return NGRAM_ESHAPE;
  if (n_tok == 0) return NGRAM_OK;
  if (!row_idx || !mem) return NGRAM_EINVAL;
  TablePtrs tp;
  st = check_tables(cfg, tables, &tp);
  if (st) return st;
  if (!aligned4(row_idx) || !aligned16(mem)) return NGRAM_EALIGN;
  return hip_status(launch_gather(cfg->table_dtype, row_idx, n_tok, cfg->n_tables, cfg->row_dim,
                                  tp, mem, static_cast<hipStream_t>(stream)));
}

size_t ngram_gate_workspace_size(const ngram_config* cfg, int64_t n_tok) {
  if (validate(cfg, false) != NGRAM_OK || n_tok < 0 || n_tok > kMaxTokens) return 0;
  return layout_for(cfg, n_tok, false).total;
}

int ngram_gate(const ngram_config* cfg, const void* hidden, int64_t hidden_branch_stride,
               const void* mem, const void* w_k, const void* w_v, const void* gamma_q,
               const void* gamma_k, int64_t n_tok, float* gates, void* u, void* workspace,
               size_t workspace_bytes, void* stream) {
  int st = validate(cfg, false);
  if (st) return st;
  if (n_tok < 0 || n_tok > kMaxTokens) return NGRAM_ESHAPE;
  int64_t h_tok = 0;
  st = check_hidden_stride(cfg, hidden_branch_stride, &h_tok);
  if (st) return st;
  if (n_tok == 0) return NGRAM_OK;
  if (!hidden || !mem || !w_k || !w_v || !gates) return NGRAM_EINVAL;
  for (const void* p : {hidden, mem, w_k, w_v, gamma_q, gamma_k, (const void*)gates, (const void*)u})
    if (!aligned16(p)) return NGRAM_EALIGN;
  const Layout L = layout_for(cfg, n_tok, false);
  if (!workspace) return NGRAM_EWORKSPACE;
  if (workspace_bytes < L.total) return NGRAM_EWORKSPACE;
  if (!aligned16(workspace)) return NGRAM_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const ProjArgs pa = proj_args(cfg, mem, w_k, w_v, hidden, h_tok, hidden_branch_stride, gamma_q,
                                gamma_k, ws, L, n_tok);
  st = hip_status(run_projection(cfg, L, pa, s));
  if (st) return st;
  ConvArgs ca = conv_args_base(cfg);
  ca.v = reinterpret_cast<const float*>(ws + L.v) + L.v_offset;
  ca.v_stride = L.v_stride;
  ca.parts = reinterpret_cast<const float*>(ws + L.parts);
  ca.np = L.plan.np;
  ca.out = u;
  ca.gates = gates;
  return hip_status(launch_gate_values(cfg->act_dtype, ca, n_tok, s));
}

int ngram_causal_conv(const ngram_config* cfg, const void* u, int32_t B, int32_t T,
                      const void* conv_w, const void* gamma_u, float* conv_state,
                      int32_t* state_pos, int32_t flags, void* out, void* stream) {
  int st = validate(cfg, false);
  if (st) return st;
  if (B < 0 || T < 0 || (int64_t)B * T > kMaxTokens) return NGRAM_ESHAPE;
  if (flags & ~NGRAM_UPDATE_STATE) return NGRAM_EINVAL;
  if ((flags & NGRAM_UPDATE_STATE) && (conv_state == nullptr || state_pos == nullptr))
    return NGRAM_EINVAL;
  if ((int64_t)B * T == 0) return NGRAM_OK;
  if (!u || !conv_w || !out) return NGRAM_EINVAL;
  for (const void* p : {u, conv_w, gamma_u, (const void*)conv_state, (const void*)out})
    if (!aligned16(p)) return NGRAM_EALIGN;
  if (!aligned4(state_pos)) return NGRAM_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ConvArgs ca = conv_args_base(cfg);
  ca.u = u;
  ca.conv_w = conv_w;
  ca.gamma_u = gamma_u;
  ca.state = conv_state;
  ca.state_pos = state_pos;
  ca.update_state = (flags & NGRAM_UPDATE_STATE) ? 1 : 0;
  ca.out = out;
  ca.B = B;
  ca.T = T;
  ca.tile = conv_tile_for(T);
  st = hip_status(launch_op_conv(cfg->act_dtype, cfg->conv_dilation, ca, s));
  if (st || !ca.update_state) return st;
  return hip_status(launch_state_update(cfg->act_dtype, false, cfg->conv_dilation, ca, s));
}

size_t ngram_forward_workspace_size(const ngram_config* cfg, int32_t B, int32_t T) {
  if (validate(cfg, false) != NGRAM_OK || B < 0 || T < 0 || (int64_t)B * T > kMaxTokens) return 0;
  return layout_for(cfg, (int64_t)B * T, true, T).total;
}

int ngram_forward_workspace_view(const ngram_config* cfg, int32_t B, int32_t T,
                                 ngram_workspace_view* view) {
  int st = validate(cfg, false);
  if (st) return st;
  if (B < 0 || T < 0 || (int64_t)B * T > kMaxTokens) return NGRAM_ESHAPE;
  if (view == nullptr) return NGRAM_EINVAL;
  const Layout L = layout_for(cfg, (int64_t)B * T, true, T);
  view->row_idx_offset = (int64_t)L.row_idx;
  view->mem_offset = (int64_t)L.e;
  view->mem_layout = L.k_split > 0 ? NGRAM_MEM_TILES16 : NGRAM_MEM_ROWS;
  view->reserved = 0;
  return NGRAM_OK;
}

int ngram_forward(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                  const int32_t* history, const int32_t* lut, const void* const* tables,
                  const void* hidden, int64_t hidden_branch_stride, const void* w_k,
                  const void* w_v, const void* conv_w, const void* gamma_q,
                  const void* gamma_k, const void* gamma_u, float* conv_state,
                  int32_t* state_pos, int32_t flags, void* out, float* gates,
                  int32_t* err_flag, void* workspace, size_t workspace_bytes, void* stream) {
  Timer tm;
  return forward_impl(cfg, raw_ids, B, T, history, lut, tables, hidden, hidden_branch_stride,
                      w_k, w_v, conv_w, gamma_q, gamma_k, gamma_u, conv_state, state_pos, flags,
                      out, gates, err_flag, workspace, workspace_bytes,
                      static_cast<hipStream_t>(stream), tm);
}

int ngram_forward_prefetch(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                           const int32_t* history, const int32_t* lut, const void* const* tables,
                           int32_t* err_flag, void* workspace, size_t workspace_bytes,
                           void* stream) {
  int st = validate(cfg, false);
  if (st) return st;
  if (B < 0 || T < 0 || (int64_t)B * T > kMaxTokens) return NGRAM_ESHAPE;
  const int64_t n_tok = (int64_t)B * T;
  if (n_tok == 0) return NGRAM_OK;
  if (!raw_ids || !lut) return NGRAM_EINVAL;
  TablePtrs tp;
  st = check_tables(cfg, tables, &tp);
  if (st) return st;
  if (!aligned4(raw_ids) || !aligned4(history) || !aligned4(lut) || !aligned4(err_flag))
    return NGRAM_EALIGN;
  const Layout L = layout_for(cfg, n_tok, true, T);
  if (!workspace || workspace_bytes < L.total) return NGRAM_EWORKSPACE;
  if (!aligned16(workspace)) return NGRAM_EALIGN;
  Timer tm;
  return launch_lookup(cfg, L, raw_ids, B, T, history, lut, tp, err_flag,
                       static_cast<char*>(workspace), static_cast<hipStream_t>(stream), tm);
}

int ngram_forward_noalloc(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                          const int32_t* history, const int32_t* lut, const void* const* tables,
                          const void* hidden, int64_t hidden_branch_stride, const void* w_k,
                          const void* w_v, const void* conv_w, const void* gamma_q,
                          const void* gamma_k, const void* gamma_u, float* conv_state,
                          int32_t* state_pos, int32_t flags, void* out, float* gates,
                          int32_t* err_flag, void* stream) {
  Timer tm;
  return forward_impl(cfg, raw_ids, B, T, history, lut, tables, hidden, hidden_branch_stride,
                      w_k, w_v, conv_w, gamma_q, gamma_k, gamma_u, conv_state, state_pos, flags,
                      out, gates, err_flag, nullptr, 0, static_cast<hipStream_t>(stream), tm,
                      true);
}

int ngram_forward_timed(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                        const int32_t* history, const int32_t* lut, const void* const* tables,
                        const void* hidden, int64_t hidden_branch_stride, const void* w_k,
                        const void* w_v, const void* conv_w, const void* gamma_q,
                        const void* gamma_k, const void* gamma_u, float* conv_state,
                        int32_t* state_pos, int32_t flags, void* out, float* gates,
                        int32_t* err_flag, void* workspace, size_t workspace_bytes,
                        void* stream, void* const* stage_events, int32_t* stage_mask) {
  if (stage_events == nullptr) return NGRAM_EINVAL;
  for (int i = 0; i < 2 * NGRAM_N_STAGES; ++i)
    if (stage_events[i] == nullptr) return NGRAM_EINVAL;
  int st;
  int mask;
  {
    Timer tm;
    tm.ev = reinterpret_cast<const hipEvent_t*>(stage_events);
    st = forward_impl(cfg, raw_ids, B, T, history, lut, tables, hidden, hidden_branch_stride,
                      w_k, w_v, conv_w, gamma_q, gamma_k, gamma_u, conv_state, state_pos, flags,
                      out, gates, err_flag, workspace, workspace_bytes,
                      static_cast<hipStream_t>(stream), tm);
    tm.close();
    mask = tm.mask;
  }
  if (stage_mask) *stage_mask = mask;
  return st;
}

size_t ngram_backward_workspace_size(const ngram_config* cfg, int32_t B, int32_t T) {
  if (validate(cfg, false) != NGRAM_OK || B < 0 || T < 0 || (int64_t)B * T > kMaxTokens) return 0;
  return bwd_layout(cfg, (int64_t)B * T).total;
}

int ngram_backward(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                   const int32_t* history, const int32_t* lut, const void* const* tables,
                   const void* hidden, int64_t hidden_branch_stride, const void* w_k,
                   const void* w_v, const void* conv_w, const void* gamma_q,
                   const void* gamma_k, const void* gamma_u, const float* conv_state,
                   const int32_t* state_pos, int32_t flags, const void* d_out,
                   float* const* d_tables, float* d_w_k, float* d_w_v, float* d_conv_w,
                   float* d_hidden, float* d_gammas, void* workspace, size_t workspace_bytes,
                   void* stream) {
  Timer tm;
  return backward_impl(cfg, raw_ids, B, T, history, lut, tables, hidden, hidden_branch_stride,
                       w_k, w_v, conv_w, gamma_q, gamma_k, gamma_u, conv_state, state_pos, flags,
                       d_out, d_tables, d_w_k, d_w_v, d_conv_w, d_hidden, d_gammas, workspace,
                       workspace_bytes, static_cast<hipStream_t>(stream), tm);
}

int ngram_backward_timed(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                         const int32_t* history, const int32_t* lut, const void* const* tables,
                         const void* hidden, int64_t hidden_branch_stride, const void* w_k,
                         const void* w_v, const void* conv_w, const void* gamma_q,
                         const void* gamma_k, const void* gamma_u, const float* conv_state,
                         const int32_t* state_pos, int32_t flags, const void* d_out,
                         float* const* d_tables, float* d_w_k, float* d_w_v, float* d_conv_w,
                         float* d_hidden, float* d_gammas, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* stage_events,
                         int32_t* stage_mask) {
  if (stage_events == nullptr) return NGRAM_EINVAL;
  for (int i = 0; i < 2 * NGRAM_N_STAGES; ++i)
    if (stage_events[i] == nullptr) return NGRAM_EINVAL;
  int st;
  int mask;
  {
    Timer tm;
    tm.ev = reinterpret_cast<const hipEvent_t*>(stage_events);
    st = backward_impl(cfg, raw_ids, B, T, history, lut, tables, hidden, hidden_branch_stride,
                       w_k, w_v, conv_w, gamma_q, gamma_k, gamma_u, conv_state, state_pos, flags,
                       d_out, d_tables, d_w_k, d_w_v, d_conv_w, d_hidden, d_gammas, workspace,
                       workspace_bytes, static_cast<hipStream_t>(stream), tm);
    tm.close();
    mask = tm.mask;
  }
  if (stage_mask) *stage_mask = mask;
  return st;
}

}  // extern "C"
