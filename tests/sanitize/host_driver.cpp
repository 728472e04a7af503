// Drives the host side of libngram.so -- configuration validation, workspace
// sizes and views, and every entry point's argument checks -- for a build
// whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer.
// Every call here is refused before any HIP call (fake device pointers are
// never dereferenced); each must return the documented status.  Test code
// only; no GPU is needed.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "ngram.h"

static int failures = 0;
#define EXPECT(call, want)                                                        \
  do {                                                                            \
    const long got_ = (long)(call);                                               \
    if (got_ != (long)(want)) {                                                   \
      fprintf(stderr, "line %d: %s = %ld, want %ld\n", __LINE__, #call, got_, (long)(want)); \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

static ngram_config qwen(int heads, int row_dim, int nb, int dtype) {
  ngram_config c;
  memset(&c, 0, sizeof c);
  c.n_orders = 2;
  c.orders[0] = 2;
  c.orders[1] = 3;
  c.heads_per_order = heads;
  c.n_tables = 2 * heads;
  static const int64_t primes[16] = {20000003, 20000023, 20000033, 20000047, 20000059, 20000063,
                                     20000069, 20000077, 20000081, 20000093, 20000107, 20000147,
                                     20000153, 20000159, 20000161, 20000171};
  for (int j = 0; j < c.n_tables; ++j) {
    c.rows[j] = primes[j];
    for (int i = 0; i < 4; ++i) c.hash_mult[j][i] = 0x9E3779B97F4A7C15ull * (j * 4 + i + 1) | 1u;
    c.table_scale[j] = 0.25f;
  }
  c.row_dim = row_dim;
  c.mem_dim = c.n_tables * row_dim;
  c.hidden_dim = 2560;
  c.n_branches = nb;
  c.conv_kernel = 4;
  c.conv_dilation = 3;
  c.vocab = 248320;
  c.vocab_compressed = 191206;
  c.pad_id = 0;
  c.rms_eps = 1e-6f;
  c.table_dtype = dtype;
  c.act_dtype = dtype == NGRAM_FP8_E4M3 ? NGRAM_BF16 : dtype;
  c.w_layout = NGRAM_W_D_MEM;
  return c;
}

int main() {
  void* fake = (void*)0x10000;
  void* odd = (void*)0x10004;
  const void* tabs[16];
  for (int j = 0; j < 16; ++j) tabs[j] = fake;

  // configurations: valid ones, then one broken field at a time
  ngram_config ok = qwen(4, 320, 1, NGRAM_BF16);
  EXPECT(ngram_config_validate(&ok), NGRAM_OK);
  ngram_config g16 = qwen(8, 160, 1, NGRAM_BF16);
  EXPECT(ngram_config_validate(&g16), NGRAM_OK);
  ngram_config mb = qwen(4, 320, 4, NGRAM_BF16);
  EXPECT(ngram_config_validate(&mb), NGRAM_OK);
  ngram_config f8 = qwen(4, 320, 1, NGRAM_FP8_E4M3);
  EXPECT(ngram_config_validate(&f8), NGRAM_OK);
  ngram_config c = ok;
  c.rows[3] = 20000001;  // 3 x 6666667
  EXPECT(ngram_config_validate(&c), NGRAM_ERANGE);
  c = ok;
  c.rows[0] = 4294967311ll;
  EXPECT(ngram_config_validate(&c), NGRAM_ERANGE);
  c = ok;
  c.n_orders = 0;
  EXPECT(ngram_config_validate(&c), NGRAM_EINVAL);
  c = ok;
  c.n_orders = 5;
  EXPECT(ngram_config_validate(&c), NGRAM_EINVAL);
  c = ok;
  c.heads_per_order = 9;
  c.n_tables = 18;
  EXPECT(ngram_config_validate(&c), NGRAM_ESHAPE);
  c = ok;
  c.row_dim = -8;
  EXPECT(ngram_config_validate(&c), NGRAM_ESHAPE);
  c = ok;
  c.hidden_dim = 1 << 30;
  EXPECT(ngram_config_validate(&c), NGRAM_ESHAPE);
  c = ok;
  c.table_dtype = 99;
  EXPECT(ngram_config_validate(&c), NGRAM_EDTYPE);
  c = ok;
  c.tune_decode_ni = 5;
  c.tune_decode_split = 3;
  EXPECT(ngram_config_validate(&c), NGRAM_EINVAL);
  c = ok;
  c.tune_proj_plan = -3;
  EXPECT(ngram_config_validate(&c), NGRAM_EINVAL);
  c = f8;
  c.table_scale[5] = -1.0f;
  EXPECT(ngram_config_validate(&c), NGRAM_EINVAL);
  EXPECT(ngram_config_validate(nullptr), NGRAM_EINVAL);

  // sizes and views over a range of shapes, including empty and oversized ones
  const int32_t shapes[][2] = {{0, 0},   {1, 1},      {256, 1}, {2048, 1}, {2049, 1},
                               {1, 262144}, {16, 8192}, {3, 77},  {-1, 4},   {1 << 20, 1 << 10}};
  for (const ngram_config* cfg : {&ok, &g16, &mb, &f8}) {
    for (const auto& s : shapes) {
      const size_t ws = ngram_forward_workspace_size(cfg, s[0], s[1]);
      ngram_workspace_view v;
      const int st = ngram_forward_workspace_view(cfg, s[0], s[1], &v);
      if (s[0] < 0 || (int64_t)s[0] * s[1] > (int64_t(1) << 28)) {
        EXPECT(ws, 0);
        EXPECT(st, NGRAM_ESHAPE);
      } else if (st == NGRAM_OK && (int64_t)s[0] * s[1] > 0) {
        if (!(v.row_idx_offset >= 0 && v.mem_offset >= 0 && (size_t)v.row_idx_offset < ws &&
              (size_t)v.mem_offset < ws)) {
          fprintf(stderr, "view outside the workspace\n");
          ++failures;
        }
      }
      (void)ngram_backward_workspace_size(cfg, s[0], s[1]);
      (void)ngram_gate_workspace_size(cfg, (int64_t)s[0] * (s[1] > 0 ? s[1] : 0));
    }
  }
  EXPECT(ngram_forward_workspace_view(&ok, 4, 4, nullptr), NGRAM_EINVAL);

  // every entry point refuses bad arguments before any launch
  ngram_config t = ok;
  const size_t need = ngram_forward_workspace_size(&t, 256, 1);
  int32_t mask = -1;
  void* ev[8] = {fake, fake, fake, fake, fake, fake, fake, fake};
  EXPECT(ngram_compress_ids(&t, nullptr, 10, (int32_t*)fake, (int32_t*)fake, nullptr, nullptr),
         NGRAM_EINVAL);
  EXPECT(ngram_compress_ids(&t, (int32_t*)fake, -1, (int32_t*)fake, (int32_t*)fake, nullptr,
                            nullptr), NGRAM_ESHAPE);
  EXPECT(ngram_hash(&t, (int32_t*)fake, 2, 4, nullptr, nullptr, nullptr), NGRAM_EINVAL);
  EXPECT(ngram_gather(&t, (int32_t*)fake, 4, nullptr, fake, nullptr), NGRAM_EINVAL);
  EXPECT(ngram_gather(&t, (int32_t*)fake, 4, tabs, odd, nullptr), NGRAM_EALIGN);
  EXPECT(ngram_gate(&t, fake, 7, fake, fake, fake, nullptr, nullptr, 16, (float*)fake, nullptr,
                    fake, 1 << 20, nullptr), NGRAM_ESHAPE);
  EXPECT(ngram_causal_conv(&t, fake, 1, 8, fake, nullptr, (float*)fake, nullptr,
                           NGRAM_UPDATE_STATE, fake, nullptr), NGRAM_EINVAL);
  EXPECT(ngram_forward(&t, (int32_t*)fake, 256, 1, nullptr, (int32_t*)fake, tabs, fake, 0, fake,
                       fake, fake, nullptr, nullptr, nullptr, nullptr, nullptr, 0, fake, nullptr,
                       nullptr, fake, need - 1, nullptr), NGRAM_EWORKSPACE);
  EXPECT(ngram_forward(&t, (int32_t*)fake, 256, 1, nullptr, (int32_t*)fake, tabs, fake, 0, fake,
                       fake, fake, nullptr, nullptr, nullptr, (float*)fake, nullptr,
                       NGRAM_UPDATE_STATE, fake, nullptr, nullptr, fake, need, nullptr),
         NGRAM_EINVAL);
  EXPECT(ngram_forward_timed(&t, (int32_t*)fake, 256, 1, nullptr, (int32_t*)fake, tabs, fake, 0,
                             fake, fake, fake, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                             fake, nullptr, nullptr, fake, need - 1, nullptr, ev, &mask),
         NGRAM_EWORKSPACE);
  EXPECT(mask, 0);
  EXPECT(ngram_forward_timed(&t, (int32_t*)fake, 256, 1, nullptr, (int32_t*)fake, tabs, fake, 0,
                             fake, fake, fake, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                             fake, nullptr, nullptr, fake, need, nullptr, nullptr, &mask),
         NGRAM_EINVAL);
  EXPECT(ngram_forward_noalloc(&t, (int32_t*)fake, 1, 8192, nullptr, (int32_t*)fake, tabs, fake, 0,
                               fake, fake, fake, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                               fake, nullptr, nullptr, nullptr), NGRAM_ESCRATCH);
  EXPECT(ngram_forward_noalloc(&t, (int32_t*)fake, 256, 1, nullptr, (int32_t*)fake, tabs, fake, 0,
                               fake, fake, fake, nullptr, nullptr, nullptr, nullptr, nullptr,
                               NGRAM_PREFETCHED, fake, nullptr, nullptr, nullptr), NGRAM_EINVAL);
  EXPECT(ngram_forward_prefetch(&t, (int32_t*)fake, 256, 1, nullptr, (int32_t*)fake, tabs, nullptr,
                                fake, need - 1, nullptr), NGRAM_EWORKSPACE);
  EXPECT(ngram_forward_prefetch(&t, (int32_t*)fake, 256, 1, nullptr, nullptr, tabs, nullptr, fake,
                                need, nullptr), NGRAM_EINVAL);
  EXPECT(ngram_forward_prefetch(&t, (int32_t*)fake, 256, 1, nullptr, (int32_t*)fake, tabs, nullptr,
                                odd, need, nullptr), NGRAM_EALIGN);
  // keeping the intermediates for a backward: a backward workspace, no prefetch
  EXPECT(ngram_forward(&t, (int32_t*)fake, 256, 1, nullptr, (int32_t*)fake, tabs, fake, 0, fake,
                       fake, fake, nullptr, nullptr, nullptr, nullptr, nullptr,
                       NGRAM_KEEP_FOR_BACKWARD, fake, nullptr, nullptr, fake, need, nullptr),
         NGRAM_EWORKSPACE);
  EXPECT(ngram_forward(&t, (int32_t*)fake, 256, 1, nullptr, (int32_t*)fake, tabs, fake, 0, fake,
                       fake, fake, nullptr, nullptr, nullptr, nullptr, nullptr,
                       NGRAM_KEEP_FOR_BACKWARD | NGRAM_PREFETCHED, fake, nullptr, nullptr, fake,
                       (size_t)1 << 40, nullptr),
         NGRAM_EINVAL);
  float* gt[16];
  for (int j = 0; j < 16; ++j) gt[j] = (float*)fake;
  EXPECT(ngram_backward(&t, (int32_t*)fake, 4, 64, nullptr, (int32_t*)fake, tabs, fake, 0, fake,
                        fake, fake, nullptr, nullptr, nullptr, nullptr, nullptr, NGRAM_UPDATE_STATE,
                        fake, gt, (float*)fake, (float*)fake, (float*)fake, nullptr, nullptr,
                        fake, 1 << 30, nullptr), NGRAM_EINVAL);
  ngram_config big = qwen(4, 320, 4, NGRAM_BF16);  // (nb+1) d mem past 2^31: refused
  big.hidden_dim = 4096;
  big.row_dim = 16384;
  big.mem_dim = 8 * 16384;
  EXPECT(ngram_backward(&big, (int32_t*)fake, 1, 64, nullptr, (int32_t*)fake, tabs, fake, 0, fake,
                        fake, fake, nullptr, nullptr, nullptr, nullptr, nullptr, 0, fake, gt,
                        (float*)fake, (float*)fake, (float*)fake, nullptr, nullptr, fake,
                        (size_t)1 << 40, nullptr), NGRAM_ESHAPE);
  EXPECT(ngram_forward(&big, (int32_t*)fake, 1, 64, nullptr, (int32_t*)fake, tabs, fake, 0, fake,
                       fake, fake, nullptr, nullptr, nullptr, nullptr, nullptr,
                       NGRAM_KEEP_FOR_BACKWARD, fake, nullptr, nullptr, fake, (size_t)1 << 40,
                       nullptr),
         NGRAM_ESHAPE);
  for (int s = -9; s <= 1; ++s) (void)ngram_status_str(s);
  EXPECT(ngram_abi_version(), 7);
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("host driver: every check ran clean\n");
  return 0;
}
