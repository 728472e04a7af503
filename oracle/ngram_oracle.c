/*
 * ORACLE for the hashed N-gram embedding layer -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU definition of what the layer computes,
 * used to check the GPU library.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.  It
 * shares no source, header, table or helper with the GPU library.
 *
 * All floating point is IEEE double on values that are exact conversions of
 * the fp32 / bf16 inputs; loops only, no BLAS, no blocking or reordering.
 *
 * Sources (page title, then the part of it followed):
 *  [A] "Qwen 4用上DeepSeek的Engram！125B MoE一张4090能跑不用量化" (yktysq.com),
 *      section "DeepSeek Engram 更复杂，Qwen 更精简": Engram's four components
 *      (tokenizer compression; multi-head hashing into prime-sized tables and
 *      concatenation; context-aware gating; kernel-4 causal conv with dilation
 *      = max n-gram order; multi-branch sharing of table and value projection).
 *  [B] "Qwen3.8-Flash-Next 深度研究：把容量从「计算」搬到「存储」" (zhichai.net),
 *      §2.3 "Embedding：N-gram Embedding": the lookup (2-gram heads on
 *      (x_{t-1}, x_t), 3-gram heads on (x_{t-2}, x_{t-1}, x_t)), concatenation
 *      into E_t, and the layer formula E_t -> K_t, V_t; g_t = Gate(Norm(Q_t),
 *      Norm(K_t)); U_t = g_t * V_t; Delta_t = U_t + SiLU(DWConv(RMSNorm(U_t))).
 *  [C] same page, §3-D lineage table: the related Over-Encoding method hashes
 *      by a modulus.
 *  [D] same page, §9.3: the FP8 release stores the N-gram table in FP8 with a
 *      per-tensor scale (a loader that dropped the scale broke the model).
 *
 * Readings where the pages leave a step open (each is the plainest one the
 * rest of the text supports):
 *  - hash: key = XOR_i (uint64 c_{t-i} * A_{j,i}) mod 2^64, row = key mod p_j,
 *    with the odd multipliers A passed in by the caller;
 *  - positions before a sequence's start take the caller's history ids, else
 *    the pad id;
 *  - RMSNorm(x) = gamma * x / sqrt(mean(x^2) + eps); the gate's scaled dot
 *    product divides by sqrt(d); the gate is the logistic sigmoid;
 *  - conv tap i multiplies position t - i*dilation, depthwise, no bias, zero
 *    before the sequence start (or the caller's normalised state rows);
 *  - FP8 table values are OCP E4M3 times the table's scale, held in E as
 *    bf16 (product rounded to fp32, then to bf16).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2 };

static double load_value(const void* base, int dtype, int64_t i) {
  if (dtype == ORC_F32) return (double)((const float*)base)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * Step 1 -- tokenizer compression [A, first component]: c = LUT[x].
 * An id outside [0, vocab) or a LUT entry outside [0, vocab_c) is invalid; it
 * becomes pad_id.  Returns the number of invalid ids.
 */
int64_t orc_compress(const int32_t* raw, int64_t n, const int32_t* lut, int32_t vocab,
                     int32_t vocab_c, int32_t pad_id, int32_t* comp) {
  int64_t bad = 0;
  for (int64_t i = 0; i < n; ++i) {
    int32_t x = raw[i];
    int32_t c = pad_id;
    if (x >= 0 && x < vocab) {
      c = lut[x];
      if (c < 0 || c >= vocab_c) {
        c = pad_id;
        ++bad;
      }
    } else {
      ++bad;
    }
    comp[i] = c;
  }
  return bad;
}

/* Compressed id at position pos of sequence b (pos may be negative). */
static int32_t context_id(const int32_t* comp, int32_t T, int32_t b, int64_t pos,
                          const int32_t* hist, int32_t hist_len, int32_t pad_id) {
  if (pos >= 0) return comp[(int64_t)b * T + pos];
  int64_t h = (int64_t)hist_len + pos; /* hist[b][hist_len-1] is position -1 */
  if (hist != NULL && h >= 0) return hist[(int64_t)b * hist_len + h];
  return pad_id;
}

/*
 * Step 2 -- n-gram keys and multi-head hashing [A, second component; B, the
 * lookup rule; C, mod hash].  For order n = orders[o] and head k, table
 * j = o*heads + k receives row
 *     key = XOR_{i=0}^{n-1} ( c_{t-i} * mult[j*4 + i] )   (mod 2^64)
 *     row = key mod rows[j].
 * row_idx is [B*T, n_tables] with n_tables = n_orders*heads.
 * hist (nullable) is [B, hist_len] compressed ids, oldest first.
 */
void orc_hash(const int32_t* comp, int32_t B, int32_t T, const int32_t* hist,
              int32_t hist_len, int32_t pad_id, int32_t n_orders, const int32_t* orders,
              int32_t heads, const int64_t* rows, const uint64_t* mult, int32_t* row_idx) {
  const int32_t n_tables = n_orders * heads;
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t t = 0; t < T; ++t) {
      int32_t* out = row_idx + ((int64_t)b * T + t) * n_tables;
      for (int32_t o = 0; o < n_orders; ++o) {
        for (int32_t k = 0; k < heads; ++k) {
          int32_t j = o * heads + k;
          uint64_t key = 0;
          for (int32_t i = 0; i < orders[o]; ++i) {
            uint64_t c = (uint64_t)(uint32_t)context_id(comp, T, b, (int64_t)t - i, hist,
                                                        hist_len, pad_id);
            key ^= c * mult[(int64_t)j * 4 + i];
          }
          out[j] = (int32_t)(key % (uint64_t)rows[j]);
        }
      }
    }
  }
}

/*
 * FP8 E4M3 (the OCP 8-bit floating-point format): sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits.  Exponent field 0 encodes the subnormals
 * m * 2^-9; exponent field 15 with mantissa 7 is NaN; there are no
 * infinities, so the largest value is 1.75 * 2^8 = 448.
 */
double orc_fp8_e4m3_value(uint32_t byte) {
  const int sign = (byte >> 7) & 1;
  const int ex = (byte >> 3) & 15;
  const int m = byte & 7;
  double v;
  if (ex == 15 && m == 7)
    v = NAN;
  else if (ex == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, ex - 7);
  return sign ? -v : v;
}

/* fp32 -> bf16 (the upper 16 bits of the fp32 pattern), round to nearest,
 * ties to even; the result is returned as the value it encodes. */
static double round_bf16(float f) {
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  const uint32_t low = bits & 0xFFFFu;
  uint32_t high = bits >> 16;
  if (low > 0x8000u || (low == 0x8000u && (high & 1u))) high += 1;
  bits = high << 16;
  float r;
  memcpy(&r, &bits, sizeof r);
  return (double)r;
}

/*
 * Step 3 -- gather and concatenate [A, second component; B, the row ids' rows
 * joined end to end into E_t]: E_t = table_0[r_0] ++ table_1[r_1]
 * ++ ... in table order (orders ascending, then heads).  e is [n_tok, mem]
 * with mem = n_tables * row_dim.  FP8 tables (dtype ORC_FP8): a row value is
 * scales[j] * decode(byte), and E holds it as bf16 -- the product rounded to
 * fp32, then to bf16, each to nearest even (the storage format's
 * definition of E; the scale is per table, [D]).
 */
void orc_gather(const int32_t* row_idx, int64_t n_tok, int32_t n_tables,
                const void* const* tables, int32_t dtype, int32_t row_dim, const float* scales,
                double* e) {
  const int64_t mem = (int64_t)n_tables * row_dim;
  for (int64_t t = 0; t < n_tok; ++t)
    for (int32_t j = 0; j < n_tables; ++j) {
      int64_t r = row_idx[t * n_tables + j];
      for (int32_t c = 0; c < row_dim; ++c) {
        double v;
        if (dtype == ORC_FP8) {
          const uint8_t byte = ((const uint8_t*)tables[j])[r * row_dim + c];
          /* exact in double (4 + 24 significant bits), then rounded to fp32 */
          const float prod = (float)(orc_fp8_e4m3_value(byte) * (double)scales[j]);
          v = round_bf16(prod);
        } else {
          v = load_value(tables[j], dtype, r * row_dim + c);
        }
        e[t * mem + (int64_t)j * row_dim + c] = v;
      }
    }
}

/*
 * Step 4 -- key / value projections [B, E_t -> K_t, V_t]: out = E @ W with W
 * stored [mem, d] row-major.  out is [n_tok, d].
 */
void orc_project(const double* e, int64_t n_tok, int32_t mem, const void* w, int32_t dtype,
                 int32_t d, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int32_t n = 0; n < d; ++n) {
      double acc = 0.0;
      for (int32_t m = 0; m < mem; ++m)
        acc += e[t * mem + m] * load_value(w, dtype, (int64_t)m * d + n);
      out[t * d + n] = acc;
    }
  }
}

/*
 * Step 5 -- context-aware gate [A, third component; B, g_t = Gate(Norm(Q_t),
 * Norm(K_t))]: the query is the layer's hidden state.
 *     q = gamma_q * h / sqrt(mean(h^2) + eps),  k^ = gamma_k * k / sqrt(mean(k^2) + eps)
 *     g = sigmoid( (q . k^) / sqrt(d) )
 * hidden row for (token t, branch b) starts at t*tok_stride + b*branch_stride
 * (branch_stride 0: one query shared by all branches).  k is [n_tok, nb, d].
 * gamma_q / gamma_k (nullable = all ones) are in the hidden's dtype.
 * gate is [n_tok, nb].
 */
void orc_gate(const void* hidden, int32_t dtype, int64_t tok_stride, int64_t branch_stride,
              const double* k, int64_t n_tok, int32_t nb, int32_t d, const void* gamma_q,
              const void* gamma_k, double eps, double* gate) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int32_t b = 0; b < nb; ++b) {
      int64_t hbase = t * tok_stride + (int64_t)b * branch_stride;
      const double* kr = k + (t * nb + b) * (int64_t)d;
      double hh = 0.0, kk = 0.0;
      for (int32_t n = 0; n < d; ++n) {
        double h = load_value(hidden, dtype, hbase + n);
        hh += h * h;
        kk += kr[n] * kr[n];
      }
      double inv_h = 1.0 / sqrt(hh / d + eps);
      double inv_k = 1.0 / sqrt(kk / d + eps);
      double dot = 0.0;
      for (int32_t n = 0; n < d; ++n) {
        double gq = gamma_q ? load_value(gamma_q, dtype, n) : 1.0;
        double gk = gamma_k ? load_value(gamma_k, dtype, n) : 1.0;
        double q = gq * load_value(hidden, dtype, hbase + n) * inv_h;
        double kn = gk * kr[n] * inv_k;
        dot += q * kn;
      }
      double z = dot / sqrt((double)d);
      gate[t * nb + b] = 1.0 / (1.0 + exp(-z));
    }
  }
}

/*
 * Step 6 -- gated value [B, U_t = g_t (.) V_t]: the value projection is shared
 * by the branches [A, multi-branch integration].  v is [n_tok, d], u is
 * [n_tok, nb, d].
 */
void orc_gated_value(const double* gate, const double* v, int64_t n_tok, int32_t nb, int32_t d,
                     double* u) {
  for (int64_t t = 0; t < n_tok; ++t)
    for (int32_t b = 0; b < nb; ++b)
      for (int32_t n = 0; n < d; ++n)
        u[(t * nb + b) * (int64_t)d + n] = gate[t * nb + b] * v[t * d + n];
}

/*
 * Step 7 -- convolution block [A, fourth component; B, Delta_t = U_t +
 * SiLU(DWConv(RMSNorm(U_t)))]:
 *     N_t     = gamma_u * U_t / sqrt(mean(U_t^2) + eps)          (per branch)
 *     C_t     = sum_{i=0}^{kernel-1} w_i (.) N_{t - i*dil}       (depthwise)
 *     Delta_t = U_t + C_t * sigmoid(C_t)
 * u and delta are [B, T, nb, d]; w is [kernel, d] in w_dtype; gamma_u
 * (nullable) in w_dtype.  A tap before the sequence start reads the caller's
 * state row (already normalised) when state != NULL -- state is
 * [B, (kernel-1)*dil, nb, d], its last row being position -1 -- else zero.
 */
void orc_conv_block(const double* u, int32_t B, int32_t T, int32_t nb, int32_t d,
                    const void* w, int32_t w_dtype, int32_t kernel, int32_t dil,
                    const void* gamma_u, double eps, const double* state, double* delta) {
  const int64_t row = (int64_t)nb * d;
  const int32_t span = (kernel - 1) * dil;
  double* nrm = (double*)malloc(sizeof(double) * (size_t)((int64_t)B * T * row));
  if (nrm == NULL) return;
  /* N_t = RMSNorm(U_t), one row per (token, branch) */
#pragma omp parallel for schedule(static)
  for (int64_t tb = 0; tb < (int64_t)B * T * nb; ++tb) {
    const double* ut = u + tb * d;
    double ss = 0.0;
    for (int32_t n = 0; n < d; ++n) ss += ut[n] * ut[n];
    double inv = 1.0 / sqrt(ss / d + eps);
    for (int32_t n = 0; n < d; ++n) {
      double g = gamma_u ? load_value(gamma_u, w_dtype, n) : 1.0;
      nrm[tb * d + n] = g * ut[n] * inv;
    }
  }
  /* C_t = sum_i w_i (.) N_{t - i*dil};  Delta_t = U_t + SiLU(C_t) */
#pragma omp parallel for collapse(2) schedule(static)
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t t = 0; t < T; ++t) {
      for (int32_t br = 0; br < nb; ++br) {
        int64_t off = ((int64_t)b * T + t) * row + (int64_t)br * d;
        for (int32_t n = 0; n < d; ++n) {
          double c = 0.0;
          for (int32_t i = 0; i < kernel; ++i) {
            int64_t p = (int64_t)t - (int64_t)i * dil;
            double nval = 0.0;
            if (p >= 0) {
              nval = nrm[((int64_t)b * T + p) * row + (int64_t)br * d + n];
            } else if (state != NULL) {
              int64_t s = (int64_t)span + p; /* row inside the state; last row is p = -1 */
              if (s >= 0) nval = state[((int64_t)b * span + s) * row + (int64_t)br * d + n];
            }
            c += load_value(w, w_dtype, (int64_t)i * d + n) * nval;
          }
          delta[off + n] = u[off + n] + c / (1.0 + exp(-c));
        }
      }
    }
  }
  free(nrm);
}

/* The normalised rows the convolution reads ([B] §2.3, RMSNorm(U_t)):
 * out[r] = gamma (.) u[r] / sqrt(mean(u[r]^2) + eps) for each of the rows
 * rows of d values; gamma (nullable = 1) in dtype.  A caller that feeds a
 * sequence in pieces keeps the last (kernel-1)*dil of these rows as the
 * state of the next piece. */
void orc_normalise_rows(const double* u, int64_t rows, int32_t d, const void* gamma,
                        int32_t dtype, double eps, double* out) {
  for (int64_t r = 0; r < rows; ++r) {
    const double* x = u + r * d;
    double ss = 0.0;
    for (int32_t n = 0; n < d; ++n) ss += x[n] * x[n];
    const double inv = 1.0 / sqrt(ss / d + eps);
    for (int32_t n = 0; n < d; ++n) {
      const double g = gamma ? load_value(gamma, dtype, n) : 1.0;
      out[r * d + n] = g * x[n] * inv;
    }
  }
}

/* ------------------------------------------------------------------------
 * Backward of the layer (the gradients a training step needs: tables, W_K,
 * W_V, conv taps, query, RMSNorm gains), each step the chain rule of the
 * forward step above it, written out with the forward's own definitions.
 * Outputs marked "accumulated" are added to, the others overwritten.
 * ------------------------------------------------------------------------ */

/* RMSNorm y = gamma (.) x / r, r = sqrt(mean(x^2) + eps), backward for one
 * row: dx = gamma (.) dy / r - x * sum(gamma dy x) / (d r^3); dgamma += dy x / r. */
static void rms_backward_row(const double* x, const double* dy, const void* gamma, int32_t dtype,
                             int32_t d, double eps, double* dx, double* dgamma) {
  double ss = 0.0;
  for (int32_t n = 0; n < d; ++n) ss += x[n] * x[n];
  const double r = sqrt(ss / d + eps);
  double s = 0.0;
  for (int32_t n = 0; n < d; ++n) {
    const double g = gamma ? load_value(gamma, dtype, n) : 1.0;
    s += g * dy[n] * x[n];
  }
  for (int32_t n = 0; n < d; ++n) {
    const double g = gamma ? load_value(gamma, dtype, n) : 1.0;
    dx[n] = g * dy[n] / r - x[n] * s / (d * r * r * r);
    if (dgamma) dgamma[n] += dy[n] * x[n] / r;
  }
}

/*
 * Backward of the conv block: Delta = U + SiLU(C), C_t = sum_i w_i (.) N_{t-i*dil},
 * N = RMSNorm(U).  d_delta [B,T,nb,d] in; d_u [B,T,nb,d] out; d_w [kernel, d]
 * and d_gamma_u [d] (nullable) accumulated.  The conv state is an input with
 * no gradient.  SiLU'(c) = s (1 + c (1 - s)), s = sigmoid(c).
 */
void orc_conv_block_backward(const double* u, int32_t B, int32_t T, int32_t nb, int32_t d,
                             const void* w, int32_t w_dtype, int32_t kernel, int32_t dil,
                             const void* gamma_u, double eps, const double* state,
                             const double* d_delta, double* d_u, double* d_w, double* d_gamma_u) {
  const int64_t row = (int64_t)nb * d;
  const int64_t n_el = (int64_t)B * T * row;
  const int32_t span = (kernel - 1) * dil;
  double* nrm = (double*)malloc(sizeof(double) * (size_t)n_el);
  double* dc = (double*)malloc(sizeof(double) * (size_t)n_el);
  double* dn = (double*)malloc(sizeof(double) * (size_t)n_el);
  if (!nrm || !dc || !dn) { free(nrm); free(dc); free(dn); return; }
  for (int64_t tb = 0; tb < (int64_t)B * T * nb; ++tb) {
    const double* ut = u + tb * d;
    double ss = 0.0;
    for (int32_t n = 0; n < d; ++n) ss += ut[n] * ut[n];
    const double inv = 1.0 / sqrt(ss / d + eps);
    for (int32_t n = 0; n < d; ++n) {
      const double g = gamma_u ? load_value(gamma_u, w_dtype, n) : 1.0;
      nrm[tb * d + n] = g * ut[n] * inv;
    }
  }
  /* N at position p of sequence b (state rows before 0, zeros past them) */
#define NVAL(b, p, br, n)                                                              \
  ((p) >= 0 ? nrm[((int64_t)(b) * T + (p)) * row + (int64_t)(br) * d + (n)]            \
   : (state != NULL && span + (p) >= 0)                                                  \
       ? state[((int64_t)(b) * span + span + (p)) * row + (int64_t)(br) * d + (n)]       \
       : 0.0)
  /* dC, the residual term of d_u, and d_w */
  for (int32_t b = 0; b < B; ++b)
    for (int32_t t = 0; t < T; ++t)
      for (int32_t br = 0; br < nb; ++br) {
        const int64_t off = ((int64_t)b * T + t) * row + (int64_t)br * d;
        for (int32_t n = 0; n < d; ++n) {
          double c = 0.0;
          for (int32_t i = 0; i < kernel; ++i)
            c += load_value(w, w_dtype, (int64_t)i * d + n) * NVAL(b, (int64_t)t - (int64_t)i * dil, br, n);
          const double s = 1.0 / (1.0 + exp(-c));
          dc[off + n] = d_delta[off + n] * s * (1.0 + c * (1.0 - s));
          d_u[off + n] = d_delta[off + n];
          for (int32_t i = 0; i < kernel; ++i)
            d_w[(int64_t)i * d + n] += dc[off + n] * NVAL(b, (int64_t)t - (int64_t)i * dil, br, n);
        }
      }
#undef NVAL
  /* dN_p = sum_i w_i (.) dC_{p + i*dil} inside the sequence */
  for (int32_t b = 0; b < B; ++b)
    for (int32_t p = 0; p < T; ++p)
      for (int32_t br = 0; br < nb; ++br)
        for (int32_t n = 0; n < d; ++n) {
          double acc = 0.0;
          for (int32_t i = 0; i < kernel; ++i) {
            const int64_t t = (int64_t)p + (int64_t)i * dil;
            if (t < T) acc += load_value(w, w_dtype, (int64_t)i * d + n) *
                              dc[((int64_t)b * T + t) * row + (int64_t)br * d + n];
          }
          dn[((int64_t)b * T + p) * row + (int64_t)br * d + n] = acc;
        }
  /* through N = RMSNorm(U) */
  double* dx = (double*)malloc(sizeof(double) * (size_t)d);
  if (dx) {
    for (int64_t tb = 0; tb < (int64_t)B * T * nb; ++tb) {
      rms_backward_row(u + tb * d, dn + tb * d, gamma_u, w_dtype, d, eps, dx, d_gamma_u);
      for (int32_t n = 0; n < d; ++n) d_u[tb * d + n] += dx[n];
    }
    free(dx);
  }
  free(nrm);
  free(dc);
  free(dn);
}

/* Backward of U = g V: d_gate [n, nb] = sum_n dU V; d_v [n, d] = sum_b g dU (overwritten). */
void orc_gated_value_backward(const double* gate, const double* v, const double* d_u,
                              int64_t n_tok, int32_t nb, int32_t d, double* d_gate, double* d_v) {
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int32_t n = 0; n < d; ++n) d_v[t * d + n] = 0.0;
    for (int32_t b = 0; b < nb; ++b) {
      const double* du = d_u + (t * nb + b) * (int64_t)d;
      double acc = 0.0;
      for (int32_t n = 0; n < d; ++n) {
        acc += du[n] * v[t * d + n];
        d_v[t * d + n] += gate[t * nb + b] * du[n];
      }
      d_gate[t * nb + b] = acc;
    }
  }
}

/*
 * Backward of the gate g = sigmoid(q . k^ / sqrt(d)), q = RMSNorm_gq(h),
 * k^ = RMSNorm_gk(K).  d_gate [n, nb] in; d_k [n, nb, d] out; d_hidden
 * (storage layout of hidden, as doubles; branches sharing a query row add
 * into it), d_gamma_q, d_gamma_k (nullable) accumulated.
 */
void orc_gate_backward(const void* hidden, int32_t dtype, int64_t tok_stride, int64_t branch_stride,
                       const double* k, int64_t n_tok, int32_t nb, int32_t d, const void* gamma_q,
                       const void* gamma_k, double eps, const double* d_gate, double* d_k,
                       double* d_hidden, double* d_gamma_q, double* d_gamma_k) {
  double* h = (double*)malloc(sizeof(double) * (size_t)d);
  double* q = (double*)malloc(sizeof(double) * (size_t)d);
  double* kn = (double*)malloc(sizeof(double) * (size_t)d);
  double* dq = (double*)malloc(sizeof(double) * (size_t)d);
  double* dkn = (double*)malloc(sizeof(double) * (size_t)d);
  double* dx = (double*)malloc(sizeof(double) * (size_t)d);
  if (h && q && kn && dq && dkn && dx) {
    const double sd = sqrt((double)d);
    for (int64_t t = 0; t < n_tok; ++t)
      for (int32_t b = 0; b < nb; ++b) {
        const int64_t hbase = t * tok_stride + (int64_t)b * branch_stride;
        const double* kr = k + (t * nb + b) * (int64_t)d;
        double hh = 0.0, kk = 0.0;
        for (int32_t n = 0; n < d; ++n) {
          h[n] = load_value(hidden, dtype, hbase + n);
          hh += h[n] * h[n];
          kk += kr[n] * kr[n];
        }
        const double inv_h = 1.0 / sqrt(hh / d + eps), inv_k = 1.0 / sqrt(kk / d + eps);
        double dot = 0.0;
        for (int32_t n = 0; n < d; ++n) {
          q[n] = (gamma_q ? load_value(gamma_q, dtype, n) : 1.0) * h[n] * inv_h;
          kn[n] = (gamma_k ? load_value(gamma_k, dtype, n) : 1.0) * kr[n] * inv_k;
          dot += q[n] * kn[n];
        }
        const double g = 1.0 / (1.0 + exp(-dot / sd));
        const double dz = d_gate[t * nb + b] * g * (1.0 - g);
        for (int32_t n = 0; n < d; ++n) {
          dq[n] = dz * kn[n] / sd;
          dkn[n] = dz * q[n] / sd;
        }
        rms_backward_row(kr, dkn, gamma_k, dtype, d, eps, d_k + (t * nb + b) * (int64_t)d,
                         d_gamma_k);
        rms_backward_row(h, dq, gamma_q, dtype, d, eps, dx, d_gamma_q);
        for (int32_t n = 0; n < d; ++n) d_hidden[hbase + n] += dx[n];
      }
  }
  free(h); free(q); free(kn); free(dq); free(dkn); free(dx);
}

/* Backward of out = E W (W [mem, d]): d_e [n, mem] += d_out W^T; d_w [mem, d] += E^T d_out. */
void orc_project_backward(const double* e, int64_t n_tok, int32_t mem, const void* w, int32_t dtype,
                          int32_t d, const double* d_out, double* d_e, double* d_w) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_tok; ++t)
    for (int32_t m = 0; m < mem; ++m) {
      double acc = 0.0;
      for (int32_t n = 0; n < d; ++n) acc += d_out[t * d + n] * load_value(w, dtype, (int64_t)m * d + n);
      d_e[t * mem + m] += acc;
    }
#pragma omp parallel for schedule(static)
  for (int32_t m = 0; m < mem; ++m)
    for (int32_t n = 0; n < d; ++n) {
      double acc = 0.0;
      for (int64_t t = 0; t < n_tok; ++t) acc += e[t * mem + m] * d_out[t * d + n];
      d_w[(int64_t)m * d + n] += acc;
    }
}

/* Backward of the gather: d_tables[j][row_idx[t][j]] += the j-th row_dim
 * slice of d_e[t] (accumulated; a row hit by several tokens sums them). */
void orc_scatter_add(const int32_t* row_idx, int64_t n_tok, int32_t n_tables, const double* d_e,
                     int32_t row_dim, double* const* d_tables) {
  const int64_t mem = (int64_t)n_tables * row_dim;
  for (int64_t t = 0; t < n_tok; ++t)
    for (int32_t j = 0; j < n_tables; ++j) {
      const int64_t r = row_idx[t * n_tables + j];
      for (int32_t c = 0; c < row_dim; ++c)
        d_tables[j][r * row_dim + c] += d_e[t * mem + (int64_t)j * row_dim + c];
    }
}
