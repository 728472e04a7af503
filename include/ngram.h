/*
 * ngram.h -- C-ABI of libngram.so, the hashed N-gram embedding layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (Engram-style "N-gram Embedding"), per token t of a sequence:
 *   1. c_t = LUT[x_t]                                   tokenizer compression
 *   2. 2-gram key (c_{t-1}, c_t), 3-gram key (c_{t-2}, c_{t-1}, c_t)
 *   3. each key hashed by K independent heads into prime-sized tables
 *   4. E_t = concatenation of the gathered rows         memory vector
 *   5. K_t = E_t W_K (one per branch), V_t = E_t W_V (shared)
 *   6. g_t = sigmoid( RMSNorm(h_t) . RMSNorm(K_t) / sqrt(d) )   one per branch
 *   7. U_t = g_t V_t
 *   8. Delta_t = U_t + SiLU( DWConv_{kernel 4, dilation = max order}( RMSNorm(U) )_t )
 * Sources: "Qwen 4用上DeepSeek的Engram！125B MoE一张4090能跑不用量化"
 * (yktysq.com), section "DeepSeek Engram 更复杂，Qwen 更精简" (the four
 * components and multi-branch integration), and "Qwen3.8-Flash-Next 深度研究"
 * (zhichai.net), §2.3 "Embedding：N-gram Embedding" (lookup rule and the
 * layer formula E_t -> K_t, V_t; g_t; U_t; Delta_t).
 *
 * Conventions for every entry point
 *  - Device pointers are borrowed for the stream-ordered duration of the call;
 *    the caller owns every buffer.  The library allocates no device memory:
 *    scratch comes from the caller's workspace (ngram_forward_noalloc alone
 *    takes it from a static device array instead; see there).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream), never synchronises, keeps no state between calls and is
 *    reentrant (ngram_forward_noalloc's shared array is the one exception).
 *    The library reads no environment variables: tuning overrides are fields
 *    of ngram_config.
 *  - All arrays are dense row-major.  Device pointers must be 16-byte aligned.
 *  - Arguments are validated on the host before any launch; a failed check
 *    returns a negative ngram_status and launches nothing.  A failed launch
 *    returns NGRAM_EHIP.  Empty inputs (zero tokens) return NGRAM_OK at once.
 *  - Invalid token ids (outside [0, vocab), or whose LUT entry lies outside
 *    [0, vocab_compressed)) are data errors found on the device: the token is
 *    treated as pad_id and, if err_flag is non-NULL, *err_flag is set to 1
 *    (never cleared by the library).
 *  - Floating point: storage is fp32 or bf16 (ngram_dtype); all arithmetic is
 *    fp32 with fp32 accumulation (MFMA for bf16 projections); outputs are
 *    rounded to the storage type to nearest-even.  Gates are always fp32.
 */
#ifndef NGRAM_H
#define NGRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NGRAM_MAX_TABLES 16
#define NGRAM_MAX_ORDER 4
#define NGRAM_MAX_BRANCHES 4

/* flags for ngram_forward / ngram_causal_conv */
#define NGRAM_ADD_RESIDUAL 1 /* out = hidden (the branch's query row) + Delta (forward only) */
#define NGRAM_UPDATE_STATE 2 /* write this call's normalised rows into the conv-state ring */
#define NGRAM_PREFETCHED 4   /* the workspace already holds the call's row ids and E
                                (ngram_forward_prefetch); forward only */
#define NGRAM_KEEP_FOR_BACKWARD 8 /* ngram_forward: leave row ids, E, K and V in the
                                     workspace for ngram_backward; ngram_backward: use
                                     them instead of recomputing (see ngram_backward) */

typedef enum ngram_status {
  NGRAM_OK = 0,
  NGRAM_EINVAL = -1,     /* NULL pointer or inconsistent configuration */
  NGRAM_ESHAPE = -2,     /* a size is out of range or not a supported multiple */
  NGRAM_EDTYPE = -3,     /* unsupported dtype or dtype combination */
  NGRAM_EALIGN = -4,     /* a device pointer is not 16-byte aligned */
  NGRAM_ERANGE = -5,     /* a table row count is not prime / too large, ids out of range */
  NGRAM_EHIP = -6,       /* a HIP launch failed */
  NGRAM_EWORKSPACE = -7, /* workspace missing or smaller than required */
  NGRAM_ESCRATCH = -8    /* ngram_forward_noalloc: the call needs more than its static scratch */
} ngram_status;

/*
 * NGRAM_FP8_E4M3 is a table storage type only: OCP FP8 E4M3 (sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent 0 holds the subnormals
 * m * 2^-9; S.1111.111 is NaN; no infinities).  Table j's row values are
 * table_scale[j] * decode(byte), and the memory vector holds each as bf16:
 * E = bf16(fp32(decode(byte) * table_scale[j])), each conversion rounding to
 * nearest even.  The FP8 release of the model stores this table in FP8 with
 * one scale per tensor, and a loader that discarded the scale degraded the
 * model without any error ("Qwen3.8-Flash-Next 深度研究" §9.3): here the
 * scale is an explicit part of every lookup.
 */
typedef enum ngram_dtype { NGRAM_F32 = 0, NGRAM_BF16 = 1, NGRAM_FP8_E4M3 = 2 } ngram_dtype;

/*
 * Storage of the projection matrices (ngram_config.w_layout).
 *   NGRAM_W_MEM_D: W_K^(b), W_V are [mem_dim, d] row-major, K = E W.
 *   NGRAM_W_D_MEM: they are [d, mem_dim] row-major (output row n holds the
 *                  mem_dim weights of K_n; the torch.nn.Linear convention),
 *                  K = E W^T.  Both operands of the product are then
 *                  contiguous along mem_dim, which the bf16 kernels stream
 *                  straight into LDS: this is the fast layout.
 */
typedef enum ngram_w_layout { NGRAM_W_MEM_D = 0, NGRAM_W_D_MEM = 1 } ngram_w_layout;

/*
 * Layer configuration (host memory, read during the call only).
 *
 * Tables: table j = o * heads_per_order + k holds the rows of head k of order
 * orders[o] (orders ascending, so 2-gram tables come first).  For the token at
 * position t its row is
 *     key = XOR_{i=0}^{n-1} ( (uint64)c_{t-i} * hash_mult[j][i] )   (mod 2^64)
 *     row = key mod rows[j]
 * with n = orders[o]; c_{t-i} for t-i < 0 comes from the history if given,
 * else pad_id.  The sources fix only that each order has K independent hash
 * heads mapping into tables of prime size, deterministically, and (in a
 * related method's lineage table) that the hash is a modulus; this
 * multiply-xor-mod form is the library's reading, the multipliers being
 * parameters of the model.
 */
typedef struct ngram_config {
  int32_t n_orders;                                      /* 1..NGRAM_MAX_ORDER */
  int32_t orders[NGRAM_MAX_ORDER];                       /* strictly ascending, 1..4 */
  int32_t heads_per_order;                               /* K >= 1 */
  int32_t n_tables;                                      /* == n_orders * K <= 16 */
  int64_t rows[NGRAM_MAX_TABLES];                        /* prime, < 2^31 */
  uint64_t hash_mult[NGRAM_MAX_TABLES][NGRAM_MAX_ORDER]; /* slot i used for i < order */
  int32_t row_dim;                                       /* values per table row */
  int32_t mem_dim;                                       /* == n_tables * row_dim */
  int32_t hidden_dim;                                    /* d */
  int32_t n_branches;                                    /* 1..NGRAM_MAX_BRANCHES */
  int32_t conv_kernel;                                   /* 4 */
  int32_t conv_dilation;                                 /* == orders[n_orders - 1] */
  int32_t vocab;                                         /* raw ids in [0, vocab) */
  int32_t vocab_compressed;                              /* LUT image in [0, vocab_compressed) */
  int32_t pad_id;                                        /* in [0, vocab_compressed) */
  float rms_eps;                                         /* >= 0, RMSNorm epsilon */
  int32_t table_dtype;                                   /* ngram_dtype */
  int32_t act_dtype;                                     /* == table_dtype; bf16 for fp8 tables */
  int32_t w_layout;                                      /* ngram_w_layout */
  float table_scale[NGRAM_MAX_TABLES];                   /* fp8 tables: finite, > 0 */
  /* Tile-plan overrides; 0 everywhere = the library's own choice.  They change
     how the work is tiled, never the result beyond fp32 summation order.
     tune_proj_plan: 1 + id of the prefill projection's tile plan (0..12) for
     bf16 with W stored [d, mem].  tune_decode_ni / tune_decode_split: the decode
     projection's 16-column blocks per workgroup (2..6) and K slices; both or
     neither, and the pair must fit (see ngram_config_validate). */
  int32_t tune_proj_plan;
  int32_t tune_decode_ni;
  int32_t tune_decode_split;
} ngram_config;

/* Human-readable name of a status code (static string). */
const char* ngram_status_str(int status);

/* Library ABI version: increments whenever a signature, a layout or the set
   of entry points changes. */
int ngram_abi_version(void);

/*
 * Check a configuration without touching the GPU.  Returns NGRAM_OK or the
 * first failing status.  Shape rules: row_dim * sizeof(table dtype) must be a
 * multiple of 16 bytes; for bf16 activations, mem_dim % 64 == 0 and
 * hidden_dim % 32 == 0; for fp32, hidden_dim % 4 == 0.  fp8 tables take bf16
 * activations, and the memory vector E is bf16.  conv_kernel must be 4 (the pages' kernel)
 * and conv_dilation the largest order.
 *
 * This is the only call that proves every rows[j] prime (deterministic
 * Miller-Rabin); call it once when a configuration is built.  The other entry
 * points repeat every check except that proof, screening rows[j] only for
 * small factors: primality shapes the hash's spread, while row ids stay below
 * rows[j] (the bound that keeps the table reads in range) for any value.
 * A decode tile-plan override must satisfy: split divides mem_dim,
 * (mem_dim / split) % 128 == 0 and 32 * ni * (mem_dim / split) <= 131072.
 */
int ngram_config_validate(const ngram_config* cfg);

/*
 * Tokenizer compression -- Engram's first component ("Qwen 4用上DeepSeek的
 * Engram", section "DeepSeek Engram 更复杂，Qwen 更精简"): comp_ids[i] =
 * lut[raw_ids[i]].
 *   raw_ids  device int32[n]
 *   lut      device int32[vocab]
 *   comp_ids device int32[n] (output)
 *   err_flag device int32, nullable: set to 1 on an invalid id
 */
int ngram_compress_ids(const ngram_config* cfg, const int32_t* raw_ids, int64_t n,
                       const int32_t* lut, int32_t* comp_ids, int32_t* err_flag, void* stream);

/*
 * N-gram keys and multi-head hashing -- Engram's second component and the
 * lookup rule of "Qwen3.8-Flash-Next 深度研究" §2.3 (2-gram heads on
 * (x_{t-1}, x_t), 3-gram heads on (x_{t-2}, x_{t-1}, x_t)).
 *   comp_ids device int32[B, T] compressed ids (output of ngram_compress_ids)
 *   history  device int32[B, max_order - 1] compressed ids before position 0,
 *            oldest first; NULL = pad_id
 *   row_idx  device int32[B, T, n_tables] (output): row of table j for token t
 * Compressed ids are not range-checked here (ngram_compress_ids does that).
 */
int ngram_hash(const ngram_config* cfg, const int32_t* comp_ids, int32_t B, int32_t T,
               const int32_t* history, int32_t* row_idx, void* stream);

/*
 * Gather and concatenation into the memory vector E_t ("Qwen3.8-Flash-Next
 * 深度研究" §2.3: the rows named by the row ids are joined end to end into
 * E_t): mem[t, j*row_dim + c] = tables[j][row_idx[t, j], c].  An exact copy.
 *   row_idx  device int32[n_tok, n_tables]; each entry must be < rows[j]
 *   tables   HOST array of n_tables device pointers, table j is
 *            [rows[j], row_dim] of table_dtype
 *   mem      device [n_tok, mem_dim] (output): table_dtype, bf16 for fp8 tables
 */
int ngram_gather(const ngram_config* cfg, const int32_t* row_idx, int64_t n_tok,
                 const void* const* tables, void* mem, void* stream);

/*
 * Context-aware gating -- Engram's third component and §2.3's
 * g_t = Gate(Norm(Q_t), Norm(K_t)), U_t = g_t (.) V_t:
 *   K^(b) = E W_K^(b), V = E W_V (fp32 accumulate), the query h^(b) is the
 *   hidden state, g = sigmoid( sum(gamma_q h/rms(h) * gamma_k K/rms(K)) / sqrt(d) )
 *   with rms(x) = sqrt(mean(x^2) + rms_eps); U^(b) = g^(b) V.
 *   hidden   device [n_tok, nbh, d] act_dtype with hidden_branch_stride == 0
 *            (nbh = 1: one query row shared by all branches) or == d
 *            (nbh = n_branches: one query row per branch)
 *   mem      device [n_tok, mem_dim] (E): table_dtype, bf16 for fp8 tables
 *   w_k      device [n_branches, mem_dim, d] act_dtype and w_v [mem_dim, d]
 *            (NGRAM_W_MEM_D), or [n_branches, d, mem_dim] and [d, mem_dim]
 *            (NGRAM_W_D_MEM)
 *   gamma_q, gamma_k  device [d] act_dtype, nullable (= 1)
 *   gates    device float[n_tok, n_branches] (output)
 *   u        device [n_tok, n_branches, d] act_dtype (output), nullable
 *   workspace device scratch of at least ngram_gate_workspace_size() bytes
 */
size_t ngram_gate_workspace_size(const ngram_config* cfg, int64_t n_tok);
int ngram_gate(const ngram_config* cfg, const void* hidden, int64_t hidden_branch_stride,
               const void* mem, const void* w_k, const void* w_v, const void* gamma_q,
               const void* gamma_k, int64_t n_tok, float* gates, void* u, void* workspace,
               size_t workspace_bytes, void* stream);

/*
 * The conv-state ring (decode, and prefill in chunks).  The convolution at
 * position t reads the normalised rows N of positions t, t - dil, t - 2 dil,
 * t - 3 dil, so a sequence that arrives in pieces needs the last R =
 * (conv_kernel - 1) * dil rows of the earlier pieces.  conv_state holds them
 * as a ring, device float[B, R, n_branches, d], together with
 * state_pos, device int32[B]: the number of positions of sequence b that came
 * before this call's first token.  The row of absolute position p lives in
 * slot p mod R.  A position before the start of the sequence (p < 0) reads
 * zeros whatever its slot holds, so the ring of a new sequence need not be
 * cleared (state_pos = 0).  A negative state_pos is read as 0.
 * state_pos NULL means state_pos = R for every sequence: slot s holds position
 * s - R, oldest first.
 * With NGRAM_UPDATE_STATE (which needs both conv_state and state_pos) the call
 * also writes the normalised rows of its last min(T, R) positions into their
 * slots (position state_pos[b] + t goes to slot (state_pos[b] + t) mod R), in
 * place, after every read of the ring it needs, and advances state_pos[b] by
 * T: the next call of the same sequences passes both on as they are, and
 * decode becomes one call per token that costs one ring row written and
 * three read per sequence and branch.
 */

/*
 * Convolution block -- Engram's fourth component (kernel 4, dilation = the
 * largest n-gram order, depthwise, causal) and §2.3's
 * Delta_t = U_t + SiLU(DWConv(RMSNorm(U_t))):
 *   N_t = gamma_u (.) U_t / rms(U_t) per branch;  C_t = sum_i conv_w[i] (.) N_{t - i*dil}
 *   (zero before position 0 unless conv_state is given);  Delta_t = U_t + C_t sigmoid(C_t)
 *   u          device [B, T, n_branches, d] act_dtype
 *   conv_w     device [conv_kernel, d] act_dtype; tap i multiplies position t - i*dil
 *   gamma_u    device [d] act_dtype, nullable (= 1)
 *   conv_state device float[B, R, n_branches, d] ring of normalised rows (see
 *              above), nullable (zeros before position 0)
 *   state_pos  device int32[B], nullable (see above); advanced in place by
 *              NGRAM_UPDATE_STATE
 *   flags      0 or NGRAM_UPDATE_STATE (which needs conv_state and state_pos)
 *   out        device [B, T, n_branches, d] act_dtype (output)
 */
int ngram_causal_conv(const ngram_config* cfg, const void* u, int32_t B, int32_t T,
                      const void* conv_w, const void* gamma_u, float* conv_state,
                      int32_t* state_pos, int32_t flags, void* out, void* stream);

/*
 * The whole layer in one call (steps 1-8 above), intermediates in fp32: K is
 * never materialised, V and U stay fp32.
 *   raw_ids   device int32[B, T]
 *   history   device int32[B, max_order - 1] RAW ids before position 0 (oldest
 *             first), compressed here; NULL = pad_id (decode passes the last
 *             tokens of each sequence)
 *   lut       device int32[vocab]
 *   tables    HOST array of n_tables device pointers (see ngram_gather)
 *   hidden, hidden_branch_stride, w_k, w_v, gamma_q, gamma_k: as ngram_gate,
 *             hidden indexed by token b*T + t
 *   conv_w, gamma_u, conv_state, state_pos: as ngram_causal_conv (with the
 *             ring, one call per new token gives the Delta_t that one call over
 *             the whole sequence gives)
 *   flags     0 or NGRAM_ADD_RESIDUAL and / or NGRAM_UPDATE_STATE and / or
 *             NGRAM_PREFETCHED (the hash and gather already ran, see
 *             ngram_forward_prefetch: raw_ids, history, lut and tables are
 *             then checked but not read) or NGRAM_KEEP_FOR_BACKWARD (training:
 *             see ngram_backward; not with NGRAM_PREFETCHED)
 *   out       device [B, T, n_branches, d] act_dtype (output): Delta_t, or
 *             hidden + Delta_t with NGRAM_ADD_RESIDUAL
 *   gates     device float[B, T, n_branches] (output), nullable
 *   err_flag  device int32, nullable (see conventions)
 *   workspace device scratch of at least ngram_forward_workspace_size() bytes;
 *             when the call's work is done it holds the call's row ids and
 *             memory vector E (ngram_forward_workspace_view)
 */
size_t ngram_forward_workspace_size(const ngram_config* cfg, int32_t B, int32_t T);
int ngram_forward(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                  const int32_t* history, const int32_t* lut, const void* const* tables,
                  const void* hidden, int64_t hidden_branch_stride, const void* w_k,
                  const void* w_v, const void* conv_w, const void* gamma_q,
                  const void* gamma_k, const void* gamma_u, float* conv_state,
                  int32_t* state_pos, int32_t flags, void* out, float* gates,
                  int32_t* err_flag, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The lookup half of ngram_forward, ahead of the rest ("Qwen3.8-Flash-Next
 * 深度研究" §2.3: the n-gram hash ids are known as soon as the tokens enter the
 * network, so the lookup can be issued early; "Qwen3.8 加了 51B 查表参数，模型
 * 开始像数据库了", section "510 亿参数不走算力主干": the lookup positions can be
 * computed in advance and the fetch overlapped with the model's other work).  Steps 1-4: compresses the
 * raw ids, hashes the n-grams and gathers E into the workspace, where
 * ngram_forward_workspace_view locates them; a later ngram_forward with the
 * same cfg, B, T and workspace and NGRAM_PREFETCHED runs steps 5-8 on them.
 * A caller that knows the ids before the layer's input is ready -- at the
 * start of the model's forward pass, the layer sitting after others -- can
 * run this on a second stream and order the forward after it with an event.
 * Arguments as ngram_forward; the workspace must stay untouched between the
 * two calls.  Returns what ngram_forward would for these arguments (and
 * NGRAM_EWORKSPACE for a workspace too small for the whole forward).
 */
int ngram_forward_prefetch(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                           const int32_t* history, const int32_t* lut, const void* const* tables,
                           int32_t* err_flag, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Where ngram_forward leaves the row ids and the memory vector of its tokens
 * in the workspace (offsets in bytes from the workspace's start; the layout
 * depends only on cfg, B and T).  After the call's work is done (stream
 * order), until the workspace is reused:
 *   row_idx_offset  int32[B*T, n_tables]: the row of table j for token b*T + t
 *   mem_offset      E, bf16 (fp8 tables widened) or fp32, in mem_layout:
 *     NGRAM_MEM_ROWS     [B*T, mem_dim] row-major
 *     NGRAM_MEM_TILES16  1 KB tiles of 16 tokens x 32 values (the decode
 *                        route, bf16): value k of token i sits at element
 *                        ((i/16) * (mem_dim/32) + k/32) * 512
 *                        + (16 * ((k%32)/8) + i%16) * 8 + k%8,
 *                        for i < 16 * ceil(B*T / 16)
 * Returns NGRAM_OK, or the status ngram_forward would return for these sizes.
 */
#define NGRAM_MEM_ROWS 0
#define NGRAM_MEM_TILES16 1
typedef struct ngram_workspace_view {
  int64_t row_idx_offset;
  int64_t mem_offset;
  int32_t mem_layout;
  int32_t reserved;
} ngram_workspace_view;
int ngram_forward_workspace_view(const ngram_config* cfg, int32_t B, int32_t T,
                                 ngram_workspace_view* view);

/*
 * Backward of ngram_forward (training): the gradients of L = sum(d_out (.) out)
 * for the tables, W_K, W_V, the conv taps, the query rows and the RMSNorm
 * gains, each step the chain rule of the forward step ("Qwen3.8-Flash-Next
 * 深度研究" §2.3).  The table gradient is the lookup's adjoint, a scatter-add
 * of dE into the rows the tokens named -- the page lists this "scatter"
 * beside the gather among the layer's fused operators (the same page, §9.4).
 *
 * Supported: bf16 activations, W stored [d, mem] (NGRAM_W_D_MEM), hidden_dim
 * a multiple of 64 and at most 4096; the tables may be bf16 or fp8.  The
 * forward intermediates (E, K, V, gates, norms) are recomputed.
 *
 *   raw_ids ... conv_state, state_pos, flags  as for ngram_forward
 *              (NGRAM_ADD_RESIDUAL: out = hidden + Delta, so d_hidden also
 *              receives d_out; the ring is only read, NGRAM_UPDATE_STATE is
 *              rejected)
 *   d_out      device [B, T, n_branches, d] bf16: dL/d(out)
 *   d_tables   HOST array of n_tables device pointers, table j an fp32
 *              [rows[j], row_dim] gradient, ACCUMULATED (+=); a row named by
 *              several tokens adds their contributions in ascending token
 *              order, so every gradient is bit-identical from run to run
 *   d_w_k      device fp32 [n_branches, d, mem_dim] (written), d_w_v fp32 [d, mem_dim]
 *   d_conv_w   device fp32 [conv_kernel, d] (written)
 *   d_hidden   device fp32, hidden's layout (written), nullable
 *   d_gammas   device fp32 [3, d]: gamma_q, gamma_k, gamma_u (written), nullable
 *   workspace  device, >= ngram_backward_workspace_size(cfg, B, T) bytes
 *
 * dK and dV enter the dE and dW products as bf16 (fp32 accumulation); the
 * other gradients are fp32 throughout.  Returns NGRAM_EDTYPE / NGRAM_ESHAPE
 * for configurations outside the supported set, otherwise as ngram_forward.
 *
 * Training without the recompute: an ngram_forward call with
 * NGRAM_KEEP_FOR_BACKWARD and a workspace of ngram_backward_workspace_size()
 * bytes leaves its row ids, E and fp32 K and V there (the prefill route is
 * taken whatever B and T are; same supported set as this call, else
 * NGRAM_EDTYPE / NGRAM_ESHAPE).  An ngram_backward with
 * NGRAM_KEEP_FOR_BACKWARD, the same cfg, B, T and workspace, then skips its
 * first stage and uses them; raw_ids, history, lut and tables are checked
 * but not read.  The backward leaves them intact, so several backward calls
 * may follow one forward.  The caller must not use the workspace for
 * anything else in between; ngram_forward_workspace_view does not describe
 * this layout.
 */
size_t ngram_backward_workspace_size(const ngram_config* cfg, int32_t B, int32_t T);
int ngram_backward(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                   const int32_t* history, const int32_t* lut, const void* const* tables,
                   const void* hidden, int64_t hidden_branch_stride, const void* w_k,
                   const void* w_v, const void* conv_w, const void* gamma_q,
                   const void* gamma_k, const void* gamma_u, const float* conv_state,
                   const int32_t* state_pos, int32_t flags, const void* d_out,
                   float* const* d_tables, float* d_w_k, float* d_w_v, float* d_conv_w,
                   float* d_hidden, float* d_gammas, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * ngram_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same work and the same kernels as ngram_forward, with the scratch taken
 * from an array the library holds in device memory (NGRAM_NOALLOC_SCRATCH_BYTES
 * per GPU, reserved when the library's code is loaded on that GPU and held
 * until the process ends) instead of a caller's workspace.  The caller still
 * passes every input and output.  The call allocates nothing: no hipMalloc,
 * hipFree or allocating library routine; the first call on a device looks up
 * that device's copy of the array (hipGetSymbolAddress) on the current device,
 * which must be the stream's.
 * Returns NGRAM_ESCRATCH, launching nothing, when the call's scratch (what
 * ngram_forward_workspace_size would ask for) exceeds the array: e.g. more
 * than about 4,000 tokens of a prefill at the Qwen dimensions.
 * Every call on one GPU shares that GPU's array and finds the previous call's
 * contents there (no kernel needs it cleared): calls that may overlap on one
 * GPU -- on different streams, or from different threads -- race and must be
 * serialised by the caller.  ngram_forward_workspace_view and
 * NGRAM_PREFETCHED (NGRAM_EINVAL) do not apply.
 */
#define NGRAM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ngram_forward_noalloc(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                          const int32_t* history, const int32_t* lut, const void* const* tables,
                          const void* hidden, int64_t hidden_branch_stride, const void* w_k,
                          const void* w_v, const void* conv_w, const void* gamma_q,
                          const void* gamma_k, const void* gamma_u, float* conv_state,
                          int32_t* state_pos, int32_t flags, void* out, float* gates,
                          int32_t* err_flag, void* stream);

/*
 * Instrumented variants for benchmarks (not part of the layer): the same work
 * as ngram_forward / ngram_backward, and each stage's kernels timed on the
 * device.  stage_events is a HOST array of 2 * NGRAM_N_STAGES hipEvent_t:
 * the first kernel of stage i stamps its begin time into stage_events[2i]
 * and every kernel of the stage its end time into stage_events[2i + 1]
 * (hipExtLaunchKernel), so hipEventElapsedTime of the pair is the stage's
 * kernel time with no event packet between the kernels.  Forward stages:
 * 0 hash, 1 gather, 2 projection, 3 gate + conv; a kernel that covers several
 * stages counts in the last of them (decode hashes and gathers in one kernel)
 * and the stages it absorbs leave their events untouched.  Backward stages:
 * 0 the recompute (hash, gather, K / V product), 1 the per-row backward, 2 the
 * dE product (with its transposes), 3 the dW products and the table
 * scatter-add.  *stage_mask (host, nullable) receives the bit mask of the
 * stages that launched a kernel.  The events are used for the duration of
 * the call only; nothing is kept.
 */
#define NGRAM_N_STAGES 4
int ngram_forward_timed(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                        const int32_t* history, const int32_t* lut, const void* const* tables,
                        const void* hidden, int64_t hidden_branch_stride, const void* w_k,
                        const void* w_v, const void* conv_w, const void* gamma_q,
                        const void* gamma_k, const void* gamma_u, float* conv_state,
                        int32_t* state_pos, int32_t flags, void* out, float* gates,
                        int32_t* err_flag, void* workspace, size_t workspace_bytes,
                        void* stream, void* const* stage_events, int32_t* stage_mask);
int ngram_backward_timed(const ngram_config* cfg, const int32_t* raw_ids, int32_t B, int32_t T,
                         const int32_t* history, const int32_t* lut, const void* const* tables,
                         const void* hidden, int64_t hidden_branch_stride, const void* w_k,
                         const void* w_v, const void* conv_w, const void* gamma_q,
                         const void* gamma_k, const void* gamma_u, const float* conv_state,
                         const int32_t* state_pos, int32_t flags, const void* d_out,
                         float* const* d_tables, float* d_w_k, float* d_w_v, float* d_conv_w,
                         float* d_hidden, float* d_gammas, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* stage_events,
                         int32_t* stage_mask);

#ifdef __cplusplus
}
#endif

#endif /* NGRAM_H */
