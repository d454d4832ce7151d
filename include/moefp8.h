/*
 * moefp8.h - C ABI of libmoefp8.so: the forward pass of a DeepSeek-V3/R1-shaped
 * Mixture-of-Experts FFN layer in blockwise FP8 on one AMD MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [R1 card]   llm-architectures-explained, "DeepSeek-R1", "Every architecture field":
 *               d_model 7168, 256 routed experts, 8 active, d_expert 2048, gated
 *               experts, 1 shared expert of width 2048, dense first layers d_ff 18432.
 *   [arch blog] onlylabs, "DeepSeek v3 and R1 Model Architecture", "Architecture
 *               Overview" (SwiGLU), "More Aggressive Mixture-of-Expert" (9 of 257
 *               active, 1 shared), "Structural change" (shared expert always on),
 *               "Local Balanced Routing to Experts" (affinity gating, routing-only
 *               bias), FP8 headings "Fine granularity quantization", "More Mantissa
 *               bits of fp8", "Better Accumulation Precision", "Online Quantization",
 *               "More customized data format and scaling factor".
 *   [aguasto]   aguasto, "DeepSeek-R1" record, "Quantization" (blockwise FP8).
 *
 * Conventions for every call:
 *   - Returns MOE_OK (0) or a negative status; moe_status_string() names it and
 *     moe_last_error() gives a message (thread-local, valid until the next call
 *     on the same thread).
 *   - Every array argument is a DEVICE pointer, allocated and owned by the
 *     caller; the library allocates nothing and keeps no state between calls
 *     (moe_ffn_forward_noalloc aside: its workspace is a static device array).
 *   - Calls enqueue kernels only (no allocation, memset, copy or synchronisation
 *     unless MOEFP8_VALIDATE is on), so they can be captured into a HIP graph; the
 *     forward's capture and replay are tested.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work and return; nothing synchronises the host.
 *   - Shapes and pointers are checked on the host before anything is enqueued;
 *     a failed check enqueues nothing.
 *   - Device data (expert ids, positions, offsets, given scores) is trusted by
 *     default: values that break a call's stated contract give undefined results
 *     and may fault the GPU.  With the environment variable MOEFP8_VALIDATE set
 *     (to anything but "" or "0") when a call is made, the calls that read such
 *     data check it on the device first, synchronise `stream`, and return
 *     MOE_ERR_INVALID_DATA, enqueuing nothing else, when an element breaks the
 *     contract (the message names the first such element and its value).  What
 *     each call checks is listed with it ("Validated:").  The checks cost one pass
 *     over the data and a stream synchronisation per call (not usable under HIP
 *     graph capture); their result word is one per GPU, so validated calls that
 *     overlap on one GPU (other streams or threads) race on it.
 *   - Layouts are row-major.  FP8 means OCP E4M3FN bytes (max 448, no inf,
 *     0x7F/0xFF NaN).  bf16 and fp8 data are passed as raw bits.
 *   - Alignment: every pointer 16-byte aligned; leading dimensions keep rows
 *     16-byte aligned.
 */
#ifndef MOEFP8_H
#define MOEFP8_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1)       /* null pointer, misalignment, bad enum, negative size   */
#define MOE_ERR_UNSUPPORTED_SHAPE (-2) /* a size the kernels do not handle (e.g. not % 128)     */
#define MOE_ERR_WORKSPACE (-3)         /* workspace missing or smaller than required            */
#define MOE_ERR_HIP (-4)               /* a HIP launch failed (hipGetLastError after enqueue)   */
#define MOE_ERR_INVALID_DATA (-5)      /* MOEFP8_VALIDATE: device data breaks the call's contract */

/* ---- element types ---- */
#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1
#define MOE_DTYPE_U8 2

/* ---- group score rule (the pages give none; see moe_route) ---- */
#define MOE_GROUP_SCORE_TOP2_SUM 0     /* sum of the two largest biased scores of the group */
#define MOE_GROUP_SCORE_MAX 1          /* largest biased score of the group                 */

/* ---- scale formats of the 1x128 / 128x128 quantisation ---- */
#define MOE_SCALE_F32 0                /* s = max(fp32(amax / 448), 2^-126), correctly rounded */
#define MOE_SCALE_UE8M0 1              /* s = smallest power of two 2^k >= amax / 448, k in
                                          [-127, 127] (an 8-bit exponent); v / s is then exact */

/* ---- flags ---- */
#define MOE_ROUTE_SCORES_GIVEN 1       /* moe_route / moe_ffn_forward: `scores` is an input   */
#define MOE_FWD_DETERMINISTIC 2        /* moe_ffn_forward: slot-ordered combine (always the case;
                                          accepted for callers that ask for it explicitly)      */

/* ---- grouped GEMM epilogues ---- */
#define MOE_EPI_STORE_F32 0            /* out f32 [M][N]                                        */
#define MOE_EPI_STORE_BF16 1           /* out bf16 [M][N], round to nearest even                */
#define MOE_EPI_SWIGLU_QUANT 2         /* N = 2W, B rows [gate; up]: out = e4m3 codes [M][W] of
                                          h = silu(gate) * up, epi->h_s f32 [M][W/128]          */
#define MOE_EPI_WEIGHTED_SCATTER_ADD 3 /* out f32 [R][N]: out[dst_row[m]] += row_weight[m] * y[m]
                                          (fp32 atomics: bits vary run to run)                  */

/* Layer configuration.  Field names follow the model config ([R1 card]). */
typedef struct moe_cfg {
  int hidden;        /* d_model; % 128 == 0                                              */
  int inter;         /* routed expert width (moe_intermediate_size); % 128 == 0           */
  int n_experts;     /* routed experts; 0 = a dense gated FFN (only the "shared" MLP)     */
  int top_k;         /* experts per token (num_experts_per_tok)                            */
  int n_shared;      /* 0 or 1 always-on gated MLP                                         */
  int inter_shared;  /* its width; % 128 == 0                                              */
  int n_group;       /* expert groups: contiguous id blocks of n_experts / n_group         */
  int topk_group;    /* groups kept per token                                              */
  int group_score;   /* MOE_GROUP_SCORE_*                                                  */
  float routed_scale;/* multiplies the normalised routed weights (1.0)                     */
  int scale_fmt;     /* MOE_SCALE_*: the activation (x and h) scales; the weights' 128x128
                        scales are expected in the same format                             */
  float norm_eps;    /* RMSNorm epsilon, used when moe_weights_t.norm_w is given           */
} moe_cfg_t;

/* Device pointers to one layer's weights.  Expert e's blocks start at
 * e * (its matrix size); scales hold one fp32 per 128x128 block.  The e4m3
 * codes are in MFMA-fragment order (see moe_pack_weights); the shapes below
 * are the logical row-major [rows][cols] of each matrix.                    */
typedef struct moe_weights {
  const uint16_t* w_router; /* bf16 [E][hidden]                                     */
  const float* bias;        /* f32 [E] routing-only bias, or NULL (= 0)             */
  const uint8_t* w13_q;     /* e4m3 [E][2*inter][hidden], rows [gate; up]           */
  const float* w13_s;       /* f32 [E][2*inter/128][hidden/128]                     */
  const uint8_t* w2_q;      /* e4m3 [E][hidden][inter]                              */
  const float* w2_s;        /* f32 [E][hidden/128][inter/128]                       */
  const uint8_t* sh_w13_q;  /* shared expert / dense MLP: e4m3 [2*inter_shared][hidden] */
  const float* sh_w13_s;    /* f32 [2*inter_shared/128][hidden/128]                 */
  const uint8_t* sh_w2_q;   /* e4m3 [hidden][inter_shared]                          */
  const float* sh_w2_s;     /* f32 [hidden/128][inter_shared/128]                   */
  const uint16_t* norm_w;   /* bf16 [hidden] RMSNorm weight applied to x first, or NULL */
} moe_weights_t;

/* Extra epilogue operands of fp8_grouped_gemm_blockscaled. */
typedef struct moe_epi {
  float* h_s;                /* SWIGLU_QUANT: f32 [M][W/128] scales of the output codes      */
  const int32_t* dst_row;    /* WEIGHTED_SCATTER_ADD: destination row of each logical row m */
  const float* row_weight;   /* WEIGHTED_SCATTER_ADD: weight per row m, or NULL (= 1)       */
  int scale_fmt;             /* MOE_SCALE_* of every scale of the call.  MOE_SCALE_UE8M0: a_s and
                                b_s hold powers of two (as fp32 values 2^k, k in [-127, 127]), which
                                the GEMM applies as the FP8 MFMA's E8M0 scale operands (or in the
                                exact bf16 conversion of the SwiGLU path) instead of promoting each
                                K block; SWIGLU_QUANT then also writes power-of-two h_s.  Scales
                                that are not powers of two give undefined results in this mode.
                                A NULL epi means MOE_SCALE_F32.                               */
} moe_epi_t;

MOE_API const char* moe_status_string(int status);
MOE_API const char* moe_last_error(void);
/* moe_validation_enabled - 1 when calls made now validate device data (MOEFP8_VALIDATE), else 0. */
MOE_API int moe_validation_enabled(void);

/* fp8_quant_1x128 - online activation quantisation ([arch blog] "Fine granularity
 * quantization", "Online Quantization").  Per row, per 128 consecutive columns:
 * amax = max |v|; s = fp32(amax / 448) (correctly rounded, at least 2^-126;
 * 1.0 for an all-zero tile), or with MOE_SCALE_UE8M0 the power of two of MOE_SCALE_UE8M0 ([arch
 * blog] "More customized data format and scaling factor");
 * q = e4m3(fp32(v / s)) rounded to nearest even, saturating.
 *   x      [rows][ld_x] of x_dtype (MOE_DTYPE_BF16 or MOE_DTYPE_F32), cols used
 *   q      e4m3 [rows][ld_q]
 *   s      f32 [rows][cols/128]
 * cols % 128 == 0; ld_x >= cols, ld_q >= cols, rows >= 0 (0: no-op).          */
MOE_API int fp8_quant_1x128(const void* x, int x_dtype, int rows, int cols, int ld_x, uint8_t* q, int ld_q, float* s,
                    int scale_fmt, void* stream);

/* fp8_quant_128x128 - weight preparation (not on the timed path): the same rule
 * over 128x128 blocks ([aguasto] "Quantization": blockwise FP8).
 *   w f32 [rows][cols] -> q e4m3 [rows][cols], s f32 [rows/128][cols/128].   */
MOE_API int fp8_quant_128x128(const float* w, int rows, int cols, uint8_t* q, float* s, int scale_fmt, void* stream);

/* fp8_rmsnorm_quant_1x128 - the RMSNorm in front of the MLP ([R1 card] facts
 * table rows "Norm placement" and "Norm type": pre-norm, RMSNorm before the
 * MLP) fused with fp8_quant_1x128.  Per row t of x:
 *   inv = fp32(1 / sqrt(S / cols + eps)) in fp64, S = sum of x^2 rounded once to fp64;
 *   y   = bf16(fp32(fp32(x * inv) * gamma))  (round to nearest even);
 *   q, s = fp8_quant_1x128 of y with scale_fmt.
 *   x bf16 [rows][ld_x]; gamma bf16 [cols]; eps >= 0;
 *   y bf16 [rows][ld_y] or NULL (the normalised rows, e.g. for the router);
 *   q e4m3 [rows][ld_q]; s f32 [rows][cols/128].
 * cols % 128 == 0; ld_x, ld_y, ld_q >= cols.                                 */
MOE_API int fp8_rmsnorm_quant_1x128(const uint16_t* x, const uint16_t* gamma, float eps, int rows, int cols, int ld_x,
                                    uint16_t* y, int ld_y, uint8_t* q, int ld_q, float* s, int scale_fmt,
                                    void* stream);

/* moe_pack_weights - reorders row-major e4m3 weights [G][N][K] into the
 * MFMA-fragment order every GEMM of this library reads (offline, like the
 * 128x128 quantisation; not on the timed path).  Block (g, n16, kb) of 2048
 * bytes holds rows 16*n16..+15 and columns 128*kb..+127 of matrix g, blocks
 * ordered by (g, n16, kb), and inside a block byte h*1024 + (16*q + r)*16 + b is
 * B[16*n16 + r][128*kb + 64*h + 16*q + b].  One wave-wide 16-byte load then
 * reads 1 KB of consecutive bytes in lane order, exactly the B operands of a
 * 16x16x128 MFMA, and a 16-row slice's whole K range is one contiguous stream.  Scales are not
 * reordered.  N % 16 == 0, K % 128 == 0; src and dst must not overlap.      */
MOE_API int moe_pack_weights(const uint8_t* src, int G, int N, int K, uint8_t* dst, void* stream);

/* moe_route - gating ([arch blog] "Local Balanced Routing to Experts").
 * Without MOE_ROUTE_SCORES_GIVEN: scores[t][e] = sigmoid(sum_d x[t][d] * w_router[e][d])
 * (bf16 operands, fp32 accumulation) is computed and written.  With it, x and
 * w_router are ignored and `scores` is read.  Then, in fp32:
 *   b = scores + bias (bias only selects); groups of n_experts/n_group contiguous
 *   experts are scored by cfg->group_score; the topk_group best groups are kept
 *   (ties: lower group index); the top_k experts by b among them are chosen
 *   (ties: lower expert index), slot j = j-th best;
 *   topk_w[t][j] = fp32(scores[t][e_j] / S) * routed_scale, S = fp32 sum of the
 *   chosen scores in slot order.
 *   x bf16 [T][hidden] or NULL; w_router bf16 [E][hidden] or NULL; bias f32 [E] or NULL;
 *   scores f32 [T][E] (in or out); topk_idx i32 [T][top_k]; topk_w f32 [T][top_k].
 * Requires n_experts % n_group == 0, topk_group <= n_group, top_k <= topk_group *
 * n_experts / n_group, n_experts <= 1024, n_group <= 64, top_k <= 64.
 * Validated: given scores and bias finite (NaN scores route arbitrarily).      */
MOE_API int moe_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int T, const moe_cfg_t* cfg,
              float* scores, int flags, int32_t* topk_idx, float* topk_w, void* stream);

/* moe_bias_update - one balancing step of the routing-only bias ([arch blog]
 * "Local Balanced Routing to Experts": the bias of an overloaded expert is
 * decreased by gamma, that of an underloaded one increased).  With load_e the
 * number of entries of topk_idx equal to e and the mean load (T*k)/E:
 *   bias[e] = fp32(bias[e] + gamma * sign(mean - load_e))   (+0 at the mean)
 *   topk_idx i32 [T][k] (entries outside [0, E) are not counted); bias f32 [E]
 *   in place; counts i32 [E] receives load_e, or NULL.
 * 1 <= E <= 1024, T >= 0, k >= 1, T*k <= 2^30.                               */
MOE_API int moe_bias_update(const int32_t* topk_idx, int T, int k, int E, float gamma, float* bias, int32_t* counts,
                            void* stream);

/* moe_permute - sort the T*k assignments a = t*k + j by expert, stably (by
 * expert, then a).  offsets[e]..offsets[e+1] is expert e's range of sorted
 * rows; sorted_assign[p] = a at sorted position p; assign_pos[a] = p.
 * Optionally gathers rows: rows_out[p] = rows_in[sorted_assign[p] / k]
 * (row_bytes each, a multiple of 16; pass NULL for both to skip).
 *   topk_idx i32 [T][k]; offsets i32 [E+1]; sorted_assign, assign_pos i32 [T*k].
 * Scratch: the call needs moe_permute_workspace_size(T, k, E) bytes in `ws`.
 * Validated: every topk_idx entry in [0, E).                                 */
MOE_API size_t moe_permute_workspace_size(int T, int k, int E);
MOE_API int moe_permute(const int32_t* topk_idx, int T, int k, int E, int32_t* offsets, int32_t* sorted_assign,
                int32_t* assign_pos, const void* rows_in, int row_bytes, void* rows_out, void* ws,
                size_t ws_bytes, void* stream);

/* moe_unpermute - the inverse of moe_permute and the routed combine.
 *   topk_w == NULL: out[t][j][:] = y_sorted[assign_pos[t*k+j]][:] (same dtype:
 *     F32, BF16 or U8), so unpermute(permute(rows)) repeats each row k times.
 *   topk_w != NULL (y_dtype F32): out bf16 [T][d] =
 *     bf16(sum_j topk_w[t][j] * y_sorted[assign_pos[t*k+j]] + shared_y[t]),
 *     summed in fp32 in slot order, shared_y f32 [T][d] or NULL (shared weight 1,
 *     [arch blog] "Structural change").  d % 4 == 0, T*k <= 2^30.
 * Validated: every assign_pos entry in [0, T*k).                            */
MOE_API int moe_unpermute(const void* y_sorted, int y_dtype, const int32_t* assign_pos, const float* topk_w,
                  const float* shared_y, int T, int k, int d, void* out, void* stream);

/* fp8_grouped_gemm_blockscaled - C_g = A_g . B_g^T for each group g, with
 * blockwise scales promoted into an fp32 accumulator once per 128-wide K block
 * ([arch blog] "Fine granularity quantization", "Better Accumulation Precision"):
 *   C[m][n] = sum_kb a_s[row(m)][kb] * b_s[g][n/128][kb] * sum_{k in kb} A[row(m)][k] B[g][n][k]
 *   a_q e4m3 [*][K], a_s f32 [*][K/128]; row(m) = a_gather[m] or m if NULL;
 *   b_q e4m3 [G][N][K] in MFMA-fragment order (moe_pack_weights), b_s f32 [G][N/128][K/128];
 *   offsets i32 [G+1] (device): group g owns logical rows offsets[g]..offsets[g+1];
 *   M_max: an upper bound of offsets[G] known on the host (sizes the launch).
 *   epilogue MOE_EPI_* with `out` and `epi` as documented at the constants.
 * N % 128 == 0 (SWIGLU_QUANT: N % 256 == 0), K % 128 == 0, G >= 1.  G = 1 with
 * offsets {0, M} is a plain block-scaled GEMM (the dense layer).
 * Validated: 0 <= offsets[0] <= ... <= offsets[G] <= M_max; a_gather[m] >= 0 and
 * (WEIGHTED_SCATTER_ADD) epi->dst_row[m] >= 0 for the rows m of the groups (the
 * arrays' row counts are not known to the call).                            */
MOE_API int fp8_grouped_gemm_blockscaled(const uint8_t* a_q, const float* a_s, const int32_t* a_gather, const uint8_t* b_q,
                                 const float* b_s, const int32_t* offsets, int G, int M_max, int N, int K,
                                 int epilogue, const moe_epi_t* epi, void* out, void* stream);

/* moe_ffn_workspace_size - bytes of device workspace moe_ffn_forward needs
 * for T tokens (host-only; 0 on invalid arguments).                         */
MOE_API size_t moe_ffn_workspace_size(int T, const moe_cfg_t* cfg);

/* moe_ffn_forward - one MoE FFN layer ([R1 card], [arch blog] "More
 * Aggressive Mixture-of-Expert", "Structural change"):
 *   x -> 1x128 e4m3; scores, routing (moe_route); permutation (moe_permute);
 *   per expert h = silu(x W_gate^T) * (x W_up^T) -> 1x128 e4m3; y = h W_down^T;
 *   out[t] = bf16(sum_j topk_w[t][j] * y[t][j] + y_shared[t]).
 * n_experts == 0 runs the dense gated FFN (x -> shared MLP -> out).
 * With w->norm_w, x first goes through the RMSNorm of fp8_rmsnorm_quant_1x128
 * (cfg->norm_eps) and the router and the experts see the normalised rows.
 * cfg->scale_fmt selects the activation scale format (x and h).
 *   x bf16 [T][hidden]; out bf16 [T][hidden];
 *   scores f32 [T][E], topk_idx i32 [T][k], topk_w f32 [T][k]: optional outputs
 *   (NULL to skip); with MOE_ROUTE_SCORES_GIVEN `scores` is an input instead.
 *   The combine is slot-ordered in fp32, so the output is bit-reproducible run to
 *   run (MOE_FWD_DETERMINISTIC is accepted and changes nothing).
 * ws: at least moe_ffn_workspace_size(T, cfg) bytes, 256-byte aligned.
 * Validated (routed layers): given scores and the routing bias finite.      */
MOE_API int moe_ffn_forward(const uint16_t* x, int T, const moe_cfg_t* cfg, const moe_weights_t* w, void* ws,
                    size_t ws_bytes, uint16_t* out, float* scores, int32_t* topk_idx, float* topk_w, int flags,
                    void* stream);

/* moe_ffn_forward_stages - moe_ffn_forward with hipEvent_t handles (passed as
 * void*, created by the caller) recorded on `stream` between its stages, for
 * live per-stage timing of the same launches:
 *   events[0] before quantising x, [1] after it, [2] after routing and the
 *   permutation, [3] after the gate/up GEMM, [4] after the down GEMM,
 *   [5] after the combine/cast.
 * n_events must be 0 (then it is moe_ffn_forward) or MOE_FWD_STAGE_EVENTS; a
 * NULL entry is not recorded (each record costs the stream a few
 * microseconds, so a caller can time one stage alone).  */
#define MOE_FWD_STAGE_EVENTS 6
MOE_API int moe_ffn_forward_stages(const uint16_t* x, int T, const moe_cfg_t* cfg, const moe_weights_t* w, void* ws,
                                   size_t ws_bytes, uint16_t* out, float* scores, int32_t* topk_idx, float* topk_w,
                                   int flags, void* const* events, int n_events, void* stream);

/* ---- FP8 backward of the grouped GEMMs ([arch blog] "First ever FP8 Precision OSS LLM
 * pre-training": the model trains with FP8 matrix multiplications; the section stops after its
 * motivation, so the following is a reading).  For a forward GEMM C_g = A_g . W_g^T over group
 * g's rows (A 1x128-quantised, W in 128x128 blocks):
 *   dgrad  dA = dC . W: fp8_quant_1x128 of dC along its contraction dimension, then
 *          fp8_grouped_gemm_blockscaled with W^T from moe_pack_weights_transposed (W's 128x128
 *          blocks read transposed, with the same scales);
 *   wgrad  dW_g = dC_g^T . A_g, a contraction over the group's rows: fp8_quant_128x1_grouped of
 *          dC and of A (128x1 tiles: per column, per 128 rows of one group), then
 *          fp8_grouped_gemm_wgrad.  ---- */

/* moe_padded_rows - an upper bound of the padded row count of M rows in G groups, each group
 * padded to a multiple of 128: (ceil(M / 128) + G) * 128 (0 on invalid arguments). */
MOE_API size_t moe_padded_rows(int M, int G);

/* fp8_quant_128x1_grouped - transposed ("128x1") tile quantisation for wgrad.  x [M][ld_x]
 * (x_dtype MOE_DTYPE_BF16 or MOE_DTYPE_F32, N columns used), rows grouped by offsets i32 [G+1]
 * (device, offsets[G] = M).  Each group is padded to a multiple of 128 rows; padded_offsets
 * i32 [G+1] (device, written) receives the padded offsets.  Output, transposed: q_t e4m3 [N][ld_q]
 * with q_t[n][padded[g] + r] the code of x[offsets[g] + r][n] (zeros in a group's padding),
 * s_t f32 [N][ld_q / 128], one scale per column and 128 padded rows, by the rule of
 * fp8_quant_1x128.  N % 128 == 0; ld_q % 128 == 0 and ld_q >= moe_padded_rows(M, G) (columns
 * past padded[G] are not written).  1 <= G <= 1024.
 * Validated: 0 = offsets[0] <= ... <= offsets[G] = M.                                    */
MOE_API int fp8_quant_128x1_grouped(const void* x, int x_dtype, int M, int N, int ld_x, const int32_t* offsets,
                                    int G, int32_t* padded_offsets, uint8_t* q_t, int ld_q, float* s_t,
                                    int scale_fmt, void* stream);

/* moe_pack_weights_transposed - weight preparation for dgrad: row-major e4m3 W [G][N][K] with
 * 128x128 block scales w_s f32 [G][N/128][K/128] -> W^T [G][K][N] in the MFMA-fragment order of
 * moe_pack_weights, and its scales wt_s f32 [G][K/128][N/128] (the same blocks, transposed).
 * N % 128 == 0, K % 128 == 0; the outputs must not overlap the inputs.                     */
MOE_API int moe_pack_weights_transposed(const uint8_t* w_q, const float* w_s, int G, int N, int K, uint8_t* wt_q,
                                        float* wt_s, void* stream);

/* fp8_grouped_gemm_wgrad - per group g:
 *   out[g][i][j] = sum over kb of a_ts[i][kb] * b_ts[j][kb] * sum_{k in kb} A_t[i][k] * B_t[j][k]
 * over the 128-wide K blocks kb of the group's padded rows [padded[g], padded[g+1]) (fp32
 * accumulation, FP8 MFMA; power-of-two scales with MOE_SCALE_UE8M0 go in as the MFMA's E8M0
 * operands).  a_t e4m3 [Na][ld], a_ts f32 [Na][ld/128], b_t e4m3 [Nb][ld], b_ts f32
 * [Nb][ld/128] (from fp8_quant_128x1_grouped); padded_offsets i32 [G+1] (device); M the rows
 * before padding (bounds the padded rows); out f32 [G][Na][Nb] (a group without rows gets
 * zeros).  Na % 128 == 0, Nb % 128 == 0, ld as for fp8_quant_128x1_grouped.
 * Validated: 0 = padded[0] <= ... <= padded[G] <= moe_padded_rows(M, G), multiples of 128. */
MOE_API int fp8_grouped_gemm_wgrad(const uint8_t* a_t, const float* a_ts, const uint8_t* b_t, const float* b_ts,
                                   const int32_t* padded_offsets, int G, int M, int Na, int Nb, int ld, float* out,
                                   int scale_fmt, void* stream);

/* moe_ffn_forward_noalloc - moe_ffn_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same launches, with the workspace taken from a static device array
 * of MOE_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on (from
 * the load of its code on that GPU until the process ends).  The call allocates
 * nothing; the caller still passes x, out and the optional routing outputs.
 *   Returns MOE_ERR_WORKSPACE (enqueuing nothing) when moe_ffn_workspace_size(T, cfg)
 *   exceeds MOE_NOALLOC_SCRATCH_BYTES (V3 layer shapes: T <= 223 tokens).
 *   The array is the current device's (the stream must belong to it).  Every call on
 *   one GPU shares that GPU's array and leaves its contents behind: calls that
 *   overlap on one GPU (other streams, other threads) race; serialise them.        */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
MOE_API int moe_ffn_forward_noalloc(const uint16_t* x, int T, const moe_cfg_t* cfg, const moe_weights_t* w,
                                    uint16_t* out, float* scores, int32_t* topk_idx, float* topk_w, int flags,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEFP8_H */
