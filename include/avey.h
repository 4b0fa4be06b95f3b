/*
 * avey.h -- C ABI of libavey.so: the Avey-B bidirectional ranker and dynamic contextualizer
 * core on AMD Instinct MI355X (gfx950).
 *
 * Sources cited below:
 *   [notes]   papernotes.org, ICLR2026 note "Avey-B: 把无注意力架构改造成双向编码器",
 *             sections 方法详解/整体框架, 关键设计 2, 关键设计 3 (eq. 6), 关键设计 4 (eq. 8).
 *   [summary] paperlayer.ai summary "Avey-B" (arXiv 2602.15814v1), sections 3 (Background),
 *             4.2, 4.3 (Neural compression) and appendix H (Ablation study).
 *
 * General conventions (all entry points)
 *   - Every pointer argument except the status string is DEVICE memory owned by the caller.
 *     The library allocates nothing, never synchronises, and no result depends on an earlier
 *     call. The one piece of state it holds is the fixed device array of
 *     avey_split_rank_noalloc (below). Calls are safe from several host threads at once; calls
 *     that share a workspace, an output buffer or that array must be ordered by the caller,
 *     e.g. by using one stream.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL means the default stream). The call
 *     returns once the kernels are enqueued.
 *   - Return value: AVEY_OK, or an AVEY_ERR_* code. Argument checks run on the host before
 *     any HIP call, so a call that fails them enqueues nothing. AVEY_ERR_HIP reports a launch
 *     error (hipGetLastError right after the launches). A fault while a kernel runs is only
 *     seen at the caller's next synchronisation.
 *   - Tensors are row-major. A [B, N, w] tensor with row stride `ld` (elements, ld >= w) has
 *     element (b, t, c) at offset (b * N + t) * ld + c. Rows t >= N are never read or written.
 *   - dtype AVEY_BF16: x, P, z and the outputs xhat/out are bf16 bit patterns (uint16),
 *     accumulation is fp32. dtype AVEY_F32: the same tensors are float32, arithmetic is fp32.
 *     scores and w are always float32; idx is always int32.
 *   - Splits: n_s = ceil(N / S). Split j holds tokens [j*S, min((j+1)*S, N)); the missing
 *     tokens of the last split are zero padding ([notes] 整体框架). Padding tokens take part
 *     neither as targets nor as candidates in MaxSim, are zero rows in X_cat, and are not
 *     mixed in the dynamic layer.
 *   - Outputs must not overlap inputs.
 *   - Empty work (B == 0 or N == 0) returns AVEY_OK and enqueues nothing; pointers may then
 *     be NULL.
 *   - Shape limits: 1 <= S <= 512. For AVEY_BF16 additionally S % 16 == 0, every ld is a
 *     multiple of 8, every tensor pointer is 16-byte aligned, the feature widths d and m_t are
 *     multiples of 8, and the enricher / fuser widths (d, m, m_h, m_t there) multiples of 64.
 *     For AVEY_F32 every tensor pointer is 4-byte aligned. Violations return AVEY_ERR_SHAPE,
 *     AVEY_ERR_ALIGN or AVEY_ERR_UNSUPPORTED.
 */
#ifndef AVEY_H
#define AVEY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AVEY_ABI_VERSION 2

/* The last enumerator widens the type's range to every int32 value, so that an unknown value a
 * caller passes is a valid avey_dtype the checks can reject (AVEY_ERR_DTYPE). */
typedef enum { AVEY_F32 = 0, AVEY_BF16 = 1, AVEY_DTYPE_RANGE_ = 0x7fffffff } avey_dtype;

typedef enum {
  AVEY_OK = 0,
  AVEY_ERR_NULL = -1,        /* a required pointer is NULL                              */
  AVEY_ERR_SHAPE = -2,       /* a size or leading dimension is out of range            */
  AVEY_ERR_DTYPE = -3,       /* unknown dtype                                          */
  AVEY_ERR_ALIGN = -4,       /* a pointer or leading dimension is misaligned           */
  AVEY_ERR_UNSUPPORTED = -5, /* valid request that this library does not implement     */
  AVEY_ERR_HIP = -6          /* the HIP runtime reported an error at launch            */
} avey_status;

/* ABI version implemented by the loaded library (AVEY_ABI_VERSION). */
int32_t avey_abi_version(void);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* avey_status_str(int32_t status);

/*
 * avey_maxsim -- all-pairs split relevance ([summary] section 3: the ranker scores every split
 * against the target split with MaxSim; [notes] 整体框架), straight from x, with no workspace.
 *
 *   scores[b, i, j] = sum over valid tokens t of split i of
 *                     max over valid tokens u of split j of cos(x_t, x_u),     for i != j
 *   scores[b, i, i] = -INFINITY
 * cos(x_t, x_u) = (x_t . x_u) / (|x_t| |x_u|), and 0 when either token is zero ([notes] 关键设计
 * 2: N(.) divides each token by its L2 norm). Padding tokens take part neither in the sum nor in
 * the max; rows t >= N of x are never read. For AVEY_BF16 the dot products and squared norms
 * accumulate in fp32 from the bf16 values; x must be finite: with a NaN or infinite token the
 * scores are unspecified.
 *
 *   x       [B, N, d] row stride ld_x, dtype dt (input)
 *   scores  [B, n_s, n_s] float32, contiguous (output)
 * Requires n_s >= 2. For AVEY_BF16, (N + 512) * ld_x < 2^30. MaxSim is not symmetric; both
 * directions of each split pair come from one pass over the pair.
 */
avey_status avey_maxsim(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d, int64_t ld_x,
                        int32_t S, float* scores, void* stream);

/*
 * Explicit-workspace scoring: the same scores as avey_maxsim from a normalised, zero-padded copy
 * of X in caller-provided device memory: n_t = N(x_t) = x_t / |x_t| (sum of squares in fp32;
 * N(0) = 0) for t < N, zero rows for the padding tokens of the last split ([notes] 关键设计 2;
 * 整体框架). Its layout is internal to the library (bf16: packed block by block in chunk planes
 * of 32 features, features padded with zeros to a multiple of 32, a block being one split, or
 * 256 consecutive tokens at S = 64 and 128; fp32: row-major n_s * S rows).
 *
 * avey_rank_workspace_bytes -- size in bytes of that workspace for (dt, B, N, d, S):
 * B * ceil(N / P) * P * d' * (2 for AVEY_BF16, 4 for AVEY_F32) with P = S (P = 256 for AVEY_BF16
 * at S = 64 and 128) and d' = d rounded up to a multiple of 32 for AVEY_BF16 (d for AVEY_F32),
 * 0 for empty work, or a negative avey_status if the shape is rejected (the same checks as
 * avey_maxsim_prepare).
 */
int64_t avey_rank_workspace_bytes(avey_dtype dt, int64_t B, int64_t N, int64_t d, int32_t S);

/*
 * avey_maxsim_prepare -- fill the workspace from x.
 *   x          [B, N, d] row stride ld_x, dtype dt (input)
 *   workspace  avey_rank_workspace_bytes(...) bytes, 16-byte aligned (output)
 * For AVEY_BF16, n_t is rounded to bf16 (round to nearest even); for AVEY_F32 it stays fp32.
 * Requires n_s >= 2.
 */
avey_status avey_maxsim_prepare(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d,
                                int64_t ld_x, int32_t S, void* workspace, void* stream);

/*
 * avey_maxsim_scores -- the scores of avey_maxsim from a workspace that avey_maxsim_prepare
 * filled (enqueued earlier) for the same (dt, B, N, d, S). With unit vectors the contraction
 * holds the cosines themselves: scores[b, i, j] = sum_t max_u n_t . n_u (dot products in fp32 of
 * the rounded n for AVEY_BF16).
 *
 *   workspace  (input, not modified)
 *   scores     [B, n_s, n_s] float32, contiguous (output)
 */
avey_status avey_maxsim_scores(const void* workspace, avey_dtype dt, int64_t B, int64_t N,
                               int64_t d, int32_t S, float* scores, void* stream);

/*
 * avey_topk_norm -- top-k selection and divide-by-max weighting ([notes] 整体框架: the ranker
 * keeps the k best candidate splits and divides their scores by the largest of them;
 * [summary] section 3).
 *
 * For each row (b, i) of scores, the candidates j != i are ordered by (score descending,
 * j ascending); NaN scores order as -INFINITY. The first k are written:
 *   idx[b, i, r] = j_r                  (int32, rank order)
 *   w[b, i, r]   = scores[b,i,j_r] / scores[b,i,j_0]   (IEEE fp32 division; w[..., 0] == 1
 *                                                       exactly when the top score is finite
 *                                                       and non-zero)
 *   scores  [B, n_s, n_s] float32 (input; the diagonal is ignored)
 *   idx, w  [B, n_s, k] int32 / float32 contiguous (outputs)
 * Requires 1 <= k <= n_s - 1.
 */
avey_status avey_topk_norm(const float* scores, int64_t B, int64_t n_s, int32_t k,
                           int32_t* idx, float* w, void* stream);

/*
 * avey_split_rank -- the bidirectional ranker: avey_maxsim, then avey_topk_norm, on the same
 * stream, with no workspace. Every argument check of both runs before the first launch.
 *   x                [B, N, d] row stride ld_x, dtype dt (input)
 *   scores, idx, w   [B, n_s, n_s], [B, n_s, k], [B, n_s, k] as described above (outputs)
 * Requires 1 <= k <= n_s - 1.
 */
avey_status avey_split_rank(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d,
                            int64_t ld_x, int32_t S, int32_t k, float* scores, int32_t* idx,
                            float* w, void* stream);

/*
 * avey_topk_norm_preceding -- the unidirectional ranker's selection ([summary] section 3: the
 * top-k preceding splits of each target split; the [summary] pretraining ablation and the
 * [notes] training-strategy section find that ranker direction the better one).
 * As avey_topk_norm, with the candidates of row i restricted to j < i. A row with fewer than
 * k candidates (i < k) is completed with idx = -1, w = 0 (empty blocks for
 * avey_select_compress); row 0 is all empty. w[..., 0] == 1 whenever row i has a candidate
 * whose score is finite and non-zero.
 */
avey_status avey_topk_norm_preceding(const float* scores, int64_t B, int64_t n_s, int32_t k,
                                     int32_t* idx, float* w, void* stream);

/*
 * avey_split_rank_noalloc -- for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops that must not call hipMalloc): the results of avey_split_rank,
 * computed through the explicit-workspace path (avey_maxsim_prepare, avey_maxsim_scores,
 * avey_topk_norm) with its workspace in a device array of AVEY_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends. Nothing is allocated.
 *   arguments and outputs as avey_split_rank; runs on the current device
 * Sequences go through the array in groups of as many as fit; a shape whose single sequence
 * needs more than AVEY_NOALLOC_SCRATCH_BYTES (avey_rank_workspace_bytes with B = 1) returns
 * AVEY_ERR_UNSUPPORTED. All calls on one GPU share its array: calls that overlap on one GPU (on
 * different streams or host threads) race and must be ordered by the caller.
 */
#define AVEY_NOALLOC_SCRATCH_BYTES (160LL << 20)
avey_status avey_split_rank_noalloc(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d,
                                    int64_t ld_x, int32_t S, int32_t k, float* scores, int32_t* idx,
                                    float* w, void* stream);

/*
 * avey_split_rank_preceding -- the unidirectional ranker: avey_maxsim, then
 * avey_topk_norm_preceding, on the same stream; arguments as avey_split_rank.
 */
avey_status avey_split_rank_preceding(const void* x, avey_dtype dt, int64_t B, int64_t N,
                                      int64_t d, int64_t ld_x, int32_t S, int32_t k, float* scores,
                                      int32_t* idx, float* w, void* stream);

/*
 * avey_select_compress -- weighted gather and neural compression ([notes] 关键设计 4, eq. 8;
 * [summary] 4.3 and appendix H).
 *
 * For each split (b, i):
 *   X_cat = [ X_i ; w[b,i,0] * X_{idx[b,i,0]} ; ... ; w[b,i,k-1] * X_{idx[b,i,k-1]} ]
 *           ((k+1)S x d; each X_j is split j as S rows with zero padding)
 *   Xhat_i = P X_cat + (residual ? X_i : 0)
 * and the valid rows of Xhat_i are written to xhat.
 *
 *   x        [B, N, d] row stride ld_x (input)
 *   idx, w   [B, n_s, k] int32 / float32 (inputs; idx in [0, n_s), or negative for an empty
 *            block of S zero rows -- the padding of avey_topk_norm_preceding; indices >= n_s
 *            are clamped to n_s - 1)
 *   P        [S, (k+1)S] contiguous, dtype dt (input)
 *   residual 0 or 1
 *   xhat     [B, N, d] row stride ld_out, dtype dt (output)
 * Requires k >= 1 (and k + 1 <= 512 for AVEY_BF16). For AVEY_BF16 the weights scale the fp32
 * accumulator between blocks, the retrieved blocks taken in ascending order of |w|; any finite
 * weight is accepted (negative, zero, above 1). A block whose |w| is below 2^-149 times the next
 * larger one's may be dropped. A NaN or infinite weight makes that split's outputs non-finite.
 * The result is rounded to bf16.
 */
avey_status avey_select_compress(const void* x, avey_dtype dt, int64_t B, int64_t N, int64_t d,
                                 int64_t ld_x, int32_t S, int32_t k, const int32_t* idx,
                                 const float* w, const void* P, int32_t residual, void* xhat,
                                 int64_t ld_out, void* stream);

/*
 * avey_dyn_context -- core of the dynamic contextualizer ([notes] 关键设计 2: mix Z_t with the
 * cosine matrix N(Z_t) N(Z_t)^T; 关键设计 3, eq. 6: divide each row by its sum plus eps).
 *
 * For each split (b, i), over its valid tokens p, q (no mask between them: bidirectional):
 *   n_p = z_p / |z_p|  (0 for a zero row)
 *   G_pq = n_p . n_q,   r_p = sum_q G_pq
 *   out_p = sum_q G_pq z_q / (r_p + eps)
 * The bias and activation of the full layer are not applied (avey_dyn_layer applies them).
 *
 *   z_tail  [B, N, m_t] row stride ld_z (input; point it at the first tail column of Z)
 *   out     [B, N, m_t] row stride ld_out, dtype dt (output)
 * For AVEY_BF16, G is rounded to bf16 for the product with z and r is summed from those
 * rounded values; the result is rounded to bf16.
 */
avey_status avey_dyn_context(const void* z_tail, avey_dtype dt, int64_t B, int64_t N, int64_t m_t,
                             int64_t ld_z, int32_t S, float eps, void* out, int64_t ld_out,
                             void* stream);

/*
 * Activation sigma of the contextualizer layers. The pages require only that it be monotone
 * ([summary] 4.2 and appendix A, relevance-monotonic updates); identity and ReLU are offered.
 */
typedef enum { AVEY_ACT_IDENTITY = 0, AVEY_ACT_RELU = 1 } avey_act;

/*
 * Row normalisation of the dynamic layer's cosine matrix G (per split, over its valid tokens):
 *   AVEY_NORM_SUM      S~_pq = G_pq / (sum_q G_pq + eps)              ([notes] 关键设计 3, eq. 6)
 *   AVEY_NORM_SOFTMAX  S~_pq = exp(G_pq) / sum_q exp(G_pq)
 *   AVEY_NORM_RMS      S~_pq = G_pq / sqrt(mean_q G_pq^2 + eps)
 *   AVEY_NORM_NONE     S~_pq = G_pq
 * The last three are the alternatives the [summary] compares (appendix B, normalisation
 * ablation; appendix H, no row-wise normalisation).
 */
typedef enum { AVEY_NORM_SUM = 0, AVEY_NORM_SOFTMAX = 1, AVEY_NORM_RMS = 2, AVEY_NORM_NONE = 3 } avey_norm;

/*
 * avey_dyn_layer -- dynamic contextualizer layer c_dyn = sigma(S~ Z_t + b) ([notes] 关键设计 2
 * and 3): the core of avey_dyn_context with the row normalisation `norm`, then for each valid
 * token p of split i
 *   out_p = act(core_p + bias[p - i S])      (one bias value per token position of a split)
 *
 *   z_tail, out, S, eps  as avey_dyn_context
 *   norm    an avey_norm (AVEY_NORM_SUM is avey_dyn_context's; other values: AVEY_ERR_SHAPE)
 *   bias    [S] float32 (input), or NULL for no bias
 *   act     an avey_act (other values: AVEY_ERR_SHAPE)
 * For AVEY_BF16 the weights S~ use G rounded to bf16 (for softmax: exp(G) rounded), the row
 * statistic is taken over those rounded values, and the bias is added to the fp32 value before
 * the activation and the single rounding to bf16.
 */
avey_status avey_dyn_layer(const void* z_tail, avey_dtype dt, int64_t B, int64_t N, int64_t m_t,
                           int64_t ld_z, int32_t S, float eps, int32_t norm, const float* bias,
                           int32_t act, void* out, int64_t ld_out, void* stream);

/*
 * avey_static_layer -- static contextualizer layer c_static = sigma(V Z_t + b) ([notes]
 * 关键设计 2: a learned linear map of the split's tail followed by the activation; [summary]
 * 4.2: its weights do not depend on the input). V mixes the S token positions of a split.
 *
 * For each split (b, i), with Z_i its S tail rows (padding rows zero):
 *   out[s][c] = act( sum_q V[s][q] Z_i[q][c] + bias[s] )
 * and the valid rows s are written.
 *
 *   z_tail  [B, N, m_t] row stride ld_z (input; point it at the first tail column of Z)
 *   V       [S, S] contiguous, dtype dt (input): V[s][q] weighs token q for output token s
 *   bias    [S] float32 (input), or NULL for no bias
 *   act     an avey_act (other values: AVEY_ERR_SHAPE)
 *   out     [B, N, m_t] row stride ld_out, dtype dt (output)
 * Computed by the kernels of avey_select_compress with no retrieved block (X_cat = Z_i, P = V,
 * no residual). For AVEY_BF16 the result is rounded to bf16 once, after bias and activation.
 */
avey_status avey_static_layer(const void* z_tail, avey_dtype dt, int64_t B, int64_t N, int64_t m_t,
                              int64_t ld_z, int32_t S, const void* V, const float* bias,
                              int32_t act, void* out, int64_t ld_out, void* stream);

/*
 * avey_enrich -- enricher of a neural-processor layer ([notes] 方法详解/整体框架: Z = sigma(X U + b),
 * a position-wise expansion from d to m features; [summary] appendix A: sigma is ReLU squared).
 *
 * For every row t < M (tokens of all sequences, flattened):  z_t = ReLU(x_t U + b)^2.
 *
 *   x     [M, d] row stride ld_x (input)
 *   U     [d, m] contiguous, dtype dt (input)
 *   b     [m] float32 (input), or NULL for none
 *   z     [M, m] row stride ld_z, dtype dt (output); its last m_t columns are the tail Z_t the
 *         contextualizer takes, the first m - m_t the bypassed head
 * For AVEY_BF16: d and m multiples of 64, m <= 4096 when b is given; fp32 accumulation, one
 * rounding to bf16 after the bias, ReLU and square.
 */
avey_status avey_enrich(const void* x, avey_dtype dt, int64_t M, int64_t d, int64_t ld_x, const void* U,
                        int64_t m, const float* b, void* z, int64_t ld_z, void* stream);

/*
 * avey_fuse -- fuser of a neural-processor layer ([notes] 方法详解/整体框架: f(Z) = [Z_h || c(Z_t)] O,
 * then a residual addition of the layer's input; [summary] section 3).
 *
 * For every row t < M:  y_t = [z_t[0 .. m_h) || c_t] O + x_t.
 *
 *   z     [M, >= m_h] row stride ld_z (input): only its first m_h columns (the head) are read
 *   c     [M, m_t] row stride ld_c (input): the contextualised tail (avey_dyn_layer,
 *         avey_static_layer)
 *   O     [m_h + m_t, d] contiguous, dtype dt (input)
 *   x     [M, d] row stride ld_x (input): the layer's input, added to the projection
 *   y     [M, d] row stride ld_y, dtype dt (output)
 * m_h may be 0 (no head). For AVEY_BF16: m_h, m_t and d multiples of 64; fp32 accumulation
 * (the residual is added exactly), one rounding to bf16.
 */
avey_status avey_fuse(const void* z, avey_dtype dt, int64_t M, int64_t m_h, int64_t ld_z, const void* c,
                      int64_t m_t, int64_t ld_c, const void* O, int64_t d, const void* x, int64_t ld_x,
                      void* y, int64_t ld_y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AVEY_H */
