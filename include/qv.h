/*
 * qv.h -- C ABI of libqv.so, the quantized speculative-verify path on AMD MI355X (gfx950).
 *
 * The calls follow the statement of the problem in two papers:
 *   [Quasar]   "Quasar: Quantized Self-Speculative Acceleration for Rapid Inference via
 *               Memory-Efficient Verification" -- a W8A8 target model verifies the draft;
 *               Sec. 3.2 (W8A8 verification via SmoothQuant), Sec. 3.3 (execution pipeline:
 *               offline weight preparation, online activation smoothing and quantisation,
 *               INT8 GEMM and dequantisation), Sec. 4.5 (the top-1 prediction decides).
 *   [HierSpec] "Speculative Decoding Meets Quantization: Compatibility Evaluation and
 *               Hierarchical Framework Design" (review page, "The reading" / "Core claim") --
 *               a W4A16 target verifies a draft of n tokens in one forward pass.
 *
 * Conventions shared by every call:
 *   - All array pointers are DEVICE memory owned by the caller.  Matrices are row-major and
 *     contiguous.  The library never allocates, frees or keeps a pointer after a call.
 *   - fp16 data is passed as uint16_t IEEE binary16 bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call is
 *     asynchronous on that stream: results are valid once the stream reaches the call.  The
 *     caller keeps its buffers alive until then.  No call synchronises the device.
 *   - Arguments are checked on the host before anything is launched; a failed check returns
 *     its error code and launches nothing.  QV_ERR_HIP means a launch was rejected by the
 *     runtime (it may also report an error left pending by earlier work on the device).
 *   - Inputs are finite (no NaN or Inf); results for non-finite inputs are unspecified.
 *   - M is the number of verified positions (last accepted token + drafts), 1 <= M <= 64.
 *
 * Workspace: qv_linear_w8a8, qv_linear_w4a16 and qv_verify_greedy may need device scratch
 * memory for split-K partial sums and arrival counters.  qv_workspace_bytes() returns the
 * size for a shape (0 = none; then `workspace` may be NULL).  The first
 * QV_WORKSPACE_COUNTER_BYTES bytes of a workspace hold counters: they must be zero before the
 * workspace is first used, and every call leaves them zero again when it completes.  Calls
 * that share a workspace must be ordered on one stream.  Workspaces must be 256-byte aligned.
 */
#ifndef QV_H
#define QV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QV_OK = 0,
  QV_ERR_NULL = 1,      /* a required pointer is NULL */
  QV_ERR_SHAPE = 2,     /* a size is outside the supported rules below */
  QV_ERR_ALIGN = 3,     /* a pointer is not aligned as required */
  QV_ERR_WORKSPACE = 4, /* workspace missing or smaller than qv_workspace_bytes() */
  QV_ERR_HIP = 5,       /* the HIP runtime rejected a launch */
  QV_ERR_SCRATCH = 6    /* the shape needs more than QV_NOALLOC_SCRATCH_BYTES (no-allocation call) */
} qv_status_t;

/* op codes for qv_workspace_bytes */
enum { QV_OP_W8A8 = 1, QV_OP_W4A16 = 2, QV_OP_VERIFY = 3, QV_OP_SAMPLE = 4, QV_OP_W4A8 = 5 };

#define QV_MAX_M 64
#define QV_W4A16_GROUP 128
/* K * 128 * 128 < 2^31: the W8A8 accumulator cannot overflow int32 for any int8 inputs. */
#define QV_W8A8_MAX_K 131008
/* Longest K of the 4-bit linears (activation offsets stay 32-bit). */
#define QV_W4A16_MAX_K 1048576
#define QV_WORKSPACE_COUNTER_BYTES 65536
/* Size of the library's static per-GPU scratch array used by qv_verify_greedy_noalloc. */
#define QV_NOALLOC_SCRATCH_BYTES (512 * 1024)

/*
 * qv_quant_act -- per-token symmetric int8 quantisation of activations, with an optional
 * online smoothing prescale ([Quasar] Sec. 3.2 and Sec. 3.3 "Online Activation Smoothing and
 * Quantization"; the per-token granularity, the symmetric [-127, 127] range and the
 * round-half-to-even rule are this library's reading, the formulas being illegible there).
 *
 * For each row m:  x'[k] = f32(x[m][k]) * inv_smooth[k]   (the product only if inv_smooth != NULL)
 *                  a     = max_k |x'[k]|
 *                  x_scale[m] = a / 127            (IEEE fp32 division, round to nearest even)
 *                  x_q[m][k]  = a == 0 ? 0 : clamp(rint(x'[k] / x_scale[m]), -127, 127)
 *
 *   x          fp16 [M][K], 16-byte aligned
 *   inv_smooth fp32 [K] per-channel smoothing multipliers or NULL, 4-byte aligned; paired
 *              with weights prepared by qv_prepare_w8 with column multipliers inv_s, they
 *              are the reciprocals of those (so that the smoothed product is unchanged)
 *   x_q        int8 [M][K], 16-byte aligned (output)
 *   x_scale    fp32 [M], 4-byte aligned (output)
 * Rules: 1 <= M <= 64, K >= 8, K % 8 == 0.
 */
qv_status_t qv_quant_act(const uint16_t* x, const float* inv_smooth, int M, int K,
                         int8_t* x_q, float* x_scale, void* stream);

/*
 * qv_prepare_w8 -- offline W8 weight preparation ([Quasar] Sec. 3.3 "Offline Weight
 * Preparation": W_hat = Q(W diag(s)^-1); Q is this library's reading, the same per-row rule
 * as qv_quant_act applied to each output channel).
 *
 * For each row n:  w'[k] = f32(w_bf16[n][k]) * inv_s[k]   (the product only if inv_s != NULL;
 *                                                         inv_s holds the entries of diag(s)^-1)
 *                  w_scale[n] = max_k |w'[k]| / 127      (IEEE fp32 division)
 *                  w_q[n][k]  = w_scale[n] == 0 ? 0 : clamp(rint(w'[k] / w_scale[n]), -127, 127)
 * The outputs are the weights and scales of qv_linear_w8a8.
 *
 *   w_bf16   bf16 bit patterns [N][K] (one row per output channel), 16-byte aligned
 *   inv_s    fp32 [K] or NULL, 4-byte aligned
 *   w_q      int8 [N][K] (output), 16-byte aligned;  w_scale fp32 [N] (output)
 * Rules: N >= 1, K >= 8, K % 8 == 0.  One launch on `stream`, no workspace.
 */
qv_status_t qv_prepare_w8(const uint16_t* w_bf16, const float* inv_s, int N, int K, int8_t* w_q,
                          float* w_scale, void* stream);

/*
 * qv_prepare_w4 -- offline 4-bit weight preparation into the format of qv_linear_w4a16 and
 * qv_linear_w4a8 ([HierSpec] review page: 4-bit weight-quantised targets; the quantiser is
 * this library's reading).  Per output channel n and 128-group g, in fp32:
 *
 *   lo = min(0, min_{k in g} w), hi = max(0, max_{k in g} w)   with w = f32(w_bf16[n][k])
 *   scales[n][g] = fp16((hi - lo) / 15), or 1 if that is 0        (round to nearest even)
 *   zeros[n][g]  = clamp(rint(-lo / s), 0, 15)                    with s = f32(scales[n][g])
 *   code(n, k)   = clamp(rint(w / s) + zeros[n][g], 0, 15)        (correctly rounded divisions)
 *   qweight[n][k / 8] nibble k % 8 = code(n, k)                   (low nibble = lowest k)
 *
 *   w_bf16   bf16 bit patterns [N][K], 16-byte aligned
 *   qweight  uint32 [N][K/8] (output), 4-byte aligned; scales fp16 [N][K/128]; zeros uint8 [N][K/128]
 * Rules: N >= 1, K >= 128, K % 128 == 0, group_size == 128.  One launch, no workspace.
 */
qv_status_t qv_prepare_w4(const uint16_t* w_bf16, int N, int K, int group_size, uint32_t* qweight,
                          uint16_t* scales, uint8_t* zeros, void* stream);

/*
 * qv_linear_w8a8 -- INT8 GEMM and dequantisation ([Quasar] Sec. 3.3 "INT8 Gemm and
 * Dequantization"; weights prepared offline as per-output-channel int8, Sec. 3.3 "Offline
 * Weight Preparation").
 *
 *   acc[m][n] = sum_k x_q[m][k] * w[n][k]                    (exact int32)
 *   y[m][n]   = fp16( f32( f32(acc[m][n]) * x_scale[m] ) * w_scale[n] )
 * two fp32 products in this order, each rounded to nearest even, then one rounding to fp16.
 *
 *   x_q      int8 [M][K] (from qv_quant_act), 16-byte aligned
 *   x_scale  fp32 [M]
 *   w        int8 [N][K] (one row per output channel), 16-byte aligned
 *   w_scale  fp32 [N]
 *   y        fp16 [M][N] (output), 16-byte aligned
 *   acc_out  int32 [M][N] (output) or NULL, 16-byte aligned
 * Rules: 1 <= M <= 64, 64 <= K <= QV_W8A8_MAX_K, K % 64 == 0, N >= 16, N % 16 == 0.  Any int8
 * values are allowed (qv_quant_act and qv_prepare_w8 produce [-127, 127]); at this K bound the
 * accumulator is exact for all of them.
 */
qv_status_t qv_linear_w8a8(const int8_t* x_q, const float* x_scale, int M, int K,
                           const int8_t* w, const float* w_scale, int N,
                           uint16_t* y, int32_t* acc_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * qv_linear_w4a16 -- weight-only 4-bit linear of the W4A16 verifier ([HierSpec], "The
 * reading": the W4A16 target verifies the draft in one forward pass; group-wise asymmetric
 * int4 with group size 128 is this library's format).
 *
 *   code(n, k) = (qweight[n][k / 8] >> (4 * (k % 8))) & 15       (low nibble = lowest k)
 *   w[n][k]    = (code(n, k) - zeros[n][k / 128]) * scales[n][k / 128]
 *   y[m][n]    = fp16( sum_k x[m][k] * w[n][k] )
 * Accumulation is in fp32.  Up to 16 tokens (with 16-byte aligned scales, 8-byte aligned
 * zeros and K % 1024 == 0) the kernel sums x * (code - zero) exactly per group and multiplies
 * the group sum by the fp32 scale; otherwise it rounds each w to fp16 (code - zero is exact)
 * before the fp16 products.  Either way results agree with the exact sum to well within 2e-3
 * of max|y|.  Split-K partial sums are added in a fixed order, so results are bitwise
 * reproducible.
 *
 *   x        fp16 [M][K], 16-byte aligned
 *   qweight  uint32 [N][K/8], 16-byte aligned
 *   scales   fp16 [N][K/128], 2-byte aligned
 *   zeros    uint8 [N][K/128], values 0..15
 *   y        fp16 [M][N] (output), 16-byte aligned
 * Rules: 1 <= M <= 64, 128 <= K <= QV_W4A16_MAX_K, K % 128 == 0, group_size == 128, N >= 16,
 * N % 16 == 0.
 */
qv_status_t qv_linear_w4a16(const uint16_t* x, int M, int K,
                            const uint32_t* qweight, const uint16_t* scales,
                            const uint8_t* zeros, int N, int group_size,
                            uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * qv_linear_w4a8 -- 4-bit weights against per-token int8 activations, on the int8 matrix
 * cores ([HierSpec], "What carries the argument" and the summary: a W4A8 target is evaluated
 * beside W4A16; its format is this library's reading: the weights of qv_linear_w4a16 and the
 * activations of qv_quant_act).
 *
 *   acc_g[m][n] = sum_{k in group g} x_q[m][k] * (code(n, k) - zeros[n][g])   (exact int32)
 *   y[m][n]     = fp16( x_scale[m] * sum_g f32(scales[n][g]) * acc_g[m][n] )
 * with code() as in qv_linear_w4a16.  The sum over groups is accumulated in fp32 (split-K
 * partials added in a fixed order, so results are bitwise reproducible) and agrees with the
 * exact value to well within 2e-3 of max|y|.
 *
 *   x_q      int8 [M][K], 16-byte aligned;  x_scale fp32 [M]
 *   qweight  uint32 [N][K/8], 16-byte aligned; scales fp16 [N][K/128]; zeros uint8 [N][K/128]
 *   y        fp16 [M][N] (output), 16-byte aligned
 *   workspace  size qv_workspace_bytes(QV_OP_W4A8, M, N, K)
 * Rules: as qv_linear_w4a16.
 */
qv_status_t qv_linear_w4a8(const int8_t* x_q, const float* x_scale, int M, int K,
                           const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                           int N, int group_size, uint16_t* y, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * qv_verify_greedy -- greedy (temperature 0) verification: the verifier's top-1 token
 * decides acceptance ([Quasar] Sec. 4.5; the mean acceptance length of Sec. 4.2 / Table 1
 * counts n_accept + 1 tokens per verify step).
 *
 *   argmax_out[m] = the lowest v with logits[m][v] == max_u logits[m][u]   (-0 == +0)
 *   n_accept      = the largest j in [0, M-1] with draft[i] == argmax_out[i] for all i < j
 * Row 0 is the last accepted token and rows 1..M-1 the drafts, so draft[i] is the token at
 * row i+1 and the step emits draft[0..n_accept-1] followed by argmax_out[n_accept].
 *
 *   logits      fp16 [M][V], 16-byte aligned
 *   draft       int32 [M-1]; may be NULL when M == 1
 *   argmax_out  int32 [M] (output)
 *   n_accept_out int32 [1] (output)
 * Rules: 1 <= M <= 64, 1 <= V <= 2^30.
 */
qv_status_t qv_verify_greedy(const uint16_t* logits, int M, int V, const int32_t* draft,
                             int32_t* argmax_out, int32_t* n_accept_out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * qv_verify_greedy_noalloc -- qv_verify_greedy without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments (minus the workspace), same results, bit for bit.
 *
 * The arrival counters and per-chunk partial results live in a static device array of
 * QV_NOALLOC_SCRATCH_BYTES inside libqv.so, one copy on each GPU the library runs on, held
 * until the process ends; the call itself allocates and frees nothing.  Its first call on a
 * device resolves that device's copy (hipGetSymbolAddress) and clears its counters with a
 * small kernel on `stream`; every call leaves them zero again.  All calls on one GPU share the
 * array: calls that may overlap on one GPU (different streams, or threads without ordering)
 * race and give undefined results; order them on one stream.
 * Rules: those of qv_verify_greedy, and 1024 + M * ceil(V / 16384) * 8 + 256 <=
 * QV_NOALLOC_SCRATCH_BYTES (V up to about 16 million at M = 64); a larger shape returns
 * QV_ERR_SCRATCH before anything is launched.
 */
qv_status_t qv_verify_greedy_noalloc(const uint16_t* logits, int M, int V, const int32_t* draft,
                                     int32_t* argmax_out, int32_t* n_accept_out, void* stream);

/*
 * qv_verify_tree -- greedy acceptance of a draft tree verified in one pass ([HierSpec],
 * "What carries the argument": the target verifies a tree draft and turns it into the
 * sequential draft it accepts; the acceptance rule below is this library's reading).
 *
 *   argmax_out[i] = as in qv_verify_greedy, for each tree node i (row i of logits)
 *   node 0 is the root (the last accepted token); node i > 0 is a draft whose parent is
 *   parent[i].  Node i is accepted iff 0 <= parent[i] < i, its parent is accepted and
 *   tokens[i] == argmax_out[parent[i]]; the root is accepted.  The accepted path runs from
 *   the root to the accepted node of greatest depth (the lowest index among equals):
 *   path_out[0..L] holds its node indices (path_out[0] = 0), path_out[L+1..M-1] = -1,
 *   accept_out[0] = L (drafts accepted) and accept_out[1] = argmax_out[path_out[L]] (the
 *   token the step emits after the accepted drafts).
 *
 *   logits      fp16 [M][V], 16-byte aligned
 *   tokens      int32 [M] (tokens[0] is ignored)
 *   parent      int32 [M] (parent[0] is ignored; an index outside [0, i) rejects node i)
 *   argmax_out  int32 [M], path_out int32 [M], accept_out int32 [2] (outputs)
 *   workspace   as for qv_verify_greedy (size qv_workspace_bytes(QV_OP_VERIFY, M, V, 0))
 * Rules: 1 <= M <= 64, 1 <= V <= 2^30.
 */
qv_status_t qv_verify_tree(const uint16_t* logits, int M, int V, const int32_t* tokens,
                           const int32_t* parent, int32_t* argmax_out, int32_t* path_out,
                           int32_t* accept_out, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * qv_verify_sample -- stochastic (temperature T > 0) verification by speculative sampling
 * ([Quasar] Sec. 3.3 "Lossless Rejection Sampling": the target distribution p recovered in
 * high precision is compared with the draft distribution q; the comparison, Eq. 2, is
 * illegible there, and this library reads it as the modified rejection sampling that Sec. 2.1
 * and the speculative-sampling abstract on the search-results page refer to).  All
 * probabilities are float64:
 *
 *   p_i = softmax(logits[i] / T)                      for rows i = 0 .. M-1
 *   q_i = softmax(draft_logits[i] / T)                for i < M-1, or, when draft_logits is
 *         NULL (a deterministic drafter), the point mass at draft[i]
 *   draft i (the token at row i+1) is accepted iff 0 <= draft[i] < V and
 *         uniforms[i] * q_i(draft[i]) < p_i(draft[i]);  n_accept = the first rejected i, or
 *         M-1 when every draft is accepted
 *   token = a draw with uniforms[M-1] from max(0, p_n - q_n) (n = n_accept < M-1; from p_n
 *         if those weights are all zero) or from p_{M-1} (n_accept = M-1), where a draw
 *         from weights w with u is the lowest v whose running sum of w exceeds u * sum(w)
 * The step emits draft[0..n_accept-1] followed by token; the emitted tokens are distributed
 * as the target's own samples at temperature T.  Results equal a sequential float64
 * evaluation except where a comparison lies within a few units in the last place of a tie.
 *
 *   logits        fp16 [M][V], 16-byte aligned (finite values; otherwise token may be -1)
 *   draft_logits  fp16 [M-1][V], 16-byte aligned, or NULL (ignored when M == 1)
 *   draft         int32 [M-1]; may be NULL when M == 1
 *   uniforms      float64 [M], values in [0, 1): the random numbers of the M-1 acceptance
 *                 tests and of the draw (the caller draws them; results are reproducible)
 *   temperature   T, finite and > 0 (T = 0 is qv_verify_greedy)
 *   result_out    int32 [2] (output) = {n_accept, token}
 *   workspace     size qv_workspace_bytes(QV_OP_SAMPLE, M, V, 0)
 * Rules: 1 <= M <= 64, 1 <= V <= 2^30.  Two kernel launches on `stream`.
 */
qv_status_t qv_verify_sample(const uint16_t* logits, int M, int V, const uint16_t* draft_logits,
                             const int32_t* draft, const double* uniforms, double temperature,
                             int32_t* result_out, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * qv_workspace_bytes -- workspace size for one call of `op` at this shape (N is V for
 * QV_OP_VERIFY and QV_OP_SAMPLE; K is ignored there).  Returns 0 when no workspace is needed, and 0 for a
 * shape the op rejects.
 */
size_t qv_workspace_bytes(int op, int M, int N, int K);

/* qv_status_str -- a static, NUL-terminated description of a status code. */
const char* qv_status_str(qv_status_t s);

/* qv_version -- library version as 10000*major + 100*minor + patch. */
int qv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QV_H */
