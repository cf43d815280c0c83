/*
 * gdn.h -- C ABI of libgdn: the gated delta-rule (GDN) linear-attention
 * recurrence on AMD Instinct MI355X (gfx950).
 *
 * The operation (standard gated delta rule, named by the "GDN CTE Kernel API
 * Reference" page in its introduction and Background; the recurrence itself is
 * not printed there):
 *
 *   S_t = e^{g_t} S_{t-1} + beta_t k_t (v_t - e^{g_t} S_{t-1}^T k_t)^T
 *   o_t = scale * S_t^T q_t
 *
 * per batch b and value head h; value head h reads key/query head
 * h / (Hv / Hk) (same page, Notes). S is [Dk][Dv], fp32.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers to contiguous row-major buffers
 *   owned by the caller. The library allocates nothing on the call path and
 *   keeps no mutable global state.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream). A GDN_OK return means the work was enqueued; device faults
 *   surface at the caller's next synchronisation.
 * - Arguments are validated on the host before anything is enqueued; on any
 *   error return nothing has been launched and no buffer has been written.
 * - q, k, v and out share the compute dtype (`dtype`); g_log, beta and the
 *   state are always fp32 (page "GDN CTE Kernel API Reference", Parameters
 *   g_log, beta, recurrent_state and Notes: the state is fp32 whatever the
 *   compute dtype).
 * - q and k must be L2-normalised per token and head (same page, Notes). This
 *   is the caller's contract and is not checked. NaN/Inf inputs are not
 *   checked either.
 * - The state is updated IN PLACE: `state_inout` holds the initial state on
 *   entry and the final state on return (same page, Parameters:
 *   recurrent_state supplied and aliased). For a zero start the caller
 *   zero-fills it.
 * - Concurrent calls that share an output or state buffer race; calls on
 *   disjoint buffers are independent.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Compute dtype of q, k, v and out. */
typedef enum {
    GDN_F32 = 0,   /* IEEE float32 operands; fp32 matrix-core products  */
    GDN_BF16 = 1   /* bfloat16 operands; fp32 accumulation and state     */
} gdn_dtype;

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,         /* a required pointer is NULL                          */
    GDN_ERR_SHAPE = 2,        /* B, Hk, Hv, S < 1, Hv % Hk != 0, or a size overflow   */
    GDN_ERR_UNSUPPORTED = 3,  /* Dk or Dv outside [16, 128] or not a multiple of 16;  *
                               * conv1d window K > 8                                 */
    GDN_ERR_DTYPE = 4,        /* dtype is not a gdn_dtype value                       */
    GDN_ERR_ALIGN = 5,        /* a tensor pointer is not 16-byte aligned              */
    GDN_ERR_ALIAS = 6,        /* out or state_inout overlaps another tensor argument  */
    GDN_ERR_WORKSPACE = 7,    /* workspace smaller than the queried size              */
    GDN_ERR_HIP = 8,          /* the HIP runtime refused a launch                     */
    GDN_ERR_VALUE = 9         /* an epsilon argument is negative or not finite, or an *
                               * unknown inverse method                              */
} gdn_status;

/* Opaque stream handle: a hipStream_t. NULL selects the null stream. */
typedef void* gdn_stream;

/*
 * gdn_chunked_prefill -- chunk-parallel prefill over S tokens.
 *
 * Follows "GDN CTE Kernel API Reference" (signature gdn_cte, Parameters,
 * Returns, Notes): the chunked form of the recurrence above, returning the
 * un-normalised output and the final state.
 *
 *   q, k        [B, Hk, S, Dk]  compute dtype, token-major, L2-normalised
 *   v           [B, Hv, S, Dv]  compute dtype
 *   g_log       [B, Hv, S]      fp32, per-token natural-log decay (<= 0)
 *   beta        [B, Hv, S]      fp32, per-token write strength in (0, 1)
 *   scale       query scaling (typically 1/sqrt(Dk)), applied on the device
 *   state_inout [B, Hv, Dk, Dv] fp32, in: initial state, out: final state
 *   out         [B, Hv, S, Dv]  compute dtype, written (head-major)
 *   workspace   device scratch of at least
 *               gdn_chunked_prefill_workspace_bytes(...) bytes; may be NULL
 *               when that size is 0
 *
 * Constraints: Hv % Hk == 0; 1 <= S <= 4194239 (byte offsets within one
 * (batch, head) stream are 32-bit). The page asks S to be a multiple of its
 * chunk length; here a partial last chunk is extended exactly, as if padded
 * with tokens of g = beta = 0 and k = q = v = 0 whose outputs are dropped.
 * 16 <= Dk, Dv <= 128, multiples of 16 (the pages' MAX_HEAD_DIM = 128,
 * Notes); all pointers 16-byte aligned; out and state_inout must not overlap
 * each other or any input. The result is deterministic run to run.
 */
gdn_status gdn_chunked_prefill(const void* q, const void* k, const void* v,
                               const float* g_log, const float* beta, float scale,
                               float* state_inout, void* out,
                               int B, int Hk, int Hv, int S, int Dk, int Dv,
                               int dtype, void* workspace, size_t workspace_bytes,
                               gdn_stream stream);

/* Intra-chunk inverse (I + A)^{-1} of the prefill: the choice the "GDN CTE
 * Kernel API Reference" page offers as `algorithm` (Parameters), here on
 * gfx950 terms. SUBSTITUTION: fp32 forward substitution on the 16x16
 * diagonal blocks (the default); NEUMANN: the exact product
 * (I - X)(I + X^2)(I + X^4)(I + X^8) of the nilpotent block X on fp32
 * matrix cores. Both merge the off-diagonal block on fp32 matrix cores. */
typedef enum {
    GDN_INV_SUBSTITUTION = 0,
    GDN_INV_NEUMANN = 1
} gdn_inverse;

/*
 * gdn_chunked_prefill_inverse -- gdn_chunked_prefill with the inverse method
 * chosen by `inverse` (a gdn_inverse value, else GDN_ERR_VALUE). Results of
 * the two methods agree to fp32 rounding of the inverse.
 */
gdn_status gdn_chunked_prefill_inverse(const void* q, const void* k, const void* v,
                                       const float* g_log, const float* beta, float scale,
                                       float* state_inout, void* out,
                                       int B, int Hk, int Hv, int S, int Dk, int Dv,
                                       int dtype, int inverse, void* workspace,
                                       size_t workspace_bytes, gdn_stream stream);

/* Device scratch bytes gdn_chunked_prefill needs for these sizes (0 when the
 * arguments are invalid or no scratch is needed). */
size_t gdn_chunked_prefill_workspace_bytes(int B, int Hk, int Hv, int S, int Dk, int Dv,
                                           int dtype);

/*
 * gdn_decode_step -- one token (S = 1) of the recurrence for every (b, h).
 *
 * The single-token recurrence that the "GDN Block TKG Kernel API Reference"
 * page places inside its decode block (introduction: "single-token
 * recurrence"), here on its own and in place.
 *
 *   q, k        [B, Hk, Dk]     compute dtype, L2-normalised
 *   v           [B, Hv, Dv]     compute dtype
 *   g_log, beta [B, Hv]         fp32
 *   state_inout [B, Hv, Dk, Dv] fp32, updated in place
 *   out         [B, Hv, Dv]     compute dtype
 *
 * Constraints as for gdn_chunked_prefill (without S).
 */
gdn_status gdn_decode_step(const void* q, const void* k, const void* v,
                           const float* g_log, const float* beta, float scale,
                           float* state_inout, void* out,
                           int B, int Hk, int Hv, int Dk, int Dv, int dtype,
                           gdn_stream stream);

/*
 * Gated entry points: the same recurrence, preceded on the device by the
 * prologue that the "GDN Block TKG Kernel API Reference" page lists ahead of
 * its single-token recurrence (introduction: "l2norm/beta/g"; Parameters
 * A_log, a per-value-head log decay, and dt_bias, a per-value-head softplus
 * bias). Per batch b, value head h and token t:
 *
 *   g_log = -exp(A_log[h]) * softplus(a[b,h,t] + dt_bias[h]),
 *           softplus(x) = ln(1 + e^x)
 *   beta  = 1 / (1 + exp(-b[b,h,t]))
 *   k_t   = k_raw_t / sqrt(sum_i k_raw_t[i]^2 + l2_eps), q_t likewise
 *           (the normalisation the "GDN CTE Kernel API Reference" page
 *           requires of its inputs, Notes; the pages give no epsilon)
 *
 * and then the recurrence above on (q_t, k_t, v_t, g_log, beta).
 *
 *   q, k        raw (un-normalised) query/key, shapes and dtype as in the
 *               ungated entry
 *   a, b        [B, Hv, S] fp32 ([B, Hv] for decode): gate pre-activations
 *   A_log       [Hv] fp32, dt_bias [Hv] fp32 (4-byte aligned suffices)
 *   l2_eps      >= 0 and finite, else GDN_ERR_VALUE; with l2_eps = 0 an
 *               all-zero q or k row gives NaN
 *
 * The normalised q, k and the gates are never written to memory: the
 * kernels fold 1/|k|, 1/|q| into per-token factors of the raw operands. All
 * other arguments, constraints and errors are those of the ungated entry;
 * out and state_inout must not overlap A_log or dt_bias either.
 */
gdn_status gdn_chunked_prefill_gated(const void* q, const void* k, const void* v,
                                     const float* a, const float* b,
                                     const float* A_log, const float* dt_bias,
                                     float scale, float l2_eps,
                                     float* state_inout, void* out,
                                     int B, int Hk, int Hv, int S, int Dk, int Dv,
                                     int dtype, void* workspace, size_t workspace_bytes,
                                     gdn_stream stream);

gdn_status gdn_decode_step_gated(const void* q, const void* k, const void* v,
                                 const float* a, const float* b,
                                 const float* A_log, const float* dt_bias,
                                 float scale, float l2_eps,
                                 float* state_inout, void* out,
                                 int B, int Hk, int Hv, int Dk, int Dv, int dtype,
                                 gdn_stream stream);

/*
 * gdn_conv1d_prefill -- depthwise causal conv1d + SiLU over T tokens and the
 * window state, the step ahead of the recurrence ("GDN Conv1D Kernel API
 * Reference": gdn_conv1d_prefill, Parameters, Returns, Notes).
 *
 *   mixed          [B, C, T]  compute dtype: raw q|k|v channels (T contiguous)
 *   conv_weight    [C, K]     fp32 depthwise weights, 1 <= K <= 8
 *   out            [B, C, T]  compute dtype, written:
 *                  out[b,c,t] = silu(sum_j w[c,j] mixed[b,c,t-(K-1)+j]),
 *                  silu(y) = y / (1 + e^{-y}), mixed = 0 before t = 0
 *   conv_state_out [B, C, K]  compute dtype, written: the last K raw tokens,
 *                  conv_state_out[b,c,j] = mixed[b,c,T-K+j] (0 where T-K+j < 0)
 *
 * The page gives no tap order, bias or window width: the weights act as a
 * squeezed depthwise convolution weight (w[c,K-1] multiplies the current
 * token), there is no bias, and K is an argument. Any T >= 1; pointers
 * 16-byte aligned; out and conv_state_out overlap nothing else.
 */
gdn_status gdn_conv1d_prefill(const void* mixed, const float* conv_weight, void* out,
                              void* conv_state_out, int B, int C, int T, int K, int dtype,
                              gdn_stream stream);

/*
 * gdn_conv1d_decode -- one token ("GDN Conv1D Kernel API Reference":
 * gdn_conv1d_decode): the window drops its oldest token and appends x, and
 * the output is silu of its K-tap dot product with the weights.
 *
 *   x                [B, C]     compute dtype, the new raw token
 *   conv_weight      [C, K]     fp32
 *   conv_state_inout [B, C, K]  compute dtype, the previous window in, the
 *                    shifted window out (in place; the page returns it as a
 *                    new tensor)
 *   out              [B, C]     compute dtype: silu(sum_j w[c,j] window[b,c,j])
 *
 * Same constraints as gdn_conv1d_prefill with T = 1.
 */
gdn_status gdn_conv1d_decode(const void* x, const float* conv_weight, void* conv_state_inout,
                             void* out, int B, int C, int K, int dtype, gdn_stream stream);

/*
 * gdn_rmsnorm_gated -- the RMSNormGated output epilogue ("GDN Block TKG Kernel
 * API Reference": introduction, "RMSNormGated"; Parameters norm_weight, the
 * gamma over head_v_dim, and W_in_z, whose projection z gates it), applied
 * to a prefill output. The page gives no formula: read as the gated RMS
 * norm over each (token, head) row of Dv values, normalised first,
 *
 *   out[b,s,h,:] = o[b,h,s,:] / sqrt(mean(o[b,h,s,:]^2) + eps)
 *                  * norm_weight * silu(z[b,s,h,:]),   silu(x) = x / (1 + e^-x)
 *
 *   o            [B, Hv, S, Dv] compute dtype: head-major, as gdn_chunked_prefill
 *                writes it
 *   z, out       [B, S, Hv, Dv] compute dtype: token-major (heads of a token
 *                adjacent), the layout of the block's output
 *   norm_weight  [Dv] fp32;  eps >= 0 and finite, else GDN_ERR_VALUE
 *
 * 16 <= Dv <= 128, a multiple of 16; pointers 16-byte aligned; out overlaps
 * no input.
 */
gdn_status gdn_rmsnorm_gated(const void* o, const void* z, const float* norm_weight, float eps,
                             void* out, int B, int Hv, int S, int Dv, int dtype,
                             gdn_stream stream);

/*
 * gdn_decode_block -- one token through the "GDN Block TKG Kernel API
 * Reference" decode layer between its input and output projections
 * (introduction), in one kernel:
 *
 *   1. conv1d decode step over the raw mixed token ("GDN Conv1D Kernel API
 *      Reference", gdn_conv1d_decode): windows shift, x = silu(w . window);
 *   2. split x into q (Hk heads of Dk), k (Hk x Dk), v (Hv x Dv), in that
 *      channel order (conv_dim = 2 key_dim + value_dim, Dimensions);
 *   3. the gated prologue and single-token recurrence of
 *      gdn_decode_step_gated (value head h reads key head h / (Hv/Hk));
 *   4. RMSNormGated of each head's Dv outputs with z and norm_weight, as in
 *      gdn_rmsnorm_gated.
 *
 *   mixed          [B, C] compute dtype, C = 2 Hk Dk + Hv Dv (raw q|k|v)
 *   z              [B, Hv Dv] compute dtype (the z projection)
 *   a, b           [B, Hv] fp32 gate pre-activations
 *   conv_state_in  [B, C, K] compute dtype, the previous windows (read)
 *   conv_state_out [B, C, K] compute dtype, the shifted windows (written; a
 *                  separate buffer, as the page returns a new conv state:
 *                  the heads of a GQA group read the same q/k windows)
 *   conv_weight    [C, K] fp32, 1 <= K <= 8
 *   A_log, dt_bias [Hv] fp32;  norm_weight [Dv] fp32
 *   scale, l2_eps, norm_eps  as in gdn_decode_step_gated / gdn_rmsnorm_gated
 *   state_inout    [B, Hv, Dk, Dv] fp32, updated in place
 *   out            [B, Hv Dv] compute dtype (token-major normalised output)
 *
 * Dk, Dv as for gdn_decode_step; pointers 16-byte aligned; the written
 * buffers (conv_state_out, state_inout, out) overlap nothing else.
 */
gdn_status gdn_decode_block(const void* mixed, const void* z, const float* a, const float* b,
                            const void* conv_state_in, void* conv_state_out,
                            const float* conv_weight, const float* A_log, const float* dt_bias,
                            const float* norm_weight, float scale, float l2_eps, float norm_eps,
                            float* state_inout, void* out,
                            int B, int Hk, int Hv, int Dk, int Dv, int K, int dtype,
                            gdn_stream stream);

/* Static, NUL-terminated description of a status code. */
const char* gdn_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
