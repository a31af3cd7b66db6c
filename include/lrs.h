/*
 * lrs.h -- C ABI of the MI355X (gfx950) linear-recurrence-scan library for
 * reinforcement-learning credit assignment.
 *
 * What is computed.  Each call evaluates one estimator over a batch of
 * rollouts of shape [num_envs, seq_len].  All seven are the same first-order
 * linear recurrence A_t = alpha_t + beta_t * A_{t+1} (its forward-time mirror
 * for the two forward estimators), solved as an associative scan with the
 * operator (a_B, b_B) (+) (a_A, b_A) = (a_B + b_B a_A, b_A b_B); each call
 * builds its alpha/beta on chip from the raw inputs and makes one pass over
 * HBM (rl-triton paper, gist.science technical summary, Methodology 1 and 2;
 * rl-triton README, Kernels table).  lrs_affine_scan_f32 exposes the bare
 * recurrence over caller-supplied alpha/beta.
 *
 * Episode boundaries (same summary, Methodology 3).  Per element (n, t):
 *   end_t   = terminated_t || truncated_t || t == seq_len-1
 *   Vnext_t = terminated_t ? 0
 *           : truncated_t  ? trunc_values[t]       (supplied bootstrap)
 *           : t == seq_len-1 ? bootstrap_value[n]  (0 if NULL)
 *           : values[t+1]
 * A terminated step has successor value 0; a truncated step uses the
 * supplied value; if both flags are set, termination wins.  The rollout-
 * window bootstrap enters the local term of step seq_len-1 only (never also
 * as a carry), and is ignored when that step is itself a cut.  The recursion
 * never continues past end_t, so no value leaks between episodes (exact for
 * finite inputs).
 *
 * Conventions shared by every call
 *   - num_envs (N) >= 1, 1 <= seq_len (T) < 2^31, N*T < 2^34.
 *   - Every array pointer is DEVICE memory owned by the caller.  Arrays of
 *     shape [N, T] are row-major with unit stride along T; per-env arrays
 *     have N elements, contiguous.  Float inputs/outputs are fp32; masks are
 *     uint8 with 0 = false, nonzero = true.  Any alignment of at least the
 *     element size is accepted; 16-byte aligned floats and 8-byte aligned
 *     masks take the vectorised fast path.
 *   - strides: NULL (every [N, T] array contiguous, row stride T), or a HOST
 *     array with one row stride per [N, T] array argument of the call -- the
 *     number of elements between the starts of consecutive rows -- in the
 *     order those arguments appear in the signature, inputs and outputs
 *     alike (for GAE: rewards, values, terminateds, truncateds,
 *     trunc_values, advantages).  0 means contiguous; otherwise the stride
 *     must be >= T.  Entries of absent (NULL) arrays are ignored.  A view
 *     such as buffer[:, :T] of a wider [N, Tmax] buffer is then read or
 *     written in place.  The vectorised fast path also needs every strided
 *     array's stride times its element size to be a multiple of the vector
 *     width (16 bytes for fp32 data, the elements per lane for masks) and T
 *     a multiple of the elements per lane; other strides take the scalar
 *     path.  The time-major (_tm_) calls take the stride between
 *     consecutive time steps (>= N).  The entries, call by call:
 *       GAE, TD(lambda) returns: rewards, values, terminateds, truncateds,
 *         trunc_values, out
 *       discounted returns: rewards, terminateds, truncateds, trunc_values, out
 *       V-trace: log_rhos, rewards, values, terminateds, truncateds,
 *         trunc_values, vs, pg_advantages
 *       Retrace: log_rhos, rewards, q_values, values, terminateds,
 *         truncateds, trunc_values, q_ret
 *       eligibility traces, prefix sums: x, dones, out
 *       affine scan: alpha, beta, reset, out
 *   - All float inputs must be finite.
 *   - Precision: coefficients and each lane's recursion are fp32; maps are
 *     composed across lanes, waves and tiles in fp32 with every lane's own
 *     product of betas formed in fp64, or wholly in fp64 when the call's
 *     betas may exceed 0.99 (sums, gamma or lambda of 1, large c_bar, and
 *     caller coefficients of lrs_affine_scan_*), where long undamped chains
 *     would accumulate fp32 rounding.  gamma*lambda (and similar products of
 *     scalars) are rounded to fp32 once, as fp32 coefficients.
 *   - gamma and lambda must lie in [0, 1].  Clip thresholds must be > 0;
 *     +INFINITY means "no clip".
 *   - workspace: caller-owned device memory of at least
 *     lrs_workspace_bytes(...) bytes, ZERO-FILLED before its first use; the
 *     library keeps it consistent from call to call afterwards, so it must
 *     not be modified between calls.  Calls that share one workspace must be
 *     ordered on one stream (concurrent use of one workspace races).  May be
 *     NULL with workspace_bytes 0 when lrs_workspace_bytes returns 0.
 *     Its first 4224 bytes are a header the calls maintain; the 32-bit word at
 *     byte offset 4 is an error word that a call sets (bit 1, value 2) if one
 *     of its carry waits gave up after its bounded number of polls (a broken
 *     workspace, or calls sharing it concurrently).  The tile whose wait gave
 *     up then takes a NaN carry: in floating-point calls every output of that
 *     tile that depends on the carry is NaN; in the int32 prefix sum the tile
 *     is summed from a carry of 0, so its sums are wrong.  The word stays set
 *     until the caller clears it; reading it after synchronising is a cheap
 *     health check.
 *   - Outputs and the workspace must not share memory with any input or with
 *     each other (checked on the host from the arrays' extents; inputs may
 *     share memory with each other); LRS_ERR_INVALID_ARG otherwise.
 *   - stream: the HIP stream to enqueue on (NULL = the null stream).  Calls
 *     are asynchronous; the library never allocates, frees or synchronises.
 *   - Errors: argument checks run on the host before anything is enqueued
 *     and return LRS_ERR_INVALID_ARG / LRS_ERR_WORKSPACE with nothing
 *     enqueued; a failed launch returns LRS_ERR_HIP.  lrs_last_error() then
 *     holds a message (per thread).  Faults inside a kernel surface at the
 *     caller's next synchronisation, as for any HIP kernel.
 */
#ifndef LRS_H
#define LRS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bit containers for the 16-bit variants: bfloat16 (1-8-7) and IEEE 754
 * binary16 (1-5-10) values, stored as their bit patterns. */
typedef uint16_t lrs_bf16;
typedef uint16_t lrs_f16;

typedef enum lrs_status {
    LRS_OK = 0,
    LRS_ERR_INVALID_ARG = 1, /* bad size, null pointer, scalar out of range */
    LRS_ERR_WORKSPACE = 2,   /* workspace missing or smaller than required */
    LRS_ERR_HIP = 3          /* a HIP runtime call failed (kernel launch)    */
} lrs_status;

typedef enum lrs_estimator {
    LRS_GAE = 0,
    LRS_VTRACE = 1,
    LRS_RETRACE = 2,
    LRS_LAMBDA_RETURNS = 3,
    LRS_DISCOUNTED_RETURNS = 4,
    LRS_ELIGIBILITY_TRACES = 5,
    LRS_PREFIX_SUM_I32 = 6,
    LRS_PREFIX_SUM_F32 = 7,
    LRS_AFFINE_SCAN = 8
} lrs_estimator;

/* Library version, encoded as major*10000 + minor*100 + patch. */
int lrs_version(void);

/* Static description of a status code (never NULL). */
const char* lrs_status_string(lrs_status s);

/* Message of the last failed call on the calling thread ("" if none). */
const char* lrs_last_error(void);

/* Bytes of workspace a call of `est` (an estimator, or LRS_AFFINE_SCAN) at
 * [num_envs, seq_len] may need, in either layout:
 * 4224 bytes plus the larger of 32 bytes per 256 elements (about 3% of one
 * fp32 array) and 24 bytes per env per 64 steps.  The same workspace serves
 * every estimator and layout at this or any smaller size.
 * Returns 0 for invalid sizes. */
size_t lrs_workspace_bytes(lrs_estimator est, int64_t num_envs, int64_t seq_len);

/* Generalized Advantage Estimation (README Kernels table, compute_gae:
 * backward scan over delta + gamma*lambda*A; Schulman et al. 2016 eq. 16):
 *   delta_t = r_t + gamma*Vnext_t - V_t
 *   A_t     = delta_t + (end_t ? 0 : gamma*lambda*A_{t+1})
 * In:  rewards, values [N,T] f32; terminateds [N,T] u8 (required);
 *      truncateds [N,T] u8 (nullable) and trunc_values [N,T] f32 (required
 *      iff truncateds); bootstrap_value [N] f32 (nullable = 0).
 * Out: advantages [N,T] f32.                                               */
lrs_status lrs_gae_f32(int64_t num_envs, int64_t seq_len,
                       const float* rewards, const float* values,
                       const uint8_t* terminateds, const uint8_t* truncateds,
                       const float* trunc_values, const float* bootstrap_value,
                       float gamma, float lambda,
                       float* advantages,
                       const int64_t* strides,
                       void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* lrs_gae_f32 for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation and results, without a workspace argument.  The carry
 * records live in a static device area of 8 MiB per GPU, held until the
 * process ends, so calls accept num_envs * seq_len <= 67075072 (the area
 * holds 4224 + 32 * ceil(num_envs * seq_len / 256) bytes) and larger ones
 * return LRS_ERR_INVALID_ARG.  The library allocates nothing in this call.
 * Every call on a GPU shares that GPU's area: calls that overlap in time on
 * one GPU race (as calls sharing a workspace do), so order them on one
 * stream.  The first call on each device clears the area with a small kernel
 * on `stream` and must not be made under graph capture (it returns
 * LRS_ERR_INVALID_ARG then); later calls may be captured.  Arguments and
 * errors otherwise as lrs_gae_f32. */
lrs_status lrs_gae_noalloc_f32(int64_t num_envs, int64_t seq_len,
                               const float* rewards, const float* values,
                               const uint8_t* terminateds, const uint8_t* truncateds,
                               const float* trunc_values, const float* bootstrap_value,
                               float gamma, float lambda,
                               float* advantages, const int64_t* strides,
                               hipStream_t stream);

/* V-trace (README Kernels table, compute_vtrace: importance-weighted targets
 * and advantages; Espeholt et al. 2018 sec. 4.1 eq. 1 with the lambda-trace of
 * sec. 4.2).  w_t = exp(log_rhos_t) = pi/mu of the taken action:
 *   rho_t = min(rho_bar, w_t), c_t = lambda*min(c_bar, w_t)
 *   A_t   = rho_t*(r_t + gamma*Vnext_t - V_t) + (end_t ? 0 : gamma*c_t*A_{t+1})
 *   vs_t  = V_t + A_t
 *   pg_t  = min(pg_rho_bar, w_t)*(r_t + gamma*(end_t ? Vnext_t : vs_{t+1}) - V_t)
 * In:  log_rhos, rewards, values [N,T] f32; masks / trunc_values / bootstrap
 *      as for GAE.  Out: vs, pg_advantages [N,T] f32 (both required).       */
lrs_status lrs_vtrace_f32(int64_t num_envs, int64_t seq_len,
                          const float* log_rhos, const float* rewards,
                          const float* values,
                          const uint8_t* terminateds, const uint8_t* truncateds,
                          const float* trunc_values, const float* bootstrap_value,
                          float gamma, float lambda,
                          float rho_bar, float c_bar, float pg_rho_bar,
                          float* vs, float* pg_advantages,
                          const int64_t* strides,
                          void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Retrace(lambda) (README Kernels table, compute_retrace: off-policy return
 * with truncated importance ratios; Munos et al. 2016).  q_values = Q(s_t,a_t),
 * values = E_pi Q(s_t,.) (trunc_values and bootstrap_value are expected
 * values too); c_{t+1} = lambda*min(c_bar, exp(log_rhos_{t+1})):
 *   G_t = r_t + gamma*(end_t ? Vnext_t : V_{t+1} + c_{t+1}*(G_{t+1} - Q_{t+1}))
 * Out: q_ret [N,T] f32.                                                     */
lrs_status lrs_retrace_f32(int64_t num_envs, int64_t seq_len,
                           const float* log_rhos, const float* rewards,
                           const float* q_values, const float* values,
                           const uint8_t* terminateds, const uint8_t* truncateds,
                           const float* trunc_values, const float* bootstrap_value,
                           float gamma, float lambda, float c_bar,
                           float* q_ret,
                           const int64_t* strides,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* TD(lambda) returns (README Kernels table, compute_lambda_returns: mixes
 * one-step TD and Monte-Carlo targets; Sutton & Barto sec. 12.1, recursive):
 *   G_t = r_t + gamma*(end_t ? Vnext_t : (1-lambda)*V_{t+1} + lambda*G_{t+1})
 * Out: returns [N,T] f32.                                                   */
lrs_status lrs_lambda_returns_f32(int64_t num_envs, int64_t seq_len,
                                  const float* rewards, const float* values,
                                  const uint8_t* terminateds, const uint8_t* truncateds,
                                  const float* trunc_values, const float* bootstrap_value,
                                  float gamma, float lambda,
                                  float* returns,
                                  const int64_t* strides,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Discounted returns (README Kernels table, compute_discounted_returns:
 * discounted reward-to-go):
 *   G_t = r_t + gamma*(end_t ? Vnext_t : G_{t+1})
 * values are never read (Vnext is 0, trunc_values or bootstrap_value).
 * Out: returns [N,T] f32.                                                   */
lrs_status lrs_discounted_returns_f32(int64_t num_envs, int64_t seq_len,
                                      const float* rewards,
                                      const uint8_t* terminateds, const uint8_t* truncateds,
                                      const float* trunc_values, const float* bootstrap_value,
                                      float gamma,
                                      float* returns,
                                      const int64_t* strides,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* Accumulating eligibility traces, forward in time (README Kernels table,
 * compute_eligibility_traces formula):
 *   e_t = x_t + (t == 0 || dones_{t-1} ? 0 : gamma*lambda*e_{t-1})
 * In:  x [N,T] f32, dones [N,T] u8 (required).  Out: traces [N,T] f32.      */
lrs_status lrs_eligibility_traces_f32(int64_t num_envs, int64_t seq_len,
                                      const float* x, const uint8_t* dones,
                                      float gamma, float lambda,
                                      float* traces,
                                      const int64_t* strides,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* Episodic inclusive prefix sum (README Kernels table,
 * compute_episodic_prefix_sum: cumulative sum with done-mask resets; same
 * reset rule as the traces):
 *   S_t = x_t + (t == 0 || dones_{t-1} ? 0 : S_{t-1})
 * The int32 variant is exact in two's-complement arithmetic (sums outside
 * the int32 range wrap modulo 2^32).                                         */
lrs_status lrs_episodic_prefix_sum_i32(int64_t num_envs, int64_t seq_len,
                                       const int32_t* x, const uint8_t* dones,
                                       int32_t* sums,
                                       const int64_t* strides,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

lrs_status lrs_episodic_prefix_sum_f32(int64_t num_envs, int64_t seq_len,
                                       const float* x, const uint8_t* dones,
                                       float* sums,
                                       const int64_t* strides,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* Generic segmented affine scan over caller-supplied coefficients: the one
 * recurrence every estimator above reduces to (gist.science technical
 * summary, Methodology 1; its Significance and Claims section names other
 * segmented affine recurrences as users), here with alpha and beta read from
 * memory instead of built on chip.  Per row n, in scan order:
 *   reverse = 0:  y_t = alpha_t + beta_t * y_{t-1}   (t = 0 .. T-1)
 *   reverse = 1:  y_t = alpha_t + beta_t * y_{t+1}   (t = T-1 .. 0)
 * The y before the row's first step in scan order is carry_in[n] (0 if
 * carry_in is NULL).  Where reset[t] is nonzero (reset may be NULL),
 * y_t = alpha_t: the beta_t * y_prev term is dropped, exactly as if
 * beta_t were 0, so nothing from before the reset reaches y_t or later.
 * Streaming a long row in windows: scan the window nearest the scan's end
 * first, then pass its outputs at the shared edge (column 0 for reverse,
 * column T-1 forward, made contiguous) as carry_in of the next window.
 * In:  alpha, beta [N,T] f32 (any finite values; |beta| > 1 may overflow);
 *      reset [N,T] u8 (nullable); carry_in [N] f32 (nullable).
 * Out: y [N,T] f32.  reverse must be 0 or 1 (else LRS_ERR_INVALID_ARG).   */
lrs_status lrs_affine_scan_f32(int64_t num_envs, int64_t seq_len,
                               const float* alpha, const float* beta,
                               const uint8_t* reset, const float* carry_in,
                               int reverse,
                               float* y,
                               const int64_t* strides,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* 16-bit storage variants of every call above (bfloat16: _bf16, IEEE half:
 * _f16).  Same operation, arguments, limits and errors as the _f32 call of
 * the same name; every floating-point stream -- the per-step inputs,
 * trunc_values, bootstrap_value, carry_in and every output -- is 16-bit,
 * while masks stay uint8 and the scalars (gamma, lambda, clips) stay float.
 * Arithmetic is exactly that of the _f32 calls: inputs widen exactly and
 * each output is rounded once to nearest even, so on the same tile schedule
 * it is the fp32 result rounded (the schedule, chosen from the shape and the
 * storage type, may differ from the _f32 call's and move the last fp32 bits).
 * Fewer bytes per element make these HBM-bound calls faster.
 * The pages serve standard formats only (gist.science summary, closing
 * limitations paragraph of its plain-language part); this storage option is
 * this library's extension of the same recurrences.  The vector fast path
 * needs 8-byte aligned data streams (2-byte alignment is accepted).       */
lrs_status lrs_gae_bf16(int64_t num_envs, int64_t seq_len,
                        const lrs_bf16* rewards, const lrs_bf16* values,
                        const uint8_t* terminateds, const uint8_t* truncateds,
                        const lrs_bf16* trunc_values, const lrs_bf16* bootstrap_value,
                        float gamma, float lambda, lrs_bf16* advantages,
                        const int64_t* strides,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_vtrace_bf16(int64_t num_envs, int64_t seq_len,
                           const lrs_bf16* log_rhos, const lrs_bf16* rewards, const lrs_bf16* values,
                           const uint8_t* terminateds, const uint8_t* truncateds,
                           const lrs_bf16* trunc_values, const lrs_bf16* bootstrap_value,
                           float gamma, float lambda,
                           float rho_bar, float c_bar, float pg_rho_bar,
                           lrs_bf16* vs, lrs_bf16* pg_advantages,
                           const int64_t* strides,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_retrace_bf16(int64_t num_envs, int64_t seq_len,
                            const lrs_bf16* log_rhos, const lrs_bf16* rewards,
                            const lrs_bf16* q_values, const lrs_bf16* values,
                            const uint8_t* terminateds, const uint8_t* truncateds,
                            const lrs_bf16* trunc_values, const lrs_bf16* bootstrap_value,
                            float gamma, float lambda, float c_bar, lrs_bf16* q_ret,
                            const int64_t* strides,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_lambda_returns_bf16(int64_t num_envs, int64_t seq_len,
                                   const lrs_bf16* rewards, const lrs_bf16* values,
                                   const uint8_t* terminateds, const uint8_t* truncateds,
                                   const lrs_bf16* trunc_values, const lrs_bf16* bootstrap_value,
                                   float gamma, float lambda, lrs_bf16* returns,
                                   const int64_t* strides,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_discounted_returns_bf16(int64_t num_envs, int64_t seq_len,
                                       const lrs_bf16* rewards,
                                       const uint8_t* terminateds, const uint8_t* truncateds,
                                       const lrs_bf16* trunc_values, const lrs_bf16* bootstrap_value,
                                       float gamma, lrs_bf16* returns,
                                       const int64_t* strides,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);
lrs_status lrs_eligibility_traces_bf16(int64_t num_envs, int64_t seq_len,
                                       const lrs_bf16* x, const uint8_t* dones,
                                       float gamma, float lambda, lrs_bf16* traces,
                                       const int64_t* strides,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);
lrs_status lrs_episodic_prefix_sum_bf16(int64_t num_envs, int64_t seq_len,
                                        const lrs_bf16* x, const uint8_t* dones, lrs_bf16* sums,
                                        const int64_t* strides,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);
lrs_status lrs_affine_scan_bf16(int64_t num_envs, int64_t seq_len,
                                const lrs_bf16* alpha, const lrs_bf16* beta,
                                const uint8_t* reset, const lrs_bf16* carry_in, int reverse,
                                lrs_bf16* y,
                                const int64_t* strides,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

lrs_status lrs_gae_f16(int64_t num_envs, int64_t seq_len,
                        const lrs_f16* rewards, const lrs_f16* values,
                        const uint8_t* terminateds, const uint8_t* truncateds,
                        const lrs_f16* trunc_values, const lrs_f16* bootstrap_value,
                        float gamma, float lambda, lrs_f16* advantages,
                        const int64_t* strides,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_vtrace_f16(int64_t num_envs, int64_t seq_len,
                           const lrs_f16* log_rhos, const lrs_f16* rewards, const lrs_f16* values,
                           const uint8_t* terminateds, const uint8_t* truncateds,
                           const lrs_f16* trunc_values, const lrs_f16* bootstrap_value,
                           float gamma, float lambda,
                           float rho_bar, float c_bar, float pg_rho_bar,
                           lrs_f16* vs, lrs_f16* pg_advantages,
                           const int64_t* strides,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_retrace_f16(int64_t num_envs, int64_t seq_len,
                            const lrs_f16* log_rhos, const lrs_f16* rewards,
                            const lrs_f16* q_values, const lrs_f16* values,
                            const uint8_t* terminateds, const uint8_t* truncateds,
                            const lrs_f16* trunc_values, const lrs_f16* bootstrap_value,
                            float gamma, float lambda, float c_bar, lrs_f16* q_ret,
                            const int64_t* strides,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_lambda_returns_f16(int64_t num_envs, int64_t seq_len,
                                   const lrs_f16* rewards, const lrs_f16* values,
                                   const uint8_t* terminateds, const uint8_t* truncateds,
                                   const lrs_f16* trunc_values, const lrs_f16* bootstrap_value,
                                   float gamma, float lambda, lrs_f16* returns,
                                   const int64_t* strides,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_discounted_returns_f16(int64_t num_envs, int64_t seq_len,
                                       const lrs_f16* rewards,
                                       const uint8_t* terminateds, const uint8_t* truncateds,
                                       const lrs_f16* trunc_values, const lrs_f16* bootstrap_value,
                                       float gamma, lrs_f16* returns,
                                       const int64_t* strides,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);
lrs_status lrs_eligibility_traces_f16(int64_t num_envs, int64_t seq_len,
                                       const lrs_f16* x, const uint8_t* dones,
                                       float gamma, float lambda, lrs_f16* traces,
                                       const int64_t* strides,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);
lrs_status lrs_episodic_prefix_sum_f16(int64_t num_envs, int64_t seq_len,
                                        const lrs_f16* x, const uint8_t* dones, lrs_f16* sums,
                                        const int64_t* strides,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);
lrs_status lrs_affine_scan_f16(int64_t num_envs, int64_t seq_len,
                                const lrs_f16* alpha, const lrs_f16* beta,
                                const uint8_t* reset, const lrs_f16* carry_in, int reverse,
                                lrs_f16* y,
                                const int64_t* strides,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Time-major variants (_tm_): every call above, for each storage type, with
 * the per-step arrays laid out [seq_len, num_envs] -- row = time step,
 * element (n, t) at t * num_envs + n, rows contiguous -- the layout of
 * rollout buffers filled one step at a time.  Per-env arrays
 * (bootstrap_value, carry_in) stay [num_envs].  Same operation, arguments,
 * limits, precision and errors as the call of the same name (num_envs must
 * also be below 2^32, and the launch -- one lane per environment, padded
 * to a multiple of 64, per 8 steps, padded to whole tiles -- must hold fewer
 * than 2^32 work items, else LRS_ERR_INVALID_ARG; with 64 or more
 * environments the size limit above already implies it, so it binds when
 * fewer than 64 environments have rows of about 2^30 steps or more, where
 * the row-major call on the same memory serves); results equal that call's
 * on the transposed arrays
 * up to fp32 re-association, bit for bit for the int32 prefix sum.  The
 * pages fix the [num_envs, seq_len] layout (README Usage); this layout is
 * this library's extension.  A lane owns one environment (loads coalesce
 * across environments) and tiles of up to 256 steps pass carries along time;
 * rows of up to 128 steps on fewer than 16384 environments take blocks of 32
 * environments that hold whole rows; no alignment beyond the element size is
 * needed.  The workspace from
 * lrs_workspace_bytes covers both layouts.  Results are deterministic run
 * to run, as for the row-major calls.                                    */
lrs_status lrs_gae_tm_f32(int64_t num_envs, int64_t seq_len,
                           const float* rewards, const float* values,
                           const uint8_t* terminateds, const uint8_t* truncateds,
                           const float* trunc_values, const float* bootstrap_value,
                           float gamma, float lambda, float* advantages,
                           const int64_t* strides,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_vtrace_tm_f32(int64_t num_envs, int64_t seq_len,
                              const float* log_rhos, const float* rewards, const float* values,
                              const uint8_t* terminateds, const uint8_t* truncateds,
                              const float* trunc_values, const float* bootstrap_value,
                              float gamma, float lambda,
                              float rho_bar, float c_bar, float pg_rho_bar,
                              float* vs, float* pg_advantages,
                              const int64_t* strides,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_retrace_tm_f32(int64_t num_envs, int64_t seq_len,
                               const float* log_rhos, const float* rewards,
                               const float* q_values, const float* values,
                               const uint8_t* terminateds, const uint8_t* truncateds,
                               const float* trunc_values, const float* bootstrap_value,
                               float gamma, float lambda, float c_bar, float* q_ret,
                               const int64_t* strides,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_lambda_returns_tm_f32(int64_t num_envs, int64_t seq_len,
                                      const float* rewards, const float* values,
                                      const uint8_t* terminateds, const uint8_t* truncateds,
                                      const float* trunc_values, const float* bootstrap_value,
                                      float gamma, float lambda, float* returns,
                                      const int64_t* strides,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);
lrs_status lrs_discounted_returns_tm_f32(int64_t num_envs, int64_t seq_len,
                                          const float* rewards,
                                          const uint8_t* terminateds, const uint8_t* truncateds,
                                          const float* trunc_values, const float* bootstrap_value,
                                          float gamma, float* returns,
                                          const int64_t* strides,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);
lrs_status lrs_eligibility_traces_tm_f32(int64_t num_envs, int64_t seq_len,
                                          const float* x, const uint8_t* dones,
                                          float gamma, float lambda, float* traces,
                                          const int64_t* strides,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);
lrs_status lrs_episodic_prefix_sum_tm_f32(int64_t num_envs, int64_t seq_len,
                                           const float* x, const uint8_t* dones, float* sums,
                                           const int64_t* strides,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream);
lrs_status lrs_affine_scan_tm_f32(int64_t num_envs, int64_t seq_len,
                                   const float* alpha, const float* beta,
                                   const uint8_t* reset, const float* carry_in, int reverse,
                                   float* y,
                                   const int64_t* strides,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_episodic_prefix_sum_tm_i32(int64_t num_envs, int64_t seq_len,
                                          const int32_t* x, const uint8_t* dones, int32_t* sums,
                                          const int64_t* strides,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);
lrs_status lrs_gae_tm_bf16(int64_t num_envs, int64_t seq_len,
                           const lrs_bf16* rewards, const lrs_bf16* values,
                           const uint8_t* terminateds, const uint8_t* truncateds,
                           const lrs_bf16* trunc_values, const lrs_bf16* bootstrap_value,
                           float gamma, float lambda, lrs_bf16* advantages,
                           const int64_t* strides,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_vtrace_tm_bf16(int64_t num_envs, int64_t seq_len,
                              const lrs_bf16* log_rhos, const lrs_bf16* rewards, const lrs_bf16* values,
                              const uint8_t* terminateds, const uint8_t* truncateds,
                              const lrs_bf16* trunc_values, const lrs_bf16* bootstrap_value,
                              float gamma, float lambda,
                              float rho_bar, float c_bar, float pg_rho_bar,
                              lrs_bf16* vs, lrs_bf16* pg_advantages,
                              const int64_t* strides,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_retrace_tm_bf16(int64_t num_envs, int64_t seq_len,
                               const lrs_bf16* log_rhos, const lrs_bf16* rewards,
                               const lrs_bf16* q_values, const lrs_bf16* values,
                               const uint8_t* terminateds, const uint8_t* truncateds,
                               const lrs_bf16* trunc_values, const lrs_bf16* bootstrap_value,
                               float gamma, float lambda, float c_bar, lrs_bf16* q_ret,
                               const int64_t* strides,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_lambda_returns_tm_bf16(int64_t num_envs, int64_t seq_len,
                                      const lrs_bf16* rewards, const lrs_bf16* values,
                                      const uint8_t* terminateds, const uint8_t* truncateds,
                                      const lrs_bf16* trunc_values, const lrs_bf16* bootstrap_value,
                                      float gamma, float lambda, lrs_bf16* returns,
                                      const int64_t* strides,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);
lrs_status lrs_discounted_returns_tm_bf16(int64_t num_envs, int64_t seq_len,
                                          const lrs_bf16* rewards,
                                          const uint8_t* terminateds, const uint8_t* truncateds,
                                          const lrs_bf16* trunc_values, const lrs_bf16* bootstrap_value,
                                          float gamma, lrs_bf16* returns,
                                          const int64_t* strides,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);
lrs_status lrs_eligibility_traces_tm_bf16(int64_t num_envs, int64_t seq_len,
                                          const lrs_bf16* x, const uint8_t* dones,
                                          float gamma, float lambda, lrs_bf16* traces,
                                          const int64_t* strides,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);
lrs_status lrs_episodic_prefix_sum_tm_bf16(int64_t num_envs, int64_t seq_len,
                                           const lrs_bf16* x, const uint8_t* dones, lrs_bf16* sums,
                                           const int64_t* strides,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream);
lrs_status lrs_affine_scan_tm_bf16(int64_t num_envs, int64_t seq_len,
                                   const lrs_bf16* alpha, const lrs_bf16* beta,
                                   const uint8_t* reset, const lrs_bf16* carry_in, int reverse,
                                   lrs_bf16* y,
                                   const int64_t* strides,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_gae_tm_f16(int64_t num_envs, int64_t seq_len,
                           const lrs_f16* rewards, const lrs_f16* values,
                           const uint8_t* terminateds, const uint8_t* truncateds,
                           const lrs_f16* trunc_values, const lrs_f16* bootstrap_value,
                           float gamma, float lambda, lrs_f16* advantages,
                           const int64_t* strides,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_vtrace_tm_f16(int64_t num_envs, int64_t seq_len,
                              const lrs_f16* log_rhos, const lrs_f16* rewards, const lrs_f16* values,
                              const uint8_t* terminateds, const uint8_t* truncateds,
                              const lrs_f16* trunc_values, const lrs_f16* bootstrap_value,
                              float gamma, float lambda,
                              float rho_bar, float c_bar, float pg_rho_bar,
                              lrs_f16* vs, lrs_f16* pg_advantages,
                              const int64_t* strides,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_retrace_tm_f16(int64_t num_envs, int64_t seq_len,
                               const lrs_f16* log_rhos, const lrs_f16* rewards,
                               const lrs_f16* q_values, const lrs_f16* values,
                               const uint8_t* terminateds, const uint8_t* truncateds,
                               const lrs_f16* trunc_values, const lrs_f16* bootstrap_value,
                               float gamma, float lambda, float c_bar, lrs_f16* q_ret,
                               const int64_t* strides,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);
lrs_status lrs_lambda_returns_tm_f16(int64_t num_envs, int64_t seq_len,
                                      const lrs_f16* rewards, const lrs_f16* values,
                                      const uint8_t* terminateds, const uint8_t* truncateds,
                                      const lrs_f16* trunc_values, const lrs_f16* bootstrap_value,
                                      float gamma, float lambda, lrs_f16* returns,
                                      const int64_t* strides,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);
lrs_status lrs_discounted_returns_tm_f16(int64_t num_envs, int64_t seq_len,
                                          const lrs_f16* rewards,
                                          const uint8_t* terminateds, const uint8_t* truncateds,
                                          const lrs_f16* trunc_values, const lrs_f16* bootstrap_value,
                                          float gamma, lrs_f16* returns,
                                          const int64_t* strides,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);
lrs_status lrs_eligibility_traces_tm_f16(int64_t num_envs, int64_t seq_len,
                                          const lrs_f16* x, const uint8_t* dones,
                                          float gamma, float lambda, lrs_f16* traces,
                                          const int64_t* strides,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);
lrs_status lrs_episodic_prefix_sum_tm_f16(int64_t num_envs, int64_t seq_len,
                                           const lrs_f16* x, const uint8_t* dones, lrs_f16* sums,
                                           const int64_t* strides,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream);
lrs_status lrs_affine_scan_tm_f16(int64_t num_envs, int64_t seq_len,
                                   const lrs_f16* alpha, const lrs_f16* beta,
                                   const uint8_t* reset, const lrs_f16* carry_in, int reverse,
                                   lrs_f16* y,
                                   const int64_t* strides,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Diagnostics and tuning (process-wide; not for concurrent use).
 * force_lookback != 0: every later call takes the multi-block carry-
 *   propagation path, even where whole rows fit in one tile.
 * elems_per_lane x waves_per_block in {4x1, 4x4, 8x4, 4x8, 16x4, 4x16, 8x16}: fix the
 *   tile (elems_per_lane * 64 * waves_per_block elements) instead of
 *   choosing it from the shape; 0 x 0 restores the automatic choice.
 * Returns LRS_ERR_INVALID_ARG for an unsupported combination.  Results stay
 * within fp32 rounding of each other across schedules (the int32 prefix sum
 * is identical). */
lrs_status lrs_debug_set_schedule(int force_lookback, int elems_per_lane,
                                  int waves_per_block);

/* Time-major calls: fix the waves per block (2, 4, 8 or 16: tiles of 16,
 * 32, 64 or 128 steps of 64 environments; 8 steps per lane), or 0 for the
 * automatic choice (which may also take blocks of 32 environments holding
 * whole rows of up to 128 steps).
 * Returns LRS_ERR_INVALID_ARG for any other value.  While 2 or 4 is set,
 * lrs_workspace_bytes reports the larger workspace such tiles need
 * (24 bytes per env per 16 or 32 steps). */
lrs_status lrs_debug_set_time_major_waves(int waves_per_block);

/* The launch a call would make, computed on the host by the same code that
 * plans and places the call's tiles (no GPU work, usable without a GPU).
 * Carries between tiles rely on one ordering: every tile a block may wait for
 * belongs to a block of lower index, which has started because a dispatch
 * starts its workgroups in index order.  This entry lets a caller check that
 * ordering for any shape and schedule setting. */
typedef struct lrs_schedule_info {
    int64_t num_blocks;       /* workgroups of the launch                          */
    int64_t num_tiles;        /* tiles; time-major: time tiles x groups            */
    int64_t tile_elems;       /* row-major: elements per tile                      */
    int64_t tile_steps;       /* time-major: steps per tile                        */
    int64_t groups;           /* time-major: environment groups (blocks per time tile) */
    int64_t envs_per_group;   /* time-major: environments per block (128, 64 or 32) */
    int32_t time_major;
    int32_t carries;          /* tiles exchange carries (look-back / time tiles > 1) */
    int32_t backward;         /* the scan runs from the end of each row            */
    int32_t tiles_per_row;    /* row-major look-back in position-major order: > 1  */
    int32_t elems_per_lane;
    int32_t waves_per_block;
    int32_t composition_fp64; /* maps composed in fp64 (betas may exceed 0.99)     */
    int32_t reserved;
} lrs_schedule_info;

enum {
    LRS_SCHED_TRUNCATED = 1,  /* backward estimators: the truncating variant; affine: reset mask */
    LRS_SCHED_REVERSE = 2,    /* affine scan: reverse direction                      */
    LRS_SCHED_TIME_MAJOR = 4, /* the _tm_ call                                       */
    LRS_SCHED_16BIT = 8       /* the _bf16 / _f16 call (not for LRS_PREFIX_SUM_I32)   */
};

/* Fills *info for a call of `est` with `flags` (LRS_SCHED_*) at
 * [num_envs, seq_len] whose betas are at most beta_max (gamma*lambda,
 * gamma, gamma*lambda*c_bar, 1 for sums, INFINITY for the affine scan), under
 * the current lrs_debug_set_* settings, and, when tile_of_block is not NULL
 * and capacity >= info->num_blocks, tile_of_block[b] = the tile block b works
 * on (time-major: time_tile * groups + group).  Returns LRS_ERR_INVALID_ARG
 * for sizes or flags the calls reject. */
lrs_status lrs_debug_schedule(lrs_estimator est, int flags, int64_t num_envs, int64_t seq_len,
                              float beta_max, lrs_schedule_info* info, uint32_t* tile_of_block,
                              int64_t capacity);

/* Measurement reference kernels (not an estimator).  kind 0: an empty kernel
 * of `blocks` workgroups of `threads` lanes (64..1024, a multiple of 64): the
 * fixed cost of a launch of that grid.  kind 1: the same grid reading
 * read_bytes from src and then writing write_bytes to dst (device memory,
 * 16-byte aligned, multiples of 16 bytes, at most 256 bytes read per lane),
 * each lane's stores waiting for its loads: the cost of a call's bytes on its
 * grid without the recurrence.  Asynchronous on `stream`. */
lrs_status lrs_debug_floor(int kind, int64_t blocks, int threads, const void* src,
                           int64_t read_bytes, void* dst, int64_t write_bytes,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LRS_H */
