/*
 * vla.h -- C ABI of the MI355X (gfx950) Variational Linear Attention library.
 *
 * The operation is the per-head VLA recurrence of "Variational Linear
 * Attention: Stable Associative Memory for Long-Context Transformers"
 * (arXiv 2605.11196), section 3.3, Eqs. (9), (10) and (11), with the initial
 * state of section 3.2 (A_0 = I / lambda0).  For every (batch b, head h), one
 * token t at a time:
 *
 *   k^ = k_t / |k_t|,  u^ = u_t / |u_t|            (a zero vector stays zero)
 *   z = A u^,  delta = 1 + u^' z,  A <- A - z z' / delta                 Eq. (9)
 *   e = v_t - S k^ (old S),  alpha^ = A k^ / |A k^| (new A),  S <- S + e alpha^'
 *                                                                         Eq. (10)
 *   zkey <- zkey + phi(k_t),  phi = ELU + 1 applied to the raw key,
 *   o_t = S phi(q_t) / max(phi(q_t)' zkey, eps)  (new S)                   Eq. (11)
 *
 * Entry points: vla_forward (T tokens; vla_forward_penalty and
 * vla_forward_memory are its two passes; vla_forward_noalloc the same forward
 * with a library-held workspace), vla_step (one decode token, state in place),
 * vla_backward (the gradients through vla_forward), vla_forward_scan
 * (vla_forward with the memory chain as a scan over chunks, for comparison),
 * the workspace-size queries and vla_status_string.
 *
 * Data layout (all row-major, contiguous, no strides):
 *   q, k, v, u : [B][H][T][d_h] of the input type (fp32 or bf16), on the device
 *   o          : [B][H][T][d_h] fp32
 *   S, A       : [B][H][d_h][d_h] fp32; S[i][j] has i = value index and
 *                j = key index (o = S phi(q)); A is stored in full (symmetric)
 *   zkey       : [B][H][d_h] fp32, the running sum of phi(k)
 * Every pointer is a device pointer and must be 16-byte aligned.
 *
 * Supported: d_h in {16, 32, 64, 96, 128}; B, H >= 1; T >= 0; finite
 * lambda0 > 0 and eps > 0.  State arithmetic is fp32 throughout; bf16 inputs
 * are widened exactly.  The kernels address one head's inputs, o, and the
 * per-chunk and per-token records in the workspace with 32-bit byte offsets, so
 * T is limited to sequences whose per-head buffers stay below 2^31 bytes (for
 * the forward at most 2,088,976 tokens at d_h = 64, 1,520,880 at 96 and
 * 1,195,696 at 128; for vla_backward, whose per-token records take
 * (4 d_h + 8) floats, 2,033,601, 1,369,568 and 1,032,444); a longer T is
 * VLA_ERR_UNSUPPORTED, also from the workspace-size queries.
 *
 * Ownership and execution: the caller owns every buffer, including the
 * device workspace of vla_forward (size from vla_forward_workspace_size); the
 * library allocates nothing and keeps no state between calls (apart from the
 * fixed device array that vla_forward_noalloc uses as its workspace).  Calls are
 * asynchronous on `stream` (a hipStream_t; NULL = the null stream) and never
 * synchronise.  Arguments are checked before anything is launched; on an
 * argument error nothing is launched and no buffer is touched.  A failed launch
 * returns VLA_ERR_HIP.  Faults inside a kernel surface at the caller's next
 * synchronisation.  NaN or Inf inputs propagate without being reported.
 * Concurrent calls that write the same buffers (a shared workspace included)
 * race.
 */
#ifndef VLA_H
#define VLA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vla_status {
    VLA_OK = 0,
    VLA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size or constant */
    VLA_ERR_UNSUPPORTED = 2,   /* d_h or dtype this library has no kernel for   */
    VLA_ERR_HIP = 3            /* a HIP runtime call or launch failed           */
} vla_status;

typedef enum vla_dtype {
    VLA_F32 = 0,
    VLA_BF16 = 1
} vla_dtype;

/*
 * vla_forward -- run T tokens of every (b, h) head in one launch.
 *
 * q, k, v, u   inputs [B][H][T][d_h] of type in_dtype (required when T > 0).
 * lambda0      penalty initialiser: the default A_0 is I / lambda0.
 * eps          floor of the readout denominator (Eq. 11).
 * o            output [B][H][T][d_h] fp32 (required when T > 0).
 * S_out, A_out, zkey_out
 *              final state [B][H][d][d], [B][H][d][d], [B][H][d]; each may be
 *              NULL to skip it.  They may alias S0, A0, zkey0 (in-place update).
 * S0, A0, zkey0
 *              initial state in the same layout, or NULL for the defaults
 *              S_0 = 0, A_0 = I / lambda0, zkey_0 = 0.  A0 must be symmetric
 *              positive definite (as every A_t of the recurrence is).
 * workspace    device scratch of at least workspace_bytes bytes, 256-byte
 *              aligned, as given by vla_forward_workspace_size for the same
 *              B, H, T, d_h (may be NULL when that size is 0).  Its contents
 *              on entry do not matter and are not meaningful on return.
 * stream       hipStream_t to launch on.
 *
 * For d_h in {64, 96, 128} and T >= 1 the sequence runs in two passes
 * (section 3.2 makes A_t the inverse of A_0^-1 + sum_{s<=t} u^_s u^_s', so
 * the penalty chain restarts at segment boundaries from that inverse, formed in
 * fp64; the memory chain then runs from the per-chunk factors the penalty
 * pass leaves in the workspace).  Results equal the token-by-token recurrence
 * up to rounding.  T == 0 launches a copy of the initial state to the
 * requested outputs.  A too small or misaligned workspace is
 * VLA_ERR_INVALID_ARG.
 */
vla_status vla_forward(const void *q, const void *k, const void *v, const void *u,
                       vla_dtype in_dtype, int B, int H, int T, int d_h,
                       float lambda0, float eps,
                       float *o, float *S_out, float *A_out, float *zkey_out,
                       const float *S0, const float *A0, const float *zkey0,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * vla_forward_penalty, vla_forward_memory -- the two passes of vla_forward for
 * d_h in {64, 96, 128} and T >= 1, for callers that schedule them apart (for
 * example the penalty pass of one batch on a second stream while the memory
 * pass of the previous batch runs).  Calling vla_forward_penalty and then
 * vla_forward_memory on the same workspace and the same inputs, in stream
 * order, gives exactly the results of vla_forward.
 *
 * vla_forward_penalty runs the penalty chain of Eq. (9) and, for every chunk of
 * 16 tokens, leaves the factors the memory chain needs (alpha^ of Eq. (10), the
 * key-sum denominators of Eq. (11)) in the workspace; it writes the final A and
 * zkey (A_out, zkey_out may be NULL).  vla_forward_memory then runs Eqs. (10)
 * and (11) from those factors and v, writing o and the final S; k^ and phi(q)
 * come from the records vla_forward_penalty left (it is the pass that reads q
 * and k), so vla_forward_memory takes neither.  Between the two calls the
 * workspace must not be used by anything else.  Arguments and errors as for
 * vla_forward; d_h in {16, 32} is VLA_ERR_UNSUPPORTED and T < 1
 * VLA_ERR_INVALID_ARG.
 */
vla_status vla_forward_penalty(const void *q, const void *k, const void *u, vla_dtype in_dtype,
                               int B, int H, int T, int d_h, float lambda0, float eps,
                               float *A_out, float *zkey_out, const float *A0,
                               const float *zkey0, void *workspace, size_t workspace_bytes,
                               void *stream);
vla_status vla_forward_memory(const void *v, vla_dtype in_dtype,
                              int B, int H, int T, int d_h, float *o, float *S_out,
                              const float *S0, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * vla_forward_workspace_size -- bytes of device workspace vla_forward needs for
 * these sizes (0 when it needs none: d_h in {16, 32}, or T == 0), in *bytes.
 * Per head it holds one record of (48 d_h + 1040) fp32 values for every chunk
 * of 16 tokens (the chunk's factors, k^ and phi(q): 16.1 KiB at d_h = 64) and,
 * when the penalty chain is split into segments, per segment the fp64 Gram
 * partial sums and the fp32 starting A and zkey; at B = 8, H = 16, T = 4096,
 * d_h = 64 the total is 546.5 MiB.  Host-only; launches nothing.  Errors:
 * VLA_ERR_INVALID_ARG (NULL bytes, bad sizes), VLA_ERR_UNSUPPORTED (d_h).
 */
vla_status vla_forward_workspace_size(int B, int H, int T, int d_h, size_t *bytes);

/*
 * vla_step -- one decode token for every (b, h) head: the same recurrence as
 * vla_forward with T = 1, continuing from the caller's state, which is updated
 * in place.  This is the streaming inference the method is built for: the
 * Portuguese technical summary of the paper ("Resumo Tecnico: Atencao Linear
 * Variacional", section 5) and the paper's section 3.5 (Table 1: O(d_h^2)
 * memory, independent of T) describe generation with a fixed-size state
 * (S, A, zkey) and no key/value cache.
 *
 * q, k, v, u   inputs [B][H][d_h] of type in_dtype.
 * S, A, zkey   in/out state [B][H][d][d], [B][H][d][d], [B][H][d] (required).
 * o            output [B][H][d_h] fp32.
 */
vla_status vla_step(const void *q, const void *k, const void *v, const void *u,
                    vla_dtype in_dtype, int B, int H, int d_h, float eps,
                    float *S, float *A, float *zkey, float *o,
                    void *stream);

/*
 * vla_forward_scan -- the same forward as vla_forward (d_h in {64, 96, 128},
 * T >= 1), with
 * the memory chain (Eqs. (10), (11)) computed as a parallel scan over chunks of
 * 16 tokens instead of a chain: section 3.4, Eq. (12), with the combine
 * corrected to the right multiplication that Eq. (10) implies
 * (S -> S F + G; (F1, G1) then (F2, G2) is (F1 F2, G1 F2 + G2)).  The penalty
 * pass is vla_forward's; each chunk's map (F, G) is formed from its factors,
 * the maps are scanned (work-efficient up- and down-sweep, d x d x d products
 * per combine) and every chunk's readout runs from its start state.  Provided
 * to measure the pages' parallel form against the chained memory pass; it
 * does O(d^3) work per chunk where the chain does O(d^2) per token.
 *
 * Arguments, outputs and errors as for vla_forward; results equal vla_forward's
 * up to rounding.  d_h other than 64, 96 or 128 is VLA_ERR_UNSUPPORTED, T < 1
 * VLA_ERR_INVALID_ARG.  workspace: at least vla_forward_scan_workspace_size
 * bytes, 256-byte aligned (vla_forward's workspace plus 2 d^2 floats per chunk
 * of each head, rounded up to a power of two chunks, plus one map per head).
 */
vla_status vla_forward_scan(const void *q, const void *k, const void *v, const void *u,
                            vla_dtype in_dtype, int B, int H, int T, int d_h,
                            float lambda0, float eps,
                            float *o, float *S_out, float *A_out, float *zkey_out,
                            const float *S0, const float *A0, const float *zkey0,
                            void *workspace, size_t workspace_bytes, void *stream);

/* vla_forward_scan_workspace_size -- bytes of workspace vla_forward_scan needs
 * (0 when T == 0).  Host-only.  Errors: VLA_ERR_INVALID_ARG (NULL bytes, bad
 * sizes), VLA_ERR_UNSUPPORTED (d_h other than 64, 96, 128). */
vla_status vla_forward_scan_workspace_size(int B, int H, int T, int d_h, size_t *bytes);

/*
 * vla_backward -- gradients of a scalar loss L through vla_forward, for every
 * (b, h) head: given the adjoints of the forward's outputs, the gradients with
 * respect to its inputs and initial state.  The pages define the forward only;
 * this is the chain rule through Eqs. (9), (10) and (11) in reverse token
 * order (section 3.3), with two conventions where no derivative exists: a zero
 * k or u (normalised to zero) passes no gradient through its normalisation, and
 * the floor of Eq. (11) passes gradient to phi(q)'zkey only where
 * phi(q)'zkey >= eps.
 *
 * q, k, v, u, in_dtype, B, H, T, d_h, lambda0, eps, S0, A0, zkey0
 *              exactly as given to vla_forward (the forward is recomputed).
 * dO           dL/do, [B][H][T][d_h] fp32 (required when T > 0).
 * dS_T, dA_T, dzkey_T
 *              dL/dS_T, dL/dA_T ([B][H][d][d], entrywise) and dL/dzkey_T
 *              ([B][H][d]) for the final state, or NULL for zero.
 * dq, dk, dv, du
 *              outputs [B][H][T][d_h] fp32 (required when T > 0): dL/dq etc.
 *              with respect to the input values as real numbers (also for
 *              bf16 inputs).
 * dS0, dzkey0  outputs dL/dS0 [B][H][d][d] and dL/dzkey0 [B][H][d], or NULL.
 * dA0          output [B][H][d][d], or NULL: the gradient with respect to A0 as
 *              a symmetric matrix, (G + G')/2 of the entrywise gradient G
 *              (A_0 must be symmetric, so only that part is meaningful).
 * workspace    device scratch of at least vla_backward_workspace_size bytes,
 *              256-byte aligned (NULL when that size is 0); it receives the
 *              forward's per-token vectors.
 * stream       hipStream_t to launch on.
 *
 * Outputs must not overlap inputs.  The forward is recomputed first, keeping
 * per token z = A_{t-1} u^, alpha^, e, zkey_t and five scalars in the workspace: for
 * d_h in {64, 96, 128} by the chunked two-pass forward of vla_forward (its o
 * passes through dq, which is then overwritten), for d_h in {16, 32} token by
 * token in the gradient kernel itself.  The reverse recurrence then runs from
 * t = T down to 1 with the states rebuilt from those vectors: for d_h in
 * {64, 96, 128} as two workgroups per head in one launch (the memory chain's
 * adjoint, and the penalty chain's, in the frame A Sigma A of the adjoint Sigma
 * of A, following it through dL/dalpha^ kept in the workspace and dL/dv), for
 * d_h in {16, 32} as one workgroup per head.  Errors as for vla_forward.
 */
vla_status vla_backward(const void *q, const void *k, const void *v, const void *u,
                        vla_dtype in_dtype, int B, int H, int T, int d_h,
                        float lambda0, float eps,
                        const float *S0, const float *A0, const float *zkey0,
                        const float *dO, const float *dS_T, const float *dA_T,
                        const float *dzkey_T,
                        float *dq, float *dk, float *dv, float *du,
                        float *dS0, float *dA0, float *dzkey0,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * vla_backward_workspace_size -- bytes of device workspace vla_backward needs:
 * (4 d_h + 8) fp32 values per token of each head, rounded up to 256 bytes,
 * and for d_h in {64, 96, 128} also the two-pass forward's workspace
 * (vla_forward_workspace_size), the forward's final S, A and zkey
 * ((2 d_h^2 + d_h) fp32 values per head), d_h fp32 values per token of each
 * head (dL/dalpha^), B H + 1 ints (synchronisation words) and d_h^2 fp32
 * values per head, each rounded up to 256 bytes (0 when T == 0).  Host-only.  Errors: VLA_ERR_INVALID_ARG (NULL bytes, bad
 * sizes), VLA_ERR_UNSUPPORTED (d_h).
 */
vla_status vla_backward_workspace_size(int B, int H, int T, int d_h, size_t *bytes);

/*
 * vla_forward_noalloc -- vla_forward for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The workspace is the library's own
 * device array of VLA_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held until the
 * process ends; the call allocates nothing.  Arguments, results and errors as
 * for vla_forward (bit-identical results), plus VLA_ERR_UNSUPPORTED when the
 * sizes need more workspace than the array holds (vla_forward_workspace_size
 * gives the need: for example B = 4, H = 8, T = 1024, d_h = 64 fits, B = 8,
 * H = 16, T = 4096 does not) and VLA_ERR_HIP if the array's device address
 * cannot be obtained.  Calls that overlap in time on one GPU share the array
 * and race: serialise them (one stream, or events between streams).
 */
#define VLA_NOALLOC_SCRATCH_BYTES (64u << 20)
vla_status vla_forward_noalloc(const void *q, const void *k, const void *v, const void *u,
                               vla_dtype in_dtype, int B, int H, int T, int d_h,
                               float lambda0, float eps,
                               float *o, float *S_out, float *A_out, float *zkey_out,
                               const float *S0, const float *A0, const float *zkey0,
                               void *stream);

/*
 * vla_baseline_forward -- the two baselines the pages compare VLA with, on the
 * same inputs and layouts (d_h in {64, 96, 128}):
 *   VLA_BASELINE_LINEAR  cumulative-sum linear attention, the recurrent form
 *                        of the "Linear Attention" wiki article: per token
 *                        S <- S + v phi(k)', zkey <- zkey + phi(k),
 *                        o = S phi(q) / (phi(q)' zkey)  (no floor; phi > 0);
 *   VLA_BASELINE_DELTA   DeltaNet as "Variational Linear Attention" section 3.5
 *                        obtains it from VLA (alpha^ replaced by the scalar gate
 *                        beta on the unit key, no A), i.e. the delta rule of the
 *                        kexue.fm article's "linear version" with eta = beta:
 *                        e = v - S k^, S <- S + beta e k^', o by Eq. (11)
 *                        (max(., eps) floor).
 * phi = ELU + 1 of the raw q and k; S [B][H][d][d] value-major as for
 * vla_forward.  beta is used by VLA_BASELINE_DELTA only (finite; 1 for the plain
 * delta rule).  S_out, zkey_out, S0, zkey0 as for vla_forward (NULL = skip /
 * zero).  workspace: at least vla_baseline_workspace_size bytes, 256-byte
 * aligned.  Errors as for vla_forward; an unknown kind or d_h in {16, 32} is
 * VLA_ERR_UNSUPPORTED.  These exist to measure VLA's constant factor and state
 * growth against them (section 3.5 Table 1, section 4.1); they share the
 * forward's memory-chain kernel.
 */
typedef enum vla_baseline {
    VLA_BASELINE_LINEAR = 0,
    VLA_BASELINE_DELTA = 1
} vla_baseline;
vla_status vla_baseline_forward(vla_baseline kind, const void *q, const void *k, const void *v,
                                vla_dtype in_dtype, int B, int H, int T, int d_h, float beta,
                                float eps, float *o, float *S_out, float *zkey_out,
                                const float *S0, const float *zkey0, void *workspace,
                                size_t workspace_bytes, void *stream);
/* bytes of workspace vla_baseline_forward needs (0 when T == 0).  Host-only. */
vla_status vla_baseline_workspace_size(int B, int H, int T, int d_h, size_t *bytes);

/* Static, human-readable text for a status code (never NULL). */
const char *vla_status_string(vla_status status);

#ifdef __cplusplus
}
#endif

#endif /* VLA_H */
