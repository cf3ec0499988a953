/*
 * linattn.h -- C ABI of the MI355X (gfx950) causal linear-attention library.
 *
 * The method (feature map phi(x) = elu(x) + 1 applied to queries and keys
 * separately, never to values):
 *
 *     S_t = a_t S_{t-1} + phi(k_t) v_t^T          (a_t = 1 when ungated)
 *     z_t = a_t z_{t-1} + phi(k_t)
 *     o_t = phi(q_t)^T S_t / (phi(q_t)^T z_t + eps)
 *
 * Sources: "Linear Attention: accumulating KV into a fixed-size state",
 * sections "Why replace softmax" (the feature map) and "State update and read
 * as equations" (the update of S and z and the normalized read); the review
 * of "Transformers are RNNs", feature-map table (elu + 1), causal-masking and
 * RNN-form tables (S_0 = 0, z_0 = 0, one token at a time) and the discussion
 * of the non-causal case; "Linear Attention: what happens when you change the
 * product order", section "The summary runs out of room" (a scalar decay of
 * the whole summary at every step); the state-space-models page, section 2
 * (the output written with j <= t, i.e. token t reads its own key and value).
 * No page adds eps; it is added after the dot product, here and in every path.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers to tensors are DEVICE pointers (hipMalloc'd or torch CUDA
 *   memory), contiguous, row-major, owned by the caller.  The library
 *   allocates and frees nothing.  Results depend only on the arguments: the
 *   library's only state across calls is the optional timing record of
 *   linattn_profile_enable / linattn_profile_read (see there; not
 *   thread-safe).
 * - Shapes follow the pages' [batch, heads, tokens, head_dim] layout:
 *   q, k [B][H][N][Dk], v [B][H][N][Dv], o [B][H][N][Dv]; the state
 *   S [B][H][Dk][Dv] (row = key component, column = value component) and
 *   z [B][H][Dk] are always fp32.
 * - dtype (LINATTN_F32 or LINATTN_BF16) is the element type of q, k, v and o.
 *   Arithmetic: bf16 inputs use bf16 matrix-core products with fp32
 *   accumulation and an fp32 state; fp32 inputs use fp32 arithmetic
 *   throughout.
 * - Dk and Dv must each be one of 16, 32, 64, 128.
 * - phi selects the feature map: LINATTN_PHI_ELU1 (the method) or
 *   LINATTN_PHI_IDENTITY (checks against the pages' post-feature-map worked
 *   examples; the caller then owns the sign of the denominator).
 * - Work is enqueued on hip_stream (a hipStream_t; NULL = the null stream).
 *   Calls return without synchronizing; results are valid once the stream
 *   has reached that point.  Calls on different streams are independent as
 *   long as their buffers are.
 * - Every argument is validated on the host before anything is launched, so
 *   an error return means nothing ran.  NaN or Inf inputs propagate; they
 *   are not checked.
 *
 * Status codes: LINATTN_OK (0) or a negative LINATTN_E* value below.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LINATTN_ABI_VERSION 4
#define LINATTN_MAX_SNAPSHOTS 256
/* Bytes of the fixed device scratch of linattn_forward_noalloc (48 MiB). */
#define LINATTN_NOALLOC_SCRATCH_BYTES 50331648u

enum linattn_dtype { LINATTN_F32 = 0, LINATTN_BF16 = 1, LINATTN_FP8_E4M3 = 2 /* state storage only */ };
enum linattn_phi { LINATTN_PHI_ELU1 = 0, LINATTN_PHI_IDENTITY = 1 };
enum linattn_kind {
    LINATTN_KIND_FORWARD = 0,
    LINATTN_KIND_GATED = 1,
    LINATTN_KIND_NONCAUSAL = 2,
    LINATTN_KIND_BACKWARD = 3,
    LINATTN_KIND_TRAIN = 4 /* linattn_forward_train: its segment states, kept for linattn_backward */
};

enum linattn_status {
    LINATTN_OK = 0,
    LINATTN_EINVAL = -1,     /* NULL required pointer, B/H/N < 1, eps < 0 or not finite, aliasing */
    LINATTN_ESHAPE = -2,     /* Dk or Dv not in {16, 32, 64, 128}, or sizes overflow 64-bit indexing */
    LINATTN_EDTYPE = -3,     /* dtype or phi not one of the enumerated values */
    LINATTN_EWORKSPACE = -4, /* workspace NULL or smaller than linattn_workspace_size() */
    LINATTN_ELAUNCH = -5     /* a HIP launch failed (the HIP error is not cleared) */
};

/*
 * Causal forward ("Transformer mode"): the whole sequence of each (b, h) in
 * parallel, with the result of the one-token-at-a-time recurrence above.
 *
 *   q, k, v   inputs, dtype `dtype`.
 *   o         output [B][H][N][Dv], dtype `dtype` (bf16: round-to-nearest-even).
 *             Must not overlap q, k or v.
 *   s_init,   initial state [B][H][Dk][Dv] and [B][H][Dk] fp32, or both NULL
 *   z_init    for S_0 = 0, z_0 = 0 (the pages' start).  Passing the final
 *             state of an earlier call resumes that sequence exactly.
 *   s_final,  if non-NULL, receive the state after token N-1 (fp32).  They may
 *   z_final   alias s_init / z_init (in-place resume); pass both or neither.
 *   eps       added to the denominator; >= 0 and finite.
 *   workspace device scratch of at least
 *             linattn_workspace_size(LINATTN_KIND_FORWARD, B, H, N, Dk, Dv, dtype)
 *             bytes (may be NULL when that size is 0).  Contents on entry do
 *             not matter; the call overwrites it.
 */
int linattn_forward(const void *q, const void *k, const void *v, void *o,
                    const float *s_init, const float *z_init,
                    float *s_final, float *z_final,
                    int B, int H, int N, int Dk, int Dv, int dtype, int phi,
                    float eps, void *workspace, size_t workspace_bytes,
                    void *hip_stream);

/*
 * Gated causal forward: as linattn_forward with the scalar decay a_t
 * multiplying the whole summary (S and z) before token t is added, so token t
 * itself is undecayed and a_0 multiplies s_init / z_init.
 *
 *   alpha     [B][H][N] fp32 per-token decay.  Values in [0, 1] are supported
 *             (0 clears the summary exactly); values above 1 make the state
 *             grow and may overflow, as the state-space-models page warns
 *             (section 3).
 * Other arguments as linattn_forward; workspace kind LINATTN_KIND_GATED.
 */
int linattn_forward_gated(const void *q, const void *k, const void *v,
                          const float *alpha, void *o,
                          const float *s_init, const float *z_init,
                          float *s_final, float *z_final,
                          int B, int H, int N, int Dk, int Dv, int dtype,
                          int phi, float eps, void *workspace,
                          size_t workspace_bytes, void *hip_stream);

/*
 * linattn_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid allocation.  It
 * takes no workspace and calls no hipMalloc, hipFree or other allocating
 * routine; the segment states that linattn_forward keeps in the workspace
 * live in a fixed device array inside the library of
 * LINATTN_NOALLOC_SCRATCH_BYTES (one per GPU, held from the library's first
 * use on that GPU until the process ends).  The caller still passes every
 * input and output, as for linattn_forward.
 *
 * - Sizes whose linattn_workspace_size(LINATTN_KIND_FORWARD, ...) exceeds
 *   LINATTN_NOALLOC_SCRATCH_BYTES are rejected with LINATTN_EWORKSPACE before
 *   anything runs (the 131072-token, 16-head, Dk = Dv = 128 case needs 35 MB).
 * - Every call on one GPU uses that GPU's one array, and the array keeps the
 *   last call's contents (nothing in it needs to start cleared: every state
 *   cell is written before it is read).  Calls that overlap in time on one GPU
 *   (on different streams, or from different host threads without ordering)
 *   race on it: the caller serializes them.
 * - The GPU is the one the stream belongs to (the current device for the
 *   NULL stream); the array's address there is looked up on the first call
 *   and kept.  LINATTN_ELAUNCH if that lookup fails.
 * - These launches are not recorded by linattn_profile_enable.
 * Results are identical to linattn_forward's on the same arguments.
 */
int linattn_forward_noalloc(const void *q, const void *k, const void *v, void *o,
                            const float *s_init, const float *z_init,
                            float *s_final, float *z_final,
                            int B, int H, int N, int Dk, int Dv, int dtype, int phi,
                            float eps, void *hip_stream);

/*
 * Causal forward (gated when alpha is non-NULL) with the split of each
 * sequence chosen by the caller.  The result is the same quantity as
 * linattn_forward(_gated): the sum of outer products does not depend on how
 * the tokens are grouped ("Linear Attention: accumulating KV into a
 * fixed-size state", section "Adding to the same state in turn"), so any split
 * gives the same outputs up to the order of the fp32 additions.
 *
 *   segments     >= 1: each sequence is cut into output segments of
 *                ceil(chunks / segments) chunks of 64 tokens (so at most
 *                `segments` of them), processed in parallel from the prefix
 *                of the earlier segments' states (1 = one sequential pass).
 *   subsegments  >= 1: each output segment's state is summed over this many
 *                parts (the largest divisor of its chunk count not above
 *                the request); only the bf16 matrix-core path uses it.
 *   workspace    at least linattn_workspace_size_planned(kind, ...,
 *                segments, subsegments) bytes, kind LINATTN_KIND_GATED when
 *                alpha is given, else LINATTN_KIND_FORWARD.
 * Other arguments as linattn_forward(_gated); LINATTN_EINVAL when segments
 * or subsegments is below 1, LINATTN_ESHAPE when the split's state cells of
 * one (b, h) (segments x parts, Dk Dv + Dk + Dv floats each) would reach
 * 1 GiB (linattn_workspace_size_planned then returns 0).  linattn_forward
 * uses a split chosen to fill the GPU.
 */
int linattn_forward_planned(const void *q, const void *k, const void *v,
                            const float *alpha, void *o,
                            const float *s_init, const float *z_init,
                            float *s_final, float *z_final,
                            int B, int H, int N, int Dk, int Dv, int dtype,
                            int phi, float eps, int segments, int subsegments,
                            void *workspace, size_t workspace_bytes,
                            void *hip_stream);

/*
 * Causal forward for training: linattn_forward that also keeps, for the
 * backward, each token's denominator den_t = phi(q_t)^T z_t + eps.
 *
 *   den       output [B][H][N] fp32.
 * o and den are required; den must not overlap q, k, v or o.
 * Restricted to the chunked bf16 path: dtype LINATTN_BF16 with Dk and Dv in
 * {64, 128} (LINATTN_ESHAPE / LINATTN_EDTYPE otherwise).  Other arguments as
 * linattn_forward.  o is the same quantity as linattn_forward's; the segment
 * states are summed in the backward's form (for elu + 1, elu(k) v^T, elu(k)
 * and v apart, so that bf16 keeps elu's bits), so the two may differ in the
 * last bit of a few outputs.
 *
 *   workspace  at least linattn_workspace_size(LINATTN_KIND_TRAIN, ...)
 *              bytes (may be NULL when that is 0).  On return it holds the
 *              forward state at the start of each segment of the sequence
 *              (S, z and the running sum of v, fp32): pass it, unchanged, as
 *              `saved` to linattn_backward on the same inputs, and the backward
 *              does not recompute them.
 */
int linattn_forward_train(const void *q, const void *k, const void *v, void *o,
                          float *den, const float *s_init, const float *z_init,
                          float *s_final, float *z_final,
                          int B, int H, int N, int Dk, int Dv, int dtype,
                          int phi, float eps, void *workspace,
                          size_t workspace_bytes, void *hip_stream);

/*
 * Backward of the causal forward (ungated): given dout = dL/dO for a loss L,
 * the gradients dq, dk, dv of L.  They are the derivative of the forward's
 * definition above (the pages give no backward formula; the quantities are
 * those of reverse-mode differentiation of the recurrence, with
 * dY_t = dout_t / den_t, dd_t = -(dout_t . o_t) / den_t:
 *   dq_t = (S_t dY_t + dd_t z_t) * phi'(q_t)
 *   dk_t = (R_t v_t + r_t) * phi'(k_t),  dv_t = R_t^T phi(k_t),
 *   R_t = sum_{u >= t} phi(q_u) dY_u^T,  r_t = sum_{u >= t} dd_u phi(q_u)).
 *
 *   q, k, v   the forward's inputs; den its output from linattn_forward_train
 *             ([B][H][N] fp32) on the same inputs and initial state.
 *   saved     NULL, or that linattn_forward_train call's workspace, unchanged
 *             since (same q, k, v, s_init, z_init, phi and sizes): the segment
 *             states are then read from it instead of being recomputed (one
 *             pass over K and V less).  Must not overlap the outputs or the
 *             workspace.
 *   dout      [B][H][N][Dv], dtype `dtype`.
 *   dq, dk    outputs [B][H][N][Dk]; dv output [B][H][N][Dv]; dtype `dtype`
 *             (bf16 round-to-nearest-even).  Must not overlap any input or
 *             each other.
 *   s_init,   the forward's initial state (both NULL for a zero start).  Its
 *   z_init    gradient is not returned.
 *   eps       the forward's eps.
 * dY is dout / den rounded to bf16 once.  dd_t is formed from the state the
 * backward carries, as -phi(q_t) . (S_t dY_t) / (phi(q_t) . z_t + eps),
 * rather than from the forward's rounded o (dq is a small difference of
 * large terms, and o's rounding would show in it).
 * Restricted like linattn_forward_train (bf16, Dk and Dv in {64, 128}).
 * Workspace kind LINATTN_KIND_BACKWARD (always needed: it holds dd).
 */
int linattn_backward(const void *q, const void *k, const void *v,
                     const float *den, const void *saved, const void *dout,
                     void *dq, void *dk, void *dv,
                     const float *s_init, const float *z_init,
                     int B, int H, int N, int Dk, int Dv, int dtype, int phi,
                     float eps, void *workspace, size_t workspace_bytes,
                     void *hip_stream);

/*
 * Delta rule ("Linear Attention: what happens when you change the product
 * order", section "The summary runs out of room": before writing, read the
 * summary with the key and write only the difference to the value, so that
 * re-reading with the same key returns the new value).  Per token:
 *   kh_t = phi(k_t) / |phi(k_t)|_2   (unit key; a zero key writes nothing)
 *   S'   = a_t S_{t-1}               (the gated form the same section names,
 *                                     Gated DeltaNet; a_t = 1 when ungated)
 *   S_t  = S' + beta_t kh_t (v_t - S'^T kh_t)^T
 *   o_t  = S_t^T phi(q_t)            (no normalizer)
 *
 *   alpha     NULL (ungated) or [B][H][N] fp32 gates in [0, 1] (a gate of 0
 *             clears the summary exactly).
 *   beta      NULL (every beta_t = 1, the page's full overwrite) or
 *             [B][H][N] fp32 write strengths.
 *   s_init    NULL (zero) or [B][H][Dk][Dv] fp32; s_final NULL or output
 *             [B][H][Dk][Dv] fp32 (may alias s_init).
 *   o         output [B][H][N][Dv] bf16; must not overlap the inputs.
 * Chunked bf16 path only (bf16, Dk and Dv in {64, 128}); no workspace.  One
 * workgroup per (b, h): the heads run in parallel, the chunks of a sequence
 * in order.
 */
int linattn_forward_delta(const void *q, const void *k, const void *v,
                          const float *alpha, const float *beta, void *o,
                          const float *s_init, float *s_final,
                          int B, int H, int N, int Dk, int Dv, int dtype,
                          int phi, void *hip_stream);

/*
 * Causal forward that also returns the summary after chosen tokens: for each
 * listed position p, S_p and z_p, the state once token p has been added (and
 * decayed, when gated).  The product-order page ("What a summary can't do")
 * notes that prefix caching and rolling back speculative tokens need a copy of
 * the summary at the exact position, since a summary cannot be cut like a KV
 * cache; these are those copies, taken in the same pass.
 *
 *   alpha      NULL (ungated) or [B][H][N] fp32 gates, as linattn_forward_gated.
 *   positions  HOST array of n_pos token indices, each in [0, N); any order,
 *              repeats allowed; 1 <= n_pos <= LINATTN_MAX_SNAPSHOTS.  The same
 *              positions apply to every (b, h).
 *   s_snap     output [B][H][n_pos][Dk][Dv] fp32; z_snap output
 *              [B][H][n_pos][Dk] fp32 (required; must not overlap the other
 *              arguments).
 * o, s_final, z_final, s_init, z_init, eps and the workspace (kind
 * LINATTN_KIND_GATED with alpha, else LINATTN_KIND_FORWARD) as
 * linattn_forward(_gated).  Restricted to the chunked bf16 path (bf16, Dk and
 * Dv in {64, 128}).  A snapshot at N - 1 equals (s_final, z_final) up to
 * summation order.
 */
int linattn_forward_snapshots(const void *q, const void *k, const void *v,
                              const float *alpha, void *o,
                              const float *s_init, const float *z_init,
                              float *s_final, float *z_final,
                              const int *positions, int n_pos,
                              float *s_snap, float *z_snap,
                              int B, int H, int N, int Dk, int Dv, int dtype,
                              int phi, float eps, void *workspace,
                              size_t workspace_bytes, void *hip_stream);

/*
 * Non-causal form: S = sum_t phi(k_t) v_t^T and z = sum_t phi(k_t) over the
 * whole sequence, computed once and read by every query:
 * o_t = phi(q_t)^T S / (phi(q_t)^T z + eps).
 *
 *   s_out, z_out  if non-NULL, receive the global S [B][H][Dk][Dv] and
 *                 z [B][H][Dk] (fp32); pass both or neither.
 * Workspace kind LINATTN_KIND_NONCAUSAL.  The reduction order over the
 * sequence is fixed, so results are bitwise reproducible.
 */
int linattn_forward_noncausal(const void *q, const void *k, const void *v,
                              void *o, float *s_out, float *z_out,
                              int B, int H, int N, int Dk, int Dv, int dtype,
                              int phi, float eps, void *workspace,
                              size_t workspace_bytes, void *hip_stream);

/*
 * One decode step ("RNN mode"): for every (b, h), update the carried state
 * in place with one new token and read it with that token's query:
 *   S <- a S + phi(k) v^T,  z <- a z + phi(k),  o = phi(q)^T S / (phi(q)^T z + eps)
 * (the read uses the updated state).
 *
 *   q, k      [B][H][Dk], dtype `dtype`;  v [B][H][Dv], dtype `dtype`.
 *   s, z      [B][H][Dk][Dv] and [B][H][Dk] fp32, read and overwritten.
 *   alpha     [B][H] fp32 decay for this step, or NULL for a = 1.
 *   o         [B][H][Dv], dtype `dtype`.  Must not overlap s or z.
 * No workspace.
 */
int linattn_decode_step(const void *q, const void *k, const void *v,
                        float *s, float *z, const float *alpha, void *o,
                        int B, int H, int Dk, int Dv, int dtype, int phi,
                        float eps, void *hip_stream);

/*
 * The decode step with the carried state stored in a narrower type: S and z
 * are read from state_dtype, the update is computed in fp32, rounded once
 * (round to nearest even) back to state_dtype, and the read uses the value as
 * stored.  The product-order page ("What a summary can't do") warns that a
 * summary rewritten every token in low precision accumulates rounding error;
 * this is that summary, at half (bf16) or a quarter (fp8) of the fp32 bytes.
 *
 *   s, z        [B][H][Dk][Dv] and [B][H][Dk] of state_dtype, IN/OUT.
 *   state_dtype LINATTN_F32 (same as linattn_decode_step), LINATTN_BF16, or
 *               LINATTN_FP8_E4M3 (OCP e4m3: 3 mantissa bits, largest finite
 *               448; a larger magnitude is stored as NaN, so an ungated sum
 *               overflows after a few hundred tokens).
 * Other arguments as linattn_decode_step.
 */
int linattn_decode_step_lowp(const void *q, const void *k, const void *v,
                             void *s, void *z, int state_dtype,
                             const float *alpha, void *o,
                             int B, int H, int Dk, int Dv, int dtype, int phi,
                             float eps, void *hip_stream);

/*
 * Workspace bytes a call of the given kind needs for these sizes (0 when the
 * call needs none).  Pure host arithmetic; returns 0 for invalid arguments.
 */
size_t linattn_workspace_size(int kind, int B, int H, int N, int Dk, int Dv, int dtype);

/* Workspace bytes of linattn_forward_planned (kind LINATTN_KIND_FORWARD or
 * LINATTN_KIND_GATED) for the requested split; 0 for invalid arguments. */
size_t linattn_workspace_size_planned(int kind, int B, int H, int N, int Dk, int Dv, int dtype,
                                      int segments, int subsegments);

/* Static string naming a status code. */
const char *linattn_status_string(int status);

/* LINATTN_ABI_VERSION of the built library. */
int linattn_abi_version(void);

/*
 * Kernel-level timing for measurement tools.  While enabled, every kernel the
 * library launches is bracketed by a pair of hipEvents recorded on the
 * caller's stream; linattn_profile_read() waits for them and reports, per
 * kernel name, the number of launches and the summed device time since the
 * last enable.  Not thread-safe: enable, run on one host thread, read.
 *
 *   linattn_profile_enable(1) clears the record and starts; (0) stops.
 *   linattn_profile_read(names, ms, counts, max) fills up to max entries
 *   (names point to static strings) and returns how many kernels were seen,
 *   or LINATTN_ELAUNCH if an event failed.
 */
int linattn_profile_enable(int on);
int linattn_profile_read(const char **names, double *total_ms, int *launches, int max);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
