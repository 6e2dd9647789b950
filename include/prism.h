/*
 * prism.h - C ABI of the PRISM rank-L gated delta-rule forward (and its backward) on
 * MI355X (gfx950).
 *
 * What is computed (per batch b and head h, state S_0 = 0 unless given, S is dv x dk):
 *
 *   anchor_t = sum_{j=0..3} conv_w[h, j, :] * v_{t-3+j}        (rows before t = 0 are 0,
 *                                                               or given: prism_fwd_state)
 *   r_{t,0}  = v_t - anchor_t
 *   r_{t,l}  = r_{t,l-1} * (1 - alpha_{t,l-1} * gamma_{t,l-1})  (element-wise), l = 1..L-1
 *   A_t      = g_t (I - beta_t k_t k_t^T)
 *   B_t      = beta_t v_t k_t^T + sum_{l=1}^{L-1} (alpha_{t,l} r_{t,l}) u_{t,l}^T
 *   S_t      = S_{t-1} A_t + B_t
 *   o_t      = S_t q_t
 *
 * Sources: the linear recurrence S_t = S_{t-1} A_t + B_t with input-only A_t, B_t
 * ("PRISM" reading notes, liuzhao09.github.io, section 2.1; Tencent Ads article,
 * section 01-二); the GDN forgetting operator (notes section 2.2; article
 * section 01-四); rank accumulation of the write (notes section 2.2; ai-engineering
 * summary "ICML 2026 | PRISM", section "PRISM 设计"); the ShortConv anchor and the
 * residual chain (notes section 2.3; article section 03-三, where the GELU is absorbed
 * into a fixed preconditioner so the chain is element-wise linear).  The pages outline
 * this form without printing the equations; the concrete form above is the one this
 * library implements and its oracle checks.
 *
 * Layout: every tensor is dense, row-major (C order), head-major [B, H, T, ...].
 *   q, k   [B, H, T, dk]         dtype dt
 *   v      [B, H, T, dv]         dtype dt
 *   g      [B, H, T]             float32, 0 < g <= 1 (decay gate)
 *   beta   [B, H, T]             float32 (GDN write / erase strength)
 *   u      [B, H, T, L-1, dk]    dtype dt;  u[..., j, :] = u_{t, j+1}
 *   alpha  [B, H, T, L]          float32;   alpha[..., l] = alpha_{t, l}
 *   gamma  [B, H, T, L-1, dv]    dtype dt;  gamma[..., j, :] = gamma_{t, j}
 *   conv_w [H, 4, dv]            float32;   tap j multiplies v_{t-3+j}
 *   o      [B, H, T, dv]         dtype dt   (output, fully overwritten)
 *   S_final[B, H, dk, dv]        float32    (output: the transpose of S_T)
 * u, alpha and gamma are not read when L == 1 (they may be NULL then); conv_w is
 * not read when L == 1 either.
 *
 * Pointers are device pointers (hipMalloc'd or equivalent).  The caller owns every
 * buffer, the workspace included.  The library allocates nothing, keeps no state
 * between calls, never synchronises, and enqueues all work on `stream`
 * (NULL = the null stream).  Outputs must not alias inputs or the workspace.
 *
 * Precision: dt = PRISM_BF16 rounds MFMA operands to bfloat16 and accumulates in
 * float32; the state stays float32.  dt = PRISM_F32 computes in float32 throughout.
 *
 * Errors: argument checks happen on the host before anything is enqueued; a
 * failed check returns an error code and enqueues nothing.  A launch failure
 * returns PRISM_ERR_HIP.  Faults inside kernels surface at the caller's next
 * synchronisation.  Not checked: g > 0, finiteness of inputs.
 */
#ifndef PRISM_H_
#define PRISM_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* hipStream_t;
struct ihipEvent_t;
typedef struct ihipEvent_t* hipEvent_t;

typedef enum {
  PRISM_OK = 0,
  PRISM_ERR_INVALID_ARG = -1,   /* NULL pointer, non-positive size, size overflow */
  PRISM_ERR_UNSUPPORTED = -2,   /* a shape / dtype combination with no kernel */
  PRISM_ERR_WORKSPACE = -3,     /* workspace NULL or smaller than required */
  PRISM_ERR_HIP = -4            /* a HIP launch or runtime call failed */
} prism_status;

/* The last two enumerators are not types: they make every int a value of prism_dtype, so an
 * unknown code can be passed across the ABI and is rejected (PRISM_ERR_INVALID_ARG or
 * PRISM_ERR_UNSUPPORTED) instead of being undefined behaviour to read. */
typedef enum {
  PRISM_F32 = 0,
  PRISM_BF16 = 1,
  PRISM_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  PRISM_DTYPE_RANGE_MAX_ = 2147483647
} prism_dtype;

/* Bytes of device workspace prism_fwd needs for these sizes; 0 when the
 * arguments are invalid or unsupported (prism_fwd then reports which).
 * Supported: B, H, T >= 1; dk and dv each in {16, 32, 64, 128} (independently);
 * chunk in {16, 32, 64}; 1 <= L <= 8; B * H <= 65535; the chunk tiles must fit the
 * 160 KB of LDS per CU (with PRISM_F32, dk = dv = 128 needs chunk <= 32).  Shapes
 * other than bfloat16 dk = dv = 64 with chunk 64 run the generic kernels. */
size_t prism_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk,
                                 prism_dtype dt);

/* The forward pass.  `chunk` is the token count of the intra-chunk UT/WY block
 * (results agree across chunk sizes up to rounding).  Returns PRISM_OK or an
 * error code; see the header comment for layout, ownership and errors. */
prism_status prism_fwd(const void* q, const void* k, const void* v,
                       const float* g, const float* beta,
                       const void* u, const float* alpha, const void* gamma,
                       const float* conv_w,
                       int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                       void* o, float* S_final,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The forward pass continued from a given state, for streaming a long sequence in pieces
 * (the fixed-size state is all the linear recurrence carries forward: Tencent Ads article,
 * section 01-二; the ShortConv anchor looks three tokens back: "PRISM" reading notes,
 * section 2.3).  Arguments as prism_fwd, plus:
 *   S0       [B, H, dk, dv] float32: the state before the first token, in the S_final
 *            layout (S_0^T); NULL = zero.  May be the same buffer as S_final.
 *   conv_in  [B, H, 3, dv] dtype dt: the values of the three tokens before the first one
 *            (oldest first), read by the anchor; NULL = zero (a sequence start).
 *   conv_out [B, H, 3, dv] dtype dt, output: the values of the last three tokens of
 *            [conv_in; v] (rows of conv_in when T < 3); NULL = not written.  May be the
 *            same buffer as conv_in.
 * Running T1 tokens and then T2 more from (S_final, conv_out) gives the same o and S_final
 * as one call over T1 + T2 tokens, up to rounding.  Workspace: prism_fwd_workspace_bytes. */
prism_status prism_fwd_state(const void* q, const void* k, const void* v,
                             const float* g, const float* beta,
                             const void* u, const float* alpha, const void* gamma,
                             const float* conv_w,
                             int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                             const float* S0, const void* conv_in,
                             void* o, float* S_final, void* conv_out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One token for every (b, h) pair, in place: the token-at-a-time form of prism_fwd_state
 * for generation and serving.  Layout (dense, row-major):
 *   q, k  [B, H, dk]  dtype dt;   v [B, H, dv] dtype dt
 *   g, beta [B, H] float32;       alpha [B, H, L] float32
 *   u     [B, H, L-1, dk] dtype dt;   gamma [B, H, L-1, dv] dtype dt;   conv_w [H, 4, dv] float32
 *   S           [B, H, dk, dv] float32, in / out: the state (the S_final layout)
 *   conv_state  [B, H, 3, dv] dtype dt, in / out: values of the previous three tokens,
 *               oldest first; the token's v is appended and the oldest row dropped.
 *               Required when L > 1; may be NULL when L == 1 (the anchor is unused).
 *   o     [B, H, dv] dtype dt, output.
 * u, alpha, gamma, conv_w may be NULL when L == 1.  Supported: dk == dv in {16, 32, 64,
 * 128}, 1 <= L <= 8.  No workspace.  Errors as prism_fwd (checked before any launch). */
prism_status prism_decode_step(const void* q, const void* k, const void* v,
                               const float* g, const float* beta,
                               const void* u, const float* alpha, const void* gamma,
                               const float* conv_w,
                               int B, int H, int dk, int dv, int L, prism_dtype dt,
                               float* S, void* conv_state, void* o, hipStream_t stream);

/* Same as prism_fwd with an explicit segment length (in chunks, >= 1) for the
 * sequence-parallel split; results agree across segment lengths up to rounding.
 * prism_fwd picks the segment length itself.  Used to test that independence. */
size_t prism_fwd_seg_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk,
                                     prism_dtype dt, int seg_chunks);
prism_status prism_fwd_seg(const void* q, const void* k, const void* v,
                           const float* g, const float* beta,
                           const void* u, const float* alpha, const void* gamma,
                           const float* conv_w,
                           int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                           void* o, float* S_final,
                           void* workspace, size_t workspace_bytes, int seg_chunks,
                           hipStream_t stream);

/* Same as prism_fwd_nl (below) with an explicit segment length in chunks (>= 1), as
 * prism_fwd_seg is to prism_fwd; used to test that independence for the nonlinear sweep.
 * Workspace: prism_fwd_nl_seg_workspace_bytes (0 for invalid arguments). */
size_t prism_fwd_nl_seg_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk,
                                        prism_dtype dt, int seg_chunks);
prism_status prism_fwd_nl_seg(const void* q, const void* k, const void* v,
                              const float* g, const float* beta,
                              const void* u, const float* alpha, const void* p,
                              const float* conv_w,
                              int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                              void* o, float* S_final,
                              void* workspace, size_t workspace_bytes, int seg_chunks,
                              hipStream_t stream);

/* Same as prism_fwd, and records four caller-created events on `stream` around
 * the launches: events[0] before the segment sweep kernel, events[1] after it,
 * events[2] after the inter-segment scan, events[3] after the output correction.
 * For per-kernel timing with hipEventElapsedTime.  events must not be NULL. */
prism_status prism_fwd_timed(const void* q, const void* k, const void* v,
                             const float* g, const float* beta,
                             const void* u, const float* alpha, const void* gamma,
                             const float* conv_w,
                             int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                             void* o, float* S_final,
                             void* workspace, size_t workspace_bytes,
                             hipEvent_t* events, hipStream_t stream);

/* The backward pass: gradients of  sum_t <d_o_t, o_t> + <dS_final, S_final>  with respect
 * to every input of prism_fwd (S_0 = 0, no ShortConv history), i.e. the reverse-mode
 * derivative that end-to-end training of the layer needs (the pages quote training
 * throughput: "PRISM" reading notes, section 3.3).  Float32 throughout.  Segment-parallel:
 * the sequence is cut into segments; since the state and its adjoint are affine in what
 * they carry (the associativity of the recurrence, reading notes section 2.1, Tencent /
 * PKU article section 01-二), one pass forms each segment's end state from zero, its
 * operator A_{t0} .. A_{t1-1} and its own adjoint contribution, two scans give every
 * segment its entering state and the adjoint arriving at its end, and a second pass runs
 * the token-by-token adjoint of all segments at once.
 *   inputs    q .. conv_w, B, H, T, dk, dv, L, dt exactly as prism_fwd
 *   d_o       [B, H, T, dv] dtype dt: gradient of o
 *   dS_final  [B, H, dk, dv] float32: gradient of S_final; NULL = zero
 * outputs (float32, the layouts of the inputs, fully overwritten):
 *   dq, dk [B, H, T, dk];  dv [B, H, T, dv];  dg, dbeta [B, H, T];
 *   du [B, H, T, L-1, dk];  dalpha [B, H, T, L];  dgamma [B, H, T, L-1, dv];
 *   dconv_w [H, 4, dv] (summed over the batch)
 * The four rank-L gradients are not written when L == 1 (they may be NULL then) and
 * are required otherwise.  Supported: dk == dv in {16, 32, 64, 128}, 1 <= L <= 8,
 * B * H <= 2^31 - 1.  Results are deterministic (fixed summation orders).  Workspace:
 * prism_bwd_workspace_bytes; it holds five float32 dk x dk matrices per segment, the
 * state every 8 tokens plus an 8-token state buffer per segment, per-segment dconv_w and
 * anchor shares, and, with dk >= 64 (dk / 32 workgroups per state), their per-token column
 * sums.  The segment length is chosen from the shape (16 to 128 tokens).  Ownership,
 * stream and errors as prism_fwd. */
size_t prism_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int L, prism_dtype dt);
prism_status prism_bwd(const void* q, const void* k, const void* v,
                       const float* g, const float* beta,
                       const void* u, const float* alpha, const void* gamma,
                       const float* conv_w,
                       int B, int H, int T, int dk, int dv, int L, prism_dtype dt,
                       const void* d_o, const float* dS_final,
                       float* dq, float* dk_out, float* dv_out, float* dg, float* dbeta,
                       float* du, float* dalpha, float* dgamma, float* dconv_w,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* prism_bwd with the segment length given: seg_len tokens per segment (a multiple of 8,
 * at least 16; the last segment may be shorter), else PRISM_ERR_INVALID_ARG.  The
 * gradients do not depend on it beyond float32 rounding; for callers that tune it and for
 * tests that reach every segment case.  Workspace: prism_bwd_seg_workspace_bytes (0 for a
 * refused shape or length). */
size_t prism_bwd_seg_workspace_bytes(int B, int H, int T, int dk, int dv, int L, prism_dtype dt, int seg_len);
prism_status prism_bwd_seg(const void* q, const void* k, const void* v,
                           const float* g, const float* beta,
                           const void* u, const float* alpha, const void* gamma,
                           const float* conv_w,
                           int B, int H, int T, int dk, int dv, int L, prism_dtype dt,
                           const void* d_o, const float* dS_final,
                           float* dq, float* dk_out, float* dv_out, float* dg, float* dbeta,
                           float* du, float* dalpha, float* dgamma, float* dconv_w, int seg_len,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The same gradients with a workspace of O(T / 64) states per pair: one pair's state walks
 * the whole sequence on dk / 16 workgroups (the forward once keeping the state every 64
 * tokens, then per 64-token block, last first, the block's forward again and its adjoint
 * steps).  Much slower than prism_bwd on long sequences; for callers with little free
 * device memory.  With dk > 16 the workspace also holds each workgroup's per-token column
 * sums, B*H * (dk/16) * T * ((2+R)*dk + 3 + R) floats (R = 1, 3 or 7 rank slots for
 * L = 1, L <= 4, L <= 8).  Arguments, layouts and errors as prism_bwd; workspace:
 * prism_bwd_lowmem_workspace_bytes. */
size_t prism_bwd_lowmem_workspace_bytes(int B, int H, int T, int dk, int dv, int L, prism_dtype dt);
prism_status prism_bwd_lowmem(const void* q, const void* k, const void* v,
                              const float* g, const float* beta,
                              const void* u, const float* alpha, const void* gamma,
                              const float* conv_w,
                              int B, int H, int T, int dk, int dv, int L, prism_dtype dt,
                              const void* d_o, const float* dS_final,
                              float* dq, float* dk_out, float* dv_out, float* dg, float* dbeta,
                              float* du, float* dalpha, float* dgamma, float* dconv_w,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The same gradients in chunked form on the matrix cores (bfloat16 inputs, dk = dv = 64):
 * the delta rule's UT / WY chunk form (Tencent / PKU article, section 01-三: each chunk
 * processed as blocks of matrix products; PRISM reading notes, sections 2.1-2.3 for the
 * rank-L writes) differentiated chunk by chunk.  Per 64-token chunk one workgroup forms the
 * chunk's operator, its end state from zero and its own adjoint contribution; two scans
 * over the chunks give every chunk its entering state and the adjoint arriving at its end; a second
 * workgroup per chunk forms every gradient from those with bfloat16 MFMA products (float32
 * sums; the unit lower triangular inverse in float32).  The operands are rounded to
 * bfloat16 like the forward's, so the gradients carry the forward's bfloat16 error
 * (a few 1e-3 of each gradient's largest entry), not prism_bwd's float32 one.  Arguments,
 * layouts and outputs as prism_bwd; dt must be PRISM_BF16 and dk = dv = 64 (else
 * PRISM_ERR_UNSUPPORTED), B * H <= 65535.  Deterministic.  Workspace:
 * prism_bwd_chunked_workspace_bytes (per chunk two float32 and 6 + L bfloat16 64 x 64
 * matrices plus 1.75 KiB, per group of four chunks six float32 64 x 64 matrices);
 * ownership, stream and errors as prism_fwd. */
size_t prism_bwd_chunked_workspace_bytes(int B, int H, int T, int dk, int dv, int L, prism_dtype dt);
prism_status prism_bwd_chunked(const void* q, const void* k, const void* v,
                               const float* g, const float* beta,
                               const void* u, const float* alpha, const void* gamma,
                               const float* conv_w,
                               int B, int H, int T, int dk, int dv, int L, prism_dtype dt,
                               const void* d_o, const float* dS_final,
                               float* dq, float* dk_out, float* dv_out, float* dg, float* dbeta,
                               float* du, float* dalpha, float* dgamma, float* dconv_w,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Nonlinear residual refinement.  PRISM's refinement layers subtract a GELU of the
 * gain-modulated residual ("PRISM" reading notes, section 2.3: greedy residual
 * subtraction, gains p from a predictor on the anchor):
 *   r_{t,l} = r_{t,l-1} - alpha_{t,l-1} * GELU(p_{t,l-1} * r_{t,l-1})   (exact erf GELU)
 * in place of the linear chain above; everything else is unchanged.  Because
 * GELU(z) = z Phi(z), this is the linear chain with gamma_{t,l} = p_{t,l} Phi(p_{t,l} r_{t,l})
 * evaluated on the chain's own residuals: the GELU folded into per-channel scaling factors
 * (Tencent Ads article, section 03-三).
 *
 * prism_nl_gain writes those factors: gamma [B, H, T, L-1, dv] (dtype dt, the layout of the
 * gamma argument above) from
 *   v [B, H, T, dv] dt;  alpha [B, H, T, L] float32;  p [B, H, T, L-1, dv] dt (slot j holds
 *   p_{t,j});  conv_w [H, 4, dv] float32;  conv_in [B, H, 3, dv] dt or NULL (as in
 *   prism_fwd_state: the values of the three tokens before the first one).
 * Each factor is rounded to dt before the chain continues with it, as the forward uses it.
 * Phi is evaluated with the erfc approximation of Abramowitz and Stegun, formula 7.1.26
 * (absolute error below 1.5e-7).
 * Feeding the factors to prism_fwd, prism_fwd_state or prism_decode_step (with the same
 * conv_in / conv_state) runs the nonlinear variant in every mode.  For L == 1 there are
 * no factors: nothing is enqueued and the pointers may be NULL.  Supported dv in
 * {16, 32, 64, 128} and B * H <= 65535 (as the forward); no workspace; gamma must not
 * alias an input.  Errors as prism_fwd. */
prism_status prism_nl_gain(const void* v, const float* alpha, const void* p, const float* conv_w,
                           const void* conv_in, int B, int H, int T, int dv, int L, prism_dtype dt,
                           void* gamma, hipStream_t stream);

/* The nonlinear-refinement forward in one call: prism_nl_gain into the front of the
 * workspace, then prism_fwd with those factors.  On the bfloat16 dk = dv = 64 and
 * dk = dv = 128, chunk 64 paths the sweep evaluates the same rounded factors in its own
 * residual chain instead (no factor pass; identical results).  Arguments as prism_fwd with the gains p in place
 * of gamma (p may be NULL when L == 1).  Workspace: prism_fwd_nl_workspace_bytes (room for
 * the factors, 256-byte aligned, plus prism_fwd_workspace_bytes). */
size_t prism_fwd_nl_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk,
                                    prism_dtype dt);
prism_status prism_fwd_nl(const void* q, const void* k, const void* v,
                          const float* g, const float* beta,
                          const void* u, const float* alpha, const void* p,
                          const float* conv_w,
                          int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                          void* o, float* S_final,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Gains from a linear predictor on the anchor, fused with the factor pass ("PRISM" reading
 * notes, section 2.3: predictors read the ShortConv anchor and emit each layer's gain):
 *   p_{t,l} = W_p[h, l] anchor_t,   W_p [H, L-1, dv, dv] bfloat16 in the (out, in) layout,
 * then the factors of prism_nl_gain from those gains.  The gains are formed on MFMA from the
 * anchor rounded to bfloat16 (float32 sums) and never written.  Other arguments as
 * prism_nl_gain.  Supported: dt = PRISM_BF16, dv in {32, 64, 128}, B * H <= 65535.  For
 * L == 1 nothing is enqueued and the pointers may be NULL. */
prism_status prism_nl_gain_pred(const void* v, const float* alpha, const void* W_p, const float* conv_w,
                                const void* conv_in, int B, int H, int T, int dv, int L, prism_dtype dt,
                                void* gamma, hipStream_t stream);

/* The nonlinear-refinement forward with predicted gains in one call: prism_nl_gain_pred into
 * the front of the workspace, then prism_fwd.  Arguments as prism_fwd with the predictor
 * weights W_p in place of gamma (NULL allowed when L == 1).  Workspace:
 * prism_fwd_nl_workspace_bytes.  Supported as prism_nl_gain_pred when L > 1. */
prism_status prism_fwd_nl_pred(const void* q, const void* k, const void* v,
                               const float* g, const float* beta,
                               const void* u, const float* alpha, const void* W_p,
                               const float* conv_w,
                               int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                               void* o, float* S_final,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The written-correction form of the refinement ("PRISM" reading notes, section 2.2: rank
 * accumulation, every refinement layer adds its correction along its own basis with its own
 * gate; section 2.3: greedy residual subtraction, the correction is a GELU of the
 * gain-modulated residual and is subtracted from the residual as it is).  With the GDN
 * forgetting and the GDN write of prism_fwd as the first component:
 *   r_{t,0}     = v_t - anchor_t
 *   delta_{t,l} = GELU(p_{t,l-1} * r_{t,l-1}),   r_{t,l} = r_{t,l-1} - delta_{t,l},  l = 1..L-1
 *   B_t         = beta_t v_t k_t^T + sum_{l=1}^{L-1} alpha_{t,l} delta_{t,l} u_{t,l}^T
 * alpha_{t,l} is layer l's gate (alpha_{t,0} is not read); p [B, H, T, L-1, dv] (dtype dt,
 * slot j holds p_{t,j}) takes gamma's place.  The exact erf GELU, as prism_nl_gain.
 *
 * prism_delta_gain writes the corrections' per-channel factors f = p Phi(p r) along this
 * chain (delta = f r), gamma's layout, each rounded to dt before the chain continues with it
 * (r <- r - f r); no alpha.  conv_in as prism_nl_gain.  For L == 1 nothing is enqueued.
 *
 * prism_fwd_delta runs that factor pass into the front of the workspace, then the forward
 * with the written-correction chain (on the bfloat16 d = 64, chunk 64 path its own sweep
 * instantiation).  Arguments as prism_fwd with p in gamma's place; workspace
 * prism_fwd_delta_workspace_bytes.  prism_fwd_delta_seg: the same with an explicit segment
 * length in chunks (as prism_fwd_seg).  Supported shapes as prism_fwd. */
prism_status prism_delta_gain(const void* v, const void* p, const float* conv_w, const void* conv_in,
                              int B, int H, int T, int dv, int L, prism_dtype dt, void* gamma,
                              hipStream_t stream);
size_t prism_fwd_delta_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk,
                                       prism_dtype dt);
prism_status prism_fwd_delta(const void* q, const void* k, const void* v,
                             const float* g, const float* beta,
                             const void* u, const float* alpha, const void* p,
                             const float* conv_w,
                             int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                             void* o, float* S_final,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);
size_t prism_fwd_delta_seg_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk,
                                           prism_dtype dt, int seg_chunks);
prism_status prism_fwd_delta_seg(const void* q, const void* k, const void* v,
                                 const float* g, const float* beta,
                                 const void* u, const float* alpha, const void* p,
                                 const float* conv_w,
                                 int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                                 void* o, float* S_final,
                                 void* workspace, size_t workspace_bytes, int seg_chunks,
                                 hipStream_t stream);

/* The predictor front end of the written-correction form ("PRISM" reading notes, section
 * 2.3, Phase 1: predictors on the ShortConv anchor emit each layer's gain, basis and gate):
 *   p_{t,l}     = W_p[h, l] anchor_t                            l = 0..L-2 (never written)
 *   u_{t,l+1}   = W_k[h, l] anchor_t / |W_k[h, l] anchor_t|     l = 0..L-2 (unit keys)
 *   alpha_{t,l} = sigmoid(W_b[h, l] . anchor_t)                 l = 0..L-1 (gates)
 * and the correction factors of prism_delta_gain from those gains, in one pass on MFMA
 * (the anchor rounded to bfloat16 as the A operand, float32 sums).
 *   W_p [H, L-1, dv, dv], W_k [H, L-1, dk, dv] ((out, in) layouts), W_b [H, L, dv]: bfloat16
 *   outputs gamma [B, H, T, L-1, dv] and u [B, H, T, L-1, dk] bfloat16, alpha [B, H, T, L]
 *   float32 (the layouts prism_fwd reads).
 * Supported: dt = PRISM_BF16, dk == dv in {32, 64, 128}, 2 <= L <= 8, B * H <= 65535.
 *
 * prism_fwd_delta_pred: the front end into the workspace, then the written-correction
 * forward with the predicted keys, gates and factors; q, k, v, g, beta and conv_w as
 * prism_fwd.  Workspace: prism_fwd_delta_pred_workspace_bytes.  Supported as
 * prism_anchor_predict. */
prism_status prism_anchor_predict(const void* v, const float* conv_w, const void* W_p, const void* W_k,
                                  const void* W_b, const void* conv_in,
                                  int B, int H, int T, int dk, int dv, int L, prism_dtype dt,
                                  void* gamma, void* u, float* alpha, hipStream_t stream);
size_t prism_fwd_delta_pred_workspace_bytes(int B, int H, int T, int dk, int dv, int L, int chunk,
                                            prism_dtype dt);
prism_status prism_fwd_delta_pred(const void* q, const void* k, const void* v,
                                  const float* g, const float* beta,
                                  const void* W_p, const void* W_k, const void* W_b,
                                  const float* conv_w,
                                  int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                                  void* o, float* S_final,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): prism_fwd without the
 * workspace arguments.  Its workspace is a static device array of
 * PRISM_NOALLOC_SCRATCH_BYTES bytes inside the library, one copy per GPU, held until the
 * process ends; the call allocates nothing (the first call on a device looks up that
 * device's copy).  Shapes whose prism_fwd_workspace_bytes exceed the array return
 * PRISM_ERR_WORKSPACE before anything is enqueued (the 16K workload, B = 2, H = 4,
 * T = 16384, d = 64, L = 4 in bfloat16, needs about 44 MB).  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other threads) race and
 * must be serialised by the caller.  Arguments, results and other errors as prism_fwd. */
#define PRISM_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t prism_noalloc_scratch_bytes(void);
prism_status prism_fwd_noalloc(const void* q, const void* k, const void* v,
                               const float* g, const float* beta,
                               const void* u, const float* alpha, const void* gamma,
                               const float* conv_w,
                               int B, int H, int T, int dk, int dv, int L, int chunk, prism_dtype dt,
                               void* o, float* S_final, hipStream_t stream);

/* A static, human-readable name of a status code. */
const char* prism_status_string(prism_status s);

/* Library version string ("major.minor.patch"). */
const char* prism_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PRISM_H_ */
