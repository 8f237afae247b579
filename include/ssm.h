/*
 * ssm.h - C ABI of the MI355X (gfx950) selective-scan library (libssm.so).
 *
 * The library computes the Mamba-1 selective state-space layer (S6): the
 * full forward scan over a sequence and the single-token recurrent decode
 * step, with hand-written HIP kernels. Definitions, in the pages' notation
 * (Delta = delta, B_t = Bt, C_t = Ct, D = Dskip):
 *
 *   dA[t,n]  = exp(delta[t] * A[n])            (A-bar, exponential rule)
 *   dBx[t,n] = delta[t] * Bt[t,n] * x[t]       (B-bar = Delta * B_t)
 *   h[t,n]   = dA[t,n] * h[t-1,n] + dBx[t,n]   (h[-1] = carried-in state or 0)
 *   y[t]     = (sum_n Ct[t,n] * h[t,n] + Dskip * x[t]) * silu(z[t])
 *   silu(z)  = z / (1 + exp(-z))
 *
 * per (batch row b, channel d). Sources: "Notas sobre Mamba"
 * (rodolfoviana.com.br), sections "Preliminares" (discretisation and the
 * first-order input rule B-bar = Delta*B), "O mecanismo de seleção (S6)"
 * (input-dependent B_t, C_t, Delta_t and the time-varying recurrence),
 * "A varredura paralela ciente do hardware" (the recurrence as an
 * associative scan over (A-bar_t, B-bar_t x_t) pairs, kept on chip, only y
 * written back), "O bloco Mamba" (the silu(z) gate); the blog post "Mamba-2
 * e State Space Duality (SSD)" (produtoramaxvision.com.br), section "Como o
 * Mamba-1 alcançou complexidade linear" (the S6 equations with the D skip and
 * the one-token forward_step on a stored state).
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers (hipMalloc'd or equivalent), owned by the
 *    caller. The library allocates nothing and may be called from several
 *    host threads; its only state is, per device, the CU count and resident
 *    workgroups of each kernel, queried once. What a scan needs from one call
 *    to the next lives in the caller's workspace.
 *  - Tensors are dense, row-major, in the shapes listed; D (channels) is the
 *    fastest axis of x, delta, z and y; N is the fastest axis of Bt, Ct, A
 *    and the state. Every base pointer must be 16-byte aligned.
 *  - dtype selects the storage type of the activations x, delta, z, Bt, Ct
 *    and y: SSM_F32 (float) or SSM_BF16 (bfloat16). A, Dskip and the state
 *    are always float. All arithmetic is float32; bfloat16 outputs are
 *    rounded to nearest even.
 *  - N (state size) must be 1, 2, 4, 8 or 16.
 *  - delta is the step AFTER the softplus (the pages apply softplus to a
 *    projection plus bias before the scan). The *_dt entry points take the
 *    step before it and apply softplus(delta_raw + dt_bias) themselves.
 *  - x is the scan's input itself; ssm_scan_fwd_conv and ssm_step_conv take
 *    it one step earlier, before the short causal convolution and SiLU of the
 *    block's x branch, and apply both themselves.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronise the host. Arguments are checked on the
 *    host before any HIP call; a failed check returns a negative status and
 *    launches nothing. SSM_ERR_HIP reports a failed launch; faults inside a
 *    kernel surface at the caller's next synchronisation.
 *  - NaN or Inf inputs are not special-cased and propagate.
 */
#ifndef SSM_H
#define SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Activation storage types. */
#define SSM_F32 0
#define SSM_BF16 1

/* Status codes. */
#define SSM_OK 0
#define SSM_ERR_NULL (-1)        /* a required pointer is NULL */
#define SSM_ERR_SHAPE (-2)       /* a size is negative or the tensor sizes overflow */
#define SSM_ERR_DTYPE (-3)       /* dtype is neither SSM_F32 nor SSM_BF16 */
#define SSM_ERR_UNSUPPORTED (-4) /* N is not 1, 2, 4, 8 or 16 */
#define SSM_ERR_ALIGN (-5)       /* a pointer is not 16-byte aligned */
#define SSM_ERR_WORKSPACE (-6)   /* workspace is NULL or smaller than required */
#define SSM_ERR_HIP (-7)         /* a HIP launch or device query failed */
#define SSM_ERR_TIMEOUT (-8)     /* reported by ssm_scan_workspace_status only: a wait of the
                                    last scan for another workgroup's results gave up */

/* Human-readable text for a status code (static storage, never NULL). */
const char *ssm_status_string(int status);

/* Library version string (static storage). */
const char *ssm_version(void);

/*
 * Scratch bytes ssm_scan_fwd needs for these sizes (0 when none). The
 * workspace holds the counters that hand work to the workgroups and, when a
 * sequence is cut into stripes scanned at the same time, each stripe's
 * summary (its end state from a zero start and its summed delta) and its end
 * state for the stripes after it, as words tagged with the call.
 *
 * The workspace must be zero-filled before its first use. After that it may
 * be reused by later calls of any size without clearing, as long as nothing
 * else writes to it in between. Its first 256 bytes are a header that the
 * kernels keep: a call reads the tag of the last finished call there, marks
 * its own words with the next value, and its last workgroup stores that value
 * back and leaves the unit counters at zero. The tag is therefore taken on the
 * device when the call runs, so a scan captured into a HIP graph may be
 * replayed any number of times, also between eager calls on the same
 * workspace.
 *
 * Order of work on long stripes (16384 tokens or more): every stripe but the
 * first scans from a zero start first, writing y, and after its entering
 * state is known walks again only until that state, decayed by exp(A * summed
 * delta), is below 2^-24 (float32 outputs, their unit roundoff) or 2^-16
 * (bfloat16 outputs, 1/256 of theirs) times every lane's largest state
 * ("Notas sobre Mamba", section "O mecanismo de seleção (S6)": the
 * recurrence is linear in the state). The stop is decided on the data only,
 * so results stay bitwise reproducible; it
 * is never taken where A > 0, delta < 0 or the entering state is not finite.
 * The environment variable SSM_STRIPE_EARLY=0 or 1, read at each call, forces
 * the two-pass order or this one (for comparison and tests).
 * Calls that share a workspace must not run at the same time (on the same
 * stream, or ordered by events).
 * Returns 0 for invalid sizes.
 */
size_t ssm_scan_workspace_bytes(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype);

/*
 * Outcome of the last ssm_scan_fwd* call that used `workspace`: waits for
 * `stream` (a hipStream_t; NULL = the null stream) to finish, then reads the
 * workspace header. When a sequence is cut into stripes scanned at the same
 * time, a stripe waits for the records of the stripes before it; that wait
 * is bounded (about 4 million polls). A wait that gives up leaves the stripe's
 * carried-in state NaN, so its y and final state, and those of every later
 * stripe of its channels, come out NaN; it also marks the header, and every
 * other wait of the same call then gives up at once. This function reports
 * that as SSM_ERR_TIMEOUT (otherwise SSM_OK, also for a workspace no scan has
 * used yet, or NULL). A timeout means the stripes could not all make progress,
 * for instance because two calls shared the workspace at the same time. The
 * next call on the workspace starts afresh. SSM_ERR_HIP: the copy or the
 * synchronisation failed; SSM_ERR_ALIGN: workspace not 16-byte aligned.
 */
int ssm_scan_workspace_status(const void *workspace, size_t workspace_bytes, void *stream);

/*
 * Selective scan forward over L tokens.
 *
 *   x, delta      (batch, L, D)  dtype      input and step (post-softplus)
 *   A             (D, N)         float      diagonal state matrix (negative)
 *   Bt, Ct        (batch, L, N)  dtype      per-token input / output vectors,
 *                                           shared by all D channels
 *   Dskip         (D)            float      skip weight; NULL = no skip term
 *   z             (batch, L, D)  dtype      gate input; NULL = no gate
 *   state_in      (batch, D, N)  float      carried-in state; NULL = zeros
 *   state_out     (batch, D, N)  float      state after token L-1; NULL = not
 *                                           written; may equal state_in
 *   y             (batch, L, D)  dtype      output (written)
 *   workspace     ssm_scan_workspace_bytes() bytes of device memory, or NULL
 *                 when that size is 0
 *
 * y must not overlap any input. batch, L or D equal to 0 is valid: nothing is
 * computed, except that state_out (if given) receives state_in or zeros when
 * L is 0. The (batch, L, D, N) expanded state is never written to memory.
 */
int ssm_scan_fwd(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                 const void *x, const void *delta, const float *A,
                 const void *Bt, const void *Ct, const float *Dskip,
                 const void *z, const float *state_in, float *state_out,
                 void *y, void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssm_scan_fwd for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc. It takes no workspace: the scan's workspace is a static device
 * array of 12 MiB inside the library, one per GPU, held until the process
 * ends. It covers every shape the tiled scan takes (its workspace is at most
 * 9 MiB); a shape that needs more (the chunked scan of large inputs whose
 * channel or Bt/Ct rows are not whole 16-byte pieces) returns
 * SSM_ERR_WORKSPACE and launches nothing. The entry point calls no hipMalloc,
 * hipFree or other allocating routine.
 *
 * Arguments, checks and status codes are those of ssm_scan_fwd without the
 * workspace. The first call on a device looks the array up and clears it with
 * a kernel on `stream`. Every call on a GPU shares that GPU's array: calls
 * that overlap in time on one GPU (other streams, other host threads) race
 * and must not be made. There is no status query for the array: a wait that
 * gives up is seen only as NaN in the outputs that depend on it.
 */
int ssm_scan_fwd_noalloc(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                         const void *x, const void *delta, const float *A,
                         const void *Bt, const void *Ct, const float *Dskip,
                         const void *z, const float *state_in, float *state_out,
                         void *y, void *stream);

/*
 * ssm_scan_fwd with the step size given before its activation: the scan uses
 * delta = softplus(delta_raw + dt_bias[d]), softplus(u) = log(1 + exp(u)).
 * The pages make the step size the softplus of a projection of the input plus
 * a bias ("Notas sobre Mamba", section "O mecanismo de seleção (S6)");
 * delta_raw is that projection, computed upstream, and dt_bias the bias.
 *
 *   delta_raw     (batch, L, D)  dtype      step size before the activation
 *   dt_bias       (D)            float      per-channel bias; NULL = zero
 *
 * Every other argument, the workspace and the status codes are those of
 * ssm_scan_fwd. The activation is computed in float32 once per (token,
 * channel). For bfloat16 activations the result is held as bfloat16 (round
 * to nearest even), the precision of a delta handed over already activated.
 */
int ssm_scan_fwd_dt(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                    const void *x, const void *delta_raw, const float *dt_bias, const float *A,
                    const void *Bt, const void *Ct, const float *Dskip,
                    const void *z, const float *state_in, float *state_out,
                    void *y, void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssm_scan_fwd_dt behind the x branch of the Mamba block: the scan's x is
 * SiLU of a short causal convolution of x_raw along the tokens, separately
 * per channel ("Notas sobre Mamba", section "O bloco Mamba": projection,
 * short depthwise convolution, SiLU, then S6; the Mamba-2 layer
 * configuration on "Mamba-2 e State Space Duality (SSD)" gives its width,
 * 4). Per (b, t, d):
 *
 *   u      = conv_b[d] + sum_{j=0..3} conv_w[d,j] * x_raw[b, t-3+j, d]
 *   x[t]   = u / (1 + exp(-u))                                   (SiLU)
 *
 * where a token before token 0 takes its raw x from conv_state. That x feeds
 * the input term and the D skip; the step size is softplus(delta_raw +
 * dt_bias) as in ssm_scan_fwd_dt.
 *
 *   x_raw         (batch, L, D)  dtype      the convolution's input
 *   conv_w        (D, 4)         float      taps; conv_w[d,3] multiplies the
 *                                           token itself, conv_w[d,0] the
 *                                           token three before it (the
 *                                           layout of a depthwise Conv1d
 *                                           weight (D, 1, 4) with left
 *                                           padding 3)
 *   conv_b        (D)            float      bias; NULL = zero
 *   conv_state    (batch, D, 3)  dtype      raw x of the three tokens before
 *                                           token 0, oldest first (to resume
 *                                           a sequence cut after an earlier
 *                                           call: that call's last three
 *                                           x_raw tokens); NULL = zeros
 *
 * Every other argument, the workspace (ssm_scan_workspace_bytes) and the
 * status codes are those of ssm_scan_fwd_dt; a NULL conv_w with a non-empty
 * input returns SSM_ERR_NULL. The convolution and SiLU are computed in
 * float32 once per (token, channel) and, for bfloat16 activations, held as
 * bfloat16 (round to nearest even) before the scan uses them. The x_raw
 * tokens the next piece of a sequence needs as conv_state are the caller's
 * own input; nothing beyond y and state_out is written.
 */
int ssm_scan_fwd_conv(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                      const void *x_raw, const float *conv_w, const float *conv_b, const void *conv_state,
                      const void *delta_raw, const float *dt_bias, const float *A,
                      const void *Bt, const void *Ct, const float *Dskip,
                      const void *z, const float *state_in, float *state_out,
                      void *y, void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssm_scan_fwd with the exponential-trapezoidal rule of "Notas sobre Mamba",
 * section "Recorrência trapezoidal": the input term blends the previous and
 * the current token's input with a per-token weight lam,
 *
 *   h[t,n] = dA[t,n] * h[t-1,n]
 *            + (1 - lam[t]) * delta[t] * dA[t,n] * Bt[t-1,n] * x[t-1]
 *            + lam[t] * delta[t] * Bt[t,n] * x[t]
 *
 * with dA, the readout, the skip term, the gate and the state as in
 * ssm_scan_fwd. lam = 1 everywhere gives ssm_scan_fwd's result; lam = 1/2 is
 * the classic trapezoidal rule. lam is the weight itself (the pages take it
 * as the sigmoid of a per-token projection, computed upstream).
 *
 *   lam           (batch, L, D)  dtype      weight per token and channel,
 *                                           normally in [0, 1]
 *   x_prev        (batch, D)     dtype      x and Bt of the token before token
 *   B_prev        (batch, N)     dtype      0 (to resume a sequence cut after
 *                                           an earlier call: that call's last
 *                                           token); both NULL = no earlier
 *                                           token (its input term is zero)
 *
 * Passing exactly one of x_prev and B_prev, or a NULL lam with a non-empty
 * input, returns SSM_ERR_NULL. Every other argument, the workspace
 * (ssm_scan_workspace_bytes) and the status codes are those of ssm_scan_fwd.
 * A long sequence may be scanned in pieces: pass each piece the previous
 * piece's state_out as state_in and its last token's x and Bt as x_prev and
 * B_prev.
 */
int ssm_scan_fwd_trap(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                      const void *x, const void *delta, const void *lam, const float *A,
                      const void *Bt, const void *Ct, const float *Dskip, const void *z,
                      const void *x_prev, const void *B_prev, const float *state_in, float *state_out,
                      void *y, void *workspace, size_t workspace_bytes, void *stream);

/*
 * One recurrent decode step for `batch` sequences (one token each), updating
 * the state in place.
 *
 *   x, delta      (batch, D)     dtype
 *   A             (D, N)         float
 *   Bt, Ct        (batch, N)     dtype
 *   Dskip         (D)            float      NULL = no skip term
 *   z             (batch, D)     dtype      NULL = no gate
 *   state         (batch, D, N)  float      read, then overwritten with the
 *                                           new state
 *   y             (batch, D)     dtype      output (written)
 *
 * Equivalent to ssm_scan_fwd with L = 1 and state_in = state_out = state.
 * Uses no workspace and keeps nothing between calls, so a sequence of steps
 * may be captured into a HIP graph and replayed.
 */
int ssm_step(int64_t batch, int64_t D, int64_t N, int dtype,
             const void *x, const void *delta, const float *A,
             const void *Bt, const void *Ct, const float *Dskip,
             const void *z, float *state, void *y, void *stream);

/*
 * ssm_step with the step size given before its activation, as in
 * ssm_scan_fwd_dt: delta = softplus(delta_raw + dt_bias[d]) in float32.
 *
 *   delta_raw     (batch, D)     dtype
 *   dt_bias       (D)            float      NULL = zero
 */
int ssm_step_dt(int64_t batch, int64_t D, int64_t N, int dtype,
                const void *x, const void *delta_raw, const float *dt_bias, const float *A,
                const void *Bt, const void *Ct, const float *Dskip,
                const void *z, float *state, void *y, void *stream);

/*
 * ssm_step_dt behind the x branch of the Mamba block, as in
 * ssm_scan_fwd_conv: x of this token is SiLU of conv_b + the taps times the
 * raw x of the three tokens before it (conv_state) and of this token
 * (x_raw); conv_state is then shifted in place to hold the raw x of the last
 * three tokens, this one last ("Notas sobre Mamba", section "O bloco Mamba";
 * the constant-size state a decode step carries is the scan state plus this
 * window).
 *
 *   x_raw         (batch, D)     dtype      the convolution's input
 *   conv_w        (D, 4)         float      taps (as in ssm_scan_fwd_conv)
 *   conv_b        (D)            float      bias; NULL = zero
 *   conv_state    (batch, D, 3)  dtype      raw x of the three tokens before,
 *                                           oldest first; read, then
 *                                           overwritten with the window that
 *                                           ends with this token
 *
 * Every other argument is that of ssm_step_dt; a NULL conv_w or conv_state
 * with a non-empty input returns SSM_ERR_NULL. T calls on tokens 0..T-1,
 * starting from a scan's conv_state and state_in, give ssm_scan_fwd_conv's y
 * and final state over those tokens.
 */
int ssm_step_conv(int64_t batch, int64_t D, int64_t N, int dtype,
                  const void *x_raw, const float *conv_w, const float *conv_b, void *conv_state,
                  const void *delta_raw, const float *dt_bias, const float *A,
                  const void *Bt, const void *Ct, const float *Dskip,
                  const void *z, float *state, void *y, void *stream);

/*
 * One decode step with the exponential-trapezoidal rule (see
 * ssm_scan_fwd_trap). The state holds h only; the caller passes the previous
 * token's x and Bt (the ones given to the previous step) as x_prev and
 * B_prev, or NULL for both at the first token of a sequence.
 *
 *   lam           (batch, D)     dtype
 *   x_prev        (batch, D)     dtype      NULL = no earlier token
 *   B_prev        (batch, N)     dtype      NULL = no earlier token
 *
 * Equivalent to ssm_scan_fwd_trap with L = 1 and state_in = state_out =
 * state. Arguments and status codes otherwise as in ssm_step.
 */
int ssm_step_trap(int64_t batch, int64_t D, int64_t N, int dtype,
                  const void *x, const void *delta, const void *lam, const float *A,
                  const void *Bt, const void *Ct, const float *Dskip, const void *z,
                  const void *x_prev, const void *B_prev, float *state, void *y, void *stream);

/*
 * Mamba-2 state space dual (SSD) layer: the selective recurrence with the
 * transition restricted to a scalar per head times the identity ("Notas sobre
 * Mamba", section "A forma dual: atenção mascarada"; "Mamba-2 e State Space
 * Duality (SSD)"). Per batch row b and head h, with group g = h / (H / G):
 *
 *   a[t]      = exp(delta[b,t,h] * A[h])
 *   S[p][n]   = a[t] * S[p][n] + delta[b,t,h] * x[b,t,h,p] * Bt[b,t,g,n]
 *   y[b,t,h,p] = sum_n Ct[b,t,g,n] * S[p][n]  (+ Dskip[h] * x[b,t,h,p])
 *
 * computed by chunks of 64 tokens: inside a chunk by the masked (attention-
 * like) dual form on the matrix cores, across chunks through the state
 * (section "O algoritmo SSD").
 *
 *   x, y          (batch, L, H, P)  bfloat16
 *   delta         (batch, L, H)     bfloat16   step after its activation
 *   A             (H)               float      negative scalar per head
 *   Bt, Ct        (batch, L, G, N)  bfloat16   shared by the H / G heads of a group
 *   Dskip         (H)               float      NULL = no skip term
 *   state_in      (batch, H, P, N)  float      NULL = zeros
 *   state_out     (batch, H, P, N)  float      NULL = not written; may equal state_in
 *
 * Supported: dtype SSM_BF16 (float accumulation; the chunk's masked matrix
 * with Dskip on its diagonal, the weighted x and the state copy that meets C
 * are rounded to bfloat16 on the way into the matrix cores), P = 64, N = 64
 * or 128, H < 8192 * 64 and G * N < 2^25 (64 tokens of x and of Bt, Ct
 * within 4 GiB); anything else returns SSM_ERR_UNSUPPORTED. H must be a
 * multiple of G (else SSM_ERR_SHAPE). Uses no
 * workspace and keeps nothing between calls. Conventions otherwise as above.
 */
int ssm_ssd_fwd(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int dtype,
                const void *x, const void *delta, const float *A, const void *Bt, const void *Ct,
                const float *Dskip, const float *state_in, float *state_out, void *y, void *stream);

/*
 * Mamba-2 SSD decode step: one token per (batch row, head) on a stored state,
 * updated in place, with the same transition, input rule and readout as
 * ssm_ssd_fwd (its recurrent form, "A forma dual: atenção mascarada"):
 *
 *   a          = exp(delta[b,h] * A[h])
 *   S[p][n]    = a * S[p][n] + delta[b,h] * x[b,h,p] * Bt[b,g,n]
 *   y[b,h,p]   = sum_n Ct[b,g,n] * S[p][n]  (+ Dskip[h] * x[b,h,p])
 *
 * with g = h / (H / G). L calls, one per token, equal one ssm_ssd_fwd call
 * over the L tokens (up to rounding).
 *
 *   x, y          (batch, H, P)     dtype
 *   delta         (batch, H)        dtype      step after its activation
 *   A, Dskip      (H)               float      Dskip NULL = no skip term
 *   Bt, Ct        (batch, G, N)     dtype
 *   state         (batch, H, P, N)  float      read and written in place
 *
 * Supported: P = 64 and N = 64 or 128, dtype SSM_F32 or SSM_BF16 (else
 * SSM_ERR_UNSUPPORTED or SSM_ERR_DTYPE); H must be a multiple of G (else
 * SSM_ERR_SHAPE). No workspace. Conventions otherwise as above.
 */
int ssm_ssd_step(int64_t batch, int64_t H, int64_t P, int64_t G, int64_t N, int dtype,
                 const void *x, const void *delta, const float *A, const void *Bt, const void *Ct,
                 const float *Dskip, float *state, void *y, void *stream);

/*
 * Scratch bytes ssm_scan_bwd, ssm_scan_bwd_dt and ssm_scan_bwd_trap need for
 * these sizes (0 for empty or invalid sizes). The gradient cuts the sequence
 * into chunks of 32 tokens; the workspace holds, per (batch row, chunk,
 * channel), the state and the gradient entering the chunk, the chunk's summed
 * delta and the states at its three inner 8-token block entries, and the
 * partial sums of dBt, dCt and dB_prev (per block of 64 to 256 channels) and
 * of dA, dDskip and ddt_bias (per chunk): about 0.75 bytes per (b, t, d, n)
 * element in all. It
 * needs no clearing: every word is written before it is read within one call.
 * Calls that share a workspace must not run at the same time.
 */
size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype);

/*
 * Gradient of ssm_scan_fwd (the Euler rule, delta given after its activation)
 * for the loss sum(dy * y) + sum(dstate * state_out). The pages give the
 * forward recurrence and recompute its states in the backward pass instead of
 * storing them ("Notas sobre Mamba", section "A varredura paralela ciente do
 * hardware"); the gradient is the chain rule through that recurrence. With
 * dA_t = exp(delta_t A) and s_t = silu(z_t) (1 without a gate), the gradient
 * of the state runs backwards,
 *
 *   G_t = Ct[t] * dy_t s_t + dA_{t+1} * G_{t+1},      G_{L-1} includes dstate,
 *
 * and every input's gradient follows from G and the recomputed states.
 *
 *   x, delta, A, Bt, Ct, Dskip, z, state_in   as passed to ssm_scan_fwd
 *   dy            (batch, L, D)  dtype      gradient of y
 *   dstate        (batch, D, N)  float      gradient of state_out; NULL = zeros
 *   dx, ddelta    (batch, L, D)  dtype      written
 *   dA            (D, N)         float      written (summed over batch and tokens)
 *   dBt, dCt      (batch, L, N)  float      written (summed over channels)
 *   dDskip        (D)            float      written when Dskip and dDskip are
 *                                           both given; NULL = not written
 *   dz            (batch, L, D)  dtype      written; required when z is given
 *   dstate_in     (batch, D, N)  float      gradient of state_in (of the zero
 *                                           start when state_in is NULL);
 *                                           NULL = not written; may equal dstate
 *   workspace     ssm_scan_bwd_workspace_bytes() bytes of device memory
 *
 * Every sum runs in a fixed order, so equal inputs give equal bits. L = 0 or
 * batch = 0 writes zeros to dA (and dDskip) and copies dstate to dstate_in.
 * Status codes as in ssm_scan_fwd; a missing required output is SSM_ERR_NULL.
 */
int ssm_scan_bwd(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                 const void *x, const void *delta, const float *A, const void *Bt, const void *Ct,
                 const float *Dskip, const void *z, const float *state_in,
                 const void *dy, const float *dstate,
                 void *dx, void *ddelta, float *dA, float *dBt, float *dCt, float *dDskip, void *dz,
                 float *dstate_in, void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssm_scan_bwd for ssm_scan_fwd_dt: the step size is given before its
 * activation, delta = softplus(delta_raw + dt_bias[d]). The gradient of the
 * raw step size is that of delta times sigmoid(delta_raw + dt_bias), the
 * derivative of softplus; the gradient of dt_bias sums it over batch and
 * tokens. For bfloat16 activations the forward rounds the activated step to
 * bfloat16; the gradient takes that rounding as the identity.
 *
 *   delta_raw     (batch, L, D)  dtype      step size before its activation
 *   dt_bias       (D)            float      NULL = zero bias
 *   ddelta_raw    (batch, L, D)  dtype      written
 *   ddt_bias      (D)            float      written; NULL = not written
 *
 * Every other argument, the workspace (ssm_scan_bwd_workspace_bytes) and the
 * status codes are those of ssm_scan_bwd.
 */
int ssm_scan_bwd_dt(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                    const void *x, const void *delta_raw, const float *dt_bias, const float *A,
                    const void *Bt, const void *Ct, const float *Dskip, const void *z, const float *state_in,
                    const void *dy, const float *dstate,
                    void *dx, void *ddelta_raw, float *ddt_bias, float *dA, float *dBt, float *dCt,
                    float *dDskip, void *dz, float *dstate_in, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * Scratch bytes ssm_scan_bwd_conv needs for these sizes (0 for invalid or
 * empty sizes): ssm_scan_bwd's, then the branch's output and its gradient
 * (two (batch, L, D) arrays of the activation dtype) and the partial sums of
 * the taps' and bias' gradients. No clearing is needed.
 */
size_t ssm_scan_bwd_conv_workspace_bytes(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype);

/*
 * ssm_scan_bwd for ssm_scan_fwd_conv: the gradient through the scan, then back
 * through SiLU and the causal width-4 convolution of the x branch ("Notas
 * sobre Mamba", section "O bloco Mamba"; the pages give the forward only, and
 * this is its chain rule). With u and x as in ssm_scan_fwd_conv and dx the
 * gradient of the scan's x,
 *
 *   du[t]          = dx[t] * s(u[t]) * (1 + u[t] * (1 - s(u[t]))),  s = sigmoid
 *   dx_raw[t]      = sum_j conv_w[d,j] * du[t+3-j]           (tokens < L)
 *   dconv_w[d,j]   = sum_{b,t} du[t] * x_raw[t-3+j]           (conv_state before 0)
 *   dconv_b[d]     = sum_{b,t} du[t]
 *   dconv_state[b,d,k] = sum_{j<=k} conv_w[d,j] * du[k-j]     (the raw x of token k-3)
 *
 * The forward rounds x to the activation dtype; the gradient takes that
 * rounding as the identity, as it does for the activated step size.
 *
 *   x_raw, conv_w, conv_b, conv_state, delta_raw, dt_bias   as passed to
 *                                           ssm_scan_fwd_conv
 *   dx_raw        (batch, L, D)  dtype      written
 *   dconv_w       (D, 4)         float      written
 *   dconv_b       (D)            float      written when conv_b is given
 *   dconv_state   (batch, D, 3)  dtype      written; NULL = not written
 *   ddelta_raw, ddt_bias          as in ssm_scan_bwd_dt
 *   workspace     ssm_scan_bwd_conv_workspace_bytes() bytes
 *
 * Every other argument and the status codes are those of ssm_scan_bwd_dt; a
 * NULL conv_w or dconv_w returns SSM_ERR_NULL. All sums over tokens and
 * channels run in a fixed order: the result is bitwise reproducible.
 */
int ssm_scan_bwd_conv(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                      const void *x_raw, const float *conv_w, const float *conv_b, const void *conv_state,
                      const void *delta_raw, const float *dt_bias, const float *A,
                      const void *Bt, const void *Ct, const float *Dskip, const void *z, const float *state_in,
                      const void *dy, const float *dstate,
                      void *dx_raw, float *dconv_w, float *dconv_b, void *dconv_state,
                      void *ddelta_raw, float *ddt_bias, float *dA, float *dBt, float *dCt,
                      float *dDskip, void *dz, float *dstate_in, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * ssm_scan_bwd for ssm_scan_fwd_trap: the gradient of the exponential-
 * trapezoidal rule ("Notas sobre Mamba", section "Recorrência trapezoidal").
 * With v_t = Bt[t] x_t, the state's gradient G_t runs back as in ssm_scan_bwd
 * (each token's update multiplies the state by dA_t in both rules); v_t enters
 * h_t with weight lam_t delta_t and h_{t+1} with (1 - lam_{t+1}) delta_{t+1}
 * dA_{t+1}, and its gradient collects both. lam's gradient is
 * delta_t sum_n G_t (v_t - dA_t v_{t-1}).
 *
 *   lam, x_prev, B_prev   as passed to ssm_scan_fwd_trap
 *   dlam          (batch, L, D)  dtype      written
 *   dx_prev       (batch, D)     dtype      gradient of x_prev   } written when
 *   dB_prev       (batch, N)     float      gradient of B_prev   } x_prev, B_prev,
 *                                           (summed over channels) both given
 *
 * Passing exactly one of x_prev and B_prev, or of dx_prev and dB_prev, or a
 * NULL lam with a non-empty input, returns SSM_ERR_NULL; L = 0 leaves dx_prev
 * and dB_prev unwritten. Every other argument, the workspace
 * (ssm_scan_bwd_workspace_bytes) and the status codes are those of
 * ssm_scan_bwd.
 */
int ssm_scan_bwd_trap(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                      const void *x, const void *delta, const void *lam, const float *A,
                      const void *Bt, const void *Ct, const float *Dskip, const void *z,
                      const void *x_prev, const void *B_prev, const float *state_in,
                      const void *dy, const float *dstate,
                      void *dx, void *ddelta, void *dlam, float *dA, float *dBt, float *dCt, float *dDskip, void *dz,
                      void *dx_prev, float *dB_prev, float *dstate_in, void *workspace, size_t workspace_bytes,
                      void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H */
