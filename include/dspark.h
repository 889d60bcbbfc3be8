/*
 * dspark.h — C ABI of the DSpark draft-and-verify round on MI355X (gfx950).
 *
 * DSpark (arXiv:2607.05147) drafts a gamma-token block with a parallel
 * backbone plus a light sequential head, scores every drafted position with
 * a confidence head, lets a hardware-aware scheduler decide how many drafts
 * of each request the target model verifies this round, and verifies them by
 * lossless rejection sampling.  This library implements the four steps that
 * sit between the backbone and the target model, as HIP kernels:
 *
 *   dspark_markov_sample  the sequential Markov-head sampling loop
 *   dspark_markov_sample_ex  the same, with the confidence head, a cancel
 *                         word and a device status word
 *   dspark_rnn_sample     the same loop with the RNN head
 *   dspark_confidence     the confidence head (linear + sigmoid, temperature)
 *   dspark_schedule       the batched prefix scheduler (Algorithm 1)
 *   dspark_schedule_ex    the same with the production admission rules
 *   dspark_schedule_noalloc  the same without a workspace (static scratch)
 *   dspark_verify         rejection-sampling verification + residual draw
 *   dspark_verify_ex      the same with the RNN head's bias vectors
 *   dspark_verify_greedy  temperature-0 (exact-match) verification
 *   dspark_acceptance     the analytic acceptance sum_v min(p_d, p_t) per position
 *   dspark_sts_fit        sequential temperature scaling with ECE and AUC
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers to row-major arrays, 16-byte
 *     aligned, on the device that is current when the call is made.  The
 *     caller owns every buffer; the library never allocates, frees or
 *     synchronises, and never reads device data on the host.
 *   - Inputs are const and are never written.  Outputs are fully
 *     overwritten.  Inputs and outputs must not alias.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and is safe to capture into a HIP graph: no
 *     allocation, no memset node, no host synchronisation.
 *   - Host-checkable preconditions (sizes, null pointers, workspace size,
 *     data type) are checked before anything is enqueued; a failed check
 *     returns an error code and enqueues nothing.  A failed launch returns
 *     DSPARK_ELAUNCH.  Conditions on device data (token ranges, confidences
 *     in [0,1], a positive non-increasing step-speed table) are the caller's
 *     obligations and are not checked.
 *   - No call keeps state between calls.  Calls on different streams with
 *     different workspaces may run concurrently, with one exception: with
 *     bf16 storage, dspark_markov_sample(_ex), and dspark_rnn_sample at the
 *     shapes where it keeps W2t on chip (dspark_rnn_sample_kernel), run all
 *     gamma positions in one persistent launch whose work groups (one per
 *     compute unit) meet at grid barriers between positions, so they need
 *     every compute unit of the device at once.  Do not overlap them with
 *     other work on the device (the library cannot see or serialise the
 *     caller's streams).  If the grid is not resident as a whole, the barrier
 *     gives up after 0.5 s instead of hanging: every x is then -1 and every
 *     lse and logit NaN (s and o of dspark_rnn_sample are then undefined),
 *     and the status word of dspark_markov_sample_ex reads DSPARK_ETIMEOUT.
 *   - dt selects the storage type of the large tensors (U, W1, W2, w, h,
 *     target): fp32 or bf16.  Arithmetic is fp32 (scheduler: fp64 and exact
 *     integers).  Random draws are inputs, drawn by the caller.
 *
 * Citations name the reading notes of the paper at zhongzhuzhou.org ("notes"),
 * the summary at caijizhuo.github.io ("caijizhuo") and the chapter at
 * llm-infra-atlas.github.io ("atlas").
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSPARK_OK = 0,
  DSPARK_EINVAL = 1,      /* a size or pointer argument is invalid            */
  DSPARK_EDTYPE = 2,      /* unsupported data type for this call / shape       */
  DSPARK_EWORKSPACE = 3,  /* workspace missing or smaller than required        */
  DSPARK_ELAUNCH = 4,     /* a kernel launch failed                            */
  DSPARK_EDEVICE = 5,     /* the current device is not a gfx950 GPU            */
  DSPARK_ETIMEOUT = 6     /* device status only: the sampler's grid barrier
                             gave up (time-out or cancel); no valid draw        */
} dspark_status;

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

/* Tokens per chunk of the two-level Gumbel draw; the chunk Gumbel tensor G
 * has ceil(V / DSPARK_CHUNK) entries per drafted position and request. */
#define DSPARK_CHUNK 16

/* Workspace selectors for dspark_workspace_size. */
typedef enum {
  DSPARK_WS_SAMPLE = 0,
  DSPARK_WS_SCHEDULE = 2,
  DSPARK_WS_VERIFY = 3,
  DSPARK_WS_VERIFY_GREEDY = 4,
  DSPARK_WS_ACCEPTANCE = 5,
  DSPARK_WS_RNN_SAMPLE = 6,
  DSPARK_WS_STS = 7         /* R = rollouts N, V = grid size, r = bins */
} dspark_ws_kind;

/*
 * dspark_markov_sample — the semi-autoregressive gamma-step sampling loop.
 *
 * Passage: notes eq (4) (bias added inside the softmax:
 * p_k(v) ∝ exp(U_k(v) + B_k(v))) and eq (5) (Markov head,
 * B(x_{k-1}, .) = W1[x_{k-1}] W2, rank r); caijizhuo section 四, the
 * sequential loop of dspark_cycle (only the sampled token is carried from
 * position to position).  Position 1 conditions on the anchor x0.
 *
 * The draw at each position is an exact two-level Gumbel-max: the
 * vocabulary is split into chunks of DSPARK_CHUNK (16) consecutive tokens;
 * the chunk is argmax_c (LSE_c + G[c]) where LSE_c is the log-sum-exp of the
 * chunk's logits, and the token is the in-chunk argmax of l_v + g[v mod 16].
 * Ties go to the lower token (up to fp32 rounding of the chunk scores).
 *
 *   U      [R][gamma][V]  dt   base logits U_k of the parallel backbone
 *   W1     [V][r]         dt   token -> r-vector table of the Markov head
 *   W2t    [V][r]         dt   W2 (r x V) stored transposed: row v of W2t
 *                              is column v of W2
 *   x0     [R]            i32  anchor tokens; -1 = no previous token (B_1 = 0)
 *   G      [gamma][ceil(V/16)][R] f32  chunk Gumbels, request-minor: the
 *                                      Gumbel of chunk c of request i at
 *                                      position k is G[(k*nC + c)*R + i]
 *   g      [R][gamma][16]         f32  in-chunk Gumbels
 *   x      [R][gamma]     i32  out: drafted tokens
 *   lse    [R][gamma]     f32  out: log sum_v exp(U_k(v) + B_k(v))
 *   logit  [R][gamma]     f32  out: U_k(x_k) + B_k(x_k)
 *   ws     workspace of at least dspark_workspace_size(DSPARK_WS_SAMPLE, ...)
 *          bytes; contents on entry are irrelevant.
 *
 * With bf16 storage the call is one persistent launch that needs the whole
 * device (see the conventions above).  If its grid barrier gives up, every
 * x is -1 and every lse and logit NaN (a sentinel: valid draws are in
 * [0, V)); dspark_markov_sample_ex also reports it in a status word.
 *
 * Limits: R >= 1, 1 <= gamma <= 64, 2 <= V < 2^24.  bf16: r in {32, 64, 128,
 * 256} (else DSPARK_EDTYPE).  fp32: 1 <= r <= 1024.
 */
dspark_status dspark_markov_sample(dspark_dtype dt, int R, int gamma, int V, int r,
                                   const void* U, const void* W1, const void* W2t,
                                   const int32_t* x0, const float* G, const float* g,
                                   int32_t* x, float* lse, float* logit,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * dspark_markov_sample_ex — dspark_markov_sample, optionally followed by the
 * confidence head on the drafted tokens, with a cancel word and a status word.
 *
 * Passage: as dspark_markov_sample and dspark_confidence (caijizhuo section
 * 四: the sequential loop computes each position's confidence from its
 * hidden state and the previous token right after drawing it).
 *
 *   dt, R, gamma, V, r, U, W1, W2t, x0, G, g, x, lse, logit, ws
 *          as in dspark_markov_sample
 *   d, h, w, T, c, z
 *          as in dspark_confidence, computed on the drafted x.  h NULL skips
 *          the confidence head (d, w, T, c and z are then ignored); with h
 *          given, w and c are required and z may be NULL.
 *   cancel [1] u32 device word or NULL.  While it is non-zero, the
 *          persistent launch's grid-barrier waits give up as on a time-out,
 *          so a caller can abandon a call that cannot complete.  It is read
 *          on the device; other paths (fp32, per-position launches) have no
 *          barrier and ignore it.
 *   status [1] i32 device word out, or NULL: DSPARK_OK, or DSPARK_ETIMEOUT
 *          when the grid barrier gave up (x = -1, lse and logit NaN; c and z
 *          are then computed on no token, x0 for the first position).
 *   events [2] hipEvent_t (host array of two events the caller created with
 *          timing enabled) or NULL.  The position sweep's start and end are
 *          recorded on them: the persistent launch's own start and end, or,
 *          on the per-position paths, around all position launches.  The
 *          key clear and the finalize step (the draws' read-out and the
 *          confidence head) are outside.  Not for use under graph capture.
 *
 * Limits: as dspark_markov_sample, and as dspark_confidence when h is given.
 */
dspark_status dspark_markov_sample_ex(dspark_dtype dt, int R, int gamma, int V, int r, int d,
                                      const void* U, const void* W1, const void* W2t,
                                      const int32_t* x0, const float* G, const float* g,
                                      const void* h, const void* w, const float* T,
                                      int32_t* x, float* lse, float* logit, float* c, float* z,
                                      const uint32_t* cancel, int32_t* status, void* const* events,
                                      void* ws, size_t ws_bytes, void* stream);

/*
 * dspark_rnn_sample — the gamma-step sampling loop with the RNN head.
 *
 * Passage: notes, "implementation two: the RNN head", eq (6); atlas, the two
 * heads.  The head keeps a state s (s_0 = 0); position k forms
 * z = [s_{k-1}; W1[x_{k-1}]; h_k] and one packed projection y = W z gives
 * s_k = sigmoid(y_g) * s_{k-1} + (1 - sigmoid(y_g)) * tanh(y_c) and the
 * bias B_k = tanh(y_o) W2; x_k is then drawn exactly as in
 * dspark_markov_sample, with the r-vector o_k = tanh(y_o) in W1[x_{k-1}]'s
 * place.  x_{-1} is the anchor x0 (-1: a W1 part of zeros).  With bf16
 * storage z enters the projection in bf16 (the state rounded from fp32 to
 * nearest, ties to even) with fp32 accumulation, the gates are fp32, and
 * o_k is rounded the same way before the bias product; with fp32 storage
 * everything is fp32.
 *
 *   U, W1, W2t, x0, G, g, x, lse, logit  as in dspark_markov_sample
 *   Wrnn  [3r][2r + d] dt: rows 0..r-1 W_g, r..2r-1 W_c, 2r..3r-1 W_o; the
 *         columns follow z (state, W1 row, hidden state)
 *   h     [R][gamma][d] dt: the backbone's hidden states
 *   s     [R][gamma][r] f32 out: the state after each position
 *   o     [R][gamma][r] dt out: each position's bias vector o_k
 *   ws    workspace of dspark_workspace_size(DSPARK_WS_RNN_SAMPLE, ...) bytes
 *
 * Limits: as dspark_markov_sample; d >= 1, and with bf16 storage d a
 * multiple of 16.
 */
dspark_status dspark_rnn_sample(dspark_dtype dt, int R, int gamma, int V, int r, int d, const void* U,
                                const void* W1, const void* W2t, const void* Wrnn, const void* h,
                                const int32_t* x0, const float* G, const float* g, int32_t* x, float* lse,
                                float* logit, float* s, void* o, void* ws, size_t ws_bytes, void* stream);

/*
 * dspark_rnn_prepare — the W1-row part of the RNN head's projection for
 * every token, computed once per set of weights.
 *
 * Passage: notes eq (6).  z's middle block is W1[x_{k-1}], so W's columns
 * r .. 2r - 1 contribute P[x_{k-1}] with P[v] = W[:, r:2r] W1[v] (3r values
 * per token: the gate, candidate and output rows).  The product is a plain
 * matrix product, bf16 inputs with fp32 accumulation, stored in fp32.
 *
 *   W1    [V][r] bf16, Wrnn [3r][2r + d] bf16 as in dspark_rnn_sample
 *   P     [V][3r] f32 out (4 * V * 3r bytes: 397 MB at V = 129280, r = 256)
 *
 * Limits: bf16 storage only (DSPARK_EDTYPE otherwise); r in {32, 64, 128,
 * 256}; 2 <= V < 2^24; d a multiple of 16.
 */
dspark_status dspark_rnn_prepare(dspark_dtype dt, int V, int r, int d, const void* W1, const void* Wrnn, float* P,
                                 void* stream);

/*
 * dspark_rnn_sample_ex — dspark_rnn_sample with P from dspark_rnn_prepare
 * (for the same W1 and Wrnn; NULL: as dspark_rnn_sample).  Where the call
 * keeps W2t on chip (dspark_rnn_sample_kernel) the step then looks the
 * W1-row part of y up in P instead of multiplying W1[x_{k-1}] by W on the
 * matrix cores; the result is the same product up to the order of the fp32
 * sums.  Other shapes, and fp32 storage, ignore P.
 */
dspark_status dspark_rnn_sample_ex(dspark_dtype dt, int R, int gamma, int V, int r, int d, const void* U,
                                   const void* W1, const void* W2t, const void* Wrnn, const void* h,
                                   const int32_t* x0, const float* G, const float* g, const float* P, int32_t* x,
                                   float* lse, float* logit, float* s, void* o, void* ws, size_t ws_bytes,
                                   void* stream);

/*
 * dspark_confidence — conditional survival of every drafted position.
 *
 * Passage: notes eq (7), c_k = sigmoid(w^T [h_k ; W1[x_{k-1}]]), and the
 * sequential temperature scaling paragraph (an order-preserving
 * per-position rescaling before the cumulative product); atlas section 4.2.
 * Computed here as z = w[:d].h_k + w[d:].W1[x_{k-1}], c = sigmoid(z / T_k),
 * with x_{k-1} = x0 at k = 1 (x0 = -1 makes the W1 part zero).
 *
 *   h   [R][gamma][d]  dt   backbone hidden states
 *   w   [d + r]        dt   weights: the h part first, then the W1 part
 *   W1  [V][r]         dt   as in dspark_markov_sample
 *   x0  [R], x [R][gamma]   i32 anchors and drafted tokens
 *   T   [gamma]        f32  per-position temperatures, or NULL for T_k = 1
 *   c   [R][gamma]     f32  out
 *   z   [R][gamma]     f32  out, may be NULL: the logit before temperature
 *
 * Limits: d a multiple of 8 (bf16) or 4 (fp32); r likewise.
 */
dspark_status dspark_confidence(dspark_dtype dt, int R, int gamma, int d, int r, int V,
                                const void* h, const void* w, const void* W1,
                                const int32_t* x0, const int32_t* x, const float* T,
                                float* c, float* z, void* stream);

/*
 * dspark_schedule — hardware-aware prefix scheduler, batched.
 *
 * Passage: notes, "hardware-aware prefix scheduler": Algorithm 1 steps 1-6
 * (cumulative survival, one pooled ranking of every (r, j), greedy admission
 * from B = R, tau = R while Theta = tau * SPS(B) strictly increases, stop at
 * the first non-increase); caijizhuo sections 三 and 四 (admit).
 * Exactness: survival is the fp64 left-to-right product of the fp32
 * confidences, quantised to a_fx = floor(a * 2^50); slots with a_fx = 0 are
 * not candidates; ties in a_fx go to the lower request, then the lower
 * position; tau is an exact integer sum and every Theta comparison is exact.
 * The result is therefore bit-exact and independent of summation order.
 *
 *   c          [R][gamma]  f32  confidences (already temperature-scaled)
 *   sps        [n_sps]     f64  sps[B-1] = SPS(B) in steps/s, positive and
 *                               non-increasing; n_sps >= R * (1 + gamma)
 *   ell        [R]         i32  out: admitted draft length l_r in 0..gamma
 *   admitted   [1]         i32  out, may be NULL: A = sum_r l_r
 *   theta_best [1]         f64  out, may be NULL:
 *                               double(tau_fx) * 2^-50 * SPS(R + A)
 *   ws         workspace of dspark_workspace_size(DSPARK_WS_SCHEDULE, ...) bytes
 *
 * Limits: R * (1 + gamma) <= 8191.
 */
dspark_status dspark_schedule(int R, int gamma, const float* c, const double* sps, int n_sps,
                              int32_t* ell, int32_t* admitted, double* theta_best,
                              void* ws, size_t ws_bytes, void* stream);

/* Admission rules of dspark_schedule_ex. */
typedef enum {
  DSPARK_SCHED_EARLY_STOP = 0,  /* Algorithm 1 as in dspark_schedule */
  DSPARK_SCHED_WHOLE_WALK = 1,  /* no early stop: the best Theta over the whole ranked walk */
  DSPARK_SCHED_CAPACITY = 2     /* fill a given capacity of K slots from the ranking */
} dspark_sched_mode;

/*
 * dspark_schedule_ex — the scheduler with a choice of admission rule: the
 * production (asynchronous) scheduler is two calls of it.
 *
 * Passage: notes, "adapting Algorithm 1 to real hardware: two conflicts" (a
 * stepped SPS curve traps the early stop at a local peak; graph replay needs
 * the verification batch before the round's confidences exist) and "the
 * asynchronous fix, and why it stays lossless" (the capacity comes from the
 * confidences of two rounds earlier with no early stop; the current round's
 * ranking decides which slots fill it); step 9 of the notes' end-to-end loop.
 * A production round t therefore runs
 *   dspark_schedule_ex(..., c_t, ..., DSPARK_SCHED_CAPACITY, K_t, ell_t, ...)
 *   dspark_schedule_ex(..., c_t, ..., DSPARK_SCHED_WHOLE_WALK, NULL, tmp, K_{t+2}, ...)
 * where the `admitted` output of the second call is the capacity two rounds
 * later (K_0 and K_1 are the caller's choice).
 *
 * Ranking, survival, Q50 quantisation, tie rules and exact Theta comparisons
 * are those of dspark_schedule.  By mode, A (the number of admitted slots) is
 *   DSPARK_SCHED_EARLY_STOP  the early stop of dspark_schedule;
 *   DSPARK_SCHED_WHOLE_WALK  the smallest m in 0..M with the largest
 *                            Theta(m) = tau_fx(m) * SPS(R + m), M the number
 *                            of candidates (a_fx > 0);
 *   DSPARK_SCHED_CAPACITY    min(max(*cap, 0), M).
 *
 *   c, sps, ell, admitted, theta_best, ws: as for dspark_schedule
 *   mode       one of dspark_sched_mode; anything else -> DSPARK_EINVAL
 *   cap        [1] i32 device pointer, read on the device: the capacity K.
 *              Required (non-NULL) for DSPARK_SCHED_CAPACITY, ignored
 *              otherwise.
 *
 * Limits: R * (1 + gamma) <= 8191.
 */
dspark_status dspark_schedule_ex(int R, int gamma, const float* c, const double* sps, int n_sps,
                                 int mode, const int32_t* cap, int32_t* ell, int32_t* admitted,
                                 double* theta_best, void* ws, size_t ws_bytes, void* stream);

/*
 * dspark_schedule_noalloc — dspark_schedule_ex without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture
 * that may not call hipMalloc, tight serving loops, and harnesses that
 * forbid allocation.  The ranked slot keys live in a static device array of
 * the library instead: 8192 slots (64 KiB) on each device the library runs
 * on, held until the process ends.  Every call on one device shares that
 * array, so calls that overlap on one device race and must be serialised by
 * the caller (one stream, or events).  Every key is rewritten before it is
 * read, so no clearing is needed between calls.  The call itself allocates
 * nothing (the array's address is looked up once per device).
 *
 *   every argument as in dspark_schedule_ex, without ws and ws_bytes
 *
 * Limits: as dspark_schedule_ex, and R * gamma <= 8192 (implied by
 * R * (1 + gamma) <= 8191); larger batches return DSPARK_EINVAL.
 */
dspark_status dspark_schedule_noalloc(int R, int gamma, const float* c, const double* sps, int n_sps,
                                      int mode, const int32_t* cap, int32_t* ell, int32_t* admitted,
                                      double* theta_best, void* stream);

/*
 * dspark_verify — lossless rejection-sampling verification.
 *
 * Passage: notes, the speculative-decoding background (accept x with
 * probability min(1, p_t(x)/p_d(x)); at the first rejection resample from
 * norm(max(0, p_t - p_d)); a bonus token from p_t when everything is
 * accepted), eq (8a)-(8c), steps 12-13 of the end-to-end loop; caijizhuo
 * section 四 steps 5-6 (row i of the target logits predicts draft i).
 * Draft i of request r is accepted iff ln u_acc[r][i] < ln p_t(x_i) -
 * ln p_d(x_i); n_acc[r] is the length of the accepted prefix (0..ell[r]).
 * next_tok[r] is the smallest v with cumsum(res)[v] > u_res[r] * sum(res),
 * res = max(0, p_t - p_d) on row n_acc[r] after a rejection, res = p_t of
 * row ell[r] otherwise; if sum(res) <= 0 the draw uses p_t of the same row.
 *
 *   target  target logits, dt: dense [R][gamma+1][V] when row0 == NULL, else
 *           a packed [rows][V] array whose rows row0[r] .. row0[r] + ell[r]
 *           belong to request r (a flattened ragged verify batch)
 *   row0    [R] i32 or NULL
 *   U, W1, W2t, x0  as in dspark_markov_sample (to rebuild p_d on the
 *           residual row)
 *   x, lse, logit   [R][gamma] outputs of dspark_markov_sample
 *   ell     [R] i32 output of dspark_schedule (read on the device)
 *   u_acc   [R][gamma] f32 uniforms in (0,1); u_res [R] f32 uniforms in (0,1)
 *   n_acc   [R] i32 out; next_tok [R] i32 out
 *   ws      workspace of dspark_workspace_size(DSPARK_WS_VERIFY, ...) bytes
 *
 * Limits: as dspark_markov_sample.
 */
dspark_status dspark_verify(dspark_dtype dt, int R, int gamma, int V, int r,
                            const void* target, const int32_t* row0,
                            const void* U, const void* W1, const void* W2t,
                            const int32_t* x0, const int32_t* x, const float* lse,
                            const float* logit, const int32_t* ell,
                            const float* u_acc, const float* u_res,
                            int32_t* n_acc, int32_t* next_tok,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * dspark_verify_greedy — verification at temperature 0.
 *
 * Passage: notes, the FAQ on greedy (temperature-0) decoding: acceptance
 * degenerates to an exact-match test of the draft token against the target's
 * argmax token (the special case of the speculative-decoding framework).
 * Reading: the argmax is the lowest token index among equal largest logits.
 * n_acc[r] = the first i < ell[r] with x[r][i] != argmax(target row i), or
 * ell[r] if every admitted draft matches; next_tok[r] = argmax of target row
 * n_acc[r] (the bonus row when everything matched).  Bit-exact: only
 * comparisons of the stored logits.
 *
 *   target, row0  as in dspark_verify
 *   x       [R][gamma] i32 draft tokens (any value; one outside [0, V) never
 *           matches)
 *   ell     [R] i32 admitted lengths (read on the device)
 *   n_acc   [R] i32 out; next_tok [R] i32 out
 *   ws      workspace of dspark_workspace_size(DSPARK_WS_VERIFY_GREEDY, ...) bytes
 *
 * Limits: as dspark_markov_sample.
 */
dspark_status dspark_verify_greedy(dspark_dtype dt, int R, int gamma, int V, const void* target,
                                   const int32_t* row0, const int32_t* x, const int32_t* ell,
                                   int32_t* n_acc, int32_t* next_tok, void* ws, size_t ws_bytes,
                                   void* stream);

/*
 * dspark_acceptance — the analytic acceptance of every drafted position.
 *
 * Passage: notes, eq (8) and its derivation (8a)-(8c), and the confidence-head
 * paragraph (the head's training label is this closed form, not sampled
 * accept/reject outcomes): c*[r][k] = sum_v min(p_d(v), p_t(v)) = 1 -
 * 0.5 ||p_d - p_t||_1, with p_d the drafter's distribution at position k
 * (U_k plus the Markov bias of x_{k-1}, normalised by lse[r][k]) and p_t the
 * softmax of target row k.  One pass over the draft and target logits of all
 * gamma positions (label generation and calibration checks).
 *
 *   target, row0  as in dspark_verify; rows 0 .. gamma-1 of every request are
 *           read (row0[r] + k when packed)
 *   U, W1, W2t, x0, x, lse  as in dspark_verify
 *   bvec    [R][gamma][r] dt or NULL: the drafter's bias vectors (the `o`
 *           output of dspark_rnn_sample) in W1[x_{k-1}]'s place
 *   c_star  [R][gamma] f32 out
 *   ws      workspace of dspark_workspace_size(DSPARK_WS_ACCEPTANCE, ...) bytes
 *
 * Limits: as dspark_markov_sample.
 */
dspark_status dspark_acceptance(dspark_dtype dt, int R, int gamma, int V, int r, const void* target,
                                const int32_t* row0, const void* U, const void* W1, const void* W2t,
                                const void* bvec, const int32_t* x0, const int32_t* x, const float* lse,
                                float* c_star, void* ws, size_t ws_bytes, void* stream);

/*
 * dspark_sts_fit — sequential temperature scaling of the confidence head
 * on a held-out set, with its calibration metrics.
 *
 * Passage: notes, "sequential temperature scaling (STS)" and the
 * per-position reliability table (ROC-AUC, ECE before and after STS);
 * paper-breakdown, the confidence-head paragraph.  For k = 1..gamma in
 * order, T_k is the grid temperature minimising the ECE of the cumulative
 * product a_k = a_{k-1} * sigmoid(z_k / T_k) (a_0 = 1) against prefix
 * survival y_k = [n_acc >= k], T_1..T_{k-1} fixed; ties go to the first
 * grid entry.  ECE: n_bins equal-width bins of [0, 1], bin min(floor(p M),
 * M - 1), ECE = (1/N) sum_b |sum_{n in b} (y_n - p_n)|.  Predictions are
 * fp32 (sigmoid(x) = 1 / (1 + exp(-x))); the bin sums are exact 64-bit
 * integers in units of 2^-32, so the fit is deterministic.  ece_before is
 * the raw chain's (every T = 1).  auc[k] is the ROC-AUC of the raw logit
 * z_k between accepted (n_acc >= k) and rejected (n_acc = k - 1) rollouts
 * that reached position k, ties counted half (NaN without both classes).
 * The count equals the pairwise definition exactly but is computed from one
 * sort of the rejected logits and rank counts: O(N log N) work in all.
 *
 *   z       [N][gamma] f32: the confidence head's logits per rollout
 *   n_acc   [N] i32: accepted prefix length of each rollout, 0..gamma
 *   grid    [n_grid] f32: candidate temperatures (> 0)
 *   T       [gamma] f32 out; ece_before, ece_after, auc [gamma] f64 out
 *   ws      workspace of dspark_workspace_size(DSPARK_WS_STS, N, gamma,
 *           n_grid, n_bins, 0) bytes
 *
 * Limits: 1 <= N <= 2^20, gamma <= 64, n_grid <= 256, n_bins <= 32.
 */
dspark_status dspark_sts_fit(int N, int gamma, const float* z, const int32_t* n_acc, const float* grid,
                             int n_grid, int n_bins, float* T, double* ece_before, double* ece_after,
                             double* auc, void* ws, size_t ws_bytes, void* stream);

/*
 * dspark_verify_ex — dspark_verify for a drafter whose bias vector is not a
 * W1 row (the RNN head).
 *
 * Passage: as dspark_verify, with eq (6)'s bias B_k = o_k W2: p_d at the
 * first rejected position n is rebuilt from U_n and the bias vector o_n,
 * bvec[r][n], instead of W1[x_{n-1}].  bvec NULL is dspark_verify.
 *
 *   bvec    [R][gamma][r] dt or NULL: the `o` output of dspark_rnn_sample
 *   every other argument as in dspark_verify
 */
dspark_status dspark_verify_ex(dspark_dtype dt, int R, int gamma, int V, int r, const void* target,
                               const int32_t* row0, const void* U, const void* W1, const void* W2t,
                               const void* bvec, const int32_t* x0, const int32_t* x, const float* lse,
                               const float* logit, const int32_t* ell, const float* u_acc, const float* u_res,
                               int32_t* n_acc, int32_t* next_tok, void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace a call needs (0 for an invalid shape).  Arguments that a
 * call does not take are ignored. */
size_t dspark_workspace_size(dspark_ws_kind kind, int R, int gamma, int V, int r, int n_sps);

/* A static, human-readable description of a status code. */
const char* dspark_status_string(dspark_status s);

/*
 * dspark_markov_sample_kernel — which kernel dspark_markov_sample(_ex) runs
 * the positions with for this shape on the current device: a static string
 * naming it and how it treats W2t, or NULL for arguments the sampling call
 * would reject or a device that is not gfx950.  With bf16 storage, R <= 128,
 * r in {32, 64, 128, 256} and at most eight 64-token tiles per compute unit
 * (V <= 131072 on 256 compute units), each work group keeps its slice of
 * W2t in registers and LDS for the whole launch; larger shapes stream W2t
 * through LDS at every position.  Enqueues nothing.
 */
const char* dspark_markov_sample_kernel(dspark_dtype dt, int R, int gamma, int V, int r);

/*
 * dspark_rnn_sample_kernel — the same for dspark_rnn_sample (DSpark reading
 * notes, "implementation two: the RNN head", eq (6)): with bf16 storage,
 * r = 256 and 33 to 128 requests, or r = 128 and 65 to 128, and W2t on chip
 * as above, one persistent launch holds W2t on chip and computes each
 * position's RNN step (o_k, s_k) between two grid barriers before that
 * position's sweep; other shapes run a step kernel and a one-position
 * sampling launch per position.  A static string, or NULL as above;
 * enqueues nothing.
 */
const char* dspark_rnn_sample_kernel(dspark_dtype dt, int R, int gamma, int V, int r);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
