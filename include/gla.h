/*
 * gla.h -- C ABI of libgla.so: chunkwise gated linear attention with a per-key-channel
 * (diagonal) decay, forward and backward, and ZeCO's segment decomposition, on one
 * MI355X (gfx950).
 *
 * The method (ZeCO, arXiv 2507.01004, as summarised on the atlas.scime.ai and
 * pith.science pages):
 *   - a sequence of T tokens is cut into P segments of L = T/P tokens;
 *   - every segment runs the gated-linear-attention recurrence from a ZERO state and
 *     produces local outputs and local states (the local pass of the paper's Algorithm 1,
 *     as the pith.science referee report describes it in major comment 1);
 *   - a decay-and-add scan over segments, split into K blocks of d_k rows, gives every
 *     segment its true incoming state: S_in[p+1] = exp(logdecay[p]) * S_in[p] + S_local[p]
 *     (the All-Scan update, pith.science "What carries the argument");
 *   - every segment's outputs are corrected with the cumulative decay (the second pass over
 *     Q, K, V of the same comment), using the linear-decomposition identity
 *     (pith.science "Assumptions", Appendix A.1);
 *   - the backward reuses the forward's global incoming states (pith.science
 *     "Assumptions", Appendix A.4).  How the state gradient crosses segments is not
 *     written on the pages; this library runs the same decay-and-add scan in reverse.
 *
 * The recurrence, per (batch b, head h), tokens t = 0..T-1, state S in R^{dk x dv}:
 *     S_t = diag(exp(g_t)) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t,   S_{-1} = h0 (zero)
 * g is the log of the decay ("log-gate"), one value per token and per d_k channel.
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers owned by the caller (for example torch tensors).
 *     The library never allocates or frees device memory and never writes inputs; the one
 *     memory it keeps is gla_chunk_fwd_noalloc's static array (256 KiB per GPU).
 *   - All tensors are contiguous, row-major:
 *       q, k, dq, dk, g, dg:   [B][H][T][dk]
 *       v, o, do, dv:          [B][H][T][dv]
 *       per-segment states:    [B][H][P][dk][dv]      (float32)
 *       per-chunk states:      [B][H][T/chunk][dk][dv] (dtype)
 *       seg_logdecay:          [B][H][P][dk]          (float32)
 *       single states (h0...): [B][H][dk][dv]         (float32)
 *   - dtype selects the element type of q, k, v, o, do, dq, dk, dv: GLA_BF16 (bfloat16)
 *     or GLA_F32 (float32).  g, dg and every state are always float32.  bf16 products
 *     run on MFMA with float32 accumulation; f32 products on the f32 MFMA.
 *   - g must be finite and <= 0 everywhere (a decay in (0, 1]); any such g is exact, however
 *     strong the decay.  gla_segment_correct relies on g <= 0 to stop a segment's correction
 *     once every channel's cumulative decay has underflowed to exactly zero in float32.  The
 *     fast kernels factor exp(b_t - b_s) inside a chunk as exp(b_t) * exp(-b_s) (b the in-chunk
 *     running sum of g) and take a chunk only if no channel decays by more than e^-40 over it;
 *     a unit (b, h, segment) holding a stronger chunk is recomputed, in the same call, by
 *     kernels that walk 16-token sub-blocks and sum the sub-block's own scores element by
 *     element with exp(b_t - b_s), an exponent that is never positive.
 *   - stream is a hipStream_t (NULL = the null stream).  Every call only enqueues work on
 *     it: no host synchronisation, no device-wide barrier.  The caller orders the calls.
 *   - Shapes, dtype, pointers, the workspace size and the supported-shape table are all checked
 *     on the host BEFORE any HIP call; a rejected call enqueues nothing.  A failed launch
 *     returns GLA_ERR_HIP.  gla_last_error() describes the last failure of the calling thread.
 *   - gla_chunk_fwd and gla_chunk_bwd take a caller-owned device workspace (see
 *     gla_workspace_size).  The call writes it before reading it, so its contents on entry do
 *     not matter; it must not be shared by calls that may run at the same time.
 *
 * Supported shapes (gla_supported() answers for a given combination):
 *   GLA_BF16: chunk in {16, 32, 64}; dk in {32, 64, 128}; dv in {32, 64, 128, 256}
 *             (chunk 16 always runs the sub-block kernels: the bf16 MFMA contracts 32 tokens)
 *   GLA_F32:  chunk in {16, 32, 64}; dk in {16, 32}; dv in {16, 32}
 *   always:   B, H, T, P >= 1 (an empty sequence is rejected with GLA_ERR_INVALID_ARG);
 *             T % P == 0; (T / P) % chunk == 0.  A sequence of another length may be padded at
 *             its end with q = k = v = do = 0 and g = 0: such tokens leave every output and
 *             gradient of the real tokens, the final state and dh0 unchanged.
 */
#ifndef GLA_H
#define GLA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GLA_OK = 0,
  GLA_ERR_INVALID_ARG = 1, /* bad shape, null pointer, bad enum value */
  GLA_ERR_UNSUPPORTED = 2, /* valid arguments, but no kernel is built for this shape */
  GLA_ERR_HIP = 3          /* a HIP launch failed */
} gla_status;

enum { GLA_F32 = 0, GLA_BF16 = 1 };
enum { GLA_FWD = 0, GLA_BWD = 1 };

/* Returns 1 if the kernels exist for (dtype, dk, dv, chunk), else 0. */
int gla_supported(int dtype, int dk, int dv, int chunk);

/* Static description of a status code. */
const char* gla_status_string(gla_status s);

/* Message of the last failure on the calling thread ("" if none). */
const char* gla_last_error(void);

/*
 * gla_workspace_size -- bytes of device workspace gla_chunk_fwd (which == GLA_FWD) or
 * gla_chunk_bwd (which == GLA_BWD) needs for the fastest schedule of these arguments.  The
 * workspace holds one int per unit (b, h, segment): which units the exact kernels recompute.
 * When B*H*P units would leave CUs idle (fewer than 256), the call cuts every segment into S
 * sub-segments (a power of 2) and the workspace also holds, per sub-segment, a float32 state
 * and log-decay for the in-call scan and its float32 result; the flags are then per
 * sub-segment (unit).  Then, when units have at least 4 chunks, the region for the re-split of
 * flagged units: R = min(256, units * xmax) slots, xmax the largest power of 2 that divides a
 * unit's chunks into pieces of at least 2; 2 + R ints, and per slot the same three float32
 * arrays.  (A unit is flagged when one of its chunks decays too fast for the fast kernels; the
 * flagged units are cut into pieces that fill the R slots and redone piece by piece, so a few
 * such units cost about as much as one piece each, not a whole unit each.)  Each of these
 * regions is rounded up to 256 bytes.
 * A smaller workspace is accepted down to B*H*P ints rounded up to 256 bytes: the call first
 * gives up the re-split, then halves S and tries the re-split again, down to no sub-segments
 * and no re-split, with the same results up to rounding.  (A caller running several calls side
 * by side on one GPU may want fewer sub-segments.)
 * Returns 0, with gla_last_error() set, if the arguments are rejected (the same checks as the
 * call itself).  Any alignment of 4 bytes or more will do.
 */
size_t gla_workspace_size(int which, int B, int H, int T, int dk, int dv, int chunk, int P, int dtype);

/*
 * gla_chunk_fwd -- local pass (the first pass of ZeCO's Algorithm 1 as the pith.science referee
 * report describes it, including the HBM state store it makes, major comment 1; chunkwise
 * form: intra-chunk decay-masked attention plus the chunk state recurrence, with K/Lambda for
 * the intra part and K*Gamma for the state update, the two forms minor comment 4 compares).
 *
 * For every segment p, starting from a ZERO state, computes
 *   o[t]                    = local output of token t (its segment's history only), dtype
 *   chunk_states[b,h,n]     = local state after chunk n (n = 0 .. T/chunk - 1 counts chunks
 *                             over the whole sequence), dtype, [B][H][T/chunk] states of
 *                             dk*dv elements in the TILED layout below
 *   seg_state[b,h,p]        = the segment's end state from a zero start, float32 [dk][dv]
 *   seg_logdecay[b,h,p,c]   = sum of g over the segment's tokens, float32
 * Inputs q, k, v (dtype), g (float32).  chunk is the tile length C of the chunkwise form.
 * Outputs are fully overwritten.  Results do not depend on chunk beyond rounding.
 * chunk_states may be NULL: a forward-only caller (no gla_chunk_bwd to follow) keeps no
 * per-chunk states, and the other results are the same, bit for bit.
 * workspace: caller device memory (scratch), gla_workspace_size(GLA_FWD, ...) bytes for the
 * fastest schedule, at least one int per unit (see gla_workspace_size).
 *
 * Tiled chunk-state layout (chunk_states only; every other state argument is row-major
 * [dk][dv]): a state is (dk/16) x (dv/16) tiles of 16 x 16.  Element (16 cb + c, 16 jb + j)
 * belongs to lane index L = 16 * (j / 4) + c of tile (cb, jb), position j % 4.  When dv/16 is
 * even, tiles (cb, 2m) and (cb, 2m + 1) are interleaved: the element sits at
 * (cb * dv/16 + 2m) * 256 + 8 L + 4 (jb - 2m) + j % 4.  When dv/16 is odd (dv = 16) it sits at
 * (cb * dv/16 + jb) * 256 + 4 L + j % 4.  A 64-lane wave holding a pair of tiles in registers
 * writes or reads it as 1024 contiguous bytes (bf16); the layout is private to the four entry
 * points (written by gla_chunk_fwd, updated by gla_segment_correct, read by gla_chunk_bwd and
 * gla_segment_correct).
 */
gla_status gla_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                         void* o, void* chunk_states, float* seg_state, float* seg_logdecay,
                         int B, int H, int T, int dk, int dv, int chunk, int P, int dtype,
                         void* workspace, size_t workspace_size, void* stream);

/*
 * gla_chunk_fwd_noalloc -- gla_chunk_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments and checks without the workspace, which here is a library-owned device array of
 * 256 KiB on each GPU (one int per unit), looked up once per device and kept until the process
 * ends.  The array holds the per-unit flags only, so the call neither cuts segments into
 * sub-segments nor re-splits flagged units; its results equal gla_chunk_fwd's up to rounding
 * (bit for bit where gla_chunk_fwd does neither).  The call allocates nothing.  B*H*P above 65536 is rejected with
 * GLA_ERR_INVALID_ARG before any HIP call.  The array's contents are written before they are
 * read, so nothing needs clearing between calls; calls that may run at the same time on one GPU
 * (two streams, two threads) share the array and race.
 */
gla_status gla_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                                 void* o, void* chunk_states, float* seg_state, float* seg_logdecay,
                                 int B, int H, int T, int dk, int dv, int chunk, int P, int dtype,
                                 void* stream);

/*
 * gla_segment_scan -- decay-and-add scan over the P segments (All-Scan update,
 * pith.science "What carries the argument"), on each of K blocks of dk/K state rows
 * independently (the results do not depend on K, bit for bit).
 *
 * reverse == 0 (forward):
 *   seg_carry[p] = state ENTERING segment p:  seg_carry[0] = h_boundary (h0; NULL = 0),
 *   seg_carry[p+1] = exp(seg_logdecay[p]) * seg_carry[p] + seg_state[p]   (row-wise)
 *   h_out (nullable) = exp(seg_logdecay[P-1]) * seg_carry[P-1] + seg_state[P-1] = S_T
 * reverse == 1 (backward; seg_state holds each segment's local state-gradient D_p):
 *   seg_carry[p] = gradient w.r.t. the state LEAVING segment p:
 *   seg_carry[P-1] = h_boundary (dL/dS_T; NULL = 0),
 *   seg_carry[p-1] = exp(seg_logdecay[p]) * seg_carry[p] + seg_state[p]
 *   h_out (nullable) = dL/dh0 = exp(seg_logdecay[0]) * seg_carry[0] + seg_state[0]
 * All float32: seg_state, seg_carry [B][H][P][dk][dv]; seg_logdecay [B][H][P][dk];
 * h_boundary, h_out [B][H][dk][dv].  seg_carry must not alias seg_state.
 * Requires 1 <= K <= dk and dk % K == 0.  Any dk, dv >= 1 are accepted.
 */
gla_status gla_segment_scan(const float* seg_state, const float* seg_logdecay,
                            const float* h_boundary, float* seg_carry, float* h_out,
                            int B, int H, int P, int dk, int dv, int K, int reverse,
                            void* stream);

/*
 * gla_segment_scan_allgather -- the same results as gla_segment_scan in the all-gather order of
 * the LASP2 baseline (mlsanity.com ZeCO page, "Key facts": LASP2 gathers every device's state
 * where All-Scan passes one accumulated state along).  Every carry is formed directly from all
 * the local states it depends on, with the decays between them summed in the log domain:
 *   reverse == 0:  seg_carry[p] = sum_{q<p} exp(sum_{q<r<p} ld[r]) seg_state[q]
 *                                 + exp(sum_{r<p} ld[r]) h_boundary;     h_out: the same at p = P
 *   reverse == 1:  seg_carry[p] = sum_{q>p} exp(sum_{p<r<q} ld[r]) seg_state[q]
 *                                 + exp(sum_{r>p} ld[r]) h_boundary;     h_out: the same at p = -1
 * (ld = seg_logdecay, row-wise per d_k channel).  Equal to the chain up to rounding: the order of
 * the sums and of the decay products differs.  O(P^2) state reads instead of O(P); no output
 * waits for another.  Arguments, layouts and errors as gla_segment_scan, without K.
 */
gla_status gla_segment_scan_allgather(const float* seg_state, const float* seg_logdecay,
                                      const float* h_boundary, float* seg_carry, float* h_out,
                                      int B, int H, int P, int dk, int dv, int reverse, void* stream);

/*
 * gla_segment_correct -- cumulative-decay correction of every segment's local results
 * (ZeCO's second pass over Q, K, V, pith.science referee report, major comment 1; the
 * atlas.scime.ai summary describes it as correcting local chunk states to global
 * states with a cumulative decay; the identity is the linear decomposition of "Assumptions").
 *
 * mode == GLA_FWD: for t in segment p, with a_t = exp(sum of g from the segment's first
 *   token through t) and S_in[p] = seg_in[p] (seg_carry of the forward scan):
 *     o[t]            += (q[t] * a_t) . S_in[p]
 *     chunk_states[n] += diag(a at the last token of chunk n) S_in[p]     (n in segment p)
 *   Uses q, g, seg_in; o and chunk_states (dtype) are in/out.  k, v, seg_grad, dk_, dv_, dg
 *   may be NULL, and so may chunk_states (a forward-only caller that kept none: then only o is
 *   corrected).  Afterwards chunk_states holds the GLOBAL state after every chunk.
 * mode == GLA_BWD: with G_p = seg_grad[p] (seg_carry of the reverse scan) and r_t = sum of g
 *   over the tokens after t up to the segment's end:
 *     dk_[t] += exp(r_t) * (G_p v[t])
 *     dv_[t] += G_p^T (exp(r_t) * k[t])
 *     dg[t]  += exp(g[t] + r_t) * rowsum(S_{t-1} * G_p)     (S_{t-1}: global state before t)
 *   S_{t-1} is rebuilt per chunk from chunk_states (global, after the GLA_FWD correction) and
 *   seg_in.  Uses k, v, g, seg_in, seg_grad, chunk_states; dk_, dv_ (dtype) and dg (float32)
 *   are in/out.  q and o may be NULL.
 */
gla_status gla_segment_correct(int mode, const void* q, const void* k, const void* v,
                               const float* g, const float* seg_in, const float* seg_grad,
                               void* o, void* chunk_states, void* dk_, void* dv_, float* dg,
                               int B, int H, int T, int dk, int dv, int chunk, int P, int dtype,
                               void* stream);

/*
 * gla_chunk_bwd -- backward of every segment given the GLOBAL states (the forward's states are
 * reused, pith.science "Assumptions", Appendix A.4; Alg. 3 loads the state from HBM and walks
 * the chunks, minor comment 5).  chunk_states must hold the global state after every chunk
 * (gla_chunk_fwd followed by gla_segment_correct(GLA_FWD)); seg_in is the forward scan's
 * seg_carry.  With do the output gradient:
 *   dq[t]          = S_t do[t] with S_t the GLOBAL state (complete, needs no correction)
 *   dk_[t], dv_[t] = gradients from segment p's own outputs (state gradient U starting at
 *                    zero at the segment's end): dk_[t] = U_t v[t], dv_[t] = U_t^T k[t]
 *   dg[t]          = sum_{t' >= t in segment} (q[t'] dq[t'] - k[t'] dk_[t'])  (float32; formed
 *                    chunk by chunk with the exact carry rowsum(S * U) at chunk boundaries,
 *                    itself formed from the chunk's own dk terms so that it cancels them to
 *                    float32 rounding under strong decay)
 *   seg_dstate[b,h,p] = D_p = gradient w.r.t. the state entering segment p from segment p's
 *                    own outputs, float32 [dk][dv]
 * q, k, v, do, chunk_states and the outputs dq, dk_, dv_ share dtype.  Outputs are fully
 * overwritten and must not alias inputs.
 * workspace: caller device memory (scratch), gla_workspace_size(GLA_BWD, ...) bytes for the
 * fastest schedule, at least one int per unit (see gla_workspace_size).
 */
gla_status gla_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                         const void* do_, const void* chunk_states, const float* seg_in,
                         void* dq, void* dk_, void* dv_, float* dg, float* seg_dstate,
                         int B, int H, int T, int dk, int dv, int chunk, int P, int dtype,
                         void* workspace, size_t workspace_size, void* stream);

/*
 * ---- The same path with the incoming states first: no correction pass ----
 *
 * In the order above, every segment runs from a zero state and the correction afterwards makes its
 * results global: a second pass over the chunks that the incoming state still reaches (the second
 * pass over Q, K, V of the pith.science referee report, major comment 1).  Under weak or no decay
 * it reaches every chunk.  The four calls below order the same decomposition the other way, as
 * LASP's devices do (elamur.ai LASP summary: the K^T V state, the right product, carries the
 * dependency between devices, and a device computes its outputs from the state it receives):
 *
 *   gla_chunk_state -> gla_segment_scan -> gla_chunk_fwd_from                        (forward)
 *   gla_chunk_dstate -> gla_segment_scan(reverse) -> gla_chunk_bwd_from             (backward)
 *
 * A state pass reads k, v, g (forward) or q, g, do (backward) of the chunks whose share of the
 * segment's end state (or of the gradient entering it) is not an exact float32 zero: it walks
 * from the segment's far end and stops once every channel's summed log-gates are below -112
 * (e^-112 underflows to 0.0f).  The corrections cost the chunks the incoming states reach; both
 * depend on the decay in the same way.  The results equal those of the correction order up to
 * rounding; seg_state, seg_logdecay and seg_dstate are the same quantities (local, from a zero
 * state), except that a segment whose walk stopped early reports, for seg_logdecay, the sum over
 * the chunks walked: every channel below -112, so its exponential is 0.0f like the full sum's.
 */

/*
 * gla_chunk_state -- each segment's local end state and summed log-gates, computed from a zero
 * start (seg_state as gla_chunk_fwd returns it, up to rounding), reading only k, v and g: the end
 * state unrolled, S = sum_t exp(x_t) k_t v_t^T with x_t the log-gates after token t, summed chunk by
 * chunk from the segment's end (the state update of the chunkwise form, S <- diag(exp(lam)) S +
 * Ktil^T V, with the decays folded into the keys).  The walk stops once every channel's x is
 * below -112: the earlier tokens' weights are then exact zeros.  seg_logdecay is the segment's
 * summed log-gates where the walk reached the segment's start; where it stopped early it is the
 * sum over the chunks walked, below -112 in every channel (the full sum is lower still, and both
 * exponentials are 0.0f, which is all gla_segment_scan takes from it).
 * Inputs k, v (dtype), g (float32), [B][H][T][d]; outputs seg_state [B][H][P][dk][dv] and
 * seg_logdecay [B][H][P][dk], float32, fully overwritten.
 * workspace: optional (NULL, or gla_workspace_size(GLA_FWD, ...) bytes): with room, segments are cut
 * into sub-segments when B*H*P < 256, as in gla_chunk_fwd.  bf16 with chunk 16 has no state-pass
 * kernel of its own; the pass then runs in chunks of 64 or 32 tokens (whichever divides the
 * segments), else GLA_ERR_UNSUPPORTED.
 */
gla_status gla_chunk_state(const void* k, const void* v, const float* g, float* seg_state, float* seg_logdecay,
                           int B, int H, int T, int dk, int dv, int chunk, int P, int dtype,
                           void* workspace, size_t workspace_size, void* stream);

/*
 * gla_chunk_fwd_from -- gla_chunk_fwd with each segment starting from its true incoming state
 * seg_in[p] (the forward gla_segment_scan's seg_carry over gla_chunk_state's results) instead of
 * zero: o and chunk_states come out GLOBAL, as after gla_segment_correct(GLA_FWD), and no
 * correction follows.  seg_in: float32 [B][H][P][dk][dv].  Other arguments, layouts, the workspace
 * and errors as gla_chunk_fwd (chunk_states may be NULL); there is no seg_state / seg_logdecay
 * output.
 */
gla_status gla_chunk_fwd_from(const void* q, const void* k, const void* v, const float* g, const float* seg_in,
                              void* o, void* chunk_states, int B, int H, int T, int dk, int dv, int chunk, int P,
                              int dtype, void* workspace, size_t workspace_size, void* stream);

/*
 * gla_chunk_dstate -- each segment's local state gradient D_p (seg_dstate exactly as gla_chunk_bwd
 * returns it, up to rounding), reading only q, g and do: the gradient recursion U <- diag(exp(lam))
 * U + Qbar^T dO unrolled, D = sum_t exp(a_t) q_t do_t^T with a_t the log-gates from the segment's
 * start through token t, summed chunk by chunk from the segment's start; the walk stops once every
 * channel's a is below -112 (the later tokens' weights are exact zeros).  Output seg_dstate float32
 * [B][H][P][dk][dv], fully overwritten.  The reverse scan takes it with gla_chunk_state's
 * seg_logdecay.  workspace and the bf16 chunk-16 rule as gla_chunk_state (GLA_BWD size).
 */
gla_status gla_chunk_dstate(const void* q, const float* g, const void* do_, float* seg_dstate, int B, int H, int T,
                            int dk, int dv, int chunk, int P, int dtype, void* workspace, size_t workspace_size,
                            void* stream);

/*
 * gla_chunk_bwd_from -- gla_chunk_bwd with each segment's backward starting from seg_grad[p], the
 * gradient w.r.t. the state leaving segment p from the later segments (the reverse gla_segment_scan's
 * seg_carry over gla_chunk_dstate's results): dq, dk, dv and dg come out GLOBAL, as after
 * gla_segment_correct(GLA_BWD), and no correction follows.  chunk_states must hold the global
 * states (gla_chunk_fwd_from) and seg_in the forward scan's seg_carry.  dg includes the
 * rowsum(S_end * seg_grad[p]) term at each segment's end.  Other arguments, layouts, the workspace
 * and errors as gla_chunk_bwd; there is no seg_dstate output.
 */
gla_status gla_chunk_bwd_from(const void* q, const void* k, const void* v, const float* g, const void* do_,
                              const void* chunk_states, const float* seg_in, const float* seg_grad, void* dq,
                              void* dk_, void* dv_, float* dg, int B, int H, int T, int dk, int dv, int chunk, int P,
                              int dtype, void* workspace, size_t workspace_size, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H */
