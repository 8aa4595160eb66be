/*
 * dlmerge.h -- C ABI of the MI355X (gfx950) DiLoCo outer-step merge.
 *
 * A merge round turns the worker checkpoints pushed after H local steps into
 * the next global model and its EMA.  Two variants are provided:
 *
 *  DL_MEAN            plain replacement averaging: each checkpoint is added
 *                     to an fp32 running sum in the order it arrives; the
 *                     new global is that sum divided by the number of
 *                     checkpoints (DiffuRefill-1B technical report, section
 *                     "Training system", Table 2, rows "Merger" and "Outer
 *                     step"; DiffuRefill-1B model card, "How it is trained",
 *                     Merging bullet).
 *  DL_DELTA_NESTEROV  fragment merge: per parameter fragment, the
 *                     participants' deltas, averaged with token weights, feed an outer
 *                     Nesterov optimizer (GradientMail post "Pythia-14M on
 *                     four rented GPUs and a bucket", section "Getting
 *                     updates through the bucket").
 *
 * Both can advance an EMA of globals in the same pass (technical report,
 * Table 2, row "Side averages"; model card, EMA bullet).
 *
 * Arithmetic.  Every step is IEEE-754 binary32, one rounding per operation,
 * round-to-nearest-even, no fused multiply-add, IEEE division, subnormals
 * kept, NaN and infinity propagated (no value is rejected).  For element j of
 * a fragment, with arrivals k = 1..N in arrival order:
 *
 *   DL_MEAN:   S = c_1 ;  S = S + c_k (k > 1) ;  g = S / N
 *   DELTA:     d = theta - c_k ; p = w_k * d ; A = p (k = 1) or A + p
 *              dbar = A / W ; m' = mu*m + dbar ; u = dbar + mu*m' ;
 *              theta' = theta - lr*u
 *   EMA:       e' = beta*e + (1 - beta)*x, x the new global (g or theta'),
 *              with (1 - beta) formed once in binary32
 *
 * where bf16 checkpoints are widened exactly to fp32, w_k is the worker's
 * int64 token count rounded once to binary32, and W is the exact int64 sum of
 * the fragment's token counts rounded once to binary32.
 *
 * Memory.  Every array argument is a DEVICE pointer to memory the caller owns
 * (e.g. a torch tensor's data_ptr()).  The library never allocates, frees or
 * copies device memory, never synchronises, and launches every kernel of a
 * round on the round's stream; the caller keeps buffers alive until that
 * stream's work is done and synchronises through the stream.  Parameters are
 * flat, contiguous vectors of n_params elements; fragment f covers elements
 * [frag_offsets[f], frag_offsets[f+1]).  Full-length buffers (acc, global,
 * momentum, ema) are indexed by those offsets; a checkpoint buffer holds only
 * its fragment's elements.  Consecutive passes over a fragment walk it in
 * alternating directions (results do not depend on it; it lets a pass find
 * the end of the previous one still cached).  Pointers must be aligned to
 * their element type;
 * when every pointer a kernel touches is 16-byte aligned the 128-bit path
 * runs, otherwise a scalar path gives the same bits.  Each span
 * [ptr, ptr + bytes) must lie inside one device allocation, which the library
 * checks with the HIP runtime before launching.
 *
 * Errors.  Every call returns DL_OK (0) or a negative status.  All checks
 * happen on the host before any launch; a call that fails them launches
 * nothing and leaves the handle unchanged.  Among them: a HIP error already
 * pending on the calling thread (hipPeekAtLastError; e.g. a failed runtime
 * call or a reported asynchronous fault) is returned as DL_E_HIP and left
 * pending for the caller, who clears it (hipGetLastError) and may retry.
 * A launch that fails is also DL_E_HIP, and then the round is failed: only
 * dl_round_end is allowed, and recovery is a new round that folds the
 * arrivals again.  A host allocation that fails is DL_E_NOMEM.  Device buffers
 * holding the global, momentum and EMA are written only by the closing calls
 * (dl_finalize_mean, dl_outer_nesterov, dl_fold_and_finalize_mean,
 * dl_fold_and_outer_nesterov, their several-arrival forms, dl_ema_update),
 * so an abandoned round changes none of them.
 *
 * Threads.  A handle is used by one host thread at a time.  Several handles
 * may be open at once (two rounds in flight, GradientMail post, "Getting
 * updates through the bucket") if their accumulator ranges do not overlap and
 * the caller orders rounds that write the same global, momentum or EMA range.
 */
#ifndef DLMERGE_H
#define DLMERGE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dl_round dl_round;   /* opaque; host memory owned by the library */

enum dl_mode {
    DL_MEAN = 0,             /* plain replacement averaging                    */
    DL_DELTA_NESTEROV = 1    /* token-weighted delta mean + outer Nesterov     */
};

enum dl_dtype {
    DL_F32 = 0,              /* IEEE binary32                                  */
    DL_BF16 = 1              /* bfloat16, widened exactly to binary32          */
};

enum dl_status {
    DL_OK = 0,
    DL_E_INVAL = -1,     /* bad argument: NULL/unknown value, range, overlap,
                            pointer outside its allocation, token overflow    */
    DL_E_STALE = -2,     /* checkpoint carries another round's tag             */
    DL_E_DUP = -3,       /* worker already folded into this fragment           */
    DL_E_QUORUM = -4,    /* closing a fragment with fewer arrivals than quorum */
    DL_E_STATE = -5,     /* call not allowed in the fragment's/round's state   */
    DL_E_ALIGN = -6,     /* pointer not aligned to its element type            */
    DL_E_HIP = -7,       /* HIP error pending before the call (nothing launched,
                            handle unchanged, error left pending), or a failed
                            launch (the round is then failed)                  */
    DL_E_CAPACITY = -8,  /* output array too small                             */
    DL_E_NOMEM = -9,     /* host memory for the round's bookkeeping exhausted  */
    DL_E_TOO_LARGE = -10 /* matrix workspace beyond the allocation-free entry
                            point's scratch (DL_NOALLOC_SCRATCH_BYTES)         */
};

/*
 * Open a merge round.  No device work.
 *
 * The merger closes a round once N or more checkpoints tagged with the
 * current round are in (technical report, Table 2, row "Merger": N is 2, or 1
 * with a single worker left or when a restarted merger first merges the
 * leftovers of dead workers, row "Recovery"); in the GradientMail run three
 * participants close a fragment's round ("Getting updates through the
 * bucket").  Quorum is a minimum: every arrival folded before the close
 * counts.
 *
 *   out           receives the handle (set to NULL on error).
 *   round_tag     the round's tag; checkpoints carrying another tag are
 *                 rejected (after a rollback the merger publishes under a
 *                 fresh round number,
 *                 technical report, "Training system", failure rule iii).
 *   mode          DL_MEAN or DL_DELTA_NESTEROV.
 *   n_params      flat parameter count, >= 1.
 *   n_frags       number of fragments, 1 <= n_frags <= 4096.
 *   frag_offsets  host array of n_frags + 1 int64: 0 = o_0 < o_1 < ... <
 *                 o_n = n_params.  Copied; the caller keeps ownership.
 *   quorum        minimum arrivals per fragment, 1 <= quorum <= max_workers.
 *   max_workers   worker ids are 0 .. max_workers-1, 1 <= max_workers <= 65536.
 *   acc           device, n_params fp32: the running sum / weighted-delta
 *                 accumulator.  Scratch owned by the caller; its contents on
 *                 entry do not matter (the first fold of a fragment
 *                 overwrites it).  Must not overlap the acc of another open
 *                 round over the same fragments.
 *   stream        hipStream_t on which every kernel of the round is launched
 *                 (NULL: the null stream).
 *
 * Errors: DL_E_INVAL (bad value or offsets), DL_E_ALIGN (acc not 4-byte
 * aligned), DL_E_NOMEM (the handle could not be allocated).
 */
int dl_round_begin(dl_round **out, uint64_t round_tag, int mode, int64_t n_params,
                   int n_frags, const int64_t *frag_offsets, int quorum, int max_workers,
                   float *acc, void *stream);

/*
 * Fold one arriving checkpoint (or fragment snapshot) into the round's
 * accumulator for fragment frag.  One kernel launch on the round's stream;
 * arrivals are folded in call order, which is the arrival order.
 *
 *   frag            fragment index, 0 <= frag < n_frags.
 *   worker_id       0 <= worker_id < max_workers; a worker is folded at
 *                   most once per fragment per round.
 *   ckpt_round_tag  must equal the round's tag.
 *   ckpt            device, fragment-length array of dtype.
 *   dtype           DL_F32 or DL_BF16.
 *   global          DL_DELTA_NESTEROV: device, full-length fp32 global the
 *                   participant trained from (deltas are theta - c); every
 *                   fold of a fragment and its close must pass the same
 *                   pointer.  DL_MEAN: must be NULL.
 *   tokens          DL_DELTA_NESTEROV: the participant's token count, > 0;
 *                   the fragment's total must stay below 2^63.  DL_MEAN:
 *                   ignored.
 *
 * Errors (all before launch): DL_E_STATE (round failed, or fragment already
 * closed), DL_E_INVAL, DL_E_STALE, DL_E_DUP, DL_E_ALIGN, DL_E_NOMEM, and
 * DL_E_HIP for an error already pending (handle unchanged); DL_E_HIP after a
 * launch failure (the round is then failed: only dl_round_end is allowed).
 */
int dl_fold_checkpoint(dl_round *r, int frag, int worker_id, uint64_t ckpt_round_tag,
                       const void *ckpt, int dtype, const float *global, int64_t tokens);

/*
 * Close fragment frag of a DL_MEAN round: write the mean of its arrivals
 * into out_global[frag range] and, if ema is not NULL, advance the EMA of
 * globals in the same pass.  One kernel launch.
 *
 *   out_global  device, full-length fp32; may be the round's acc (in place),
 *               otherwise must not overlap it.
 *   ema         device, full-length fp32 in/out, or NULL; must not overlap
 *               acc or out_global.
 *   beta        EMA weight of the old EMA (0.9 on the pages).
 *
 * Errors: DL_E_STATE (wrong mode, already closed, round failed),
 * DL_E_QUORUM (fewer arrivals than quorum), DL_E_INVAL, DL_E_ALIGN, DL_E_HIP.
 */
int dl_finalize_mean(dl_round *r, int frag, float *out_global, float *ema, float beta);

/*
 * Close fragment frag of a DL_DELTA_NESTEROV round: token-weighted mean delta
 * from the accumulator, outer Nesterov step on global and momentum, and, if
 * ema is not NULL, the EMA of the new global, all in one pass.  Momentum 0
 * and learning rate 1 give plain parameter averaging (GradientMail post,
 * "What might explain the loss difference", second follow-up run).
 *
 *   global    device, full-length fp32 in/out; the pointer the folds used.
 *   momentum  device, full-length fp32 in/out (zero before the first round);
 *             must not overlap acc, global or ema.
 *   lr, mu    outer learning rate and momentum (0.7 and 0.9 on the pages).
 *   ema, beta as in dl_finalize_mean.
 *
 * Errors: DL_E_STATE, DL_E_QUORUM, DL_E_INVAL, DL_E_ALIGN, DL_E_HIP.
 */
int dl_outer_nesterov(dl_round *r, int frag, float *global, float *momentum, float lr,
                      float mu, float *ema, float beta);

/*
 * Fold the fragment's last expected arrival and close the fragment in the
 * same pass: identical results, bit for bit, to dl_fold_checkpoint followed
 * by dl_finalize_mean, with one kernel launch instead of two.  The sum is
 * completed in registers and not written back to acc (acc's fragment range
 * is unspecified afterwards), so the pass moves 8 bytes per element fewer.
 * For the merger that closes as soon as every expected worker of the round
 * is in; a round closed by its grace timer uses dl_finalize_mean.  If this
 * is the fragment's first arrival (quorum 1), the mean is that checkpoint.
 *
 * Arguments as in dl_fold_checkpoint and dl_finalize_mean; the quorum check
 * counts this arrival.  ckpt must not overlap out_global or ema.
 *
 * Errors: those of both calls; nothing is launched and the handle is
 * unchanged on any error but a failed launch (DL_E_HIP, round failed).
 */
int dl_fold_and_finalize_mean(dl_round *r, int frag, int worker_id, uint64_t ckpt_round_tag,
                              const void *ckpt, int dtype, float *out_global, float *ema,
                              float beta);

/*
 * Fold the fragment's last expected arrival (token-weighted delta) and take
 * the outer Nesterov step (+ EMA) in the same pass: identical results, bit
 * for bit, to dl_fold_checkpoint followed by dl_outer_nesterov, with one
 * kernel launch instead of two.  The global is read once for both the delta
 * and the update and the accumulator is not written back (acc's fragment
 * range is unspecified afterwards): 12 bytes per element fewer than the two
 * calls.  The token total used is the exact sum including this arrival.
 *
 * Arguments as in dl_fold_checkpoint and dl_outer_nesterov; `global` must be
 * the pointer earlier folds of the fragment used.  ckpt must not overlap
 * global, momentum or ema.
 *
 * Errors: those of both calls; nothing is launched and the handle is
 * unchanged on any error but a failed launch (DL_E_HIP, round failed).
 */
int dl_fold_and_outer_nesterov(dl_round *r, int frag, int worker_id, uint64_t ckpt_round_tag,
                               const void *ckpt, int dtype, int64_t tokens, float *global,
                               float *momentum, float lr, float mu, float *ema, float beta);

/*
 * Fold several arrivals of fragment frag in one pass.  A merger that holds
 * more than one checkpoint of the fragment at once (they came in while it
 * waited for the quorum or the grace timer, or a restarted merger finds the
 * leftovers of the round, technical report, Table 2, rows "Merger" and
 * "Recovery") reads the accumulator and the global once for all of them
 * instead of once per arrival.  Results are identical, bit for bit, to
 * `count` dl_fold_checkpoint calls in array order, which is taken as the
 * arrival order (model card, "How it is trained", Merging bullet).
 *
 *   count            number of arrivals, 1 <= count <= max_workers.
 *   worker_ids       host array of count worker ids (distinct, and not yet
 *                    folded into the fragment).
 *   ckpt_round_tags  host array of count tags, each equal to the round's.
 *   ckpts            host array of count device pointers, each a
 *                    fragment-length array of dtype (one dtype for all).
 *                    Checkpoints may overlap one another (they are only
 *                    read), not acc or global.
 *   global, dtype    as in dl_fold_checkpoint.
 *   tokens           DL_DELTA_NESTEROV: host array of count token counts,
 *                    each > 0.  DL_MEAN: ignored (may be NULL).
 *
 * The host arrays are read during the call only.  The kernels take at most 8
 * arrivals per pass; a larger count runs ceil(count / 8) passes, each
 * arrival still folded in order.  Every arrival is checked as the single
 * call would check it, after those before it; on any error nothing is
 * launched and the handle is unchanged (first failing arrival's status).
 *
 * Errors: those of dl_fold_checkpoint, and DL_E_INVAL for count out of range
 * or a NULL array.
 */
int dl_fold_checkpoints(dl_round *r, int frag, int count, const int *worker_ids,
                        const uint64_t *ckpt_round_tags, const void *const *ckpts, int dtype,
                        const float *global, const int64_t *tokens);

/*
 * dl_fold_checkpoints followed by dl_finalize_mean, the last pass folding and
 * closing at once (one pass for up to 8 arrivals): the round's whole merge of
 * a fragment when every checkpoint is already in.  Bit-identical to the
 * separate calls; acc's fragment range is unspecified afterwards, as in
 * dl_fold_and_finalize_mean.  The quorum check counts this call's arrivals.
 * No checkpoint may overlap out_global or ema.
 *
 * Errors: those of dl_fold_checkpoints and dl_finalize_mean; nothing is
 * launched and the handle is unchanged on any error but a failed launch.
 */
int dl_fold_checkpoints_and_finalize_mean(dl_round *r, int frag, int count,
                                          const int *worker_ids, const uint64_t *ckpt_round_tags,
                                          const void *const *ckpts, int dtype, float *out_global,
                                          float *ema, float beta);

/*
 * dl_fold_checkpoints followed by dl_outer_nesterov, the last pass folding
 * and taking the outer step (+ EMA) at once: with every arrival of a
 * fragment in hand, each buffer (global, momentum, EMA and the checkpoints)
 * is read once and global, momentum and EMA written once per round.
 * Bit-identical to the separate calls; the token total is the exact sum over
 * the fragment's arrivals including this call's.  No checkpoint may overlap
 * global, momentum or ema.
 *
 * Errors: those of dl_fold_checkpoints and dl_outer_nesterov; nothing is
 * launched and the handle is unchanged on any error but a failed launch.
 */
int dl_fold_checkpoints_and_outer_nesterov(dl_round *r, int frag, int count,
                                           const int *worker_ids,
                                           const uint64_t *ckpt_round_tags,
                                           const void *const *ckpts, int dtype,
                                           const int64_t *tokens, float *global, float *momentum,
                                           float lr, float mu, float *ema, float beta);

/*
 * Stand-alone EMA of globals: ema[j] = beta*ema[j] + (1-beta)*global[j] for
 * j < n, on stream (technical report, Table 2, row "Side averages").
 * n = 0 is a no-op.  ema and global must not overlap.
 *
 * Errors: DL_E_INVAL, DL_E_ALIGN, DL_E_HIP.
 */
int dl_ema_update(float *ema, const float *global, int64_t n, float beta, void *stream);

/*
 * Side averages of the globals (technical report, "Training system", Table 2,
 * row "Side averages": besides the EMA, the merger keeps a uniform average
 * (SWA) of the globals and periodic snapshots in the final stretch; section
 * "Data and schedule": the published model is the equal-weight average of
 * the 130 globals committed between steps ~181k and 200k; section "The final stretch",
 * Table 5: averages of the last 3 and the last 5 snapshots).  These calls
 * keep no state: the caller owns the running sum and its count (so the
 * average survives a restart of the merger) and orders the calls on stream.
 */

/*
 * Fold one committed global into the uniform-average running fp32 sum, in
 * commit order: sum[j] = global[j] if folded_before == 0, else
 * sum[j] + global[j].  n = 0 is a no-op.  sum and global must not overlap.
 * Errors: DL_E_INVAL, DL_E_ALIGN, DL_E_HIP.
 */
int dl_swa_fold(float *sum, const float *global, int64_t n, int64_t folded_before,
                void *stream);

/*
 * out[j] = sum[j] / count (IEEE division; count rounded once to binary32),
 * count >= 1 the number of globals folded.  out may be sum (in place),
 * otherwise must not overlap it.  Errors: DL_E_INVAL, DL_E_ALIGN, DL_E_HIP.
 */
int dl_swa_average(float *out, const float *sum, int64_t n, int64_t count, void *stream);

/* Most snapshots dl_snapshot_average reads in one pass. */
#define DL_MAX_SNAPSHOTS 16

/*
 * Mean of k snapshots in one pass, summed in the order given (oldest first):
 * out[j] = (((s_0[j] + s_1[j]) + ...) + s_{k-1}[j]) / k in binary32, the same
 * bits as folding them one by one into a running sum and dividing.
 * snapshots: host array of k device pointers (n fp32 each), 1 <= k <=
 * DL_MAX_SNAPSHOTS.  out must not overlap any snapshot.  n = 0 is a no-op.
 * Errors: DL_E_INVAL, DL_E_ALIGN, DL_E_HIP.
 */
int dl_snapshot_average(float *out, const float *const *snapshots, int k, int64_t n,
                        void *stream);

/*
 * Worker-side adoption that keeps local drift (DiffuRefill-1B technical
 * report, "What we measured", "Distributed optimisation"; model card, "What
 * the run taught"): instead of replacing its weights by the new global, the
 * worker keeps the progress it made since its push:
 *     theta[j] = theta[j] + (global[j] - pushed[j])
 * with the difference rounded first.  The report measured it worse than
 * plain replacement (which is a copy of the global and needs no kernel).
 *
 *   theta         device, n fp32 in/out: the worker's current weights.
 *   global        device, n fp32: the new global.
 *   pushed        device, n elements of pushed_dtype (DL_F32 or DL_BF16):
 *                 the checkpoint the worker pushed.
 * theta must not overlap global or pushed.  n = 0 is a no-op.
 * Errors: DL_E_INVAL, DL_E_ALIGN, DL_E_HIP.
 */
int dl_adopt_keep_drift(float *theta, const float *global, const void *pushed, int pushed_dtype,
                        int64_t n, void *stream);

/*
 * Outer orthogonalisation (DiffuRefill-1B technical report, "What we
 * measured", "Optimisers": the polar factor takes the place of the averaged
 * outer update; it was a gain in a run on the 4-worker stand).  For one weight matrix
 * of rows x cols (row-major fp32) whose averaged update is A = U S V^T (thin
 * SVD), the polar factor is P = U V^T.  It is reached by a Newton-Schulz
 * iteration on fp32 MFMA: X_0 = A / ||A||_F, then `quintic_steps` steps of
 * X <- X (a I + b G + c G^2) with (a, b, c) = (3.4445, -4.7750, 2.0315) and
 * `cubic_steps` steps of X <- X (1.5 I - 0.5 G), G = X^T X (X X^T and M X for
 * rows < cols).  With 12 + 6 steps every singular value s with
 * s >= 1.4e-7 ||A||_F reaches 1 within fp32 rounding; directions below that
 * are left small.  Results are deterministic (fixed reduction order).
 *
 * The caller provides a device workspace of dl_polar_workspace_bytes bytes,
 * 256-byte aligned (the library never allocates); it must not overlap any
 * argument.  Calls on one stream may share a workspace.
 */

/* Workspace bytes for a rows x cols matrix (rows, cols >= 1).  DL_E_INVAL. */
int dl_polar_workspace_bytes(int64_t rows, int64_t cols, int64_t *bytes);

/* Workspace bytes for a batch of 1 <= batch <= DL_MAX_BATCH rows x cols
 * matrices (dl_outer_orthogonal_step_batch).  DL_E_INVAL. */
#define DL_MAX_BATCH 64
int dl_polar_workspace_bytes_batch(int64_t rows, int64_t cols, int batch, int64_t *bytes);

/*
 * out = polar factor of `update` (both rows x cols, device fp32; out may be
 * update, otherwise they must not overlap).  1 <= quintic + cubic steps,
 * each <= 64.  Errors: DL_E_INVAL (sizes, steps, workspace too small or
 * overlapping, spans), DL_E_ALIGN, DL_E_HIP.
 */
int dl_polar_factor(float *out, const float *update, int64_t rows, int64_t cols,
                    int quintic_steps, int cubic_steps, void *workspace,
                    int64_t workspace_bytes, void *stream);

/*
 * One outer step with the orthogonalised update, for one weight matrix:
 *     theta = theta - scale * P(theta - averaged)
 * where `averaged` is the round's plain mean of the workers (dl_finalize_mean)
 * and theta the global the workers trained from, so theta - averaged is the
 * averaged update.  With P replaced by the identity and scale 1 this would
 * be plain replacement (theta = averaged).  The pages give no scale; the
 * caller chooses it.  theta, averaged: device, rows x cols fp32, disjoint.
 * Errors: as dl_polar_factor.
 */
int dl_outer_orthogonal_step(float *theta, const float *averaged, int64_t rows, int64_t cols,
                             float scale, int quintic_steps, int cubic_steps, void *workspace,
                             int64_t workspace_bytes, void *stream);

/*
 * dl_outer_orthogonal_step for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument; the library's own scratch is used
 * instead, and the call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine).
 *
 * The scratch is a file-scope device array of DL_NOALLOC_SCRATCH_BYTES
 * (192 MiB) that every GPU the entry point runs on holds until the process
 * ends.  A matrix fits when dl_polar_workspace_bytes(rows, cols) is at most
 * that: every weight matrix of DiffuRefill-1B but its 73,760 x 2048
 * embedding, and every one of Pythia-14M.  No part of the scratch needs to
 * start at zero; every value is written before it is read within a call.
 *
 * Calls on one GPU share its scratch.  Calls whose work overlaps in time on
 * one GPU (different streams, or host threads without ordering) race and
 * give undefined results; calls in one stream's order are safe.  The
 * calling thread's current device must be the stream's device (NULL: the
 * current device's null stream).
 *
 * Same arguments and results as dl_outer_orthogonal_step, bit for bit (same
 * kernels, same workspace layout).  Errors: DL_E_TOO_LARGE (the matrix's
 * workspace exceeds the scratch), DL_E_INVAL (sizes, steps, overlapping or
 * out-of-allocation spans, a stream of another device), DL_E_ALIGN,
 * DL_E_HIP.
 */
#define DL_NOALLOC_SCRATCH_BYTES (192LL << 20)
int dl_outer_orthogonal_step_noalloc(float *theta, const float *averaged, int64_t rows,
                                     int64_t cols, float scale, int quintic_steps,
                                     int cubic_steps, void *stream);

/*
 * The same step for a batch of equally shaped weight matrices (the model's
 * matrices of one kind, e.g. every layer's attention projections): theta[b]
 * = theta[b] - scale * P(theta[b] - averaged[b]) for b < batch.  The
 * batch's products run as one launch each, which fills the GPU where one
 * matrix's products would not.  theta and averaged are host arrays of
 * `batch` device pointers; no theta may overlap any other argument matrix
 * or the workspace (dl_polar_workspace_bytes_batch bytes).  With batch 1
 * this is dl_outer_orthogonal_step; with more, the products are cut into
 * workgroups differently, so results agree with the one-matrix call to
 * rounding, not bit for bit.  Errors: as dl_polar_factor.
 */
int dl_outer_orthogonal_step_batch(float *const *theta, const float *const *averaged, int batch,
                                   int64_t rows, int64_t cols, float scale, int quintic_steps,
                                   int cubic_steps, void *workspace, int64_t workspace_bytes,
                                   void *stream);

enum dl_matmul_form {
    DL_TN = 0,   /* C[i][j] = sum_k A[k*lda + i] * B[k*ldb + j] */
    DL_NT = 1    /* C[i][j] = sum_k A[i*lda + k] * B[j*ldb + k] */
};

/*
 * The fp32 MFMA product the orthogonalisation is built from, with its fused
 * epilogue:  C[i][j] = alpha * sum + beta * Y[i][j] + (i == j ? diag : 0)
 * for i < m, j < n, C and Y with leading dimension ldc (Y may be NULL or
 * equal C; otherwise it must not overlap C; C must not overlap A or B).
 * Accumulation is fp32 on MFMA; results are deterministic for a given call.
 *
 * symmetric = 1 (m == n) declares the result symmetric (A^T A, A A^T, or the
 * product of a symmetric matrix with itself) and Y symmetric or NULL: only
 * the upper triangle is computed and the lower one is its mirror image.
 *
 * workspace: device memory (256-byte aligned, disjoint from every other
 * argument) or NULL.  With at least dl_matmul_workspace_bytes bytes the work
 * (output tiles x K) is spread evenly over the workgroups the GPU holds at
 * once, and tiles cut between workgroups are summed in K order through the
 * workspace (few output tiles over a long K: K cut into ranges, every tile
 * in pieces, summed in K order); a smaller workspace may still hold the
 * stream-K split's pieces; otherwise, or without one, every workgroup
 * computes one whole output tile.  Products large enough to fill the GPU
 * with 256 x 256 tiles, with K a multiple of 16 and 16-byte aligned operand
 * rows (and, when symmetric, m a multiple of 256 and 16-byte aligned result
 * rows; with a nonzero diag, m and n multiples of 256), run those tiles on a
 * large-tile kernel instead (the last round's tiles possibly cut along K and
 * summed in K order through the workspace) and the ragged rest as above.  The plans give different (each
 * deterministic) summation orders.  m = 0 or n = 0 is a no-op.  Errors:
 * DL_E_INVAL (also: symmetric with m != n), DL_E_ALIGN, DL_E_HIP.
 */
int dl_matmul_workspace_bytes(int64_t m, int64_t n, int64_t k, int symmetric, int64_t *bytes);
int dl_matmul_f32(int form, const float *a, int64_t lda, const float *b, int64_t ldb, int64_t m,
                  int64_t n, int64_t k, float *c, int64_t ldc, const float *y, float alpha,
                  float beta, float diag, int symmetric, void *workspace,
                  int64_t workspace_bytes, void *stream);

/*
 * A batch of 1 <= batch <= DL_MAX_BATCH such products in one launch: matrix
 * b reads a + b*stride_a, b + b*stride_b (and y + b*stride_y, which is
 * either that matrix's own result or overlaps no result) and writes
 * c + b*stride_c (strides in elements, >= 0; the results must not overlap:
 * stride_c covers one result).  The workspace is that of
 * dl_matmul_workspace_bytes_batch; dl_matmul_f32 is the batch of one.
 * Errors: as dl_matmul_f32.
 */
int dl_matmul_workspace_bytes_batch(int64_t m, int64_t n, int64_t k, int symmetric, int batch,
                                    int64_t *bytes);

/*
 * *large = 1 when a batch of such products with 16-byte aligned, contiguous
 * operands (leading dimension k), diag = 0 and workspace_bytes of workspace
 * runs its main block on the large-tile kernel, else 0 (either form: the
 * rule does not depend on it).  For reports and tests; nothing is launched.  Errors:
 * as dl_matmul_workspace_bytes_batch, and DL_E_INVAL for a negative
 * workspace_bytes or a NULL large.
 */
int dl_matmul_large_tiles(int64_t m, int64_t n, int64_t k, int symmetric, int batch,
                          int64_t workspace_bytes, int *large);
int dl_matmul_f32_batch(int form, const float *a, int64_t lda, int64_t stride_a, const float *b,
                        int64_t ldb, int64_t stride_b, int64_t m, int64_t n, int64_t k, float *c,
                        int64_t ldc, int64_t stride_c, const float *y, int64_t stride_y,
                        float alpha, float beta, float diag, int symmetric, int batch,
                        void *workspace, int64_t workspace_bytes, void *stream);

/* Element range [offset, offset + length) of fragment frag.  DL_E_INVAL. */
int dl_frag_range(const dl_round *r, int frag, int64_t *offset, int64_t *length);

/*
 * Workers folded into fragment frag so far, in arrival order (round logs
 * identify participants, GradientMail post, "Getting updates through the
 * bucket").  *count receives the number; if workers is not NULL it receives
 * the ids and must hold capacity >= *count entries, else DL_E_CAPACITY.
 */
int dl_round_participants(const dl_round *r, int frag, int *count, int *workers,
                          int capacity);

/* Exact int64 sum of the token counts folded into fragment frag. DL_E_INVAL. */
int dl_round_tokens(const dl_round *r, int frag, int64_t *total_tokens);

/*
 * Release the handle (NULL is allowed).  Touches no device buffer and does
 * not wait for the stream: work already launched still completes.  A failed
 * round is recovered by a new round that re-folds the same arrivals in the
 * same order, which gives identical bits (the GradientMail post rebuilds a
 * failed round from its mailbox and then retries it, "Getting updates through
 * the bucket").
 */
int dl_round_end(dl_round *r);

/* Static description of a status code; never NULL. */
const char *dl_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* DLMERGE_H */
