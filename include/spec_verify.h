/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) verify-and-commit library for
 * batch speculative decoding.
 *
 * One call per step of the step's hot path; each call is a hand-written HIP
 * kernel.  Sources (web pages, cited by title and section):
 *   [Forensics]   "Correctness Forensics for Batch Speculative Decoding:
 *                 Diagnosing the Ragged Tensor Problem" (paper summary),
 *                 sections 3, 3.1, 3.2, App. B, App. D.
 *   [Walkthrough] zero-to-sglang "Chapter 10 Speculative Decoding (Code
 *                 Walkthrough)", sections 3.3, 4.1, 5.1, 5.2.
 *   [Atlas]       "Speculative decoding: proposals and verified output" (Atlas
 *                 lesson), The mechanism; Acceptance and rejection correction;
 *                 Interfaces.
 *   [Design]      speculative-decoding-real "Design Document", Standard Greedy
 *                 Algorithm; KV Cache Synchronization.
 *
 * Conventions shared by every call
 *   - Every array argument is a DEVICE pointer owned by the caller; the library
 *     allocates, frees and keeps nothing.  Scalars are host values.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream).  It returns after enqueueing its kernel, with no host sync.
 *   - Host-checkable argument errors return a negative code before anything is
 *     enqueued and before any HIP runtime call.  A failed kernel launch returns
 *     SPEC_EHIP.  Data-dependent anomalies never fail a call: they set per-
 *     sequence status bits (SPEC_ST_*).
 *   - Output arrays must not overlap input arrays or each other.
 *   - Workspaces ("ws") are device memory of at least the queried size, 256-byte
 *     aligned, holding per-call partial results.  Calls that may run at the
 *     same time (different streams) need different workspaces.
 *   - The greedy and the stochastic verification workspaces also carry the
 *     completion flags of their single launch: such a workspace must be
 *     zero-filled before its first use (e.g. hipMemset, torch.zeros) and no
 *     call of another kind may write into it; every completed call leaves it
 *     zero-filled again.  A greedy workspace may be shared with tree
 *     verification, whose workspace is of the same kind.  For verification
 *     from logits only the last
 *     spec_verify_sample_workspace_bytes(B, k, V) bytes are such flags; the
 *     leading part is rewritten by every call (so a workspace taken over from
 *     calls of another B, k or V is zero-filled again first).  Every other
 *     workspace's contents on entry are ignored.
 *   - A greedy verify call is one launch: streaming workgroups publish per-
 *     chunk results and one workgroup of the same launch commits them; tree
 *     verification does the same over whole trees.  Calls whose rows need
 *     more chunk results than that workgroup holds at once (more than 16384
 *     per sequence, or 1024 per tree) launch a streaming pass and a commit
 *     pass, synchronised by the stream order.
 *   - A stochastic verify call is one launch too: streaming workgroups publish
 *     the chunk masses of the row each sequence draws from, and one workgroup
 *     per sequence of the same launch, dispatched after them, draws.  The
 *     stochastic tree verification's workspace, when given, is of the same
 *     kind.  Verification from logits with top-k (K <= 256) takes two
 *     launches: the slices' candidate lists, then the row statistics and,
 *     in the same launch, the draw from the lists; with top-p alone a launch
 *     of the slices' exact weights comes between them.
 *   - Token ids are int32 in [0, V).  Layouts are row-major, last index fastest.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *spec_stream_t; /* hipStream_t */

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

/* return codes */
#define SPEC_OK 0
#define SPEC_EINVAL (-1)     /* bad pointer, size, alignment or overlap */
#define SPEC_EWORKSPACE (-2) /* ws_bytes below the queried size, or ws misaligned */
#define SPEC_ECAPACITY (-3)  /* a size exceeds a documented maximum */
#define SPEC_EHIP (-4)       /* the HIP runtime reported an error at launch */

/* per-sequence status bits (status[b]) */
#define SPEC_ST_DRAFT_OOR 1   /* a draft id outside [0, V): counted as mismatch / rejection */
#define SPEC_ST_Q_ZERO 2      /* q_j(x) == 0 at a proposed x: a = 1 if p_j(x) > 0, else 0 */
#define SPEC_ST_RESID_ZERO 4  /* the row drawn from had no positive mass; fallback used */
#define SPEC_ST_NONFINITE 8   /* a gathered probability or a drawn row's mass is not finite */
#define SPEC_ST_BAD_STATE 16  /* commit: n_b outside [0, E] or e_b outside [0, k+1] */
#define SPEC_ST_CAPACITY 32   /* commit: E < 0 or E + k + 1 > C */
#define SPEC_ST_INCOMPLETE 64 /* greedy or stochastic verify: a chunk result did not arrive
                                 within the call's wait bound (seconds); this sequence's
                                 outputs are unspecified (not expected in normal operation) */

#define SPEC_MAX_K 127          /* largest number of proposals k per sequence */
#define SPEC_GROUP_MAX_N 4096   /* largest window for spec_group_same_length */
#define SPEC_PROC_MAX_V 524288  /* largest vocabulary for the processed-distribution calls */
#define SPEC_TREE_MAX_N 256     /* largest candidate tree (nodes per sequence) */

/* Human-readable name of a return code. */
const char *spec_strerror(int code);

/* Bound on the polls of the single-launch greedy and tree verification's
 * committing workgroup (each poll is one round trip to memory, plus about
 * 0.2 us); polls <= 0 restores the default (about 4 s).  It applies to calls
 * launched afterwards, from any thread, and returns the previous setting
 * (0: the default).  Meant for tests of the incomplete path: a tiny bound
 * makes the commit stop waiting, count the chunk results still missing as
 * empty chunks and mark those sequences SPEC_ST_INCOMPLETE, while every
 * workgroup still ends normally. */
int spec_set_wait_bound(int polls);

/* ------------------------------------------------------------------------ *
 * Greedy verification.
 * [Walkthrough] 3.3 (row alignment) and 4.1 (greedy commitment); [Forensics]
 * App. D (BatchVerify).  Row j of sequence b verifies draft j; row k is the
 * bonus row (in a full-prefix forward over L confirmed tokens these are rows
 * L-1 .. L+k-1).  For each sequence: emit t_j = argmax(row j) for j = 0, 1, ...
 * and stop after emitting EOS, after emitting `remaining[b]` tokens, or after
 * the first j with t_j != draft[b, j]; if no stop happened, also emit
 * argmax(row k).  remaining[b] == 0 emits nothing; a negative remaining[b]
 * means no budget.  Ties: the lowest index among equal maxima; -0 == +0; a row
 * of -inf gives index 0; NaN inputs give unspecified results.
 *
 *   logits      [B, k+1, V] of dt (bf16 or f32), element-aligned
 *   draft       [B, k] int32
 *   eos_id      EOS token id, or -1 for none
 *   remaining   [B] int32 output budget, or NULL for none
 *   accept_len  [B]   out: number of accepted drafts m_b
 *   emit_count  [B]   out: number of emitted tokens e_b (0 .. k+1)
 *   out_tokens  [B, k+1] out: emitted tokens, -1 after the first e_b
 *   emit_offsets[B+1] out or NULL: exclusive prefix sum of emit_count
 *   status      [B]   out or NULL: SPEC_ST_DRAFT_OOR if any draft[b, j] is
 *                     outside [0, V)
 *   ws          workspace of spec_verify_greedy_workspace_bytes(B, k, V, dt),
 *               zero-filled before its first use (see the conventions above)
 *   status      also SPEC_ST_INCOMPLETE if the commit stopped waiting for a
 *               chunk result (a bound of seconds that normal operation never
 *               reaches; see spec_set_wait_bound).  Chunk results may still
 *               land in the workspace after such a call: zero-fill it again
 *               before its next use.
 * Errors: SPEC_EINVAL for NULL required pointers, B < 1, k < 1, V < 1,
 * V >= 2^31 - 1 or a misaligned logits pointer; SPEC_ECAPACITY for
 * k > SPEC_MAX_K; SPEC_EWORKSPACE.
 * ------------------------------------------------------------------------ */
size_t spec_verify_greedy_workspace_bytes(int B, int k, int V, spec_dtype dt);
int spec_verify_greedy(const void *logits, spec_dtype dt, int B, int k, int V,
                       const int32_t *draft, int32_t eos_id, const int32_t *remaining,
                       int32_t *accept_len, int32_t *emit_count, int32_t *out_tokens,
                       int32_t *emit_offsets, int32_t *status,
                       void *ws, size_t ws_bytes, spec_stream_t stream);

/* ------------------------------------------------------------------------ *
 * Greedy verification that allocates nothing and takes no workspace.
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, outputs and errors as spec_verify_greedy without ws / ws_bytes;
 * the chunk results live in a static device array of
 * SPEC_GREEDY_SCRATCH_BYTES per GPU (held until the process ends), so a call
 * needs spec_verify_greedy_workspace_bytes(B, k, V, dt) <=
 * SPEC_GREEDY_SCRATCH_BYTES, else it returns SPEC_ECAPACITY.  It launches the
 * streaming pass and the commit pass (two launches; no memory needs clearing
 * first).  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (different streams, threads) race and give undefined
 * results; calls in one stream are ordered and safe.  SPEC_EHIP if the
 * array's device address cannot be obtained.
 * ------------------------------------------------------------------------ */
#define SPEC_GREEDY_SCRATCH_BYTES (8u << 20)
int spec_verify_greedy_noalloc(const void *logits, spec_dtype dt, int B, int k, int V,
                               const int32_t *draft, int32_t eos_id, const int32_t *remaining,
                               int32_t *accept_len, int32_t *emit_count, int32_t *out_tokens,
                               int32_t *emit_offsets, int32_t *status, spec_stream_t stream);

/* ------------------------------------------------------------------------ *
 * Stochastic (Leviathan-style) verification.
 * [Atlas] The mechanism steps 2-5 and Acceptance and rejection correction;
 * [Walkthrough] 5.1.  For j = 0, 1, ...: x = draft[b, j],
 * a = min(1, p[b,j,x] / q[b,j,x]) (one IEEE float32 division); accept x iff
 * uniforms[b, j] < a.  At the first rejection emit one token drawn from the
 * positive residual r = max(p[b,j,:] - q[b,j,:], 0) and stop; after k
 * acceptances emit one token drawn from p[b,k,:].  A draw from mass vector r
 * with uniform u = uniforms[b, k] returns the smallest v whose inclusive prefix
 * sum exceeds u * S, S = sum(r) (both accumulated in float64 from the float32
 * r_v); if rounding leaves no such v, the last v with r_v > 0.  EOS and the
 * budget stop the round as in greedy verification (no draw after such a stop).
 * A residual with no positive mass falls back to drawing from p[b,j,:]
 * (SPEC_ST_RESID_ZERO); a row with no positive mass yields token 0.
 * q[b,j,x] == 0 gives a = 1 if p[b,j,x] > 0 else 0 (SPEC_ST_Q_ZERO); a draft id
 * outside [0, V) is rejected (SPEC_ST_DRAFT_OOR).
 *
 *   p           [B, k+1, V] float32 target probabilities (used as given)
 *   q           [B, k, V]   float32 draft probabilities
 *   draft       [B, k] int32
 *   uniforms    [B, k+1] float32 in [0, 1): u[b, j<k] decide acceptance,
 *               u[b, k] is the single draw for the correction or the bonus
 *   final_mass  [B] float64 out or NULL: S of the row drawn from, 0 if no draw
 *   other arguments as in spec_verify_greedy
 *   ws          workspace of spec_verify_sample_workspace_bytes(B, k, V)
 * Errors: as spec_verify_greedy (p, q, uniforms must be 4-byte aligned).
 * ------------------------------------------------------------------------ */
size_t spec_verify_sample_workspace_bytes(int B, int k, int V);
int spec_verify_sample(const float *p, const float *q, const int32_t *draft,
                       const float *uniforms, int B, int k, int V,
                       int32_t eos_id, const int32_t *remaining,
                       int32_t *accept_len, int32_t *emit_count, int32_t *out_tokens,
                       int32_t *emit_offsets, double *final_mass, int32_t *status,
                       void *ws, size_t ws_bytes, spec_stream_t stream);

/* ------------------------------------------------------------------------ *
 * Processed sampling distributions from raw logits.
 * [Walkthrough] 5.1: p and q must be the distributions actually sampled from;
 * when temperature, top-k or top-p is applied, the processed probabilities
 * are the ones verified.  The pages do not define the operations; the usual
 * definitions are used, in this order, for each row z of V logits:
 *   w(v)  = exp((z(v) - max z) / T)  (0 for z(v) = -inf), T = temperature > 0;
 *   top-k (top_k >= 1; 0 = off): keep v iff z(v) >= the top_k-th largest
 *         logit of the row, counting repeats (ties at the boundary are kept);
 *   top-p (0 < top_p < 1; 1 = off), among the top-k survivors: keep v iff the
 *         weight of the kept entries with a strictly larger logit is below
 *         top_p times their total weight (ties at the boundary are kept);
 *   p'(v) = w(v) / (sum of the kept w), 0 for dropped entries and for rows
 *         with no weight.
 * Arithmetic: w in float32, the accurate expf of (z - max z) / T with the
 * argument's rounding errors (the difference's, the product by 1/T's and that
 * of 1/T itself) folded back in to first order, so a weight is within
 * 2^-23 + 2^-24 relative of exp((z - max z) / T) whatever the argument; sums
 * and the top-p comparison use the weights truncated to 2^-40 units and added
 * exactly, so results are reproducible run to run.  Against a float64
 * evaluation, p' agrees to a relative 4.8e-7 + 9.1e-13 * V, and a top-p
 * boundary can differ only where the weight above it is within about
 * V * 2^-40 of top_p times the total.
 * Logits must be finite or -inf.
 *
 * spec_process_logits -- processes R rows:
 *   logits         [R, V] float32 or bf16 (dt), element-aligned
 *   probs          [R, V] float32 out or NULL: p'
 *   row_max        [R] float32 out or NULL: max z
 *   row_threshold  [R] float32 out or NULL: the smallest kept logit
 *   row_mass       [R] float64 out or NULL: sum of the kept w
 *   ws             workspace of spec_process_workspace_bytes(R, V)
 * Errors: SPEC_EINVAL for NULL logits or ws, R < 1, V < 1 or V >
 * SPEC_PROC_MAX_V, T not positive and finite, top_k < 0, top_p outside
 * (0, 1], misalignment or overlap; SPEC_EWORKSPACE.
 *
 * spec_verify_sample_logits -- stochastic verification (as spec_verify_sample)
 * on p' = processed target logits and q' = processed draft logits, both with
 * the same temperature, top_k and top_p; the processed rows are never stored.
 *   target_logits  [B, k+1, V] float32 or bf16 (dt)
 *   draft_logits   [B, k, V]   same dtype
 *   other arguments as in spec_verify_sample
 *   ws             workspace of spec_verify_sample_logits_workspace_bytes(B, k, V)
 * Errors: as spec_verify_sample, plus the processing errors above.
 * ------------------------------------------------------------------------ */
size_t spec_process_workspace_bytes(int R, int V);
int spec_process_logits(const void *logits, spec_dtype dt, int R, int V, float temperature,
                        int top_k, float top_p, float *probs, float *row_max,
                        float *row_threshold, double *row_mass, void *ws, size_t ws_bytes,
                        spec_stream_t stream);
size_t spec_verify_sample_logits_workspace_bytes(int B, int k, int V);
int spec_verify_sample_logits(const void *target_logits, const void *draft_logits, spec_dtype dt,
                              int B, int k, int V, float temperature, int top_k, float top_p,
                              const int32_t *draft, const float *uniforms, int32_t eos_id,
                              const int32_t *remaining, int32_t *accept_len,
                              int32_t *emit_count, int32_t *out_tokens, int32_t *emit_offsets,
                              double *final_mass, int32_t *status, void *ws, size_t ws_bytes,
                              spec_stream_t stream);

/* ------------------------------------------------------------------------ *
 * Commit: realign the contiguous left-padded KV cache, position ids and mask.
 * [Forensics] section 3 / 3.1 (rectangular alignment, position-id contiguity,
 * position/KV correspondence) and App. B (realignment keeps retained entries,
 * drops rejected ones, rebuilds positions from the mask; no shift under
 * uniform acceptance); App. D and [Walkthrough] 5.2 (the last emitted token
 * has no KV yet).
 * Before the call, sequence b's n_b cached rows sit at columns [E - n_b, E) of
 * every (layer, K/V, head) plane and the verify forward has written its k+1
 * slots at [E, E + k + 1).  With e_b = emit_count[b], M = max_b e_b and
 * E' = E + M, the call keeps the first e_b slots and moves columns
 * [E - n_b, E + e_b) to [E' - n_b - e_b, E'), in place (a right shift by
 * M - e_b columns; sequences with e_b == M do not move, and cells outside the
 * destination range are not written).  Then, over all C columns,
 * mask[b, c] = 1 iff E' - n'_b <= c < E' (n'_b = n_b + e_b), and
 * pos[b, c] = c - (E' - n'_b) there, 0 elsewhere.
 *
 *   kv          [L][2][B][H][C][D] of dt, modified in place
 *   k           proposals per sequence (the forward wrote k+1 slots)
 *   end_col     device scalar E (int32)
 *   kv_len_in   [B] int32 n_b
 *   emit_count  [B] int32 e_b (as written by a verify call)
 *   end_col_out device scalar out: E'
 *   kv_len_out  [B] out: n'_b
 *   pos_ids     [B, C] int32 out
 *   mask        [B, C] int32 out (1 / 0)
 *   bytes_moved device int64 out or NULL: sum over moved sequences of
 *               2 * n'_b * (L * 2 * H * D * element size)
 *   status      [B] out or NULL
 * If E < 0 or E + k + 1 > C (SPEC_ST_CAPACITY on every sequence) or some n_b
 * is outside [0, E] or e_b outside [0, k+1] (SPEC_ST_BAD_STATE on it), the call
 * writes only `status` and changes nothing else.
 * Errors: SPEC_EINVAL for NULL required pointers, L, B, H, C, D or k < 1, a kv
 * pointer not aligned to the element size, or outputs overlapping inputs.
 * ------------------------------------------------------------------------ */
int spec_commit_realign_kv(void *kv, spec_dtype dt, int L, int B, int H, int C, int D, int k,
                           const int32_t *end_col, const int32_t *kv_len_in,
                           const int32_t *emit_count, int32_t *end_col_out,
                           int32_t *kv_len_out, int32_t *pos_ids, int32_t *mask,
                           int64_t *bytes_moved, int32_t *status, spec_stream_t stream);

/* ------------------------------------------------------------------------ *
 * Ragged caches and the unpad-append-repad fallback.
 * [Forensics] 3.2: EXSPEC keeps sequences in ragged states and batches
 * sequences of identical length (no realignment); when no same-length group
 * forms it falls back to unpad-append-repad.  The ragged caches form one pool
 * [L][2][N][H][Cs][D] in which pool sequence s holds its rows at columns
 * [0, n_s) of each (layer, K/V, head) plane; a batch is B pool sequences
 * index[0..B) (distinct), in a rectangle [L][2][B][H][C][D].
 *
 * spec_repad_kv -- copies member i's rows [0, kv_len[i]) of pool sequence
 * index[i] to columns [E - kv_len[i], E) of rectangle sequence i, E the device
 * scalar end_col (left padding: cells outside those ranges are not written).
 *
 * spec_unpad_kv -- after the verify forward wrote k+1 slots at [E, E + k + 1)
 * of the rectangle and a verify call gave emit_count, copies member i's rows
 * [E - kv_len[i], E + emit_count[i]) (its cached rows and the slots it keeps,
 * as in spec_commit_realign_kv) to columns [0, kv_len[i] + emit_count[i]) of
 * its pool sequence, and writes kv_len_out[i] = kv_len[i] + emit_count[i].
 *
 *   pool        [L][2][N][H][Cs][D] of dt (read by repad, written by unpad)
 *   rect        [L][2][B][H][C][D] of dt (written by repad, read by unpad)
 *   index       [B] int32 pool sequence of each member
 *   kv_len      [B] int32 cached rows n_i of each member
 *   emit_count  [B] int32 (unpad)
 *   end_col     device scalar E (int32)
 *   kv_len_out  [B] int32 out (unpad): n_i + e_i (n_i for a rejected member)
 *   status      [B] out or NULL: SPEC_ST_CAPACITY if E < 0 or E > C;
 *               SPEC_ST_BAD_STATE if index[i] is outside [0, N), n_i outside
 *               [0, E], or (unpad) e_i < 0, E + e_i > C or n_i + e_i > Cs;
 *               such members are not copied.
 * Errors: SPEC_EINVAL for NULL required pointers, sizes < 1, buffers not
 * aligned to the element size, or outputs overlapping inputs.
 * ------------------------------------------------------------------------ */
int spec_repad_kv(const void *pool, void *rect, spec_dtype dt, int L, int N, int H, int Cs, int D,
                  int B, int C, const int32_t *index, const int32_t *kv_len, const int32_t *end_col,
                  int32_t *status, spec_stream_t stream);
int spec_unpad_kv(const void *rect, void *pool, spec_dtype dt, int L, int N, int H, int Cs, int D,
                  int B, int C, const int32_t *index, const int32_t *kv_len, const int32_t *emit_count,
                  const int32_t *end_col, int32_t *kv_len_out, int32_t *status, spec_stream_t stream);

/* ------------------------------------------------------------------------ *
 * Draft-cache re-sync.
 * [Design] Standard Greedy Algorithm step 7 and "KV Cache Synchronization":
 * after each step the draft model's cache must hold the accepted prefix,
 * copying the accepted entries (rather than re-running the draft).  An
 * autoregressive draft that proposed k tokens consumed the last confirmed token
 * and d_1..d_{k-1}, so its forward wrote k slots at columns [E, E + k) of its
 * own left-padded rectangle.  Sequence b keeps the first min(e_b, k) of them
 * (after full acceptance the draft has no entry for d_k yet and stays one
 * entry behind the target), and the rectangle is right-aligned to
 * E' = E + max_b min(e_b, k), exactly as spec_commit_realign_kv does with
 * min(e_b, k) kept slots:
 *   n'_b = n_b + min(e_b, k); bytes_moved counts the sequences that shift.
 *   kv          [L][2][B][H][C][D] draft cache (its own L, H, D), in place
 *   emit_count  [B] the target verification's e_b, in [0, k + 1]
 *   pos_ids, mask  [B, C] out or NULL (each may be NULL independently)
 *   other arguments as in spec_commit_realign_kv; needs E + k <= C.
 * Errors and status bits as spec_commit_realign_kv (SPEC_ST_CAPACITY when
 * E + k > C).
 * ------------------------------------------------------------------------ */
int spec_resync_draft_kv(void *kv, spec_dtype dt, int L, int B, int H, int C, int D, int k,
                         const int32_t *end_col, const int32_t *kv_len_in,
                         const int32_t *emit_count, int32_t *end_col_out, int32_t *kv_len_out,
                         int32_t *pos_ids, int32_t *mask, int64_t *bytes_moved, int32_t *status,
                         spec_stream_t stream);

/* ------------------------------------------------------------------------ *
 * Commit for a variable-length (paged) KV layout: rollback only.
 * [Forensics] section 2 and App. F: variable-length layouts need no
 * repadding, but rejected tokens must be rolled back in the position ids and
 * the KV cache.  In a paged cache that moves no KV bytes.  Before the verify
 * forward sequence b held n_b rows and the caller gave it pages for the k + 1
 * forward slots, so its first a_b = ceil((n_b + k + 1) / page_size) block-table
 * entries are in use.  It keeps n'_b = n_b + e_b rows (the last emitted token
 * has no KV yet, App. D); its next input position is n'_b; the entries
 * ceil(n'_b / page_size) .. a_b - 1 are released.
 *   kv_len_in      [B] n_b            emit_count [B] e_b in [0, k + 1]
 *   block_table    [B, max_pages] int32 page ids (row b lists b's pages in order)
 *   kv_len_out     [B] out: n'_b (also the next input position)
 *   pages_kept     [B] out: ceil(n'_b / page_size)
 *   freed_pages    out, room for B * ceil((k + 1) / page_size) ids: the
 *                  released entries, block-table order, sequences in order
 *   freed_offsets  [B + 1] out: sequence b's released ids are
 *                  freed_pages[freed_offsets[b] .. freed_offsets[b + 1])
 *   status         [B] out or NULL: SPEC_ST_BAD_STATE (n_b < 0 or e_b outside
 *                  [0, k + 1]) or SPEC_ST_CAPACITY (a_b > max_pages); such a
 *                  sequence keeps n_b and releases nothing.
 * Errors: SPEC_EINVAL for NULL required pointers, B, k, page_size or
 * max_pages < 1, sizes that overflow int32, overlapping outputs.
 * ------------------------------------------------------------------------ */
int spec_commit_paged(int B, int k, int page_size, int max_pages, const int32_t *kv_len_in,
                      const int32_t *emit_count, const int32_t *block_table, int32_t *kv_len_out,
                      int32_t *pages_kept, int32_t *freed_pages, int32_t *freed_offsets,
                      int32_t *status, spec_stream_t stream);

/* ------------------------------------------------------------------------ *
 * Greedy verification of a candidate tree, and compaction of its KV slots.
 * [Forensics] section 5 names tree-structured verification and [Walkthrough]
 * 5.2 the fields a tree verifier records (draft tokens, positions, a
 * visibility mask, retrieve_* links) without an algorithm.  Reading: the
 * greedy rule of [Walkthrough] 4.1 applied along the tree.  Each sequence has
 * N nodes in topological order; node 0 is the root (the last confirmed token)
 * and node i > 0 proposes draft[b, i]; first_child / next_sibling (-1 = none)
 * list each node's children in order, links pointing forward (to a larger
 * index below N).  Row i of the logits is the target's distribution after the
 * path ending at node i.  From the root: t = argmax of the current node's row
 * (lowest index on ties); the first child proposing t is accepted and becomes
 * the current node; otherwise t is emitted (correction, or bonus at a leaf)
 * and the round stops.  EOS and the budget stop it as in spec_verify_greedy.
 * A linear chain (node i's only child is i + 1) is exactly spec_verify_greedy.
 *
 * spec_verify_tree:
 *   logits       [B, N, V] float32 or bf16
 *   draft, first_child, next_sibling  [B, N] int32 (draft[b, 0] is ignored)
 *   out_tokens   [B, N] out, -1 padded; accept_len, emit_count [B] out
 *   path         [B, N] out, -1 padded: the nodes whose rows were read, from
 *                the root, one per emitted token (their KV slots are kept)
 *   emit_offsets [B + 1] out or NULL; status [B] out or NULL
 *                (SPEC_ST_DRAFT_OOR; SPEC_ST_BAD_STATE for links that do not
 *                point forward inside the tree: that sequence emits nothing;
 *                SPEC_ST_INCOMPLETE as in spec_verify_greedy, with the same
 *                zero-fill of the workspace before its next use)
 *   ws           workspace of spec_verify_tree_workspace_bytes(B, N, V, dt)
 * Errors: as spec_verify_greedy; SPEC_ECAPACITY for N > SPEC_TREE_MAX_N.
 *
 * spec_compact_tree_kv: the tree forward wrote node i's KV at column E + i of
 * the left-padded cache [L][2][B][H][C][D]; sequence b's slots
 * path[b, 0..e_b-1] are moved, in order, to columns E .. E + e_b - 1 (in
 * place), after which spec_commit_realign_kv(k = N - 1) commits as usual.
 *   end_col      device int32 E; path, emit_count as returned above
 *   status       [B] out or NULL: SPEC_ST_BAD_STATE when E + N > C, e_b is
 *                outside [0, N] or the path does not start at 0 and increase
 *                (that sequence is left unchanged)
 * Errors: SPEC_EINVAL for NULL pointers, sizes < 1, misalignment, overflow;
 * SPEC_ECAPACITY for N > SPEC_TREE_MAX_N.
 * ------------------------------------------------------------------------ */
size_t spec_verify_tree_workspace_bytes(int B, int N, int V, spec_dtype dt);
int spec_verify_tree(const void *logits, spec_dtype dt, int B, int N, int V, const int32_t *draft,
                     const int32_t *first_child, const int32_t *next_sibling, int32_t eos_id,
                     const int32_t *remaining, int32_t *accept_len, int32_t *emit_count,
                     int32_t *out_tokens, int32_t *path, int32_t *emit_offsets, int32_t *status,
                     void *ws, size_t ws_bytes, spec_stream_t stream);
int spec_compact_tree_kv(void *kv, spec_dtype dt, int L, int B, int H, int C, int D, int N,
                         const int32_t *end_col, const int32_t *path, const int32_t *emit_count,
                         int32_t *status, spec_stream_t stream);

/* ------------------------------------------------------------------------ *
 * Stochastic verification of a candidate tree.
 * [Forensics] 5 names tree verification and [Walkthrough] 5.2 lists the draft
 * tokens and their draft probabilities among a tree verifier's fields, but
 * neither gives the sampling rule.  This call implements multi-draft
 * speculative sampling: the children of a node, drawn independently from the
 * draft's distribution q at that node, are tried in sibling order against the
 * current residual of the target row there ([Atlas] Acceptance and rejection
 * correction; [Walkthrough] 5.1); every rejection replaces the residual by the
 * normalised positive part of (residual - q); an accepted child becomes the
 * current node; when no child is accepted, or at a leaf, one token is drawn
 * from the current residual and the round stops.  Every emitted token then
 * follows the target's row at its node.  A chain tree is exactly
 * spec_verify_sample.
 *   Residual mass vectors at the current node after i rejections: R_0 = p as
 *   given; R_1 = max(p - q, 0) in float32; R_j = max(R_{j-1} - q * m_{j-1}, 0)
 *   in float64 with m_j = sum of R_j (each operation separately rounded).  The
 *   first try compares u with min(1, p(x)/q(x)) (one float32 division); a try
 *   after i >= 1 rejections compares u with min(1, R_i(x) / (m_i * q(x))) in
 *   float64.  A rejection whose residual has no mass keeps the previous one
 *   (SPEC_ST_RESID_ZERO); a non-finite residual mass ends the round with token 0
 *   (SPEC_ST_NONFINITE).  Draws are the inverse CDF of spec_verify_sample.
 *   Trees, links, EOS, the budget and SPEC_ST_BAD_STATE are as in
 *   spec_verify_tree; q(x) == 0 and out-of-range drafts as in
 *   spec_verify_sample.
 *
 *   p            [B, N, V] float32: p[b, i] is the target's distribution after
 *                the path ending at node i
 *   q            [B, N, V] float32: q[b, i] is the draft's distribution at node
 *                i, which its children were drawn from (unused at leaves)
 *   draft, first_child, next_sibling  [B, N] int32 (draft[b, 0] is ignored)
 *   uniforms     [B, N] float32 in [0, 1): u[b, c] (c >= 1) decides the try
 *                of node c; u[b, 0] is the single draw
 *   out_tokens   [B, N] out, -1 padded; accept_len, emit_count [B] out
 *   path         [B, N] out, -1 padded: the nodes whose rows were read (their
 *                KV slots are kept; spec_compact_tree_kv applies)
 *   emit_offsets [B + 1] out or NULL; final_mass [B] float64 out or NULL: the
 *                mass S of the vector drawn from, 0 without a draw
 *   status       [B] out or NULL
 *   ws           NULL, or a workspace of
 *                spec_verify_tree_sample_workspace_bytes(B, N, V) bytes
 *                (zero-filled on first use, left zero-filled by every call;
 *                it carries completion flags, so no other kind of call may
 *                write into it)
 * Each sequence's tree is walked by one workgroup; each rejection reads the
 * node's p and q rows once.  With a workspace, and when the query returns a
 * nonzero size (small batches), up to 16 workgroups per sequence share those
 * passes, exchanging chunk masses through the workspace; the results are the
 * same.  The query returns 0 for shapes that run one workgroup per sequence
 * (then ws may be NULL or anything: it is not used).
 * Errors: SPEC_EINVAL for NULL required pointers, B, N or V < 1, misaligned
 * p, q or uniforms (4 bytes), overlapping outputs; SPEC_ECAPACITY for
 * N > SPEC_TREE_MAX_N or V > 4194304; SPEC_EWORKSPACE for a non-NULL ws
 * smaller than the query or not 256-byte aligned (when the query is nonzero).
 * ------------------------------------------------------------------------ */
size_t spec_verify_tree_sample_workspace_bytes(int B, int N, int V);
int spec_verify_tree_sample(const float *p, const float *q, const int32_t *draft,
                            const int32_t *first_child, const int32_t *next_sibling,
                            const float *uniforms, int B, int N, int V, int32_t eos_id,
                            const int32_t *remaining, int32_t *accept_len, int32_t *emit_count,
                            int32_t *out_tokens, int32_t *path, int32_t *emit_offsets,
                            double *final_mass, int32_t *status, void *ws, size_t ws_bytes,
                            spec_stream_t stream);

/* ------------------------------------------------------------------------ *
 * Same-length grouping of a window of ragged sequences.
 * [Forensics] 3.2 (EXSPEC: batches of identical-length sequences drawn from a
 * window larger than the batch size, with unpad-append-repad as the fallback).
 * The scheduler's own algorithm body is not given on the page; this call
 * implements the following reading.  Order the window's indices by
 * (length, index); cut each run of equal lengths into floor(count / B) full
 * batches, plus one smaller same-length batch if the remainder is at least
 * min_group, else send the remainder to a fallback list (in (length, index)
 * order); cut the fallback list into mixed batches of B (the last may be
 * short).  Same-length batches come first, in ascending length.
 *
 *   lengths     [N] int32 (any values)
 *   perm        [N] out: window indices in batch order
 *   batch_start [N + 1] out: batch t is perm[batch_start[t] .. batch_start[t+1])
 *   batch_len   [N] out: the shared length of batch t, or -1 for a mixed batch
 *   num_batches device int32 out
 *   num_grouped device int32 out: sequences placed in same-length batches
 * Entries of batch_start / batch_len past num_batches are not written.  With
 * N == 0, lengths, perm and batch_len may be NULL (nothing is read or written
 * there) and the call writes batch_start[0] = 0 and two zero counts.
 * Errors: SPEC_EINVAL for NULL pointers, N < 0, B < 1, min_group < 1;
 * SPEC_ECAPACITY for N > SPEC_GROUP_MAX_N.
 * ------------------------------------------------------------------------ */
int spec_group_same_length(const int32_t *lengths, int N, int B, int min_group,
                           int32_t *perm, int32_t *batch_start, int32_t *batch_len,
                           int32_t *num_batches, int32_t *num_grouped,
                           spec_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
