/*
 * rssm.h -- C ABI of librssm.so, the ReplaySSM decode-time state engine for
 * AMD MI355X (gfx950).
 *
 * Source of the method: "ReplaySSM: Cache SSM Inputs, Not State" (arXiv
 * abstract, mlsanity.com index page) and the frontier.agentik-os.com
 * explainer "ReplaySSM for hybrid SSM-Transformer stacks".  The state of a
 * sequence is a checkpoint plus a ring buffer of the SSM inputs received
 * since the checkpoint; outputs come from the checkpoint and a replay over
 * the buffer, so the state is not written on ordinary steps; a periodic
 * commit folds the buffer into a new checkpoint; speculative rollback only
 * moves the buffer tail; verification computes draft outputs from one
 * checkpoint read; a low-precision checkpoint may serve the output reads
 * while an fp32 checkpoint alone receives the folds.
 *
 * Layer types: Mamba-2 (SSD) and Gated DeltaNet (GDN), the two the pages
 * implement.  Their recurrences (not printed on the pages, which say so under
 * "What is not documented"; textbook forms of the layers listed under
 * "Builds on"):
 *   Mamba-2, head h, group g = h*G/H:  a = exp(dt*A_h);
 *       h_t = a h_{t-1} + dt x_t B_t^T  (P x N);   y_t = h_t C_t + D_h x_t
 *   GDN, head h:  S_t = alpha S_{t-1} (I - beta k k^T) + beta v k^T  (dv x dk);
 *       o_t = S_t q_t
 *
 * Conventions common to every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates and frees nothing, keeps no global state, and never
 *    synchronises implicitly (except rssm_status, which says so).
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *    null stream) and is asynchronous.  Calls on one layer must be ordered
 *    on one stream; distinct layers may be driven concurrently.
 *  - Apart from rssm_status, a call enqueues kernel launches and nothing else
 *    (no memset, copy or allocation), and the arrival counters are back at
 *    zero when each launch ends.  A sequence of calls may therefore be
 *    captured into a HIP graph on `stream` and replayed; the replay reads the
 *    captured pointers, so new inputs are written into the same buffers.
 *  - Row-major layouts, innermost index contiguous.  Tensors read or written
 *    with 16-byte vector accesses must be 16-byte aligned (EALIGN otherwise).
 *  - batch == 0 is valid: the call validates the descriptor's enums,
 *    dimensions and counts, and returns RSSM_OK without launching anything.
 *    Every per-sequence array then holds no elements and may be NULL.
 *  - Return codes (host-detected, returned before any launch, no side
 *    effects) are the RSSM_E* values below.  Errors that depend on device
 *    data (per-sequence buffer lengths) are reported through the layer's
 *    sticky `status` word instead.  For ring overflow, rollback past the
 *    checkpoint and unusable indices (RSSM_STATUS_INDEX, checked by every
 *    call that reads them) the offending sequence is left unchanged (no
 *    append, no fold, no index change) and its outputs are written as quiet
 *    NaN (commit and prefill leave their outputs and state untouched).
 */
#ifndef RSSM_H
#define RSSM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RSSM_ABI_VERSION 11
#define RSSM_ARRIVE_STRIDE 32   /* uint32 elements between two sequences' counters */
#define RSSM_NOALLOC_MAX_BATCH 4096  /* sequences served by rssm_mamba2_step_noalloc    */

/* ---- host return codes ------------------------------------------------- */
#define RSSM_OK            0
#define RSSM_EINVAL       (-1) /* null pointer, bad enum, bad or inconsistent dims */
#define RSSM_EUNSUPPORTED (-2) /* shape / scheme combination not instantiated     */
#define RSSM_EALIGN       (-3) /* a 16-byte-accessed pointer is misaligned         */
#define RSSM_ERANGE       (-4) /* n_pos < 1 or > capacity, n_tok < 1, min_len < 0  */
#define RSSM_EHIP         (-5) /* the HIP runtime reported a launch/copy error     */

/* ---- sticky device status bits (layer->status[0]) ---------------------- */
#define RSSM_STATUS_OVERFLOW  1u /* an append would exceed `capacity` entries       */
#define RSSM_STATUS_ROLLBACK  2u /* n_reject < 0 or n_reject > len (past checkpoint)*/
#define RSSM_STATUS_NONFINITE 4u /* non-finite state met while quantising to E4M3   */
#define RSSM_STATUS_INDEX     8u /* a sequence's indices are unusable: len < 0,      */
                                 /* len > capacity or ckpt_pos < 0                   */
/* On RSSM_STATUS_NONFINITE the head's E4M3 scale is set to 1 and its codes
 * saturate (+-inf -> +-448, NaN stays NaN); the fp32 checkpoint and the
 * indices are updated as for any commit or prefill.  bf16 copies carry inf
 * and NaN natively and raise no bit. */

typedef enum { RSSM_MAMBA2 = 1, RSSM_GDN = 2 } rssm_kind;

/* rssm_layer.flags (explainer, "How to think about using it": buffers per
 * layer or shared).  The layers of one model see the same tokens, rollbacks
 * and commits, so their buffer indices move in lockstep and may live in one
 * set of arrays.  A layer with RSSM_LAYER_INDEX_READONLY reads ckpt_pos and
 * len but never writes them and uses no arrival counters (arrive may be
 * NULL); its per-sequence errors are raised as usual.  Give every layer of a
 * stack the same ckpt_pos/len arrays, set the flag on all but one, and make
 * each call (step, commit, verify, append, prefill, rollback) on the layer
 * without the flag after the same call on the others, on the same stream:
 * that call moves the shared indices for the whole stack.  rssm_rollback on a
 * read-only layer validates its arguments and does nothing. */
#define RSSM_LAYER_INDEX_READONLY 1u

/* Checkpoint precision scheme (explainer, "Separate precisions for serving vs
 * updating state"; abstract: the low-precision copy serves outputs, the
 * higher-precision checkpoint alone serves recurrent updates). */
typedef enum {
  RSSM_F32 = 0,    /* one fp32 checkpoint serves outputs and receives folds        */
  RSSM_DUAL = 1,   /* ckpt_lp serves outputs; ckpt (fp32) alone receives folds;    */
                   /* each commit re-quantises ckpt_lp from the new fp32 state     */
  RSSM_SHARED = 2  /* ckpt_lp is the only checkpoint: outputs read it, commits     */
                   /* fold from its dequantised value and re-quantise (comparator) */
} rssm_scheme;

typedef enum {
  RSSM_LP_NONE = 0,
  RSSM_BF16 = 1,   /* bfloat16, round to nearest even                              */
  RSSM_E4M3 = 2    /* OCP FP8 E4M3 with one fp32 scale per (sequence, head):       */
                   /* scale = amax|S|/448 (1 if amax == 0), code = E4M3(S/scale),  */
                   /* saturating, round to nearest even; value = code * scale      */
} rssm_lp;

/*
 * One SSM layer's state, all device memory owned by the caller.
 *
 * Dimensions
 *   batch     sequences;  nheads  heads per sequence
 *   ngroups   Mamba-2: groups sharing B and C (head h uses group h*ngroups/nheads,
 *             nheads % ngroups == 0);  GDN: must be 1
 *   dim_v     Mamba-2: headdim P;  GDN: dv  (rows of the state)
 *   dim_k     Mamba-2: dstate N;   GDN: dk  (columns of the state)
 *   capacity  ring slots per sequence (1..16; a Mamba-2 layer with an fp32
 *             checkpoint may have up to 32 for rssm_mamba2_step[_noalloc],
 *             rssm_commit and rssm_rollback, the calls of plain decoding;
 *             every other call returns RSSM_EUNSUPPORTED above 16); entry j
 *             since the checkpoint lives in slot (ckpt_pos + j) % capacity
 *   Instantiated: Mamba-2 P=64, N=128; GDN dk=dv=128; all schemes for both;
 *   batch * nheads <= 2^30 - 1 (RSSM_EUNSUPPORTED above: some launches take
 *   two workgroups per head).
 *
 * Checkpoints  [batch][nheads][dim_v][dim_k]
 *   ckpt      fp32; required for F32 and DUAL, NULL for SHARED
 *   ckpt_lp   uint16 bf16 bits or uint8 E4M3 codes; required for DUAL/SHARED
 *   lp_scale  fp32 [batch][nheads]; required for E4M3
 * Per-head parameters (Mamba-2 only): A[nheads] (negative decay rate),
 *   D[nheads] (skip); NULL for GDN.
 * Ring buffers (fp32)
 *   Mamba-2: ring[0] = x  [batch][nheads][capacity][P]
 *            ring[1] = B  [batch][ngroups][capacity][N]
 *            ring[2] = dt [batch][nheads][capacity]      ring[3] unused (NULL)
 *   GDN:     ring[0] = k  [batch][nheads][capacity][dk]
 *            ring[1] = v  [batch][nheads][capacity][dv]
 *            ring[2] = alpha, ring[3] = beta  [batch][nheads][capacity]
 *   (C and q are not buffered: only the current token's output uses them.)
 * Indices
 *   ckpt_pos  int64 [batch]  absolute token position of the checkpoint
 *   len       int32 [batch]  entries buffered since the checkpoint
 *   arrive    uint32 [batch][RSSM_ARRIVE_STRIDE] scratch counters (element
 *             [b][0] is sequence b's; one 128-byte line per sequence, because
 *             atomics to one line are serialised); must be zero before the
 *             first call and are left zero by every call, whatever the
 *             indices hold (the last workgroup of a sequence to finish
 *             updates its indices)
 *   status    uint32 [1]     sticky RSSM_STATUS_* bits
 */
typedef struct rssm_layer {
  int32_t kind, scheme, lp_dtype;
  int32_t batch, nheads, ngroups, dim_v, dim_k, capacity;
  int32_t flags;      /* 0 or RSSM_LAYER_INDEX_READONLY; other bits: RSSM_EINVAL */
  float* ckpt;
  void* ckpt_lp;
  float* lp_scale;
  const float* A;
  const float* D;
  float* ring[4];
  int64_t* ckpt_pos;
  int32_t* len;
  uint32_t* arrive;
  uint32_t* status;
} rssm_layer;

/* Per-position inputs for rssm_verify / rssm_prefill / rssm_eager_step.
 * Unused members NULL.
 * Mamba-2: x [n][batch][H][P], B and C [n][batch][G][N], dt [n][batch][H]
 * GDN:     q, k [n][batch][H][dk], v [n][batch][H][dv], alpha, beta [n][batch][H]
 * (n = n_pos for verify, n_tok for prefill, 1 for eager_step). */
typedef struct rssm_inputs {
  const float *x, *B, *C, *dt;
  const float *q, *k, *v, *alpha, *beta;
} rssm_inputs;

/*
 * rssm_mamba2_step -- one decode token for every sequence of a Mamba-2 layer.
 * Explainer "Compute outputs without eagerly updating the checkpoint": append
 * the step's SSM input to the buffer, then compute the output from the
 * checkpoint and a replay over the buffer; the checkpoint is not written.
 *   y_t = Gamma_{c+1..t} h_c C_t + sum_i Gamma_{i+1..t} dt_i (B_i . C_t) x_i + D x_t
 *   with Gamma_{m..n} = exp(A * sum_{j=m..n} dt_j), i over the buffered entries
 *   including this one.
 * x [batch][H][P], B and C [batch][G][N], dt [batch][H] (the discretisation
 * step, already positive: no bias or softplus is applied); y [batch][H][P].
 * commit_after != 0: after computing y, fold the whole buffer (this entry
 * included) into the fp32 checkpoint in the same pass over the state and
 * reset the buffer (explainer, "Periodically commit a new checkpoint").
 * Per sequence, len + 1 > capacity sets RSSM_STATUS_OVERFLOW (y = NaN, no
 * append).  Output reads use ckpt (F32) or ckpt_lp (DUAL, SHARED; E4M3 values
 * are code * lp_scale).  commit_after is supported for F32 and DUAL
 * (RSSM_EUNSUPPORTED for SHARED; use rssm_commit).  Under DUAL the committing
 * step reads the fp32 checkpoint, which it folds anyway, and takes its output
 * from it; afterwards ckpt_lp holds the image of the new fp32 checkpoint, as
 * after rssm_commit.
 */
int rssm_mamba2_step(const rssm_layer* L, const float* x, const float* B,
                     const float* C, const float* dt, float* y,
                     int commit_after, void* stream);

/*
 * rssm_mamba2_step_noalloc -- rssm_mamba2_step for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops that
 * must not allocate, harnesses that forbid it.  Same arguments, results and
 * errors as rssm_mamba2_step, except that the arrival counters are the
 * library's own instead of L->arrive (ignored, may be NULL): a file-scope
 * device array with room for RSSM_NOALLOC_MAX_BATCH sequences (512 KiB on each
 * device that runs the call, held until the process ends).  The call first
 * zeroes the counters of sequences 0..batch-1 with a small kernel on
 * `stream`, then launches the step; it allocates nothing and calls no memset
 * or copy.  batch > RSSM_NOALLOC_MAX_BATCH gives RSSM_ERANGE.  Every call on a
 * device shares that device's counters: calls that overlap in time on one
 * device (other streams, other threads) race and corrupt each other's index
 * updates; serialise them.
 */
int rssm_mamba2_step_noalloc(const rssm_layer* L, const float* x, const float* B,
                             const float* C, const float* dt, float* y,
                             int commit_after, void* stream);

/*
 * rssm_gdn_step -- one decode token for every sequence of a GDN layer.
 * Same contract as rssm_mamba2_step.  The output is formed by carrying the
 * query backwards through the buffered entries (newest first):
 *   s_i = beta_i (k_i . q);  q <- alpha_i (q - s_i k_i);   o_t = S_c q + sum_i s_i v_i
 * q, k [batch][H][dk] (unit-norm is the caller's business), v [batch][H][dv],
 * alpha, beta [batch][H]; o [batch][H][dv].
 * Output reads use ckpt (F32) or ckpt_lp (DUAL, SHARED).  commit_after as
 * for rssm_mamba2_step (F32 and DUAL).
 */
int rssm_gdn_step(const rssm_layer* L, const float* q, const float* k,
                  const float* v, const float* alpha, const float* beta,
                  float* o, int commit_after, void* stream);

/*
 * rssm_commit -- fold buffers into new checkpoints (explainer, "Periodically
 * commit a new checkpoint": apply the recurrence from the checkpoint across
 * every buffered input, write the result as the new checkpoint, reset the
 * buffer).  A sequence is folded when mask == NULL or mask[b] != 0, and
 * len[b] >= min_len.  Then ckpt_pos += len, len = 0.
 *   F32:    ckpt <- fold(ckpt)
 *   DUAL:   ckpt <- fold(ckpt);  ckpt_lp <- Q(ckpt)      (fp32 alone is updated)
 *   SHARED: ckpt_lp <- Q(fold(deQ(ckpt_lp)))
 * A selected sequence with len == 0 keeps its fp32 state; under DUAL its
 * low-precision copy is refreshed from fp32 (use min_len = 0 once to
 * initialise ckpt_lp).  mask: device uint8 [batch] or NULL.
 */
int rssm_commit(const rssm_layer* L, const uint8_t* mask, int min_len,
                void* stream);

/*
 * rssm_verify -- verification of n_pos draft tokens by their outputs alone
 * (abstract; explainer "Cheap speculative decoding rollback": draft outputs
 * are recomputed from the checkpoint and the buffered inputs, and no
 * intermediate state is stored or reloaded).  Appends the n_pos draft
 * inputs at entries len..len+n_pos-1 and writes, for every draft position j,
 * the output the layer would produce after drafts 0..j, reading the
 * checkpoint once.  No state is written; len += n_pos.
 * in: see rssm_inputs (leading [n_pos]); out [n_pos][batch][H][dim_v].
 * 1 <= n_pos <= min(8, capacity) (RSSM_ERANGE).  Per sequence,
 * len + n_pos > capacity sets RSSM_STATUS_OVERFLOW (outputs NaN, no append).
 * Mamba-2 and GDN, all schemes (DUAL and SHARED read ckpt_lp).
 */
int rssm_verify(const rssm_layer* L, int n_pos, const rssm_inputs* in,
                float* out, void* stream);

/*
 * rssm_verify_commit -- rssm_verify preceded, for every sequence whose buffer
 * holds len >= min_len entries, by the commit of those entries (explainer,
 * "Periodically commit a new checkpoint"), both from one read of the
 * checkpoint: the kernel folds the buffered entries into the checkpoint
 * while it streams it for the draft outputs, so a speculative loop that
 * commits a full buffer at its next verify reads the state once per round
 * instead of twice in the rounds that commit.  For such a sequence
 * ckpt_pos += len and len = n_pos afterwards (the drafts keep their ring
 * slots); for the others len += n_pos as in rssm_verify.  Outputs, indices
 * and checkpoints equal rssm_commit(L, NULL, min_len) followed by
 * rssm_verify, up to fp32 rounding of the outputs.  Both layer types, F32
 * checkpoints only (RSSM_EUNSUPPORTED otherwise); min_len >= 1 (RSSM_ERANGE);
 * other arguments and errors as for rssm_verify (an overflowing sequence is
 * neither committed nor appended).
 */
int rssm_verify_commit(const rssm_layer* L, int n_pos, const rssm_inputs* in, float* out,
                       int min_len, void* stream);

/*
 * rssm_rollback_verify_commit -- rssm_rollback(L, n_reject) followed by
 * rssm_verify_commit(L, n_pos, in, out, min_len), in one launch.  A
 * speculative loop passes each round's rejection counts with the next
 * round's drafts: a rollback only moves the buffer tail (explainer, "Cheap
 * speculative decoding rollback"), and the verify reads the buffer indices
 * anyway, so it applies len -= n_reject before it folds and appends.
 * Indices, rings, checkpoints, outputs and status bits are bitwise those of
 * the two calls, errors included: a sequence whose n_reject[b] is < 0 or
 * > len sets RSSM_STATUS_ROLLBACK and keeps its len, and is then verified
 * as rssm_verify_commit would verify it; a valid rollback stands when the
 * drafts then overflow (RSSM_STATUS_OVERFLOW, outputs NaN, no append).
 * n_reject: device int32 [batch], caller-owned, read only; NULL is
 * RSSM_EINVAL.  On a layer with RSSM_LAYER_INDEX_READONLY the rejections are
 * applied to the indices the call reads and nothing is written: the layer
 * that owns the shared indices applies the same rollback when its own call,
 * the last of the stack, runs (rssm_rollback alone does nothing there).  A min_len above the capacity never folds (a fused rollback
 * with plain verification).  Other arguments and errors as for
 * rssm_verify_commit (F32 checkpoints only).
 */
int rssm_rollback_verify_commit(const rssm_layer* L, const int32_t* n_reject, int n_pos,
                                const rssm_inputs* in, float* out, int min_len, void* stream);

/*
 * rssm_verify_tree -- output-only verification of a tree of drafts from one
 * checkpoint read (explainer, "Why this matters for agentic systems now":
 * replay from a shared checkpoint along different input buffers, then
 * discard branches by moving pointers).  Draft j hangs below draft
 * parent[j] (parent[j] < j), or below the buffer tail when parent[j] == -1;
 * its output is the layer output after the buffered entries and the drafts
 * on its path (root first, j last).  parent: HOST int32 [n_nodes], the same
 * tree for every sequence; in: as rssm_verify with leading [n_nodes];
 * out [n_nodes][batch][H][dim_v].  Nothing is appended and no index changes:
 * the caller appends the accepted path with rssm_append_path; rejected
 * branches are never written.  1 <= n_nodes <= min(8, capacity)
 * (RSSM_ERANGE); a bad parent gives RSSM_EINVAL.  Per sequence,
 * len + n_nodes > capacity sets RSSM_STATUS_OVERFLOW (outputs NaN).
 */
int rssm_verify_tree(const rssm_layer* L, int n_nodes, const int32_t* parent,
                     const rssm_inputs* in, float* out, void* stream);

/*
 * rssm_verify_tree_commit -- rssm_verify_tree preceded, for every sequence
 * whose buffer holds len >= min_len entries, by the commit of those entries,
 * both from one read of the checkpoint (as rssm_verify_commit does for a
 * chain).  For such a sequence ckpt_pos += len and len = 0 afterwards; the
 * caller then appends the accepted path with rssm_append_path at the new
 * buffer's entries 0..  With a chain parent array (-1, 0, 1, ...) it serves a
 * speculative loop that writes only the accepted drafts to the ring: no
 * rejected draft is appended and no rollback is needed.  Outputs, indices and
 * checkpoints equal rssm_commit(L, NULL, min_len) followed by
 * rssm_verify_tree, up to fp32 rounding of the outputs.  F32 checkpoints only
 * (RSSM_EUNSUPPORTED otherwise); min_len >= 1 (RSSM_ERANGE); other arguments
 * and errors as for rssm_verify_tree (an overflowing sequence is not folded).
 */
int rssm_verify_tree_commit(const rssm_layer* L, int n_nodes, const int32_t* parent,
                            const rssm_inputs* in, float* out, int min_len, void* stream);

/*
 * rssm_append_path -- append, for every sequence b, the inputs of drafts
 * path[b][0 .. path_len[b]) (indices into the verify inputs `in`, leading
 * [n_nodes]) at the buffer tail, in that order: len += path_len[b].  For
 * an accepted root-to-node path of rssm_verify_tree this leaves the layer as
 * plain decoding of the accepted tokens would.  path: device int32
 * [batch][depth]; path_len: device int32 [batch], 0..depth.
 * 1 <= depth <= n_nodes <= 8 (RSSM_ERANGE).  Per sequence, a path that
 * overflows the ring or names a draft outside 0..n_nodes-1 sets
 * RSSM_STATUS_OVERFLOW and leaves the sequence unchanged.  Uses x, B, dt
 * (Mamba-2) or k, v, alpha, beta (GDN) of `in`; x and B (k and v) are read
 * with 16-byte accesses and must be 16-byte aligned (RSSM_EALIGN).
 */
int rssm_append_path(const rssm_layer* L, int n_nodes, const int32_t* path,
                     const int32_t* path_len, int depth, const rssm_inputs* in,
                     void* stream);

/*
 * rssm_prefill -- fold a prompt into the checkpoint of every selected
 * sequence.  The pages describe decode only; a prefill is read as a commit
 * over a long buffer (explainer, "Periodically commit a new checkpoint":
 * apply the recurrence from the checkpoint across the inputs and store the
 * result) whose prompt tokens also get their outputs.  A sequence is selected
 * when mask == NULL or mask[b] != 0 (mask: device uint8 [batch]).  For a
 * selected sequence the state continues from its checkpoint over its len
 * buffered entries (oldest first; they get no output) and then over the
 * n_tok prompt tokens of `in` (leading [n_tok], laid out as for rssm_verify);
 * out[t] (leading [n_tok], laid out as rssm_verify's; may be NULL) receives
 * prompt token t's output, the value plain decoding of the same tokens gives.
 * Afterwards ckpt_pos += len + n_tok and len = 0.
 *   F32:    ckpt <- fold(ckpt)
 *   DUAL:   ckpt <- fold(ckpt);  ckpt_lp <- Q(ckpt)   (outputs from fp32)
 *   SHARED: ckpt_lp <- Q(fold(deQ(ckpt_lp)))         (outputs from the decoded copy)
 * The state stays on chip in fp32 for the whole prompt: one read and one
 * write of the checkpoint per call.  Unselected sequences, and their rows of
 * out, are not touched.  n_tok >= 1 (RSSM_ERANGE).  Mamba-2 uses x, B, dt
 * and, when out != NULL, C; GDN uses k, v, alpha, beta and, when out != NULL,
 * q.  An E4M3 tile holding NaN or an infinity sets RSSM_STATUS_NONFINITE.
 */
int rssm_prefill(const rssm_layer* L, int n_tok, const rssm_inputs* in, float* out,
                 const uint8_t* mask, void* stream);

/*
 * rssm_rollback -- reject the last n_reject[b] buffered entries of every
 * sequence by moving the buffer tail: len -= n_reject (explainer, "Cheap
 * speculative decoding rollback": rejecting k tokens only moves the tail
 * back by k; the checkpoint is left as it was).
 * Ring contents and checkpoints are not touched.  n_reject: device int32
 * [batch].  n_reject < 0 or > len sets RSSM_STATUS_ROLLBACK and leaves that
 * sequence unchanged.
 */
int rssm_rollback(const rssm_layer* L, const int32_t* n_reject, void* stream);

/*
 * rssm_eager_step -- the eager baseline the pages compare against (explainer,
 * "What ReplaySSM is solving": read the entire state, update it with the
 * current input, write it back, every step).  Rewrites the checkpoint in
 * place and writes the step output; rings and indices are ignored.
 * in: one token (n = 1); out: y [batch][H][P] or o [batch][H][dv].
 * F32 and DUAL update the fp32 checkpoint `ckpt`.  SHARED is the comparator
 * that keeps the recurrent state in low precision only (explainer, "What
 * ReplaySSM is solving": the rounding then feeds every later update): ckpt_lp
 * is decoded, updated in fp32, the output is taken from the updated values,
 * and the result is re-encoded into ckpt_lp (and lp_scale).
 */
int rssm_eager_step(const rssm_layer* L, const rssm_inputs* in, float* out,
                    void* stream);

/*
 * rssm_status -- synchronise `stream`, copy the layer's sticky status word to
 * *bits (host pointer), then clear it on the device.  Blocking.
 */
int rssm_status(const rssm_layer* L, uint32_t* bits, void* stream);

/* Static description of a return code.  Never NULL. */
const char* rssm_strerror(int code);

/*
 * rssm_eager_spec_round / rssm_eager_spec_accept -- the eager comparator for
 * speculative decoding.  Without a checkpoint and an input buffer, verifying
 * drafts while keeping the option to roll back means materialising the state
 * after every draft (Abstract: ReplaySSM verifies drafts from their outputs
 * without materialising intermediate states).  The comparator keeps each
 * sequence's state in a ring of n_pos + 1 caller-owned state slots
 * (`slots`: device fp32 [n_pos + 1][batch][H][dim_v][dim_k]); cur[b] (device
 * int32 [batch], 0..n_pos) names the slot holding sequence b's state.
 *   round:  read slot cur[b] once, apply drafts j = 0..n_pos-1 with the eager
 *           recurrence, write out[j] (laid out as rssm_verify's) and the state
 *           after draft j to slot (cur[b] + 1 + j) % (n_pos + 1);
 *   accept: cur[b] = (cur[b] + n_accept[b]) % (n_pos + 1), n_accept device
 *           int32 [batch] in 0..n_pos; the state after the last accepted draft
 *           becomes current.
 * One state read and n_pos state writes per round, against ReplaySSM's one
 * read.  n_pos must be the same in both calls and in every round on the same
 * slots.  F32 layers only (RSSM_EUNSUPPORTED otherwise); 1 <= n_pos <= 8
 * (RSSM_ERANGE).  The layer's rings, indices and checkpoint are not used.  A
 * cur[b] or n_accept[b] out of range sets RSSM_STATUS_ROLLBACK and leaves the
 * sequence unchanged (its outputs NaN).  Inputs as for rssm_verify.
 */
int rssm_eager_spec_round(const rssm_layer* L, int n_pos, const rssm_inputs* in, float* out,
                          float* slots, const int32_t* cur, void* stream);
int rssm_eager_spec_accept(const rssm_layer* L, int n_pos, int32_t* cur, const int32_t* n_accept,
                           void* stream);

/*
 * rssm_probe_stream -- a measurement utility, not part of the method: streams
 * `bytes` (a multiple of 32 KiB, 16-byte aligned) from `src` with the replay
 * step's workgroup shape and load pattern (256 threads, 32 KiB per
 * workgroup, 16-byte nontemporal loads).  dst != NULL: copies to dst (same
 * size and alignment).  dst == NULL: reads only and writes one float per
 * wave to `sink` (device, bytes / 8 KiB floats).  Gives the streaming ceilings
 * against which the state kernels' HBM fractions can be read.
 * RSSM_EINVAL for NULL src (or sink when dst is NULL), RSSM_EALIGN, RSSM_ERANGE
 * for a size that is not a positive multiple of 32 KiB.
 */
int rssm_probe_stream(const void* src, void* dst, float* sink, int64_t bytes, void* stream);

/*
 * rssm_probe_stream_tiles -- as rssm_probe_stream with a choice of workgroup
 * tile: tile_bytes = 32768 is rssm_probe_stream; tile_bytes = 4096 gives every
 * thread of a 256-thread workgroup a single 16-byte load (a pure stream whose
 * waves live for one memory round trip; the fastest read shape measured on
 * the MI355X, shown next to the step's own shape).  `bytes` must be a
 * positive multiple of tile_bytes.  With dst == NULL the sink holds one float
 * per wave (bytes / (tile_bytes / 4) floats): check != 0 writes every wave's
 * XOR fold of its words there, as rssm_probe_stream does; check == 0 (for
 * timing) writes only the folds that equal 0x9E3779B9, so that the read
 * stream carries no stores.  RSSM_EUNSUPPORTED for another tile size; other
 * errors as for rssm_probe_stream.
 */
int rssm_probe_stream_tiles(const void* src, void* dst, float* sink, int64_t bytes,
                           int32_t tile_bytes, int32_t check, void* stream);

/* RSSM_ABI_VERSION of the loaded library. */
int rssm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RSSM_H */
