/*
 * dlm.h -- C ABI of the per-iteration parallel-decoding step of a masked
 * diffusion language model, for AMD Instinct MI355X (gfx950).
 *
 * Sources.  The step follows the dInfer explainer (91haoming.cn, a summary of
 * arXiv 2510.08666):
 *   - decoding-strategy component: positions are fixed by the model's
 *     confidence in each position's text, with three strategies -- threshold
 *     decoding, hierarchical decoding (split the regions still to fill
 *     recursively and fix region centres first) and credit decoding (a credit
 *     per position and candidate, accumulated across iterations);
 *   - diffusion-iteration manager: fixed-size blocks are handled in turn;
 *     a block of L positions is the unit of one step.
 * One step = LM head z = h W^T over every row of the block, per-row candidate
 * (arg-max, lowest id on ties) and confidence (largest softmax probability),
 * then the sequence's commit policy, with at least one commit per step while
 * a position is still masked.
 *
 * Conventions for every entry point.
 *   - Tensors are dense, row-major, caller-owned DEVICE memory unless stated.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = null stream);
 *     calls are asynchronous: errors found while the kernels run surface on
 *     the stream, HIP-style.
 *   - Arguments are validated on the host BEFORE any HIP call; on a non-zero
 *     status nothing is enqueued and nothing is written.  dlm_last_error()
 *     then returns a message (thread-local).
 *   - The library never allocates device memory in these calls.  Its only
 *     mutable global state is the static scratch of dlm_decode_step_noalloc;
 *     calls of the other entry points on different streams must use
 *     different workspaces.
 */
#ifndef DLM_H
#define DLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DLM_VERSION_STRING "0.6.0"

#define DLM_MAX_SEQS 256   /* sequences per call                                  */
#define DLM_MAX_L 64       /* positions per block: one wavefront lane per position */
#define DLM_CREDIT_SLOTS 4 /* tracked (token, credit) candidates per position      */
#define DLM_MAX_RULES 8    /* distinct dlm_seq_policy values per call              */
#define DLM_MAX_TOPK 8     /* candidates per row in the top-k export               */
#define DLM_MAX_SHARDS 256 /* vocabulary shards one dlm_merge_commit call merges    */

/* Status codes. */
enum {
  DLM_OK = 0,
  DLM_ERR_NULL = -1,      /* a required pointer is NULL                              */
  DLM_ERR_DTYPE = -2,     /* dtype is not DLM_F32 / DLM_BF16                         */
  DLM_ERR_SHAPE = -3,     /* B, L, H or V outside the supported range                */
  DLM_ERR_POLICY = -4,    /* bad policy kind / parameter, or too many distinct rules */
  DLM_ERR_WORKSPACE = -5, /* workspace smaller than dlm_workspace_bytes()            */
  DLM_ERR_HIP = -6        /* the HIP runtime refused a launch                        */
};

/* Element type of hidden and W_vocab (both the same). */
enum { DLM_F32 = 0, DLM_BF16 = 1 };

/* Commit strategies (explainer, decoding-strategy component). */
enum { DLM_THRESHOLD = 0, DLM_HIERARCHICAL = 1, DLM_CREDIT = 2 };

/* dlm_policy.flags */
enum {
  /* A sequence whose mask is empty on entry starts its next block first: the
   * mask row is refilled with ones and its credit slots are cleared (explainer,
   * diffusion-iteration manager: fixed-size blocks in turn).  Without it such a
   * sequence commits nothing and nothing of it changes except out_tokens. */
  DLM_AUTO_ADVANCE = 1u
};

/* One tracked candidate of a position; token -1 marks an empty slot (credit 0). */
typedef struct {
  int32_t token;
  float credit;
} dlm_credit_slot;

/* The rule one sequence is decoded with. */
typedef struct {
  int32_t kind;      /* DLM_THRESHOLD / DLM_HIERARCHICAL / DLM_CREDIT                     */
  float threshold;   /* threshold, hierarchical: tau on conf; credit: theta on score     */
  float decay;       /* credit only: per-iteration credit factor, 0 <= decay < 1          */
  int32_t max_depth; /* hierarchical only: split depth limit, 0 = unbounded (runs = 1)    */
  int32_t eos_token; /* end token for early stop (needs dlm_policy.seq_done), -1 = none  */
} dlm_seq_policy;

/*
 * Early stop on the end token (explainer, engineering paragraph: once an end token appears in
 * the generated text the computation that would follow it is skipped).  With
 * dlm_policy.seq_done set, a sequence whose rule names an end token keeps a state:
 *   DLM_SEQ_RUNNING       decoding;
 *   DLM_SEQ_EOS_IN_BLOCK  the end token was committed in the current block;
 *   DLM_SEQ_FINISHED      the block containing the end token is complete: the sequence commits
 *                         nothing more, its mask and credit stay as they are and
 *                         DLM_AUTO_ADVANCE starts no new block for it (the caller resets the
 *                         state to reuse the slot).
 * A step that commits the end token also commits every still-masked position after the first
 * such position, and every position after it committed by that step carries the end token
 * (dlm_decode_step reports it in out_tokens; dlm_commit's caller applies it to its tokens).
 */
enum { DLM_SEQ_RUNNING = 0, DLM_SEQ_FINISHED = 1, DLM_SEQ_EOS_IN_BLOCK = 2 };

/* Shapes, per-sequence rules and launch context of one call. */
typedef struct {
  int64_t B;                 /* sequences, 1..DLM_MAX_SEQS                                 */
  int64_t L;                 /* positions per block, 1..DLM_MAX_L                          */
  int64_t H;                 /* hidden size, multiple of 32 (limits: see dlm_workspace_bytes) */
  int64_t V;                 /* vocabulary size, >= 1                                      */
  int32_t dtype;             /* DLM_F32 or DLM_BF16                                        */
  uint32_t flags;            /* DLM_AUTO_ADVANCE                                           */
  const dlm_seq_policy* seq; /* HOST array [B]; at most DLM_MAX_RULES distinct entries     */
  void* workspace;           /* device scratch, >= dlm_workspace_bytes(B, L, H, V, dtype)   */
  size_t workspace_bytes;    /* its size; must be zero-filled before its first use, and
                                serves calls of one shape (B, L, H, V, dtype, topk): another
                                shape needs its own workspace or a dlm_workspace_init first  */
  void* stream;              /* hipStream_t                                                */
  float* out_conf;           /* optional device [B][L]: confidence of every row, or NULL   */
  float* out_gap;            /* optional device [B][L]: top-1 minus top-2 logit, or NULL   */
  uint8_t* seq_done;         /* optional device [B], in/out: early-stop state (DLM_SEQ_*);
                                NULL disables early stop for every sequence                 */
  int32_t topk;              /* top-k export: 0 = off, 1..DLM_MAX_TOPK candidates per row   */
  int32_t* out_topk_tokens;  /* device [B][L][topk] int32 when topk > 0 (see below)         */
  float* out_topk_prob;      /* optional device [B][L][topk] float, or NULL                 */
  void* head_events[2];      /* optional hipEvent_t pair, each may be NULL (see below)      */
} dlm_policy;


/*
 * Timing the vocabulary head alone (dlm_decode_step and dlm_token_stats; the other calls ignore
 * the field).  head_events[0] is recorded on the stream right before the launch of the kernel
 * that streams W_vocab, head_events[1] right after it: the step kernel itself up to 64 rows (it
 * also merges and commits), the GEMM-shaped head beyond (between the hidden-row packing and the
 * merge + commit kernel).  The events are the caller's (created with hipEventCreate or a
 * framework's event type); hipEventElapsedTime of the pair is that kernel's duration.  A failed
 * record returns DLM_ERR_HIP.
 */

/*
 * Top-k candidate export (policy->topk > 0; dlm_decode_step, dlm_decode_steps and
 * dlm_token_stats).  The explainer's diffusion-iteration manager carries the information of the
 * candidates a step does not choose into the next iteration; the step exports that raw material
 * from the same pass over W_vocab.  For EVERY row (masked or not):
 *   out_topk_tokens[r][i]  the token with the i-th largest logit (float32), ties to the lower
 *                          id, so entry 0 is the candidate in out_tokens;
 *   out_topk_prob[r][i]    its softmax probability over the whole vocabulary,
 *                          exp(z - max z) / sum_v exp(z_v - max z), so entry 0 is the confidence;
 *   entries past V         token -1, probability 0.
 * The workspace must hold dlm_workspace_bytes_topk(B, L, H, V, dtype, topk) bytes.  Up to 64
 * rows (and in float32) the streaming LM head folds the lists next to the statistics in its one
 * kernel.  Beyond 64 bfloat16 rows with H % 256 == 0 and V < 2^22 the GEMM-shaped head keeps,
 * per row, lists of its best 16-logit chunks, and the finalizer recomputes (bit-identically) the
 * rare chunk that may hold a second top-k token; the extra workspace there is 64 bytes per row
 * (rows padded to the 512-row group) and GEMM workgroup: 8 MiB at 512 rows.
 * Errors: topk outside 0..DLM_MAX_TOPK gives DLM_ERR_POLICY, topk > 0 with out_topk_tokens NULL
 * gives DLM_ERR_NULL, a workspace smaller than the top-k size gives DLM_ERR_WORKSPACE.
 */

/*
 * One decode step.
 *   hidden       [B][L][H]   dtype    block hidden states (row b*L + l)
 *   W_vocab      [V][H]      dtype    vocabulary head
 *   mask_state   [B][L]      uint8    in/out: 1 = still masked; only 1 -> 0 changes
 *                                     (plus the refill of DLM_AUTO_ADVANCE)
 *   credit_state [B][L][4]   slots    in/out; only rows masked on entry change.
 *                                     May be NULL iff no sequence uses DLM_CREDIT.
 *   policy                            shapes, rules, workspace, stream, diagnostics
 *   out_tokens   [B][L]      int32    candidate (arg-max token) of EVERY row
 *   out_commit   [B][L]      uint8    1 where this call fixed the position
 * Every row goes through the LM head; the [B][L][V] logits never reach memory.
 * The workspace carries completion counters (one per call, or one per sequence beyond 64 rows)
 * that each call leaves at zero.
 * hidden and W_vocab must be finite: the kernels are built without NaN handling, so
 * NaN or Inf inputs give unspecified (but in-bounds, non-faulting) results.
 */
int dlm_decode_step(const void* hidden, const void* W_vocab, uint8_t* mask_state,
                    dlm_credit_slot* credit_state, const dlm_policy* policy, int32_t* out_tokens,
                    uint8_t* out_commit);

/*
 * dlm_decode_step for callers that cannot allocate device memory (code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid hipMalloc): the same step, with the workspace
 * taken from a static device array of DLM_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on (until the process ends) instead of policy->workspace.  policy->workspace and
 * workspace_bytes are ignored; every other argument and field means what it means for
 * dlm_decode_step, and the results are the same bits.
 *   - The array starts with a fixed 8 KB counter region; the rest of the workspace follows it.
 *     Shapes that need more than DLM_NOALLOC_SCRATCH_BYTES in that layout (the workspace of
 *     dlm_decode_step / dlm_workspace_bytes_topk plus at most 8 KB) give DLM_ERR_WORKSPACE
 *     before anything is enqueued.  Blocks of up to 16 x 32 rows at V = 157184, H = 2048 fit
 *     without the top-k export (4.2 MB), and one sequence of 32 rows with it (0.7 MB).
 *   - The call allocates and frees nothing.  The first call on a device looks up that device's
 *     copy of the array and enqueues a fill kernel on `stream` that zeroes its counter region;
 *     every call leaves the counters at zero again, so calls of different shapes may follow one
 *     another freely.
 *   - The current device (hipSetDevice) must be the device of `stream` and of the buffers.
 *   - All calls on one GPU share its array: calls that overlap in time on one GPU (different
 *     streams or threads without ordering between them) race and give wrong results.
 */
#define DLM_NOALLOC_SCRATCH_BYTES (8u << 20)
int dlm_decode_step_noalloc(const void* hidden, const void* W_vocab, uint8_t* mask_state,
                            dlm_credit_slot* credit_state, const dlm_policy* policy, int32_t* out_tokens,
                            uint8_t* out_commit);

/*
 * N decode steps enqueued back to back on policy->stream with no host work between them: the
 * iterations of a block run device-resident (the explainer's system-level optimisations remove
 * the idle time between diffusion iterations).  Step n reads hidden_steps[n], the hidden states
 * staged for that iteration, and writes out_tokens_steps[n] / out_commit_steps[n]; mask_state
 * and credit_state carry over on the device from one step to the next, and with
 * DLM_AUTO_ADVANCE a sequence whose block completed starts the next block in the following
 * step.  The result equals n_steps calls of dlm_decode_step.
 *   hidden_steps      [n_steps][B][L][H]  dtype
 *   out_tokens_steps  [n_steps][B][L]     int32
 *   out_commit_steps  [n_steps][B][L]     uint8
 *   n_steps           >= 1 (DLM_ERR_SHAPE otherwise)
 * policy->out_conf / out_gap, if set, hold the last step's values; with policy->topk > 0,
 * out_topk_tokens / out_topk_prob are [n_steps][B][L][topk], step n at offset n*B*L*topk.  Everything is validated
 * before the first launch; on error nothing is enqueued.  The call allocates nothing, waits for
 * nothing and records no memset, so it may be captured into a HIP graph and replayed.
 */
int dlm_decode_steps(const void* hidden_steps, const void* W_vocab, uint8_t* mask_state,
                     dlm_credit_slot* credit_state, const dlm_policy* policy, int64_t n_steps,
                     int32_t* out_tokens_steps, uint8_t* out_commit_steps);

/*
 * LM head + per-row statistics only (no commit): for every row, the
 * confidence, the candidate token and the top-2 logit gap, and with
 * policy->topk > 0 the top-k export.  policy->seq, flags, out_conf and
 * out_gap are ignored; out_gap may be NULL.
 */
int dlm_token_stats(const void* hidden, const void* W_vocab, const dlm_policy* policy,
                    float* out_conf, int32_t* out_tokens, float* out_gap);

/*
 * Commit policies only, from given per-row confidences and candidates
 * (conf [B][L] float, tokens [B][L] int32, device).  Same state semantics as
 * dlm_decode_step; out_tokens of that call equals `tokens` here.  policy->H,
 * V, dtype, workspace, out_conf, out_gap and the top-k fields are ignored.
 */
int dlm_commit(const float* conf, const int32_t* tokens, uint8_t* mask_state,
               dlm_credit_slot* credit_state, const dlm_policy* policy, uint8_t* out_commit);

/*
 * Vocabulary-sharded head (tensor parallelism over the vocabulary).  The explainer splits the
 * model over GPUs so that one request uses all of them; for the head, GPU g holds the contiguous
 * vocabulary range of shard g and produces one record per row, the records of all shards are
 * all-gathered (B*L * 16 bytes per GPU), and every GPU merges them identically and commits.
 * These two calls are the per-GPU parts; the exchange between them is the caller's.
 */
typedef struct {
  float max_logit;    /* largest logit over the shard                                      */
  float sum_exp;      /* sum over the shard of exp(z - max_logit), >= 1                    */
  int32_t token;      /* lowest GLOBAL token id attaining max_logit                        */
  float second_logit; /* second-largest logit of the shard, with multiplicity (-inf if the
                         shard has one token)                                              */
} dlm_shard_record;   /* 16 bytes */

/*
 * One GPU's share: the LM head over W_shard = rows [v_begin, v_begin + policy->V) of the full
 * vocabulary head, one record per row.
 *   hidden       [B][L][H]   dtype
 *   W_shard      [V][H]      dtype             policy->V = the shard's size
 *   v_begin      first global token id of the shard: >= 0, v_begin + V <= 2^31 - 1
 *   out_records  [B][L]      dlm_shard_record  16-byte aligned
 * policy->seq, flags, out_conf, out_gap and seq_done are ignored; topk must be 0
 * (DLM_ERR_POLICY otherwise).  Workspace: dlm_workspace_bytes(B, L, H, V_shard, dtype).
 */
int dlm_shard_stats(const void* hidden, const void* W_shard, int64_t v_begin, const dlm_policy* policy,
                    dlm_shard_record* out_records);

/*
 * The merge + commit after the exchange: records [n_shards][B][L] (shard g's out_records, the
 * shards in vocabulary order, as an all-gather leaves them) are merged per row in shard order by
 * the same merge the single-GPU head applies to its workgroups' records (largest logit, rescaled
 * sum, lowest id among the maxima, runner-up), then the commit policies run exactly as in
 * dlm_decode_step (same state semantics, out_conf / out_gap / seq_done included).
 *   n_shards     1..DLM_MAX_SHARDS (DLM_ERR_SHAPE otherwise)
 *   records      16-byte aligned (DLM_ERR_SHAPE otherwise)
 * policy->V is the FULL vocabulary (end tokens are checked against it); policy->H, dtype,
 * workspace and the top-k fields are ignored.  Every GPU that merges the same records in the
 * same order reaches the same mask, credit and outputs.
 */
int dlm_merge_commit(const dlm_shard_record* records, int64_t n_shards, uint8_t* mask_state,
                     dlm_credit_slot* credit_state, const dlm_policy* policy, int32_t* out_tokens,
                     uint8_t* out_commit);

/* Workspace bytes a call with these shapes needs (0 if the shapes are unsupported). */
size_t dlm_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t V, int32_t dtype);

/* Same for a call with policy->topk = topk (0 if unsupported or topk outside 0..DLM_MAX_TOPK);
   topk = 0 gives dlm_workspace_bytes. */
size_t dlm_workspace_bytes_topk(int64_t B, int64_t L, int64_t H, int64_t V, int32_t dtype, int32_t topk);

/* Zero-fill a workspace on `stream` (a fill kernel, safe under graph capture). */
int dlm_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Message of the last non-zero status on this thread ("" if none). */
const char* dlm_last_error(void);

/* Library version, DLM_VERSION_STRING. */
const char* dlm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DLM_H */
