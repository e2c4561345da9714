/*
 * ra.h -- C ABI of libringattn: one context-parallel rank's share of blockwise causal
 * self-attention (the ring "p2p" mode), on one AMD Instinct MI355X (gfx950).
 *
 * The method (pages cited by title and section):
 *  - Ring attention, p2p mode: K/V chunks circulate around the CP ring; each step a rank
 *    folds the chunk it holds into its running output with a single-pass online softmax,
 *    and the backward recomputes probabilities and returns K/V gradients to the chunk's
 *    owner.  InfiniTrain pull request "Feat: Context Parallel", section 主要改动 (main
 *    changes), the mode table; lecture note "上下文并行", section "朴素 Ring Attention".
 *  - Sequence layouts: contiguous (default) or zigzag head/tail pairing of 2*cp chunks
 *    ("Feat: Context Parallel" 主要改动; "上下文并行" section "Zig-Zag Ring Attention").
 *  - GQA: n_rep = heads_q / heads_kv; query head h reads key/value head h / n_rep, handled
 *    inside the kernels instead of a repeated-heads copy ("Feat: Context Parallel", review
 *    thread on the attention helper and its RepeatKVHeads gradient grouping).
 *  - Scope: fixed-length, equally split, causal self-attention ("Feat: Context Parallel",
 *    section 实现边界 (implementation boundary)).
 *
 * Conventions for every entry point:
 *  - Tensors are B,H,S,D contiguous with D innermost.  "rows" counts sequence positions of
 *    one (batch, head).  Element type of q/k/v/o/dO/dq/dk/dv is problem->dtype (fp32 or
 *    bf16); statistics (m, l, lse, delta) and accumulators are always fp32.
 *  - Pointers: all tensor pointers are caller-owned DEVICE memory on the context's device,
 *    16-byte aligned.  ra_problem / ra_pair pointers and out-parameters are HOST memory.
 *    The library allocates no device memory: scratch comes from a caller workspace sized
 *    by ra_workspace_size.
 *  - Streams: `stream`, `compute`, `staging` are hipStream_t values passed as void*
 *    (NULL = the legacy default stream).  All device work is enqueued asynchronously.
 *  - Errors: every call returns ra_status and never throws or aborts across the ABI.
 *    Arguments are validated on the host before anything is enqueued, so a call that
 *    returns RA_ERR_INVALID / RA_ERR_UNSUPPORTED / RA_ERR_WORKSPACE enqueued nothing.
 *    RA_ERR_DEVICE reports a HIP launch/runtime failure; faults in already-enqueued work
 *    surface at the caller's next synchronisation.  ra_last_error() gives a thread-local
 *    human-readable message for the last failing call on the calling thread.
 */
#ifndef RINGATTN_RA_H
#define RINGATTN_RA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_ERR_INVALID = 1,      /* bad argument: shape, pointer, alignment, rank, pair list */
  RA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head_dim, dtype) */
  RA_ERR_DEVICE = 3,       /* HIP runtime / launch failure */
  RA_ERR_WORKSPACE = 4     /* workspace too small */
} ra_status;

typedef enum { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;
typedef enum { RA_CONTIGUOUS = 0, RA_ZIGZAG = 1 } ra_layout;

/* Mask kind of one (Q block, K/V block) pair.
 *  FULL: every key visible to every query (the K/V block lies wholly in the past).
 *  DIAG: q_len == kv_len and local key j is visible to local query i iff j <= i.
 *  SKIP: no key visible; the pair is a no-op. */
typedef enum { RA_MASK_FULL = 0, RA_MASK_DIAG = 1, RA_MASK_SKIP = 2 } ra_mask;

/* The full-sequence problem.  Rank r's Q slice has seq_len / cp_size rows. */
typedef struct {
  int64_t batch;
  int64_t seq_len;    /* full sequence length S */
  int64_t heads_q;
  int64_t heads_kv;   /* heads_q % heads_kv == 0 */
  int64_t head_dim;   /* 64 or 128 */
  int32_t cp_size;    /* simulated context-parallel degree, >= 1 */
  int32_t layout;     /* ra_layout */
  int32_t dtype;      /* ra_dtype */
  float scale;        /* softmax scale; 0 selects 1/sqrt(head_dim) */
  /* Optional restrictions of the causal mask (the transformers context-parallel page lists
   * sliding-window and chunked attention among the masks rebuilt over the whole sequence).
   * With window W > 0 query position t also needs t - j < W of key position j (itself and the
   * W - 1 keys before it); with attn_chunk C > 0 it needs j / C == t / C (keys of its own
   * chunk of C positions).  0 disables either. */
  int64_t window;
  int64_t attn_chunk;
} ra_problem;

/* One pair: Q rows [q_row0, q_row0+q_len) of the Q operand against K/V rows
 * [kv_row0, kv_row0+kv_len) of the K/V operand, with a mask kind. */
typedef struct {
  int64_t q_row0;
  int64_t kv_row0;
  int64_t q_len;
  int64_t kv_len;
  int32_t mask;       /* ra_mask */
  int32_t reserved;   /* must be 0 */
  /* Full-sequence positions of query row q_row0 and key row kv_row0 (rows of a pair are
   * consecutive positions).  Read only when problem->window or problem->attn_chunk is set;
   * ra_plan_step fills them. */
  int64_t q_pos0;
  int64_t kv_pos0;
} ra_pair;

typedef struct ra_context ra_context;

/* ---- host-only helpers (no GPU needed) ------------------------------------------------ */

const char* ra_version(void);
const char* ra_status_str(int32_t status);
/* Thread-local message of the last failing call on this thread ("" if none). */
const char* ra_last_error(void);

/* Checks the problem and a rank against the scope the pages fix: fixed-length, equally split,
 * causal self-attention ("Feat: Context Parallel", section 实现边界), MHA or GQA with
 * n_rep = heads_q / heads_kv ("Feat: Context Parallel", review thread on the attention helper),
 * zigzag splitting into 2 * cp_size chunks ("上下文并行", Zig-Zag Ring Attention).  So:
 * heads_q % heads_kv == 0, seq_len % cp_size == 0 (and % (2*cp_size) for zigzag),
 * 0 <= rank < cp_size, positive sizes, a known dtype/layout, finite scale >= 0, window and
 * attn_chunk >= 0: RA_ERR_INVALID otherwise.  head_dim outside {64,128} and
 * batch * heads_q > 65535 return RA_ERR_UNSUPPORTED.  Every entry point that takes a problem
 * applies these checks first. */
ra_status ra_validate(const ra_problem* problem, int32_t rank);

/* Ring step plan ("上下文并行", "朴素 Ring Attention": each round a rank sends its K/V to the
 * next rank and receives the previous rank's, so at step `step` rank `rank` holds the chunk of
 * owner (rank - step) mod cp; the zigzag per-step rule is the table in "Zig-Zag Ring
 * Attention").  Writes the owner and up to 4 pairs (SKIP pairs included, so a plan can be
 * audited): contiguous gives 1 pair (DIAG at step 0, FULL for 1 <= step <= rank, SKIP after);
 * zigzag gives 4 pairs over the half-chunks (Q_lo,K_lo), (Q_lo,K_hi), (Q_hi,K_lo), (Q_hi,K_hi).
 * q rows are offsets in the rank's Q slice, kv rows offsets in the owner's K/V chunk. */
ra_status ra_plan_step(const ra_problem* problem, int32_t rank, int32_t step, int32_t* owner,
                       ra_pair pairs[4], int32_t* n_pairs);

/* Workspace bytes needed by ra_rank_view_fwd (pass = 0), ra_rank_view_bwd (pass = 1) or
 * ra_rank_view_fwd_split (pass = 2). */
ra_status ra_workspace_size(const ra_problem* problem, int32_t pass, size_t* bytes);

/* ---- context ----------------------------------------------------------------------- */

/* Creates a context bound to HIP device `device` (events, device properties).  The context
 * may be used from one host thread at a time. */
ra_status ra_create(int32_t device, ra_context** out);
void ra_destroy(ra_context* ctx);

/* Debugging aids of a context: flags (0 when the context is created, the production setting).
 * RA_DEBUG_POISON_SLOTS: the rank views (ra_rank_view_fwd, ra_rank_view_bwd) fill a staging slot
 *   with NaN on the staging stream as soon as the work that reads it has finished, i.e. after its
 *   slot_free events ("Feat: Context Parallel" 主要改动: events manage the K/V lifetime across
 *   streams): before each refill and, after the ring, every slot the ring used.  The ring orders
 *   every read of a slot before that fill, so results do not change; a read that escaped the
 *   events would see NaN (the fill word 0x7FC07FC0 is NaN as two bf16 values and as an fp32).
 *   When such a call's stream has drained, the slots in its workspace hold NaN.
 * RA_DEBUG_ROCTX: the rank views mark the ring loop and each ring step with roctx ranges
 *   ("ra fwd step 3 owner 12 (slot 0)", ...) for rocprofv3 --marker-trace; the roctx library is
 *   opened on first use, and where it is absent the flag does nothing.
 * RA_ERR_INVALID for a NULL context or unknown bits. */
#define RA_DEBUG_POISON_SLOTS 1u
#define RA_DEBUG_ROCTX 2u
ra_status ra_set_debug(ra_context* ctx, uint32_t flags);

/* ---- device entry points -------------------------------------------------------------- */

/* Layout permutation ("Feat: Context Parallel" 主要改动; "上下文并行" "Zig-Zag Ring
 * Attention"): copies, bit-exactly, the slices of ranks [rank_begin, rank_begin+rank_count)
 * out of the full-sequence tensor `full` (batch, heads, seq_len, head_dim) into `out`
 * (batch, heads, rank_count * seq_len/cp, head_dim), owner after owner.  rank_count = cp
 * gives the owner-major ring order used for k_ring / v_ring; rank_count = 1 gives one rank's
 * slice.  `heads` is heads_q or heads_kv.  ra_layout_scatter is the exact inverse (writes
 * only the rows of those ranks into `full`). */
ra_status ra_layout_gather(ra_context* ctx, const ra_problem* problem, int32_t rank_begin,
                           int32_t rank_count, int64_t heads, const void* full, void* out,
                           void* stream);
ra_status ra_layout_scatter(ra_context* ctx, const ra_problem* problem, int32_t rank_begin,
                            int32_t rank_count, int64_t heads, const void* in, void* full,
                            void* stream);

/* Ulysses re-shard, the on-GPU half of the all-to-all that turns a sequence shard into a head
 * shard and back ("上下文并行", section Ulysses: the all-to-all exchanges sequence sharding
 * for head sharding before attention and reverses it after).  cp = problem->cp_size is the
 * all-to-all degree; it must divide `heads` (heads_q or heads_kv) and seq_len.  With
 * Hh = heads / cp and Sc = seq_len / cp, the tensors are (element type problem->dtype):
 *   sequence shard  (batch, heads, Sc, head_dim)          rank r holds positions r Sc ..
 *   exchange buffer (cp, batch, Hh, Sc, head_dim)          block j goes to / came from rank j
 *   head shard      (batch, Hh, seq_len, head_dim)         rank r holds heads r Hh ..
 * RA_A2A_SEQ_PACK:    sequence shard -> send buffer (block j = this shard's heads of rank j)
 * RA_A2A_HEAD_UNPACK: receive buffer (block j = rank j's positions) -> head shard
 * RA_A2A_HEAD_PACK:   head shard -> send buffer (block j = positions of rank j)
 * RA_A2A_SEQ_UNPACK:  receive buffer (block j = heads of rank j) -> sequence shard
 * The all-to-all itself (receive block j on rank r = send block r of rank j) is the
 * collective and not part of this library.  A pure permutation: bit-exact.  src and dst must
 * not overlap (each spans batch * heads * seq_len/cp * head_dim elements); RA_ERR_INVALID
 * otherwise, for an unknown step, or heads not divisible by cp. */
typedef enum {
  RA_A2A_SEQ_PACK = 0,
  RA_A2A_HEAD_UNPACK = 1,
  RA_A2A_HEAD_PACK = 2,
  RA_A2A_SEQ_UNPACK = 3
} ra_a2a_step;

ra_status ra_ulysses_reshard(ra_context* ctx, const ra_problem* problem, int32_t step,
                             int64_t heads, const void* src, void* dst, void* stream);

/* The ring's receive on one GPU ("上下文并行", 朴素 Ring Attention: each step a rank receives
 * the previous rank's K/V chunk; "Feat: Context Parallel" 主要改动: a separate stream carries
 * it): copies owner `owner`'s K and V chunk, (batch, heads_kv, seq_len/cp, head_dim) each, out
 * of the owner-major ring tensors k_ring / v_ring (batch, heads_kv, seq_len, head_dim) into
 * `dst`, K first, then V.  The rank views stage every chunk but their own this way.  Bit-exact.
 * RA_ERR_INVALID for an owner outside [0, cp_size) or NULL / misaligned pointers. */
ra_status ra_stage_kv(ra_context* ctx, const ra_problem* problem, int32_t owner,
                      const void* k_ring, const void* v_ring, void* dst, void* stream);

/* Empty online-softmax state for (batch, heads_q, rows): U = 0, m = -inf, l = 0. */
ra_status ra_state_init(ra_context* ctx, const ra_problem* problem, int64_t rows, float* U,
                        float* m, float* l, void* stream);

/* Chunk forward ("上下文并行", "朴素 Ring Attention": safe softmax and the
 * FlashAttention-2-style update of the output, row max and row sum per K/V block).
 * q: (batch, heads_q, q_rows, head_dim); k, v: (batch, heads_kv, kv_rows, head_dim).
 * State (fp32, in/out): m (batch, heads_q, q_rows) is the row's reference point (natural-log
 * units), l (batch, heads_q, q_rows) the row sum of exp(score - m) and U (batch, heads_q,
 * q_rows, head_dim) the unnormalised output sum of exp(score - m) v, so m + ln l is the row's
 * log-sum-exp and U / l its output.  m is at least the row max minus 8 ln 2: the bf16 kernel
 * moves m only when a key block's max exceeds it by more than 8 ln 2 (so exp(score - m) <= 256),
 * which skips most rescales of U; the empty state is (U = 0, m = -inf, l = 0).
 * Every non-SKIP pair is folded into its rows exactly once; pairs may share Q rows, but the
 * Q ranges of two pairs must be identical or disjoint.  Rows no pair touches, and SKIP
 * pairs, leave the state bit-unchanged.  bf16 path: Q K^T and P V on bf16 MFMA with fp32
 * accumulation, P rounded to bf16 only as the MFMA operand.  fp32 path: fp32 throughout. */
ra_status ra_chunk_fwd(ra_context* ctx, const ra_problem* problem, const void* q, int64_t q_rows,
                       const void* k, const void* v, int64_t kv_rows, const ra_pair* pairs,
                       int32_t n_pairs, float* U, float* m, float* l, void* stream);

/* Folds an independently computed, normalised partial (o_part fp32 (batch, heads_q, rows,
 * head_dim), lse_part fp32 (batch, heads_q, rows), -inf = empty) into the state: the partial
 * is the state (U = o_part, m = lse_part, l = 1) ("上下文并行", "朴素 Ring Attention",
 * order independence; Megatron's separate softmax_lse update stream in "Zig-Zag Ring
 * Attention"). */
ra_status ra_lse_merge(ra_context* ctx, const ra_problem* problem, int64_t rows,
                       const float* o_part, const float* lse_part, float* U, float* m, float* l,
                       void* stream);

/* O = U / l in problem->dtype (bf16 rounded to nearest even after normalisation, per
 * "Feat: Context Parallel" section 数值精度) and lse = m + ln l (fp32).  Rows with l = 0
 * give O = 0 and lse = -inf. */
ra_status ra_fwd_finalize(ra_context* ctx, const ra_problem* problem, int64_t rows,
                          const float* U, const float* m, const float* l, void* o, float* lse,
                          void* stream);

/* Backward pre-pass: delta = rowsum(dO * O) in fp32, (batch, heads_q, rows).  The p2p backward
 * recomputes the probabilities from the saved log-sum-exp ("Feat: Context Parallel", 主要改动);
 * the gradient of the softmax then needs, per query row, the inner product of the row's output
 * and output gradient, which this computes once for all ring steps.  o and dO: (batch, heads_q,
 * rows, head_dim) in problem->dtype; delta: caller-owned fp32 device memory, overwritten.
 * RA_ERR_INVALID for NULL or misaligned pointers or rows < 0. */
ra_status ra_bwd_preprocess(ra_context* ctx, const ra_problem* problem, int64_t rows,
                            const void* o, const void* dO, float* delta, void* stream);

/* Chunk backward with probability recompute ("Feat: Context Parallel" 主要改动, p2p mode):
 * for every non-SKIP pair, P = exp(scale*Q K^T - lse), dP = dO V^T, dS = P (dP - delta), and
 *   dq_acc += scale * dS K,  dk_acc += scale * dS^T Q,  dv_acc += P^T dO  (fp32, ADDED to).
 * q, dO: (batch, heads_q, q_rows, head_dim); lse, delta: (batch, heads_q, q_rows) fp32;
 * k, v: (batch, heads_kv, kv_rows, head_dim); dq_acc like q, dk_acc/dv_acc like k (fp32).
 * dk/dv of a key/value head sum the contributions of all heads_q/heads_kv query heads that
 * read it, inside the kernel.  Accumulation uses fp32 atomics: summation order varies.
 * Gradients that are not needed may be left out: dq_acc = NULL computes dK and dV only;
 * dk_acc = dv_acc = NULL computes dQ only (the bf16 path then runs one kernel instead of two).
 * RA_ERR_INVALID if only one of dk_acc, dv_acc is NULL or all three are. */
ra_status ra_chunk_bwd(ra_context* ctx, const ra_problem* problem, const void* q, const void* dO,
                       const float* lse, const float* delta, int64_t q_rows, const void* k,
                       const void* v, int64_t kv_rows, const ra_pair* pairs, int32_t n_pairs,
                       float* dq_acc, float* dk_acc, float* dv_acc, void* stream);

/* Chunk backward with stored dS: the same gradients as ra_chunk_bwd (all three required), formed
 * by five contractions instead of seven.  The dK/dV kernel, which forms dS = P (dP - delta) for
 * its dK contraction anyway, also writes scale * dS (bf16, the very operand of that contraction)
 * into `scratch`; a second kernel then forms dQ += (scale dS) K as a plain contraction that
 * streams the stored dS, instead of recomputing S and dP per query row ("Feat: Context
 * Parallel" 主要改动: the p2p backward recomputes P from the saved log-sum-exp once per chunk
 * pair).  Arguments as for ra_chunk_bwd, plus `scratch`: caller-owned device memory of at least
 * ra_chunk_bwd_ds_size bytes (16-byte aligned; its contents on entry do not matter; it must not
 * be reused by other work until this call's work has finished on `stream`).  The two kernels can
 * be run as two calls: dq_acc = NULL runs only the first (dK, dV, and dS into the scratch);
 * dk_acc = dv_acc = NULL runs only the second, which reads the scratch a first-phase call with
 * the same arguments filled.  For fp32 problems the scratch is not used (size 0) and the call
 * runs the fp32 backward, which needs all three gradients (RA_ERR_UNSUPPORTED otherwise).
 * RA_ERR_WORKSPACE if scratch_bytes is too small; RA_ERR_INVALID for NULL or misaligned
 * pointers, only one of dk_acc / dv_acc, no gradient at all, or a bad pair list. */
ra_status ra_chunk_bwd_ds_size(const ra_problem* problem, int64_t q_rows, int64_t kv_rows,
                               const ra_pair* pairs, int32_t n_pairs, size_t* bytes);
ra_status ra_chunk_bwd_ds(ra_context* ctx, const ra_problem* problem, const void* q,
                          const void* dO, const float* lse, const float* delta, int64_t q_rows,
                          const void* k, const void* v, int64_t kv_rows, const ra_pair* pairs,
                          int32_t n_pairs, float* dq_acc, float* dk_acc, float* dv_acc,
                          void* scratch, size_t scratch_bytes, void* stream);

/* The same call for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): ra_chunk_bwd_ds with the scratch taken
 * from a static device array of RA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every
 * GPU it runs on until the process ends (its address is looked up once per device, in ra_create).
 * The call allocates nothing.  Every call on a GPU shares that GPU's array, which keeps the last
 * call's dS: calls that overlap on one GPU (on different streams, or from several threads or
 * contexts) race, and a second-phase call (dk_acc = dv_acc = NULL) reads whatever the last
 * first-phase call on that GPU wrote.  RA_ERR_WORKSPACE when ra_chunk_bwd_ds_size exceeds
 * RA_NOALLOC_SCRATCH_BYTES; otherwise arguments, results and errors as for ra_chunk_bwd_ds. */
#define RA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ra_status ra_chunk_bwd_ds_noalloc(ra_context* ctx, const ra_problem* problem, const void* q,
                                  const void* dO, const float* lse, const float* delta,
                                  int64_t q_rows, const void* k, const void* v, int64_t kv_rows,
                                  const ra_pair* pairs, int32_t n_pairs, float* dq_acc,
                                  float* dk_acc, float* dv_acc, void* stream);

/* Casts n fp32 values to problem->dtype (round to nearest even for bf16): the backward's
 * final step for dQ / dK / dV accumulators. */
ra_status ra_cast_from_f32(ra_context* ctx, const ra_problem* problem, int64_t n,
                           const float* src, void* dst, void* stream);

/* Rank-view forward: the whole ring for rank `rank` on one GPU.
 * q_slice: the rank's Q slice (batch, heads_q, S/cp, head_dim) in slice order (see
 * ra_layout_gather with rank_count = 1).  k_ring, v_ring: all owners' K/V in owner-major
 * ring order (batch, heads_kv, S, head_dim) (ra_layout_gather with rank_count = cp).
 * Outputs o_slice (like q_slice) and lse_slice (batch, heads_q, S/cp) fp32.
 * For step i = 0..cp-1 the chunk of owner (rank - i) mod cp is copied into one of two
 * workspace slots on `staging` (the stand-in for the ring receive) while step i-1 computes on
 * `compute`; events order slot reuse.  A step whose pairs are all SKIP neither stages nor
 * computes.  With two or more staged steps, those staged in slot 1 fold into a second running
 * state on a context stream, concurrently with the other steps, and the two states are merged
 * before the finalize; which state a step uses depends only on its slot, so the result is the
 * same for any timing.  All work is ordered before later work on `compute`.
 * Workspace: ra_workspace_size(problem, 0).  compute and staging may be equal. */
ra_status ra_rank_view_fwd(ra_context* ctx, const ra_problem* problem, int32_t rank,
                           const void* q_slice, const void* k_ring, const void* v_ring,
                           void* o_slice, float* lse_slice, void* workspace,
                           size_t workspace_bytes, void* compute, void* staging);

/* All-gather mode with split-KV ("上下文并行", 基本思想: the all_gather variant gathers every
 * K/V chunk and computes with the local Q; Megatron's separate stream that updates the
 * softmax_lse, "Zig-Zag Ring Attention").  k_all / v_all hold the gathered K/V in the same
 * owner-major order as k_ring / v_ring.  Every chunk the rank's queries see is computed
 * independently into its own partial online-softmax state, the chunk launches spread over the
 * context's own streams so that they can run concurrently; each partial is then merged into
 * the running state on the `merge` stream (in step order) and the result finalised there, as
 * in ra_rank_view_fwd.  Outputs equal ra_rank_view_fwd's up to summation order.  Workspace:
 * ra_workspace_size(problem, 2, ...) bytes (the running state and one partial state per
 * step).  `merge` may be NULL (merges on the compute stream).  The call returns once all work
 * is enqueued; `compute` is ordered after all of it.  RA_ERR_UNSUPPORTED for cp_size > 64. */
ra_status ra_rank_view_fwd_split(ra_context* ctx, const ra_problem* problem, int32_t rank,
                                 const void* q_slice, const void* k_all, const void* v_all,
                                 void* o_slice, float* lse_slice, void* workspace,
                                 size_t workspace_bytes, void* compute, void* merge);

/* Rank-view backward.  Inputs as for the forward plus o_slice / lse_slice from it and
 * dO_slice (like q_slice).  Outputs dq_slice (like q_slice) and dk_ring, dv_ring
 * (batch, heads_kv, S, head_dim) in owner-major ring order: this rank's contribution to every
 * owner's K/V gradient (rows of chunks this rank never attends to are zero); summing dk_ring
 * over all ranks gives the full-sequence gradient -- the ring's return-to-owner.
 * Staging and slot reuse as for the forward.  In the bf16 path each step's dQ kernel runs on a
 * context stream (in step order: the steps add into the same dQ rows) and the dK/dV kernels of
 * the steps staged in slot 1 on a second one (steps write different owners' rows).  An owner's
 * rows of dk_ring / dv_ring are written right after its step, on that step's stream; both
 * context streams are joined into `compute` before the dQ cast, so all work is ordered before
 * later work on `compute`.  dK/dV sums over the query heads of a group use fp32 atomics, whose order (and so
 * the last bits of dk_ring, dv_ring) can vary from run to run.
 * Workspace: ra_workspace_size(problem, 1). */
ra_status ra_rank_view_bwd(ra_context* ctx, const ra_problem* problem, int32_t rank,
                           const void* q_slice, const void* k_ring, const void* v_ring,
                           const void* o_slice, const float* lse_slice, const void* dO_slice,
                           void* dq_slice, void* dk_ring, void* dv_ring, void* workspace,
                           size_t workspace_bytes, void* compute, void* staging);

#ifdef __cplusplus
}
#endif

#endif /* RINGATTN_RA_H */
