// Internal interface between the host driver (ra_host.cpp), the planning core (ra_plan.cpp)
// and the gfx950 kernels (kern_*.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <climits>

#include <string>

#include "ra.h"

namespace ra {

// ---- error reporting (thread-local message, see ra_last_error) -------------------------
ra_status fail(ra_status code, const char* fmt, ...);
void clear_error();

// ---- resolved problem --------------------------------------------------------------------
struct Shape {
  int64_t B, S, Hq, Hkv, D, n_rep;
  int32_t cp, layout, dtype;
  float scale;      // resolved (never 0)
  int64_t window, attn_chunk;  // mask restrictions, 0 = off
  int64_t esize;    // bytes per element of the storage dtype
  int64_t chunk;    // rows of one rank slice, S / cp
  int64_t nchunks;  // cp (contiguous) or 2*cp (zigzag)
  int64_t crow;     // rows of one layout chunk, S / nchunks
};

// Validates the problem only (no rank).  Fills *out on success.
ra_status resolve(const ra_problem* p, Shape* out);
// Validates a rank against a resolved shape.
ra_status check_rank(const Shape& s, int32_t rank);
// Pair-list validation for chunk entry points (bounds, DIAG q_len == kv_len, identical or
// disjoint Q ranges when by_q, identical or disjoint K/V ranges otherwise).
ra_status check_pairs(const ra_pair* pairs, int32_t n, int64_t q_rows, int64_t kv_rows);
// Plan of one ring step (always fills the SKIP pairs too).
void plan_step(const Shape& s, int32_t rank, int32_t step, int32_t* owner, ra_pair pairs[4],
               int32_t* n);
// First global row of layout chunk `c`; rank r's slice holds chunk r (contiguous) or chunks
// r and 2cp-1-r (zigzag), in that order.
int64_t slice_chunk(const Shape& s, int32_t rank, int32_t which);

// Workspace carve-up, shared by ra_workspace_size and the rank-view drivers.
// Forward: the running state; with two staging slots a second state (U2, m2, l2) for the steps
// staged in slot 1, merged into the first after the ring (two states let consecutive steps run
// concurrently); then the slots.
struct FwdWs { size_t U, m, l, U2, m2, l2, slot[2], total; bool two; };
struct BwdWs { size_t dq, dk, dv, delta, slot[2], ds[2], ds_bytes, total; };
FwdWs fwd_ws(const Shape& s);
// Split-KV forward: the running state, then one partial state per ring step (cp of them).
struct SplitWs { size_t U, m, l, part, part_stride, total; };
SplitWs split_ws(const Shape& s);
BwdWs bwd_ws(const Shape& s);

// ---- kernel parameter blocks -------------------------------------------------------------
// A group of pairs that share one row range on the "outer" side: Q rows for the forward
// (each workgroup owns a Q tile), K/V rows for the backward (each workgroup owns a K/V tile).
struct KRange {
  int64_t row0, len;      // outer rows
  int64_t tile0, ntiles;  // first linear tile index and tile count of this range
  int32_t npairs;
  int32_t pair[4];        // indices into KParams::pairs
  int32_t reverse;        // visit tiles last-to-first (heaviest first)
  int32_t pad_;
};

struct KPair {
  int64_t q_row0, kv_row0, q_len, kv_len;
  int32_t mask, pad_;
  int64_t q_pos0, kv_pos0;  // sequence positions of the first query / key row
  // Backward with stored dS: the pair's dS^T block starts ds_off elements into KParams::ds; it
  // holds, per (batch, query head), ds_rows rows (keys; kv_len rounded up to 128) of ds_ld
  // elements (queries; q_len rounded up to 128).
  int64_t ds_off, ds_rows, ds_ld;
};

struct KParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dO;
  const float* lse;
  const float* delta;
  float* U;   // fwd state / dq_acc
  float* m;
  float* l;
  float* dk;  // bwd accumulators
  float* dv;
  void* ds;   // bwd: bf16 dS scratch (see KPair::ds_off); NULL = not stored
  int64_t q_head_rows;    // head stride (rows) of q, dO, U, m, l, lse, delta, dq
  int64_t kv_head_rows;   // head stride (rows) of k, v
  int64_t dkv_head_rows;  // head stride (rows) of dk, dv
  int32_t B, Hq, Hkv, n_rep, D;
  float scale;            // softmax scale
  float scale_log2;       // scale * log2(e)
  int64_t window;         // sliding window (0 = none)
  int64_t attn_chunk;     // attention chunk (0 = none)
  int32_t fresh;          // forward: start every row from the empty state instead of loading U, m, l
  int32_t q_per_wg;       // dK/dV kernel (D = 128): query heads of one key/value group per workgroup (0 or 1: one)
  int32_t dq_qblocks;     // dQ-from-stored-dS kernel: 32-query blocks per wavefront (2, or 0 / 1: one)
  int32_t nranges;
  int64_t tiles_per_head;
  KRange ranges[4];
  KPair pairs[4];
};

// Query heads per workgroup of the D = 128 dK/dV kernel (call after build_ranges): two heads of a
// key/value group share one workgroup's K/V prologue and dK/dV atomics when the launch has more
// than 256 workgroups (one per CU) -- never more rounds of workgroups (ceil(n / 512) twice-longer
// rounds against ceil(n / 256)), half the fixed costs; at 256 or fewer it would lengthen the one
// round.
inline int32_t kv_heads_per_wg(const KParams& kp) {
  const int64_t n = (int64_t)kp.B * kp.Hq * kp.tiles_per_head;
  return (kp.D == 128 && kp.n_rep % 2 == 0 && n > 256) ? 2 : 1;
}

// Builds the range table: groups non-SKIP pairs by their outer range and assigns tiles of
// `tile_rows` rows.  by_q selects the forward grouping (Q ranges) or the backward (K/V).
void build_ranges(KParams* kp, const ra_pair* pairs, int32_t n, bool by_q, int64_t tile_rows);
// Lays out the stored-dS scratch of a pair list (bytes; 0 when no pair computes) and, when kp is
// given, fills the pairs' ds_off / ds_rows / ds_ld (call after build_ranges).  Each non-SKIP pair
// gets B * Hq * ds_rows * ds_ld bf16 values (dS^T, key-major), ds_rows = kv_len rounded up to
// 128 (the dK/dV workgroup's key granule) and ds_ld = q_len rounded up to 128, blocks 256-byte
// aligned.
size_t ds_layout(const Shape& s, const ra_pair* pairs, int32_t n, KParams* kp);
// Largest ds_layout over the ring steps of a rank view (the size of one dS buffer).
size_t ds_step_max(const Shape& s, int32_t rank);
// Above this size per step the rank-view backward recomputes S and dP for dQ instead of storing
// dS (the Qwen3-shaped single-chunk share would need 34 GB).
constexpr size_t kDsCap = (size_t)8 << 30;

// Lowest key position visible to query position t under the window / chunk restrictions
// (INT64_MIN when neither is set); the causal bound is key <= t.  constexpr: usable on the
// host and, implicitly, in device code.
constexpr int64_t lowest_key(int64_t t, int64_t window, int64_t attn_chunk) {
  int64_t lo = INT64_MIN;
  if (window > 0) lo = t - window + 1;
  if (attn_chunk > 0) {
    const int64_t c = (t / attn_chunk) * attn_chunk;
    lo = lo > c ? lo : c;
  }
  return lo;
}

// Highest query position that sees key position j under the window / chunk restrictions
// (INT64_MAX when neither is set); the causal bound is query >= j.
constexpr int64_t highest_query(int64_t j, int64_t window, int64_t attn_chunk) {
  int64_t hi = INT64_MAX;
  if (window > 0) hi = j + window - 1;
  if (attn_chunk > 0) {
    const int64_t c = (j / attn_chunk + 1) * attn_chunk - 1;
    hi = hi < c ? hi : c;
  }
  return hi;
}

// ---- launchers (kern_*.hip); all return hipError_t as int ----------------------------------
int launch_chunk_fwd_bf16(const KParams& kp, void* stream);
// Backward as two launches: `kv` has K/V-major ranges (dK, dV), `q` Q-major ranges (dQ).
// With `fork` (hipStream_t side, hipEvent_t fork, hipEvent_t join) the dQ launch goes to `side`
// after a fork event, so the two kernels can run at once, and the caller's stream then waits
// for it through `join`; with join == nullptr it does not, and the caller joins later.
struct BwdFork { void* side; void* fork; void* join; };
int launch_chunk_bwd_bf16(const KParams& kv, const KParams& q, void* stream, const BwdFork* fork);
// Backward with stored dS: the dK/dV kernel (kv.ds set) writes dS^T, then the dQ kernel reads it
// (q.ds set, Q-major ranges): dq += dS K.  With `fork` the dQ kernel runs on `side` after the
// dK/dV kernel (fork event recorded after it), joined into `stream` when fork->join is set.
int launch_chunk_bwd_ds_bf16(const KParams& kv, const KParams& q, void* stream, const BwdFork* fork);
// Device address of this GPU's copy of the static scratch of ra_chunk_bwd_ds_noalloc (looked up
// once per device; `device` must be current).  Returns a hipError_t.
constexpr int kMaxDevices = 64;
int noalloc_scratch_address(int device, void** out);
int launch_chunk_fwd_f32(const KParams& kp, void* stream);
int launch_chunk_bwd_f32(const KParams& kp, void* stream);
constexpr int64_t kFwdTileRows = 128;   // Q rows per forward workgroup (bf16 MFMA kernel)
constexpr int64_t kFwdPPTileRows = 256; // Q rows per workgroup of the ping-pong forward (D = 128)
constexpr int64_t kBwdTileRows = 128;   // K/V rows per dK/dV workgroup (bf16 MFMA kernel)
constexpr int64_t kBwdPPTileRows = 256; // K/V rows per dK/dV workgroup of the ping-pong kernel (D = 128)
constexpr int64_t kBwdQTileRows = 128;  // Q rows per dQ workgroup (bf16 MFMA kernel)
constexpr int64_t kBwdDsTileRows = 128; // Q rows per workgroup of the dQ-from-stored-dS kernel
                                         // with one query block per wavefront (twice with two)
constexpr int64_t kBwdDsWideMin = 512;   // workgroups the two-block dQ grid needs to be chosen
constexpr int64_t kF32FwdTileRows = 1;  // one row per workgroup in the fp32 path
constexpr int64_t kF32BwdTileRows = 1;

int launch_layout(const Shape& s, int32_t rank_begin, int32_t rank_count, int64_t heads,
                  const void* src, void* dst, bool gather, void* stream);
int launch_state_init(int64_t nrows, int64_t D, float* U, float* m, float* l, void* stream);
// Ulysses re-shard step (ra_a2a_step) over `heads` heads; cp divides heads and S.
int launch_reshard(const Shape& s, int32_t step, int64_t heads, const void* src, void* dst, void* stream);
int launch_lse_merge(int64_t nrows, int64_t D, const float* o_part, const float* lse_part,
                     float* U, float* m, float* l, void* stream);
// Folds an unnormalised partial state (Up, mp, lp) into (U, m, l): the merge of the normalised
// partial (Up / lp, mp + ln lp) written without the division.
int launch_state_merge(int64_t nrows, int64_t D, const float* Up, const float* mp, const float* lp,
                       float* U, float* m, float* l, void* stream);
int launch_fwd_finalize(int64_t nrows, int64_t D, int32_t dtype, const float* U, const float* m,
                        const float* l, void* o, float* lse, void* stream);
// launch_state_merge of (Ub, mb, lb) into (Ua, ma, la) followed by launch_fwd_finalize, in one
// pass that does not write the merged state.
int launch_merge_finalize(int64_t nrows, int64_t D, int32_t dtype, const float* Ub, const float* mb,
                          const float* lb, const float* Ua, const float* ma, const float* la, void* o,
                          float* lse, void* stream);
int launch_bwd_preprocess(int64_t nrows, int64_t D, int32_t dtype, const void* o,
                          const void* dO, float* delta, void* stream);
int launch_cast_from_f32(int64_t n, int32_t dtype, const float* src, void* dst, void* stream);
int launch_fill_zero(int64_t n_floats, float* dst, void* stream);
// `blocks` blocks of block_bytes (a multiple of 16) zeroed, pitch_bytes apart.
int launch_zero2d(void* dst, int64_t pitch_bytes, int64_t block_bytes, int64_t blocks, void* stream);
// Fills blocks x block_bytes (a multiple of 16) spaced pitch_bytes apart with one 32-bit word.
int launch_fill2d(void* dst, int64_t pitch_bytes, int64_t block_bytes, int64_t blocks, uint32_t word,
                  void* stream);
// `blocks` blocks of `block` fp32 values (a multiple of 4) cast to dtype; source and destination
// blocks start `pitch` elements apart.
int launch_cast2d(const float* src, void* dst, int64_t pitch, int64_t block, int64_t blocks, int32_t dtype,
                  void* stream);
// Copies `blocks` blocks of `block_bytes` from src (pitch src_pitch) to dst (pitch dst_pitch).
int launch_copy2d(const void* src, int64_t src_pitch, void* dst, int64_t dst_pitch,
                  int64_t block_bytes, int64_t blocks, void* stream);

}  // namespace ra
