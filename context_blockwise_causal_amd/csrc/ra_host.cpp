// Host driver of libringattn: the C ABI device entry points, argument validation and the
// rank-view ring loop with side-stream staging.
//
// Ring on one GPU (lecture note "上下文并行", "朴素 Ring Attention" walk-through; InfiniTrain
// "Feat: Context Parallel" 主要改动, dual compute streams with events managing cross-stream K/V
// lifetime): at step i rank r computes with the chunk of owner (r - i) mod cp.  Step 0 uses
// the rank's own chunk in place.  For later steps the chunk is copied into one of two
// workspace slots on the staging stream -- the stand-in for the ring receive -- while the
// previous step computes on the compute stream.  Event slot_ready[s] orders "copy into slot s"
// before "compute from slot s"; event slot_free[s] orders "compute from slot s" before the next
// copy into it.
#include <dlfcn.h>
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <mutex>

#include "ra_internal.h"

// Streams of the split-KV forward: its chunk launches are independent and run on a small pool
// of the context's own streams (default priority), so that several can occupy the GPU at once.
constexpr int kPoolStreams = 4;
constexpr int kMaxSteps = 64;

struct ra_context {
  int device;
  hipEvent_t start;
  hipEvent_t ready[2];
  hipEvent_t freed[2];
  hipStream_t pool[kPoolStreams];
  hipEvent_t done[kMaxSteps];  // chunk i of a split-KV forward has finished
  hipEvent_t fin;              // the split-KV forward's merges and finalize have finished
  hipEvent_t bfork, bjoin;     // the backward's dQ kernel on a pool stream beside dK/dV
  hipEvent_t qfreed[2];        // the backward ring's dQ kernels have finished reading a slot
  hipEvent_t ajoin;            // the ring's second compute stream has finished
  hipEvent_t dslocal;          // the backward's local-step dQ kernel has read its dS buffer
  void* noalloc_scratch;       // this device's static scratch (ra_chunk_bwd_ds_noalloc)
  hipEvent_t poisoned;         // the end-of-ring slot poisoning has been enqueued (debug mode)
  uint32_t debug;              // RA_DEBUG_* flags
};

namespace ra {
namespace {

// Orders `side` before `main` (record on side, wait on main) when it goes out of scope while
// armed: every return path of a driver that forked work onto a context stream joins it, so
// that even after an error all enqueued work is ordered before later work on the caller's
// stream.  The success path joins explicitly (reporting errors) and disarms it.
struct JoinGuard {
  hipEvent_t ev;
  hipStream_t side, main;
  bool armed;
  void join_now() {
    if (armed) {
      (void)hipEventRecord(ev, side);
      (void)hipStreamWaitEvent(main, ev, 0);
    }
    armed = false;
  }
  ~JoinGuard() { join_now(); }
};

struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

// roctx ranges (RA_DEBUG_ROCTX): the marker library is opened on first use, so that the library
// has no link-time dependency on it; without it the ranges are no-ops.
struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};

const Roctx& roctx() {
  static Roctx r;
  static std::once_flag once;
  std::call_once(once, [] {
    for (const char* name : {"librocprofiler-sdk-roctx.so.1", "libroctx64.so.4"}) {
      void* h = dlopen(name, RTLD_NOW | RTLD_LOCAL);
      if (!h) continue;
      r.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
      r.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
      if (r.push && r.pop) return;  // kept open for the life of the process
      r.push = nullptr;
      r.pop = nullptr;
      dlclose(h);
    }
  });
  return r;
}

// A roctx range from construction to destruction (when `on` and the library is there).
struct Range {
  bool on = false;
  Range(bool enable, const char* fmt, ...) {
    if (!enable || !roctx().push) return;
    char msg[96];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, sizeof msg, fmt, ap);
    va_end(ap);
    on = roctx().push(msg) >= 0;
  }
  ~Range() {
    if (on) (void)roctx().pop();
  }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

ra_status dev_err(int e, const char* what) {
  if (e == 0) return RA_OK;
  return fail(RA_ERR_DEVICE, "%s: %s", what, hipGetErrorString((hipError_t)e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

ra_status need_ptrs(std::initializer_list<const void*> ps) {
  int i = 0;
  for (const void* p : ps) {
    if (!p) return fail(RA_ERR_INVALID, "pointer argument %d is NULL", i);
    if (!aligned16(p)) return fail(RA_ERR_INVALID, "pointer argument %d is not 16-byte aligned", i);
    ++i;
  }
  return RA_OK;
}

ra_status common(ra_context* ctx, const ra_problem* prob, Shape* s) {
  clear_error();
  if (!ctx) return fail(RA_ERR_INVALID, "context is NULL");
  return resolve(prob, s);
}

KParams base_params(const Shape& s) {
  KParams kp{};
  kp.B = (int32_t)s.B;
  kp.Hq = (int32_t)s.Hq;
  kp.Hkv = (int32_t)s.Hkv;
  kp.n_rep = (int32_t)s.n_rep;
  kp.D = (int32_t)s.D;
  kp.scale = s.scale;
  kp.scale_log2 = s.scale * 1.4426950408889634f;
  kp.window = s.window;
  kp.attn_chunk = s.attn_chunk;
  return kp;
}

int run_fwd(const Shape& s, KParams& kp, const ra_pair* pairs, int32_t n, void* stream) {
  if (s.dtype == RA_BF16) {
    build_ranges(&kp, pairs, n, true, s.D == 128 ? kFwdPPTileRows : kFwdTileRows);
    return kp.nranges ? launch_chunk_fwd_bf16(kp, stream) : 0;
  }
  build_ranges(&kp, pairs, n, true, kF32FwdTileRows);
  return kp.nranges ? launch_chunk_fwd_f32(kp, stream) : 0;
}

int run_bwd(const Shape& s, KParams& kp, const ra_pair* pairs, int32_t n, void* stream,
            const BwdFork* fork) {
  if (s.dtype == RA_BF16) {
    KParams kq = kp;
    build_ranges(&kp, pairs, n, false, s.D == 128 ? kBwdPPTileRows : kBwdTileRows);
    kp.q_per_wg = kv_heads_per_wg(kp);
    build_ranges(&kq, pairs, n, true, kBwdQTileRows);
    return kp.nranges ? launch_chunk_bwd_bf16(kp, kq, stream, fork) : 0;
  }
  build_ranges(&kp, pairs, n, true, kF32BwdTileRows);
  return kp.nranges ? launch_chunk_bwd_f32(kp, stream) : 0;
}

// Backward with stored dS (bf16): `ds` holds at least ds_layout(s, pairs, n) bytes.
int run_bwd_ds(const Shape& s, KParams& kp, const ra_pair* pairs, int32_t n, void* ds, void* stream,
               const BwdFork* fork) {
  KParams kq = kp;
  build_ranges(&kp, pairs, n, false, s.D == 128 ? kBwdPPTileRows : kBwdTileRows);
  kp.q_per_wg = kv_heads_per_wg(kp);
  // dQ kernel: two query blocks per wavefront (each K^T operand read from LDS feeds two MFMAs)
  // while the wider tiles still give a grid of several workgroups per CU; else one
  build_ranges(&kq, pairs, n, true, 2 * kBwdDsTileRows);
  kq.dq_qblocks = 2;
  if ((int64_t)kq.B * kq.Hq * kq.tiles_per_head < kBwdDsWideMin) {
    build_ranges(&kq, pairs, n, true, kBwdDsTileRows);
    kq.dq_qblocks = 1;
  }
  ds_layout(s, pairs, n, &kp);
  ds_layout(s, pairs, n, &kq);
  kp.ds = ds;
  kq.ds = ds;
  return kp.nranges ? launch_chunk_bwd_ds_bf16(kp, kq, stream, fork) : 0;
}

// The ring's receive on one GPU: owner's K and V chunk, (B, Hkv, S/cp, D) each, copied out of the
// owner-major ring tensors into `dst` (K then V).
int stage_copy(const Shape& s, int32_t owner, const void* k_ring, const void* v_ring, void* dst,
               hipStream_t stream) {
  const int64_t chunk_bytes = s.chunk * s.D * s.esize;  // one (b, kv head) block of a chunk
  const int64_t head_bytes = s.S * s.D * s.esize;       // pitch of the ring tensors
  const int64_t half = s.B * s.Hkv * chunk_bytes;
  const int64_t off = (int64_t)owner * chunk_bytes;
  int e;
  if ((e = launch_copy2d((const char*)k_ring + off, head_bytes, dst, chunk_bytes, chunk_bytes, s.B * s.Hkv,
                         stream)))
    return e;
  return launch_copy2d((const char*)v_ring + off, head_bytes, (char*)dst + half, chunk_bytes, chunk_bytes,
                       s.B * s.Hkv, stream);
}

bool any_compute(const ra_pair* pairs, int32_t n) {
  for (int i = 0; i < n; ++i)
    if (pairs[i].mask != RA_MASK_SKIP && pairs[i].q_len > 0 && pairs[i].kv_len > 0) return true;
  return false;
}

// Ring steps after the local one that have work (the steps the ring loop stages).
int staged_steps(const Shape& s, int32_t rank) {
  int n = 0;
  for (int32_t i = 1; i < s.cp; ++i) {
    int32_t owner, np;
    ra_pair pairs[4];
    plan_step(s, rank, i, &owner, pairs, &np);
    if (any_compute(pairs, np)) ++n;
  }
  return n;
}

// The ring loop shared by both passes.  `step_fn(stream, slot, kv_k, kv_v, kv_head_rows, owner,
// pairs, n)` (slot -1 for the local step) enqueues one step's compute on `stream` and, when `side`
// is not NULL, part of it on `side`, which the caller joins after the loop.  With `alt` set, the
// steps staged in slot 1 run on `alt` instead of the compute stream (only for steps that do not
// depend on each other); the loop joins `alt` into the compute stream before it returns.  A slot
// is refilled only once all the work that reads it has finished.  Debug flags of the context:
// RA_DEBUG_POISON_SLOTS fills a slot with NaN on the staging stream once that work has finished
// (before each refill, and both slots after the last step, joined into the compute stream);
// RA_DEBUG_ROCTX marks the loop and each step with roctx ranges named after `pass`.
template <class StepFn>
ra_status ring_loop(ra_context* ctx, const char* pass, const Shape& s, int32_t rank, const void* k_ring,
                    const void* v_ring, char* slot0, char* slot1, hipStream_t cs, hipStream_t ss,
                    hipStream_t side, hipStream_t alt, StepFn step_fn) {
  const bool poison = (ctx->debug & RA_DEBUG_POISON_SLOTS) != 0;
  const bool marks = (ctx->debug & RA_DEBUG_ROCTX) != 0;
  Range loop_range(marks, "ra %s rank %d ring", pass, (int)rank);
  struct Step { int32_t i, owner, n; ra_pair pairs[4]; };
  Step staged[64];
  int nstaged = 0;
  Step local{};
  bool have_local = false;
  // cp is bounded by the caller (<= 64 supported by this loop)
  for (int32_t i = 0; i < s.cp; ++i) {
    Step st{};
    st.i = i;
    plan_step(s, rank, i, &st.owner, st.pairs, &st.n);
    if (!any_compute(st.pairs, st.n)) continue;
    if (i == 0) {
      local = st;
      have_local = true;
    } else {
      staged[nstaged++] = st;
    }
  }
  const int64_t row_bytes = s.D * s.esize;
  const int64_t chunk_bytes = s.chunk * row_bytes;       // one (b, kv head) block of a chunk
  const int64_t slot_half = s.B * s.Hkv * chunk_bytes;   // K part of a slot; V follows
  char* slots[2] = {slot0, slot1};
  int e;
  // NaN as bf16 pairs and as fp32 words
  auto fill_nan = [&](int sl) { return launch_fill2d(slots[sl], 0, 2 * slot_half, 1, 0x7FC07FC0u, ss); };

  auto issue_copy = [&](int k) -> ra_status {
    const int sl = k & 1;
    if (k >= 2 && (e = (int)hipStreamWaitEvent(ss, ctx->freed[sl], 0))) return dev_err(e, "wait slot_free");
    if (k >= 2 && side && (e = (int)hipStreamWaitEvent(ss, ctx->qfreed[sl], 0)))
      return dev_err(e, "wait slot_free (side)");
    if (k >= 2 && poison && (e = fill_nan(sl))) return dev_err(e, "poison slot");
    if ((e = stage_copy(s, staged[k].owner, k_ring, v_ring, slots[sl], ss))) return dev_err(e, "staging copy");
    if ((e = (int)hipEventRecord(ctx->ready[sl], ss))) return dev_err(e, "record slot_ready");
    return RA_OK;
  };

  ra_status st;
  const bool use_alt = alt && alt != cs && nstaged > 1;
  hipStream_t kvs[2] = {cs, use_alt ? alt : cs};
  JoinGuard alt_join{ctx->ajoin, alt, cs, use_alt};
  if ((nstaged > 0 && ss != cs) || use_alt) {
    // The slots may still be read by earlier work on the compute stream, and the second compute
    // stream starts after everything the caller queued before the loop.
    if ((e = (int)hipEventRecord(ctx->start, cs))) return dev_err(e, "record start");
    if (nstaged > 0 && ss != cs && (e = (int)hipStreamWaitEvent(ss, ctx->start, 0))) return dev_err(e, "wait start");
    if (use_alt && (e = (int)hipStreamWaitEvent(alt, ctx->start, 0))) return dev_err(e, "wait start (alt)");
  }
  if (nstaged > 0 && (st = issue_copy(0)) != RA_OK) return st;
  if (have_local) {
    Range r(marks, "ra %s step 0 owner %d (local)", pass, (int)local.owner);
    const int64_t off = (int64_t)rank * chunk_bytes;
    if ((e = step_fn(cs, -1, (const char*)k_ring + off, (const char*)v_ring + off, s.S, local.owner,
                     local.pairs, local.n)))
      return dev_err(e, "chunk kernel (local step)");
  }
  for (int k = 0; k < nstaged; ++k) {
    Range r(marks, "ra %s step %d owner %d (slot %d)", pass, (int)staged[k].i, (int)staged[k].owner, k & 1);
    if (k + 1 < nstaged && (st = issue_copy(k + 1)) != RA_OK) return st;
    const int sl = k & 1;
    const hipStream_t t = kvs[sl];
    if ((e = (int)hipStreamWaitEvent(t, ctx->ready[sl], 0))) return dev_err(e, "wait slot_ready");
    if ((e = step_fn(t, sl, slots[sl], slots[sl] + slot_half, s.chunk, staged[k].owner, staged[k].pairs,
                     staged[k].n)))
      return dev_err(e, "chunk kernel (staged step)");
    if ((e = (int)hipEventRecord(ctx->freed[sl], t))) return dev_err(e, "record slot_free");
    if (side && (e = (int)hipEventRecord(ctx->qfreed[sl], side))) return dev_err(e, "record slot_free (side)");
  }
  if (use_alt) {
    alt_join.armed = false;
    if ((e = (int)hipEventRecord(ctx->ajoin, alt))) return dev_err(e, "record alt join");
    if ((e = (int)hipStreamWaitEvent(cs, ctx->ajoin, 0))) return dev_err(e, "wait alt join");
  }
  if (poison && nstaged > 0) {
    // both slots after their last readers; the compute stream (the caller's) then waits for the
    // fills, so that they are ordered before whatever the caller does with the workspace next
    for (int sl = 0; sl < (nstaged > 1 ? 2 : 1); ++sl) {
      if ((e = (int)hipStreamWaitEvent(ss, ctx->freed[sl], 0))) return dev_err(e, "wait slot_free");
      if (side && (e = (int)hipStreamWaitEvent(ss, ctx->qfreed[sl], 0))) return dev_err(e, "wait slot_free (side)");
      if ((e = fill_nan(sl))) return dev_err(e, "poison slot");
    }
    if (ss != cs) {
      if ((e = (int)hipEventRecord(ctx->poisoned, ss))) return dev_err(e, "record poison");
      if ((e = (int)hipStreamWaitEvent(cs, ctx->poisoned, 0))) return dev_err(e, "wait poison");
    }
  }
  return RA_OK;
}

}  // namespace
}  // namespace ra

namespace ra {
namespace {

// Destroys the context's events and streams that exist (all of them after a successful
// ra_create, those created so far after a failed one; the rest are null), then the context.
// The caller has made the context's device current.
void release(ra_context* c) {
  auto ev = [](hipEvent_t x) { if (x) (void)hipEventDestroy(x); };
  ev(c->start);
  for (int i = 0; i < 2; ++i) {
    ev(c->ready[i]);
    ev(c->freed[i]);
    ev(c->qfreed[i]);
  }
  ev(c->ajoin);
  ev(c->dslocal);
  for (int i = 0; i < kMaxSteps; ++i) ev(c->done[i]);
  ev(c->fin);
  ev(c->bfork);
  ev(c->bjoin);
  ev(c->poisoned);
  for (int i = 0; i < kPoolStreams; ++i)
    if (c->pool[i]) (void)hipStreamDestroy(c->pool[i]);
  delete c;
}

}  // namespace
}  // namespace ra

using namespace ra;

extern "C" {

ra_status ra_create(int32_t device, ra_context** out) {
  clear_error();
  if (!out) return fail(RA_ERR_INVALID, "out is NULL");
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return fail(RA_ERR_DEVICE, "no HIP device");
  if (device < 0 || device >= n) return fail(RA_ERR_INVALID, "device %d outside [0, %d)", device, n);
  DeviceGuard g(device);
  if (!g.ok) return fail(RA_ERR_DEVICE, "hipSetDevice(%d) failed", device);
  ra_context* c = new ra_context();
  c->device = device;
  hipError_t e = hipEventCreateWithFlags(&c->start, hipEventDisableTiming);
  for (int i = 0; i < 2 && e == hipSuccess; ++i) {
    e = hipEventCreateWithFlags(&c->ready[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->freed[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->qfreed[i], hipEventDisableTiming);
  }
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ajoin, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->dslocal, hipEventDisableTiming);
  for (int i = 0; i < kMaxSteps && e == hipSuccess; ++i)
    e = hipEventCreateWithFlags(&c->done[i], hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->fin, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->bfork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->bjoin, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->poisoned, hipEventDisableTiming);
  for (int i = 0; i < kPoolStreams && e == hipSuccess; ++i)
    e = hipStreamCreateWithFlags(&c->pool[i], hipStreamNonBlocking);
  if (e != hipSuccess) {
    release(c);  // the handles created before the failure
    return fail(RA_ERR_DEVICE, "event or stream creation failed: %s", hipGetErrorString(e));
  }
  // the static scratch's address on this device (the device is current here)
  if ((e = (hipError_t)noalloc_scratch_address(device, &c->noalloc_scratch)) != hipSuccess) {
    release(c);
    return fail(RA_ERR_DEVICE, "address of the static scratch on device %d: %s", device, hipGetErrorString(e));
  }
  *out = c;
  return RA_OK;
}

void ra_destroy(ra_context* c) {
  if (!c) return;
  DeviceGuard g(c->device);
  release(c);
}

ra_status ra_set_debug(ra_context* ctx, uint32_t flags) {
  clear_error();
  if (!ctx) return fail(RA_ERR_INVALID, "context is NULL");
  if (flags & ~(uint32_t)(RA_DEBUG_POISON_SLOTS | RA_DEBUG_ROCTX))
    return fail(RA_ERR_INVALID, "unknown debug flags 0x%x", (unsigned)flags);
  ctx->debug = flags;
  return RA_OK;
}

ra_status ra_layout_gather(ra_context* ctx, const ra_problem* prob, int32_t rank_begin,
                           int32_t rank_count, int64_t heads, const void* full, void* out,
                           void* stream) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if (rank_count < 1 || rank_begin < 0 || rank_begin + rank_count > s.cp)
    return fail(RA_ERR_INVALID, "rank range [%d, %d) outside [0, %d)", rank_begin,
                rank_begin + rank_count, s.cp);
  if (heads != s.Hq && heads != s.Hkv) return fail(RA_ERR_INVALID, "heads must be heads_q or heads_kv");
  if ((st = need_ptrs({full, out})) != RA_OK) return st;
  if (rank_count * s.chunk > (int64_t)UINT32_MAX / 64)
    return fail(RA_ERR_UNSUPPORTED, "too many rows for one layout launch");
  DeviceGuard g(ctx->device);
  return dev_err(launch_layout(s, rank_begin, rank_count, heads, full, out, true, stream), "layout gather");
}

ra_status ra_layout_scatter(ra_context* ctx, const ra_problem* prob, int32_t rank_begin,
                            int32_t rank_count, int64_t heads, const void* in, void* full,
                            void* stream) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if (rank_count < 1 || rank_begin < 0 || rank_begin + rank_count > s.cp)
    return fail(RA_ERR_INVALID, "rank range [%d, %d) outside [0, %d)", rank_begin,
                rank_begin + rank_count, s.cp);
  if (heads != s.Hq && heads != s.Hkv) return fail(RA_ERR_INVALID, "heads must be heads_q or heads_kv");
  if ((st = need_ptrs({in, full})) != RA_OK) return st;
  if (rank_count * s.chunk > (int64_t)UINT32_MAX / 64)
    return fail(RA_ERR_UNSUPPORTED, "too many rows for one layout launch");
  DeviceGuard g(ctx->device);
  return dev_err(launch_layout(s, rank_begin, rank_count, heads, in, full, false, stream), "layout scatter");
}

ra_status ra_ulysses_reshard(ra_context* ctx, const ra_problem* prob, int32_t step, int64_t heads,
                             const void* src, void* dst, void* stream) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if (step < RA_A2A_SEQ_PACK || step > RA_A2A_SEQ_UNPACK) return fail(RA_ERR_INVALID, "unknown re-shard step %d", step);
  if (heads != s.Hq && heads != s.Hkv) return fail(RA_ERR_INVALID, "heads must be heads_q or heads_kv");
  if (heads % s.cp) return fail(RA_ERR_INVALID, "heads (%lld) must be divisible by cp_size (%d)", (long long)heads, s.cp);
  if ((st = need_ptrs({src, dst})) != RA_OK) return st;
  // every re-shard step reads and writes batch * heads * seq_len/cp * head_dim elements
  const uintptr_t nbytes = (uintptr_t)(s.B * heads * s.chunk * s.D * s.esize);
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + nbytes && b < a + nbytes) return fail(RA_ERR_INVALID, "re-shard src and dst overlap");
  DeviceGuard g(ctx->device);
  return dev_err(launch_reshard(s, step, heads, src, dst, stream), "ulysses re-shard");
}

ra_status ra_stage_kv(ra_context* ctx, const ra_problem* prob, int32_t owner, const void* k_ring,
                      const void* v_ring, void* dst, void* stream) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if ((st = check_rank(s, owner)) != RA_OK) return st;
  if ((st = need_ptrs({k_ring, v_ring, dst})) != RA_OK) return st;
  DeviceGuard g(ctx->device);
  return dev_err(stage_copy(s, owner, k_ring, v_ring, dst, (hipStream_t)stream), "staging copy");
}

ra_status ra_state_init(ra_context* ctx, const ra_problem* prob, int64_t rows, float* U, float* m,
                        float* l, void* stream) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if (rows < 0) return fail(RA_ERR_INVALID, "rows must be >= 0");
  if ((st = need_ptrs({U, m, l})) != RA_OK) return st;
  DeviceGuard g(ctx->device);
  return dev_err(launch_state_init(s.B * s.Hq * rows, s.D, U, m, l, stream), "state init");
}

ra_status ra_chunk_fwd(ra_context* ctx, const ra_problem* prob, const void* q, int64_t q_rows,
                       const void* k, const void* v, int64_t kv_rows, const ra_pair* pairs,
                       int32_t n_pairs, float* U, float* m, float* l, void* stream) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if (q_rows < 0 || kv_rows < 0) return fail(RA_ERR_INVALID, "row counts must be >= 0");
  if ((st = check_pairs(pairs, n_pairs, q_rows, kv_rows)) != RA_OK) return st;
  if ((st = need_ptrs({q, k, v, U, m, l})) != RA_OK) return st;
  KParams kp = base_params(s);
  kp.q = q; kp.k = k; kp.v = v; kp.U = U; kp.m = m; kp.l = l;
  kp.q_head_rows = q_rows;
  kp.kv_head_rows = kv_rows;
  kp.dkv_head_rows = kv_rows;
  DeviceGuard g(ctx->device);
  return dev_err(run_fwd(s, kp, pairs, n_pairs, stream), "chunk forward");
}

ra_status ra_lse_merge(ra_context* ctx, const ra_problem* prob, int64_t rows, const float* o_part,
                       const float* lse_part, float* U, float* m, float* l, void* stream) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if (rows < 0) return fail(RA_ERR_INVALID, "rows must be >= 0");
  if ((st = need_ptrs({o_part, lse_part, U, m, l})) != RA_OK) return st;
  DeviceGuard g(ctx->device);
  return dev_err(launch_lse_merge(s.B * s.Hq * rows, s.D, o_part, lse_part, U, m, l, stream), "lse merge");
}

ra_status ra_fwd_finalize(ra_context* ctx, const ra_problem* prob, int64_t rows, const float* U,
                          const float* m, const float* l, void* o, float* lse, void* stream) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if (rows < 0) return fail(RA_ERR_INVALID, "rows must be >= 0");
  if ((st = need_ptrs({U, m, l, o, lse})) != RA_OK) return st;
  DeviceGuard g(ctx->device);
  return dev_err(launch_fwd_finalize(s.B * s.Hq * rows, s.D, s.dtype, U, m, l, o, lse, stream),
                 "forward finalize");
}

ra_status ra_bwd_preprocess(ra_context* ctx, const ra_problem* prob, int64_t rows, const void* o,
                            const void* dO, float* delta, void* stream) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if (rows < 0) return fail(RA_ERR_INVALID, "rows must be >= 0");
  if ((st = need_ptrs({o, dO, delta})) != RA_OK) return st;
  DeviceGuard g(ctx->device);
  return dev_err(launch_bwd_preprocess(s.B * s.Hq * rows, s.D, s.dtype, o, dO, delta, stream),
                 "backward preprocess");
}

ra_status ra_chunk_bwd(ra_context* ctx, const ra_problem* prob, const void* q, const void* dO,
                       const float* lse, const float* delta, int64_t q_rows, const void* k,
                       const void* v, int64_t kv_rows, const ra_pair* pairs, int32_t n_pairs,
                       float* dq_acc, float* dk_acc, float* dv_acc, void* stream) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if (q_rows < 0 || kv_rows < 0) return fail(RA_ERR_INVALID, "row counts must be >= 0");
  if ((st = check_pairs(pairs, n_pairs, q_rows, kv_rows)) != RA_OK) return st;
  if ((st = need_ptrs({q, dO, lse, delta, k, v})) != RA_OK) return st;
  // dq_acc may be NULL (no dQ), or dk_acc and dv_acc together (no dK, dV); not all three.
  if ((dk_acc == nullptr) != (dv_acc == nullptr))
    return fail(RA_ERR_INVALID, "dk_acc and dv_acc must both be given or both be NULL");
  if (!dq_acc && !dk_acc) return fail(RA_ERR_INVALID, "no gradient requested (dq_acc, dk_acc, dv_acc all NULL)");
  if (dq_acc && (st = need_ptrs({dq_acc})) != RA_OK) return st;
  if (dk_acc && (st = need_ptrs({dk_acc, dv_acc})) != RA_OK) return st;
  KParams kp = base_params(s);
  kp.q = q; kp.dO = dO; kp.lse = lse; kp.delta = delta; kp.k = k; kp.v = v;
  kp.U = dq_acc; kp.dk = dk_acc; kp.dv = dv_acc;
  kp.q_head_rows = q_rows;
  kp.kv_head_rows = kv_rows;
  kp.dkv_head_rows = kv_rows;
  DeviceGuard g(ctx->device);
  const BwdFork fork{ctx->pool[0], ctx->bfork, ctx->bjoin};
  return dev_err(run_bwd(s, kp, pairs, n_pairs, stream, &fork), "chunk backward");
}

ra_status ra_chunk_bwd_ds_size(const ra_problem* prob, int64_t q_rows, int64_t kv_rows,
                               const ra_pair* pairs, int32_t n_pairs, size_t* bytes) {
  clear_error();
  Shape s;
  ra_status st = resolve(prob, &s);
  if (st != RA_OK) return st;
  if (!bytes) return fail(RA_ERR_INVALID, "bytes is NULL");
  if (q_rows < 0 || kv_rows < 0) return fail(RA_ERR_INVALID, "row counts must be >= 0");
  if ((st = check_pairs(pairs, n_pairs, q_rows, kv_rows)) != RA_OK) return st;
  *bytes = s.dtype == RA_BF16 ? ds_layout(s, pairs, n_pairs, nullptr) : 0;
  return RA_OK;
}

namespace ra {
namespace {

// ra_chunk_bwd_ds and ra_chunk_bwd_ds_noalloc: the same call with the scratch given (`fixed` =
// false: a caller buffer, too small is RA_ERR_WORKSPACE) or the static one (`fixed` = true).
ra_status chunk_bwd_ds(ra_context* ctx, const ra_problem* prob, const void* q, const void* dO,
                       const float* lse, const float* delta, int64_t q_rows, const void* k,
                       const void* v, int64_t kv_rows, const ra_pair* pairs, int32_t n_pairs,
                       float* dq_acc, float* dk_acc, float* dv_acc, void* scratch,
                       size_t scratch_bytes, void* stream, bool fixed) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if (q_rows < 0 || kv_rows < 0) return fail(RA_ERR_INVALID, "row counts must be >= 0");
  if ((st = check_pairs(pairs, n_pairs, q_rows, kv_rows)) != RA_OK) return st;
  if ((st = need_ptrs({q, dO, lse, delta, k, v})) != RA_OK) return st;
  if ((dk_acc == nullptr) != (dv_acc == nullptr))
    return fail(RA_ERR_INVALID, "dk_acc and dv_acc must both be given or both be NULL");
  if (!dq_acc && !dk_acc) return fail(RA_ERR_INVALID, "no gradient requested (dq_acc, dk_acc, dv_acc all NULL)");
  if (dq_acc && (st = need_ptrs({dq_acc})) != RA_OK) return st;
  if (dk_acc && (st = need_ptrs({dk_acc, dv_acc})) != RA_OK) return st;
  KParams kp = base_params(s);
  kp.q = q; kp.dO = dO; kp.lse = lse; kp.delta = delta; kp.k = k; kp.v = v;
  kp.U = dq_acc; kp.dk = dk_acc; kp.dv = dv_acc;
  kp.q_head_rows = q_rows;
  kp.kv_head_rows = kv_rows;
  kp.dkv_head_rows = kv_rows;
  if (s.dtype != RA_BF16) {  // the fp32 path forms dQ in its single kernel: no scratch
    if (!dq_acc || !dk_acc)
      return fail(RA_ERR_UNSUPPORTED, "the fp32 path computes all three gradients in one pass");
    DeviceGuard g(ctx->device);
    return dev_err(run_bwd(s, kp, pairs, n_pairs, stream, nullptr), "chunk backward");
  }
  const size_t need = ds_layout(s, pairs, n_pairs, nullptr);
  if (fixed) {
    if (need > scratch_bytes)
      return fail(RA_ERR_WORKSPACE, "the stored dS needs %zu bytes; the static scratch holds %zu", need,
                  scratch_bytes);
  } else {
    if (need > 0 && (!scratch || !aligned16(scratch)))
      return fail(RA_ERR_INVALID, "scratch is NULL or not 16-byte aligned");
    if (scratch_bytes < need)
      return fail(RA_ERR_WORKSPACE, "scratch has %zu bytes, needs %zu", scratch_bytes, need);
  }
  DeviceGuard g(ctx->device);
  return dev_err(run_bwd_ds(s, kp, pairs, n_pairs, scratch, stream, nullptr), "chunk backward (stored dS)");
}

}  // namespace
}  // namespace ra

ra_status ra_chunk_bwd_ds(ra_context* ctx, const ra_problem* prob, const void* q, const void* dO,
                          const float* lse, const float* delta, int64_t q_rows, const void* k,
                          const void* v, int64_t kv_rows, const ra_pair* pairs, int32_t n_pairs,
                          float* dq_acc, float* dk_acc, float* dv_acc, void* scratch,
                          size_t scratch_bytes, void* stream) {
  return ra::chunk_bwd_ds(ctx, prob, q, dO, lse, delta, q_rows, k, v, kv_rows, pairs, n_pairs, dq_acc,
                          dk_acc, dv_acc, scratch, scratch_bytes, stream, false);
}

ra_status ra_chunk_bwd_ds_noalloc(ra_context* ctx, const ra_problem* prob, const void* q,
                                  const void* dO, const float* lse, const float* delta,
                                  int64_t q_rows, const void* k, const void* v, int64_t kv_rows,
                                  const ra_pair* pairs, int32_t n_pairs, float* dq_acc,
                                  float* dk_acc, float* dv_acc, void* stream) {
  clear_error();
  if (!ctx) return ra::fail(RA_ERR_INVALID, "context is NULL");
  return ra::chunk_bwd_ds(ctx, prob, q, dO, lse, delta, q_rows, k, v, kv_rows, pairs, n_pairs, dq_acc,
                          dk_acc, dv_acc, ctx->noalloc_scratch, RA_NOALLOC_SCRATCH_BYTES, stream, true);
}

ra_status ra_cast_from_f32(ra_context* ctx, const ra_problem* prob, int64_t n, const float* src,
                           void* dst, void* stream) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if (n < 0 || n % 4) return fail(RA_ERR_INVALID, "n must be a non-negative multiple of 4");
  if ((st = need_ptrs({src, dst})) != RA_OK) return st;
  DeviceGuard g(ctx->device);
  return dev_err(launch_cast_from_f32(n, s.dtype, src, dst, stream), "cast");
}

ra_status ra_rank_view_fwd(ra_context* ctx, const ra_problem* prob, int32_t rank,
                           const void* q_slice, const void* k_ring, const void* v_ring,
                           void* o_slice, float* lse_slice, void* workspace,
                           size_t workspace_bytes, void* compute, void* staging) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if ((st = check_rank(s, rank)) != RA_OK) return st;
  if (s.cp > 64) return fail(RA_ERR_UNSUPPORTED, "cp_size above 64 is not supported by the rank view");
  if ((st = need_ptrs({q_slice, k_ring, v_ring, o_slice, lse_slice})) != RA_OK) return st;
  const FwdWs W = fwd_ws(s);
  if (!workspace || !aligned16(workspace)) return fail(RA_ERR_INVALID, "workspace is NULL or misaligned");
  if (workspace_bytes < W.total)
    return fail(RA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, W.total);
  char* ws = static_cast<char*>(workspace);
  float* U = reinterpret_cast<float*>(ws + W.U);
  float* m = reinterpret_cast<float*>(ws + W.m);
  float* l = reinterpret_cast<float*>(ws + W.l);
  hipStream_t cs = (hipStream_t)compute;
  hipStream_t ss = staging ? (hipStream_t)staging : cs;
  DeviceGuard g(ctx->device);
  int e;
  const int64_t rows = s.B * s.Hq * s.chunk;
  // Consecutive steps fold into the same rows, so one running state would chain every step's
  // kernel to the previous one.  With two or more staged steps, the steps staged in slot 1 fold
  // into a second state on a second stream, concurrently with the others, and the two states
  // are merged after the ring (online softmax is exact in any grouping).  Which state a step
  // uses depends only on its slot, so the result does not depend on timing.
  const bool two = W.two && staged_steps(s, rank) >= 2;
  float* U2 = reinterpret_cast<float*>(ws + W.U2);
  float* m2 = reinterpret_cast<float*>(ws + W.m2);
  float* l2 = reinterpret_cast<float*>(ws + W.l2);
  // The first step (the local one, which the ring loop runs first) has pairs covering every row
  // of the slice (its diagonal pairs are never skipped), so it starts from the empty state
  // instead of reading an initialised one.  The second state is initialised: its steps may
  // leave rows untouched.
  if (two && (e = launch_state_init(rows, s.D, U2, m2, l2, cs))) return dev_err(e, "state init");
  KParams kp = base_params(s);
  kp.q = q_slice;
  kp.q_head_rows = s.chunk;
  bool first = true;
  auto step = [&](hipStream_t t, int slot, const void* k, const void* v, int64_t kv_head_rows,
                  int32_t owner, const ra_pair* pairs, int32_t n) -> int {
    (void)owner;
    (void)slot;
    const bool b = t != cs;  // slot-1 steps run on the second stream
    kp.U = b ? U2 : U; kp.m = b ? m2 : m; kp.l = b ? l2 : l;
    kp.fresh = first ? 1 : 0;
    first = false;
    kp.k = k; kp.v = v;
    kp.kv_head_rows = kv_head_rows;
    kp.dkv_head_rows = kv_head_rows;
    return run_fwd(s, kp, pairs, n, t);
  };
  if ((st = ring_loop(ctx, "fwd", s, rank, k_ring, v_ring, ws + W.slot[0], ws + W.slot[1], cs, ss, nullptr,
                      two ? ctx->pool[1] : nullptr, step)) != RA_OK)
    return st;
  if (two)
    return dev_err(launch_merge_finalize(rows, s.D, s.dtype, U2, m2, l2, U, m, l, o_slice, lse_slice, cs),
                   "forward merge and finalize");
  return dev_err(launch_fwd_finalize(rows, s.D, s.dtype, U, m, l, o_slice, lse_slice, cs),
                 "forward finalize");
}

ra_status ra_rank_view_fwd_split(ra_context* ctx, const ra_problem* prob, int32_t rank,
                                 const void* q_slice, const void* k_all, const void* v_all,
                                 void* o_slice, float* lse_slice, void* workspace,
                                 size_t workspace_bytes, void* compute, void* merge) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if ((st = check_rank(s, rank)) != RA_OK) return st;
  if (s.cp > kMaxSteps) return fail(RA_ERR_UNSUPPORTED, "cp_size above %d is not supported", kMaxSteps);
  if ((st = need_ptrs({q_slice, k_all, v_all, o_slice, lse_slice})) != RA_OK) return st;
  const SplitWs W = split_ws(s);
  if (!workspace || !aligned16(workspace)) return fail(RA_ERR_INVALID, "workspace is NULL or misaligned");
  if (workspace_bytes < W.total)
    return fail(RA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, W.total);
  char* ws = static_cast<char*>(workspace);
  hipStream_t cs = (hipStream_t)compute;
  hipStream_t ms = merge ? (hipStream_t)merge : cs;
  DeviceGuard g(ctx->device);
  int e;
  const int64_t rows = s.B * s.Hq * s.chunk;
  const int64_t chunk_bytes = s.chunk * s.D * s.esize;
  float* U = reinterpret_cast<float*>(ws + W.U);
  float* m = reinterpret_cast<float*>(ws + W.m);
  float* l = reinterpret_cast<float*>(ws + W.l);
  // everything starts after the caller's earlier work on the compute stream
  if ((e = (int)hipEventRecord(ctx->start, cs))) return dev_err(e, "record start");
  for (int i = 0; i < kPoolStreams; ++i)
    if ((e = (int)hipStreamWaitEvent(ctx->pool[i], ctx->start, 0))) return dev_err(e, "pool wait start");
  if (ms != cs && (e = (int)hipStreamWaitEvent(ms, ctx->start, 0))) return dev_err(e, "merge wait start");
  // on an error return, the pool streams and the merge stream are still joined into `compute`
  JoinGuard pool_join[kPoolStreams] = {};
  for (int i = 0; i < kPoolStreams; ++i) pool_join[i] = JoinGuard{ctx->ajoin, ctx->pool[i], cs, false};
  for (int i = 0; i < kPoolStreams; ++i) pool_join[i].armed = true;
  JoinGuard merge_join{ctx->fin, ms, cs, ms != cs};
  if ((e = launch_state_init(rows, s.D, U, m, l, ms))) return dev_err(e, "state init");
  int np = 0;
  for (int32_t i = 0; i < s.cp; ++i) {
    int32_t owner, n;
    ra_pair pairs[4];
    plan_step(s, rank, i, &owner, pairs, &n);
    if (!any_compute(pairs, n)) continue;
    // partial state of this chunk, computed on a pool stream straight from the gathered K/V
    char* part = ws + W.part + (size_t)np * W.part_stride;
    float* Up = reinterpret_cast<float*>(part);
    float* mp = reinterpret_cast<float*>(part + W.m);
    float* lp = reinterpret_cast<float*>(part + W.l);
    hipStream_t ps = ctx->pool[np % kPoolStreams];
    if ((e = launch_state_init(rows, s.D, Up, mp, lp, ps))) return dev_err(e, "partial state init");
    KParams kp = base_params(s);
    kp.q = q_slice; kp.U = Up; kp.m = mp; kp.l = lp;
    kp.q_head_rows = s.chunk;
    kp.k = (const char*)k_all + owner * chunk_bytes;
    kp.v = (const char*)v_all + owner * chunk_bytes;
    kp.kv_head_rows = s.S;
    kp.dkv_head_rows = s.S;
    if ((e = run_fwd(s, kp, pairs, n, ps))) return dev_err(e, "chunk kernel (split)");
    if ((e = (int)hipEventRecord(ctx->done[np], ps))) return dev_err(e, "record chunk done");
    // its merge into the running state, on the merge stream, in step order
    if ((e = (int)hipStreamWaitEvent(ms, ctx->done[np], 0))) return dev_err(e, "merge wait chunk");
    if ((e = launch_state_merge(rows, s.D, Up, mp, lp, U, m, l, ms))) return dev_err(e, "state merge");
    ++np;
  }
  if ((e = launch_fwd_finalize(rows, s.D, s.dtype, U, m, l, o_slice, lse_slice, ms)))
    return dev_err(e, "forward finalize");
  // every pool stream's work is ordered before the merge stream's (done events)
  for (int i = 0; i < kPoolStreams; ++i) pool_join[i].armed = false;
  merge_join.armed = false;
  if (ms != cs) {
    if ((e = (int)hipEventRecord(ctx->fin, ms))) return dev_err(e, "record fin");
    if ((e = (int)hipStreamWaitEvent(cs, ctx->fin, 0))) return dev_err(e, "compute wait fin");
  }
  return RA_OK;
}

ra_status ra_rank_view_bwd(ra_context* ctx, const ra_problem* prob, int32_t rank,
                           const void* q_slice, const void* k_ring, const void* v_ring,
                           const void* o_slice, const float* lse_slice, const void* dO_slice,
                           void* dq_slice, void* dk_ring, void* dv_ring, void* workspace,
                           size_t workspace_bytes, void* compute, void* staging) {
  Shape s;
  ra_status st = common(ctx, prob, &s);
  if (st != RA_OK) return st;
  if ((st = check_rank(s, rank)) != RA_OK) return st;
  if (s.cp > 64) return fail(RA_ERR_UNSUPPORTED, "cp_size above 64 is not supported by the rank view");
  if ((st = need_ptrs({q_slice, k_ring, v_ring, o_slice, lse_slice, dO_slice, dq_slice, dk_ring,
                       dv_ring})) != RA_OK)
    return st;
  const BwdWs W = bwd_ws(s);
  if (!workspace || !aligned16(workspace)) return fail(RA_ERR_INVALID, "workspace is NULL or misaligned");
  if (workspace_bytes < W.total)
    return fail(RA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, W.total);
  char* ws = static_cast<char*>(workspace);
  float* dq = reinterpret_cast<float*>(ws + W.dq);
  float* dk = reinterpret_cast<float*>(ws + W.dk);
  float* dv = reinterpret_cast<float*>(ws + W.dv);
  float* delta = reinterpret_cast<float*>(ws + W.delta);
  hipStream_t cs = (hipStream_t)compute;
  hipStream_t ss = staging ? (hipStream_t)staging : cs;
  DeviceGuard g(ctx->device);
  int e;
  const int64_t rows = s.B * s.Hq * s.chunk;
  if ((e = launch_fill_zero(rows * s.D, dq, cs))) return dev_err(e, "zero dq");
  if ((e = launch_bwd_preprocess(rows, s.D, s.dtype, o_slice, dO_slice, delta, cs)))
    return dev_err(e, "backward preprocess");
  KParams kp = base_params(s);
  kp.q = q_slice; kp.dO = dO_slice; kp.lse = lse_slice; kp.delta = delta; kp.U = dq;
  kp.q_head_rows = s.chunk;
  kp.dkv_head_rows = s.S;
  // The dQ kernels run on a pool stream beside the dK/dV kernels and are joined once, after the
  // ring: a step's dK/dV kernel can start while the previous step's dQ kernel drains.  The dQ
  // kernels stay in order on their stream (each adds into the same dq rows).  The dK/dV kernels
  // of different steps write different owners' rows, so in the bf16 path the steps staged in
  // slot 1 run theirs on a second pool stream, beside those of the compute stream.
  hipStream_t side = ctx->pool[0];
  const BwdFork fork{side, ctx->bfork, nullptr};
  JoinGuard side_join{ctx->bjoin, side, cs, true};
  // Each owner's chunk is the K/V of exactly one ring step, so its dK/dV rows are complete once
  // that step's dK/dV kernel has run (the dQ kernels do not touch them): the rows are zeroed
  // just before it and cast into dk_ring / dv_ring just after it, on the same stream -- the
  // ring's return of the K/V gradients to their owner, overlapping the later steps.
  const int64_t blk = s.chunk * s.D;  // one owner's rows of one (batch, kv head)
  const int64_t pitch = s.S * s.D;    // head stride of the ring-ordered tensors
  const int64_t nkvh = s.B * s.Hkv;
  bool visited[64] = {};
  // bf16: the dK/dV kernel stores dS into one of two buffers (the local step and the steps staged
  // in slot 1 use buffer 1, slot-0 steps buffer 0) and the step's dQ kernel reads it on `side`.
  // A staged step's buffer is free once the dQ kernel two steps back has run: its staging copy
  // already waited for that (the slot's side event).  The local step shares buffer 1 with the
  // first slot-1 step, which waits for the local dQ kernel explicitly.
  const bool use_ds = s.dtype == RA_BF16 && W.ds_bytes > 0;
  bool local_recorded = false, local_waited = false;
  auto step = [&](hipStream_t t, int slot, const void* k, const void* v, int64_t kv_head_rows,
                  int32_t owner, const ra_pair* pairs, int32_t n) -> int {
    kp.k = k; kp.v = v;
    kp.kv_head_rows = kv_head_rows;
    float* const dko = dk + (int64_t)owner * blk;
    float* const dvo = dv + (int64_t)owner * blk;
    int r;
    if ((r = launch_zero2d(dko, pitch * 4, blk * 4, nkvh, t))) return r;
    if ((r = launch_zero2d(dvo, pitch * 4, blk * 4, nkvh, t))) return r;
    kp.dk = dko;
    kp.dv = dvo;
    if (use_ds) {
      const int buf = slot == 0 ? 0 : 1;
      if (slot == 1 && local_recorded && !local_waited) {
        if ((r = (int)hipStreamWaitEvent(t, ctx->dslocal, 0))) return r;
        local_waited = true;
      }
      if ((r = run_bwd_ds(s, kp, pairs, n, ws + W.ds[buf], t, &fork))) return r;
      if (slot < 0) {
        if ((r = (int)hipEventRecord(ctx->dslocal, side))) return r;
        local_recorded = true;
      }
    } else if ((r = run_bwd(s, kp, pairs, n, t, &fork))) {
      return r;
    }
    visited[owner] = true;
    const int64_t off = (int64_t)owner * blk * s.esize;
    if ((r = launch_cast2d(dko, static_cast<char*>(dk_ring) + off, pitch, blk, nkvh, s.dtype, t))) return r;
    return launch_cast2d(dvo, static_cast<char*>(dv_ring) + off, pitch, blk, nkvh, s.dtype, t);
  };
  // (the fp32 path adds dQ inside its single kernel: its steps stay on one stream)
  if ((st = ring_loop(ctx, "bwd", s, rank, k_ring, v_ring, ws + W.slot[0], ws + W.slot[1], cs, ss, side,
                      s.dtype == RA_BF16 ? ctx->pool[1] : nullptr, step)) != RA_OK)
    return st;
  side_join.armed = false;
  if ((e = (int)hipEventRecord(ctx->bjoin, side))) return dev_err(e, "record dq join");
  if ((e = (int)hipStreamWaitEvent(cs, ctx->bjoin, 0))) return dev_err(e, "wait dq join");
  if ((e = launch_cast_from_f32(rows * s.D, s.dtype, dq, dq_slice, cs))) return dev_err(e, "cast dq");
  // owners whose chunk no step attends to (skipped steps) get zero gradients
  for (int32_t o = 0; o < s.cp; ++o) {
    if (visited[o]) continue;
    const int64_t off = (int64_t)o * blk * s.esize;
    if ((e = launch_zero2d(static_cast<char*>(dk_ring) + off, pitch * s.esize, blk * s.esize, nkvh, cs)))
      return dev_err(e, "zero dk");
    if ((e = launch_zero2d(static_cast<char*>(dv_ring) + off, pitch * s.esize, blk * s.esize, nkvh, cs)))
      return dev_err(e, "zero dv");
  }
  return RA_OK;
}

}  // extern "C"
