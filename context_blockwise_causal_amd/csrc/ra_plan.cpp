// Host-only core of libringattn: validation, ring step planning, workspace carve-up and the
// per-launch range tables.  Plain C++17 with no HIP calls, so every function here can be
// exercised on a machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>

#include "ra_internal.h"

namespace ra {

static thread_local std::string g_last_error;

ra_status fail(ra_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

const char* last_error_cstr() { return g_last_error.c_str(); }

ra_status resolve(const ra_problem* p, Shape* out) {
  if (!p) return fail(RA_ERR_INVALID, "problem is NULL");
  if (p->batch <= 0 || p->seq_len <= 0 || p->heads_q <= 0 || p->heads_kv <= 0 || p->head_dim <= 0)
    return fail(RA_ERR_INVALID, "batch, seq_len, heads and head_dim must be positive");
  if (p->cp_size <= 0) return fail(RA_ERR_INVALID, "cp_size must be >= 1");
  if (p->layout != RA_CONTIGUOUS && p->layout != RA_ZIGZAG)
    return fail(RA_ERR_INVALID, "unknown layout %d", (int)p->layout);
  if (p->dtype != RA_F32 && p->dtype != RA_BF16)
    return fail(RA_ERR_INVALID, "unknown dtype %d", (int)p->dtype);
  if (p->heads_q % p->heads_kv)
    return fail(RA_ERR_INVALID, "heads_q (%lld) must be a multiple of heads_kv (%lld)",
                (long long)p->heads_q, (long long)p->heads_kv);
  const int64_t nchunks = p->layout == RA_ZIGZAG ? 2 * (int64_t)p->cp_size : p->cp_size;
  if (p->seq_len % nchunks)
    return fail(RA_ERR_INVALID, "seq_len (%lld) must split into %lld equal chunks",
                (long long)p->seq_len, (long long)nchunks);
  if (!(p->scale >= 0.0f) || isinf(p->scale))
    return fail(RA_ERR_INVALID, "scale must be finite and >= 0 (0 selects 1/sqrt(head_dim))");
  if (p->window < 0 || p->attn_chunk < 0)
    return fail(RA_ERR_INVALID, "window and attn_chunk must be >= 0 (0 = off)");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim %lld is not supported (64 or 128)",
                (long long)p->head_dim);
  // Index arithmetic in the kernels uses 64-bit offsets, but tile counts per launch use
  // 32-bit grid indices.
  const int64_t rows = p->batch * p->heads_q * (p->seq_len / p->cp_size);
  if (rows > (int64_t(1) << 40)) return fail(RA_ERR_UNSUPPORTED, "problem too large");
  // The row-wise kernels (layout, staging copy, re-shard) put one (batch, head) per grid row,
  // and a grid's y dimension holds at most 65535.
  if (p->batch * p->heads_q > 65535)
    return fail(RA_ERR_UNSUPPORTED, "batch * heads_q (%lld) above 65535", (long long)(p->batch * p->heads_q));
  Shape s;
  s.B = p->batch;
  s.S = p->seq_len;
  s.Hq = p->heads_q;
  s.Hkv = p->heads_kv;
  s.D = p->head_dim;
  s.n_rep = p->heads_q / p->heads_kv;
  s.cp = p->cp_size;
  s.layout = p->layout;
  s.dtype = p->dtype;
  s.scale = p->scale > 0.0f ? p->scale : (float)(1.0 / sqrt((double)p->head_dim));
  s.window = p->window;
  s.attn_chunk = p->attn_chunk;
  s.esize = p->dtype == RA_BF16 ? 2 : 4;
  s.chunk = p->seq_len / p->cp_size;
  s.nchunks = nchunks;
  s.crow = p->seq_len / nchunks;
  if (out) *out = s;
  return RA_OK;
}

ra_status check_rank(const Shape& s, int32_t rank) {
  if (rank < 0 || rank >= s.cp)
    return fail(RA_ERR_INVALID, "rank %d outside [0, %d)", (int)rank, (int)s.cp);
  return RA_OK;
}

int64_t slice_chunk(const Shape& s, int32_t rank, int32_t which) {
  if (s.layout == RA_CONTIGUOUS) return (int64_t)rank * s.crow;
  const int64_t c = which == 0 ? rank : 2 * (int64_t)s.cp - 1 - rank;
  return c * s.crow;
}

// A FULL pair whose every key lies below the first query's lowest visible key (window or
// attention chunk) has no visible key at all: the lowest visible key grows with the query.
static void restrict_pairs(const Shape& s, ra_pair* pairs, int32_t n) {
  if (s.window <= 0 && s.attn_chunk <= 0) return;
  for (int i = 0; i < n; ++i) {
    ra_pair& p = pairs[i];
    if (p.mask != RA_MASK_FULL) continue;
    if (lowest_key(p.q_pos0, s.window, s.attn_chunk) > p.kv_pos0 + p.kv_len - 1) p.mask = RA_MASK_SKIP;
  }
}

void plan_step(const Shape& s, int32_t rank, int32_t step, int32_t* owner, ra_pair pairs[4],
               int32_t* n) {
  // Ring direction: K/V move to the next rank each step, so the chunk held at step i was
  // owned by rank (rank - i) mod cp.
  *owner = (int32_t)(((int64_t)rank - step) % s.cp + s.cp) % s.cp;
  if (s.layout == RA_CONTIGUOUS) {
    const int32_t kind = step == 0 ? RA_MASK_DIAG : (step <= rank ? RA_MASK_FULL : RA_MASK_SKIP);
    pairs[0] = ra_pair{0, 0, s.chunk, s.chunk, kind, 0, (int64_t)rank * s.chunk, (int64_t)*owner * s.chunk};
    *n = 1;
    restrict_pairs(s, pairs, *n);
    return;
  }
  // Zigzag: the slice is [chunk r | chunk 2cp-1-r]; the held K/V is [chunk o | chunk 2cp-1-o].
  // Step 0 is causal attention over the rank's own tokens; for 1 <= step <= rank the second
  // K/V half lies in the future of every query; for step > rank the first Q half precedes
  // every key.
  const int64_t h = s.crow;
  int32_t ll, lh, hl, hh;
  if (step == 0) {
    ll = RA_MASK_DIAG; lh = RA_MASK_SKIP; hl = RA_MASK_FULL; hh = RA_MASK_DIAG;
  } else if (step <= rank) {
    ll = RA_MASK_FULL; lh = RA_MASK_SKIP; hl = RA_MASK_FULL; hh = RA_MASK_SKIP;
  } else {
    ll = RA_MASK_SKIP; lh = RA_MASK_SKIP; hl = RA_MASK_FULL; hh = RA_MASK_FULL;
  }
  const int64_t qlo = (int64_t)rank * h, qhi = (2 * (int64_t)s.cp - 1 - rank) * h;
  const int64_t klo = (int64_t)*owner * h, khi = (2 * (int64_t)s.cp - 1 - *owner) * h;
  pairs[0] = ra_pair{0, 0, h, h, ll, 0, qlo, klo};
  pairs[1] = ra_pair{0, h, h, h, lh, 0, qlo, khi};
  pairs[2] = ra_pair{h, 0, h, h, hl, 0, qhi, klo};
  pairs[3] = ra_pair{h, h, h, h, hh, 0, qhi, khi};
  *n = 4;
  restrict_pairs(s, pairs, *n);
}

static bool same_or_disjoint(int64_t a0, int64_t al, int64_t b0, int64_t bl) {
  if (a0 == b0 && al == bl) return true;
  return a0 + al <= b0 || b0 + bl <= a0;
}

ra_status check_pairs(const ra_pair* pairs, int32_t n, int64_t q_rows, int64_t kv_rows) {
  if (n < 0 || n > 4) return fail(RA_ERR_INVALID, "n_pairs must be in [0, 4]");
  if (n > 0 && !pairs) return fail(RA_ERR_INVALID, "pairs is NULL");
  for (int i = 0; i < n; ++i) {
    const ra_pair& p = pairs[i];
    if (p.mask != RA_MASK_FULL && p.mask != RA_MASK_DIAG && p.mask != RA_MASK_SKIP)
      return fail(RA_ERR_INVALID, "pair %d: unknown mask kind %d", i, (int)p.mask);
    if (p.reserved != 0) return fail(RA_ERR_INVALID, "pair %d: reserved field must be 0", i);
    if (p.q_row0 < 0 || p.kv_row0 < 0 || p.q_len < 0 || p.kv_len < 0)
      return fail(RA_ERR_INVALID, "pair %d: negative row or length", i);
    if (p.q_row0 + p.q_len > q_rows || p.kv_row0 + p.kv_len > kv_rows)
      return fail(RA_ERR_INVALID, "pair %d: rows out of range (q %lld+%lld > %lld or kv %lld+%lld > %lld)",
                  i, (long long)p.q_row0, (long long)p.q_len, (long long)q_rows,
                  (long long)p.kv_row0, (long long)p.kv_len, (long long)kv_rows);
    if (p.mask == RA_MASK_DIAG && p.q_len != p.kv_len)
      return fail(RA_ERR_INVALID, "pair %d: a diagonal pair needs q_len == kv_len", i);
    if (p.q_pos0 < 0 || p.kv_pos0 < 0) return fail(RA_ERR_INVALID, "pair %d: negative position", i);
  }
  for (int i = 0; i < n; ++i) {
    if (pairs[i].mask == RA_MASK_SKIP) continue;
    for (int j = i + 1; j < n; ++j) {
      if (pairs[j].mask == RA_MASK_SKIP) continue;
      if (!same_or_disjoint(pairs[i].q_row0, pairs[i].q_len, pairs[j].q_row0, pairs[j].q_len))
        return fail(RA_ERR_INVALID, "pairs %d and %d: Q ranges overlap without being equal", i, j);
      if (!same_or_disjoint(pairs[i].kv_row0, pairs[i].kv_len, pairs[j].kv_row0, pairs[j].kv_len))
        return fail(RA_ERR_INVALID, "pairs %d and %d: K/V ranges overlap without being equal", i, j);
    }
  }
  return RA_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

FwdWs fwd_ws(const Shape& s) {
  FwdWs w;
  const size_t rows = (size_t)(s.B * s.Hq * s.chunk);
  const size_t slot = (size_t)(s.B * s.Hkv * s.chunk * s.D * s.esize) * 2;  // K then V
  const int nslots = s.cp > 2 ? 2 : (int)s.cp - 1;
  size_t off = 0;
  w.U = off; off += align256(rows * s.D * 4);
  w.m = off; off += align256(rows * 4);
  w.l = off; off += align256(rows * 4);
  w.two = nslots == 2;
  w.U2 = off; if (w.two) off += align256(rows * s.D * 4);
  w.m2 = off; if (w.two) off += align256(rows * 4);
  w.l2 = off; if (w.two) off += align256(rows * 4);
  for (int i = 0; i < 2; ++i) {
    w.slot[i] = off;
    if (i < nslots) off += align256(slot);
  }
  w.total = off;
  return w;
}

SplitWs split_ws(const Shape& s) {
  SplitWs w;
  const size_t rows = (size_t)(s.B * s.Hq * s.chunk);
  const size_t state = align256(rows * s.D * 4) + 2 * align256(rows * 4);
  w.U = 0;
  w.m = align256(rows * s.D * 4);
  w.l = w.m + align256(rows * 4);
  w.part = state;
  w.part_stride = state;
  w.total = state * (size_t)(1 + s.cp);
  return w;
}

size_t ds_layout(const Shape& s, const ra_pair* pairs, int32_t n, KParams* kp) {
  size_t off = 0;  // elements
  for (int i = 0; i < n; ++i) {
    const ra_pair& p = pairs[i];
    if (p.mask == RA_MASK_SKIP || p.q_len == 0 || p.kv_len == 0) continue;
    const int64_t rows = (p.kv_len + 127) / 128 * 128, ld = (p.q_len + 127) / 128 * 128;
    if (kp) {
      kp->pairs[i].ds_off = (int64_t)off;
      kp->pairs[i].ds_rows = rows;
      kp->pairs[i].ds_ld = ld;
    }
    off += align256((size_t)(s.B * s.Hq * rows * ld) * 2) / 2;
  }
  return off * 2;
}

size_t ds_step_max(const Shape& s, int32_t rank) {
  size_t mx = 0;
  for (int32_t i = 0; i < s.cp; ++i) {
    int32_t owner, n;
    ra_pair pairs[4];
    plan_step(s, rank, i, &owner, pairs, &n);
    const size_t b = ds_layout(s, pairs, n, nullptr);
    mx = b > mx ? b : mx;
  }
  return mx;
}

BwdWs bwd_ws(const Shape& s) {
  BwdWs w;
  const size_t rows = (size_t)(s.B * s.Hq * s.chunk);
  const size_t kvel = (size_t)(s.B * s.Hkv * s.S * s.D);
  const size_t slot = (size_t)(s.B * s.Hkv * s.chunk * s.D * s.esize) * 2;
  const int nslots = s.cp > 2 ? 2 : (int)s.cp - 1;
  size_t off = 0;
  w.dq = off; off += align256(rows * s.D * 4);
  w.dk = off; off += align256(kvel * 4);
  w.dv = off; off += align256(kvel * 4);
  w.delta = off; off += align256(rows * 4);
  for (int i = 0; i < 2; ++i) {
    w.slot[i] = off;
    if (i < nslots) off += align256(slot);
  }
  // Two dS buffers for the bf16 path: a step's dQ kernel reads its buffer while the next step's
  // dK/dV kernel fills the other.  The largest step over all ranks sizes them, so that the
  // workspace size does not depend on the rank.
  w.ds_bytes = 0;
  if (s.dtype == RA_BF16) {
    for (int32_t r = 0; r < s.cp; ++r) {
      const size_t b = ds_step_max(s, r);
      w.ds_bytes = b > w.ds_bytes ? b : w.ds_bytes;
    }
    if (w.ds_bytes > kDsCap) w.ds_bytes = 0;  // recompute path
  }
  for (int i = 0; i < 2; ++i) {
    w.ds[i] = off;
    off += align256(w.ds_bytes);
  }
  w.total = off;
  return w;
}

void build_ranges(KParams* kp, const ra_pair* pairs, int32_t n, bool by_q, int64_t tile_rows) {
  struct R { int64_t row0, len, weight; int npairs; int pair[4]; bool diag; };
  R rs[4];
  int nr = 0;
  for (int i = 0; i < n; ++i) {
    const ra_pair& p = pairs[i];
    kp->pairs[i] = KPair{p.q_row0, p.kv_row0, p.q_len, p.kv_len, p.mask, 0, p.q_pos0, p.kv_pos0, 0, 0};
    if (p.mask == RA_MASK_SKIP || p.q_len == 0 || p.kv_len == 0) continue;
    const int64_t r0 = by_q ? p.q_row0 : p.kv_row0;
    const int64_t rl = by_q ? p.q_len : p.kv_len;
    int found = -1;
    for (int j = 0; j < nr; ++j)
      if (rs[j].row0 == r0 && rs[j].len == rl) found = j;
    if (found < 0) {
      found = nr++;
      rs[found] = R{r0, rl, 0, 0, {0, 0, 0, 0}, false};
    }
    R& r = rs[found];
    r.pair[r.npairs++] = i;
    r.weight += by_q ? p.kv_len : p.q_len;
    r.diag = r.diag || p.mask == RA_MASK_DIAG;
  }
  // Heaviest range first, so long-running workgroups start early.
  std::stable_sort(rs, rs + nr, [](const R& a, const R& b) { return a.weight > b.weight; });
  int64_t t = 0;
  for (int j = 0; j < nr; ++j) {
    KRange& k = kp->ranges[j];
    k.row0 = rs[j].row0;
    k.len = rs[j].len;
    k.tile0 = t;
    k.ntiles = (rs[j].len + tile_rows - 1) / tile_rows;
    k.npairs = rs[j].npairs;
    for (int q = 0; q < 4; ++q) k.pair[q] = q < rs[j].npairs ? rs[j].pair[q] : 0;
    // Forward: a diagonal pair gives the last Q tiles the most keys.  Backward: it gives the
    // first K/V tiles the most queries, so the natural order is already heaviest first.
    k.reverse = (by_q && rs[j].diag) ? 1 : 0;
    k.pad_ = 0;
    t += k.ntiles;
  }
  kp->nranges = nr;
  kp->tiles_per_head = t;
}

}  // namespace ra

// ---- public host-only entry points ------------------------------------------------------

extern "C" {

const char* ra_version(void) { return "libringattn 0.1 (gfx950)"; }

const char* ra_status_str(int32_t st) {
  switch (st) {
    case RA_OK: return "RA_OK";
    case RA_ERR_INVALID: return "RA_ERR_INVALID";
    case RA_ERR_UNSUPPORTED: return "RA_ERR_UNSUPPORTED";
    case RA_ERR_DEVICE: return "RA_ERR_DEVICE";
    case RA_ERR_WORKSPACE: return "RA_ERR_WORKSPACE";
    default: return "RA_ERR_UNKNOWN";
  }
}

}  // extern "C"

namespace ra { const char* last_error_cstr(); }

extern "C" {

const char* ra_last_error(void) { return ra::last_error_cstr(); }

ra_status ra_validate(const ra_problem* problem, int32_t rank) {
  ra::clear_error();
  ra::Shape s;
  ra_status st = ra::resolve(problem, &s);
  if (st != RA_OK) return st;
  return ra::check_rank(s, rank);
}

ra_status ra_plan_step(const ra_problem* problem, int32_t rank, int32_t step, int32_t* owner,
                       ra_pair pairs[4], int32_t* n_pairs) {
  ra::clear_error();
  ra::Shape s;
  ra_status st = ra::resolve(problem, &s);
  if (st != RA_OK) return st;
  if ((st = ra::check_rank(s, rank)) != RA_OK) return st;
  if (step < 0 || step >= s.cp)
    return ra::fail(RA_ERR_INVALID, "step %d outside [0, %d)", (int)step, (int)s.cp);
  if (!owner || !pairs || !n_pairs) return ra::fail(RA_ERR_INVALID, "NULL output pointer");
  ra::plan_step(s, rank, step, owner, pairs, n_pairs);
  return RA_OK;
}

ra_status ra_workspace_size(const ra_problem* problem, int32_t pass, size_t* bytes) {
  ra::clear_error();
  ra::Shape s;
  ra_status st = ra::resolve(problem, &s);
  if (st != RA_OK) return st;
  if (!bytes) return ra::fail(RA_ERR_INVALID, "bytes is NULL");
  if (pass == 0) *bytes = ra::fwd_ws(s).total;
  else if (pass == 1) *bytes = ra::bwd_ws(s).total;
  else if (pass == 2) *bytes = ra::split_ws(s).total;
  else return ra::fail(RA_ERR_INVALID, "pass must be 0 (forward), 1 (backward) or 2 (split-KV forward)");
  return RA_OK;
}

}  // extern "C"
