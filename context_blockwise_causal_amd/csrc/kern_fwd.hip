// Chunk forward on bf16 MFMA (gfx950): folds K/V blocks into the running online-softmax
// state (U, m, l) of a tile of query rows.
//
// Method: lecture note "上下文并行", section "朴素 Ring Attention": the safe softmax (row
// max subtracted) and the FlashAttention-2-style update of the output block per K/V block,
// which lets a rank fold the ring's chunks one at a time in any order.  Numerics per
// "Feat: Context Parallel" section 数值精度: statistics and accumulation stay fp32, the
// probabilities are rounded to bf16 only as the MFMA operand.
//
// Layout of the work (one workgroup = 4 wavefronts = 128 query rows of one (batch, head)):
//  * Each wavefront owns 32 query rows.  Scores are computed transposed, S^T = K Q^T, on
//    v_mfma_f32_32x32x16_bf16 so that a lane owns one query (column) and holds 16 keys per
//    32-key block in registers: the row max and row sum are in-register reductions plus a
//    single exchange with the other lane half.
//  * The output is accumulated transposed too, O^T += V^T P^T: the probabilities stay in the
//    registers they were computed in (the K rows are fed in perm32 order for that) and the
//    per-query rescale factor is one scalar per lane.
//  * K/V tiles of 64 keys are staged in LDS, double buffered, shared by the 4 wavefronts, and
//    filled by direct global->LDS loads issued one tile ahead (no VGPR staging).  The tiles are
//    unpadded and chunk-swizzled, so K row reads, V^T transposed reads (ds_read_b64_tr_b16)
//    and tile writes are free of bank conflicts.
//  * exp2 with the softmax scale folded into log2(e): p = 2^(s*scale*log2e - m2), one FMA.
//  * Lazy rescaling: the per-row reference m2 only moves when a tile's max exceeds it by more
//    than 2^8, so the O^T rescale (D/2 multiplies per lane) is skipped on almost every tile.
#include "kern_common.h"

namespace ra {
namespace {

constexpr int kNT = 256;  // threads per workgroup
constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per K/V tile
constexpr float kLazyLog2 = 8.0f;  // allowed growth of a row max before U and l are rescaled

template <int D>
struct FwdCfg {
  static constexpr int KK = D / 16;                    // k-steps of S^T over the head dim
  static constexpr int DB = D / 32;                    // 32-row blocks of O^T
  static constexpr int TILE = kBN * D;                 // elements of one K (or V) LDS tile
};

template <int D>
__global__ __launch_bounds__(kNT, 2) void chunk_fwd_bf16_kernel(const KParams p) {
  using C = FwdCfg<D>;
  // Two K/V buffers as four distinct LDS objects: the tile loop is unrolled by two so that every
  // step reads one pair of objects while direct loads fill the other, and the compiler can tell
  // that those loads do not alias the reads (no wait on them before the step's LDS reads).
  __shared__ __attribute__((aligned(16))) u16 k0[C::TILE], v0[C::TILE], k1[C::TILE], v1[C::TILE];

  const TileRef tr = map_tile(p, kBM);
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int qi = 32 * w + lq;  // this lane's query row within the tile
  const bool qvalid = qi < tr.nrows;
  const int64_t qrow = (((int64_t)tr.b * p.Hq + tr.hq) * p.q_head_rows) + tr.row0 + qi;
  const int64_t kvhead = ((int64_t)tr.b * p.Hkv + tr.g) * p.kv_head_rows;
  const u16* __restrict__ Q = reinterpret_cast<const u16*>(p.q);
  const u16* __restrict__ Kg = reinterpret_cast<const u16*>(p.k);
  const u16* __restrict__ Vg = reinterpret_cast<const u16*>(p.v);

  // B operand of S^T = K Q^T: lane holds Q[query][kk*16 + 8*hh .. +8].
  bf16x8 qreg[C::KK];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk) {
    if (qvalid)
      qreg[kk] = *reinterpret_cast<const bf16x8*>(Q + qrow * D + kk * 16 + 8 * hh);
    else
      qreg[kk] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }

  // Running state of this lane's query, O^T accumulator layout: oacc[db][4j+i] holds
  // U[query][32*db + 8*j + 4*hh + i].
  f32x16 oacc[C::DB];
  float m2 = -__builtin_inff(), lsum = 0.f;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
  if (qvalid && !p.fresh) {
    m2 = p.m[qrow] * kLog2e;
    lsum = p.l[qrow];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 u = *reinterpret_cast<const f32x4*>(p.U + qrow * D + 32 * db + 8 * j + 4 * hh);
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[db][4 * j + i] = u[i];
      }
  }

  // K row fed to A-operand row lq of each 32-key block (perm32), and the operand addresses.
  const RowAddr ka0 = make_row_addr(perm32(lq), hh, D);
  const RowAddr ka1 = make_row_addr(32 + perm32(lq), hh, D);
  const TrAddr va = make_tr_addr(lane, D);
  const KRange& R = p.ranges[tr.range];
  for (int pi = 0; pi < R.npairs; ++pi) {
    const KPair pr = p.pairs[R.pair[pi]];
    const bool diag = pr.mask == RA_MASK_DIAG;
    const int64_t qloc0 = tr.row0 - pr.q_row0;  // pair-local index of the tile's first query
    const int64_t iq = qloc0 + qi;              // pair-local index of this lane's query
    int64_t key_end = pr.kv_len;
    if (diag && qloc0 + tr.nrows < key_end) key_end = qloc0 + tr.nrows;
    const int nkt = (int)((key_end + kBN - 1) / kBN);
    const u16* Kp = Kg + (kvhead + pr.kv_row0) * D;
    const u16* Vp = Vg + (kvhead + pr.kv_row0) * D;
    const int64_t wq_first = qloc0 + 32 * w;  // pair-local index of the wavefront's first query
    const bool wave_has_rows = 32 * w < tr.nrows;
    // Window / attention-chunk restriction: pair-local index of the lowest key this lane's
    // query sees (non-decreasing in the query), and its range over the wavefront and the tile.
    const bool has_lo = p.window > 0 || p.attn_chunk > 0;
    int64_t lo = 0, wave_lo = 0, wave_lo_max = 0, kt0 = 0;
    if (has_lo) {
      lo = lowest_key(pr.q_pos0 + iq, p.window, p.attn_chunk) - pr.kv_pos0;
      wave_lo = lowest_key(pr.q_pos0 + wq_first, p.window, p.attn_chunk) - pr.kv_pos0;
      wave_lo_max = lowest_key(pr.q_pos0 + wq_first + 31, p.window, p.attn_chunk) - pr.kv_pos0;
      const int64_t tile_lo = lowest_key(pr.q_pos0 + qloc0, p.window, p.attn_chunk) - pr.kv_pos0;
      kt0 = tile_lo > 0 ? tile_lo / kBN : 0;  // key tiles below every query's lowest key are skipped
    }

    // One key tile: issue the next tile's loads into (nk, nv), then compute on (kb, vb).
    auto step = [&](const u16* kb, const u16* vb, u16* nk, u16* nv, int kt) {
      const int64_t kbase = (int64_t)kt * kBN;
      if (kt + 1 < nkt) {
        issue_tile<D, kBN, 4>(Kp + (kbase + kBN) * D, pr.kv_len - kbase - kBN, nk);
        issue_tile<D, kBN, 4>(Vp + (kbase + kBN) * D, pr.kv_len - kbase - kBN, nv);
      }
      // Skip the math when the whole tile lies in the future of every query of this wave, or
      // below every query's lowest visible key.
      const bool active = wave_has_rows && !(diag && kbase > wq_first + 31) &&
                          !(has_lo && kbase + kBN - 1 < wave_lo);
      if (active) {
        // The two 32-key blocks' accumulation chains are interleaved, so that each MFMA's
        // operand read has the other chain's MFMA to hide behind.
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
          for (int b = 0; b < 2; ++b) s[b] = mfma32(row_operand(kb, b ? ka1 : ka0, kk), qreg[kk], s[b]);
        // Keys past the pair, or after this lane's query in a diagonal pair, are excluded; kmax
        // is the last visible key of the tile (only edge tiles take the masked path).
        const bool edge = (kbase + kBN > pr.kv_len) || (diag && kbase + kBN - 1 > wq_first) ||
                          (has_lo && kbase < wave_lo_max);
        if (edge) {
          const int64_t lim = diag ? (iq < pr.kv_len - 1 ? iq : pr.kv_len - 1) : pr.kv_len - 1;
          const int kmax = (int)(lim - kbase < -1 ? -1 : (lim - kbase > kBN - 1 ? kBN - 1 : lim - kbase));
          const int kmin = has_lo ? (int)(lo - kbase < 0 ? 0 : (lo - kbase > kBN ? kBN : lo - kbase)) : 0;
          // key of register r in block b is 32 b + perm_reg_row(r, 0) + 8 hh: compare the
          // compile-time part against kmax - 8 hh and kmin - 8 hh
          const int kmh = kmax - 8 * hh, kml = kmin - 8 * hh;
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = b * 32 + perm_reg_row(r, 0);
              if (key > kmh || key < kml) s[b][r] = -__builtin_inff();
            }
        }
        float mx = -__builtin_inff();
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
        mx = xor32_max(mx) * p.scale_log2;
        // Lazy rescale: the reference m2 moves only when a row's tile max exceeds it by more
        // than kLazyLog2, so exp2(score - m2) <= 2^kLazyLog2 and U, l stay consistent with m2.
        const bool grow = mx > m2 + kLazyLog2;
        if (__ballot(grow)) {
          const float mnew = grow ? mx : m2;
          const float alpha = mnew == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m2 - mnew);
          lsum *= alpha;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
          m2 = mnew;
        }
        const float nbase = m2 == -__builtin_inff() ? 0.f : -m2;
        float rs = 0.f;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(fmaf(s[b][r], p.scale_log2, nbase));
            s[b][r] = e;
            rs += e;
          }
        rs = xor32_sum(rs);
        lsum += rs;

        // B operand P^T for key step c (16 keys): registers 8*(c&1) .. +8 of block c>>1.
        bf16x8 pb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          bf16x8 t;
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = (__bf16)s[c >> 1][8 * (c & 1) + e];
          pb[c] = t;
        }
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            // A operand V^T: lane holds V[16c + 8hh + e][32db + lq], e = 0..7 (transposed read).
            oacc[db] = mfma32(tr_operand(vb, va, D, c, db), pb[c], oacc[db]);
      }
      wait_vmem();
      __syncthreads();
    };

    if (kt0 >= nkt) continue;  // uniform over the workgroup
    issue_tile<D, kBN, 4>(Kp + kt0 * kBN * D, pr.kv_len - kt0 * kBN, k0);
    issue_tile<D, kBN, 4>(Vp + kt0 * kBN * D, pr.kv_len - kt0 * kBN, v0);
    wait_vmem();
    __syncthreads();
    for (int kt = (int)kt0; kt < nkt; kt += 2) {
      step(k0, v0, k1, v1, kt);
      if (kt + 1 < nkt) step(k1, v1, k0, v0, kt + 1);
    }
  }

  if (qvalid) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = oacc[db][4 * j + i];
        *reinterpret_cast<f32x4*>(p.U + qrow * D + 32 * db + 8 * j + 4 * hh) = u;
      }
    if (hh == 0) {
      p.m[qrow] = m2 * kLn2;
      p.l[qrow] = lsum;
    }
  }
}

// ======================================================================= forward, ping-pong
//
// The same computation with two teams of 4 wavefronts per workgroup (8 wavefronts, two per SIMD,
// one of each team), each team owning 128 query rows; both teams walk the same K/V tiles.  A
// wavefront's tile is split into a matrix phase (O^T += V^T P^T of the previous tile, then S^T of
// this tile) and a vector phase (mask, row max, lazy rescale, exp2, row sum, P^T as bf16).  The
// teams run these phases half a tile apart between workgroup barriers, so that on every SIMD one
// wavefront issues MFMAs while the other does its softmax.  K/V tiles rotate through four LDS
// buffers, loaded by the first team two tiles ahead with buffer loads to LDS (which, unlike the
// global form, leave the compiler's waits for LDS reads exact).
//
// The loop is bound by instruction issue more than by any one unit, so its reads carry no address
// arithmetic: the tile loop is unrolled over the four buffers, the four K tiles lie in the first
// 64 KB of LDS and the four V tiles after them, and each operand read is a register formed once
// per lane plus a compile-time offset (the buffer, the key step) in the instruction.

template <int N>
struct Step {
  static constexpr int value = N;
};

constexpr int kPPRows = 256;  // query rows per workgroup (two teams of 128)
constexpr int kPPNT = 512;    // threads per workgroup

template <int D>
__global__ __launch_bounds__(kPPNT, 2) void chunk_fwd_pp_kernel(const KParams p) {
  using C = FwdCfg<D>;
  // K tile b at lds + b TILE, V tile b at lds + (4 + b) TILE
  __shared__ __attribute__((aligned(16))) u16 lds[8 * C::TILE];

  const TileRef tr = map_tile(p, kPPRows);
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int team = w >> 2;
  const int qi = 32 * w + lq;  // this lane's query row within the tile
  const bool qvalid = qi < tr.nrows;
  const int64_t qrow = (((int64_t)tr.b * p.Hq + tr.hq) * p.q_head_rows) + tr.row0 + qi;
  const int64_t kvhead = ((int64_t)tr.b * p.Hkv + tr.g) * p.kv_head_rows;
  const u16* __restrict__ Q = reinterpret_cast<const u16*>(p.q);
  const u16* __restrict__ Kg = reinterpret_cast<const u16*>(p.k);
  const u16* __restrict__ Vg = reinterpret_cast<const u16*>(p.v);

  bf16x8 qreg[C::KK];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk) {
    if (qvalid)
      qreg[kk] = *reinterpret_cast<const bf16x8*>(Q + qrow * D + kk * 16 + 8 * hh);
    else
      qreg[kk] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }
  f32x16 oacc[C::DB];
  float m2 = -__builtin_inff(), lsum = 0.f;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
  if (qvalid && !p.fresh) {
    m2 = p.m[qrow] * kLog2e;
    lsum = p.l[qrow];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 u = *reinterpret_cast<const f32x4*>(p.U + qrow * D + 32 * db + 8 * j + 4 * hh);
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[db][4 * j + i] = u[i];
      }
  }

  // Per-lane byte offsets of the operand reads, formed once: the K row operand of 16-deep step kk
  // within a K tile (the row 32 further, with the same swizzle, is 64 D bytes on) and the two
  // halves of the transposed V operand of d block db (key step c adds 32 c D bytes), the latter
  // measured from the K tile of the same buffer index, 8 TILE bytes before its V tile, so that
  // the buffer's offset stays within the reach of the instruction's immediate.
  int kb[C::KK], vb[C::DB][2];
  {
    const RowAddr ka = make_row_addr(perm32(lq), hh, D);
    const TrAddr va = make_tr_addr(lane, D);
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      kb[kk] = (ka.base + ((16 * kk) ^ ka.g8)) * 2;
      asm volatile("" : "+v"(kb[kk]));
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      vb[db][0] = (va.lo ^ (db << 5)) * 2 + 8 * C::TILE;
      vb[db][1] = (va.hi ^ (db << 5)) * 2 + 8 * C::TILE;
      asm volatile("" : "+v"(vb[db][0]), "+v"(vb[db][1]));
    }
  }
  const KRange& R = p.ranges[tr.range];
  for (int pi = 0; pi < R.npairs; ++pi) {
    const KPair pr = p.pairs[R.pair[pi]];
    const bool diag = pr.mask == RA_MASK_DIAG;
    const int64_t qloc0 = tr.row0 - pr.q_row0;
    const int64_t iq = qloc0 + qi;
    int64_t key_end = pr.kv_len;
    if (diag && qloc0 + tr.nrows < key_end) key_end = qloc0 + tr.nrows;
    const int nkt = (int)((key_end + kBN - 1) / kBN);
    const u16* Kp = Kg + (kvhead + pr.kv_row0) * D;
    const u16* Vp = Vg + (kvhead + pr.kv_row0) * D;
    const int64_t wq_first = qloc0 + 32 * w;
    const bool has_lo = p.window > 0 || p.attn_chunk > 0;
    int64_t lo = 0, wave_lo = 0, wave_lo_max = 0, kt0 = 0;
    if (has_lo) {
      lo = lowest_key(pr.q_pos0 + iq, p.window, p.attn_chunk) - pr.kv_pos0;
      wave_lo = lowest_key(pr.q_pos0 + wq_first, p.window, p.attn_chunk) - pr.kv_pos0;
      wave_lo_max = lowest_key(pr.q_pos0 + wq_first + 31, p.window, p.attn_chunk) - pr.kv_pos0;
      const int64_t tile_lo = lowest_key(pr.q_pos0 + qloc0, p.window, p.attn_chunk) - pr.kv_pos0;
      kt0 = tile_lo > 0 ? tile_lo / kBN : 0;
    }
    if (kt0 >= nkt) continue;  // uniform over the workgroup
    const int niter = nkt - (int)kt0;
    // Tiles that take the mask, as bounds on the tile index t (kept in scalar registers): t >= t_hi
    // when the tile runs past the pair's end or, on a diagonal pair, past this wavefront's first
    // query; t < t_lo when it starts below the lowest visible key of the wavefront's last query.
    int64_t kt_hi = pr.kv_len / kBN;
    if (diag && (wq_first + 1) / kBN < kt_hi) kt_hi = (wq_first + 1) / kBN;
    const int64_t kt_lo = has_lo && wave_lo_max > 0 ? (wave_lo_max + kBN - 1) / kBN : 0;
    const int t_hi = (int)(kt_hi - kt0 < niter ? kt_hi - kt0 : niter);
    const int t_lo = (int)(kt_lo - kt0 > 0 ? kt_lo - kt0 : 0);

    // The first team loads key tile kt (K then V, rows past the pair repeat its last row): 16
    // one-KB instructions per tile, 8 per wavefront.
    auto load = [&](int64_t kt, u16* __restrict__ Bk, u16* __restrict__ Bv) {
      const int64_t k0 = kt * kBN;
      const int last = (int)(pr.kv_len - k0 < kBN ? pr.kv_len - k0 : kBN) - 1;
      const auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)(Kp + k0 * D), 0, kBN * D * 2, kBufRsrcWord3);
      const auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)(Vp + k0 * D), 0, kBN * D * 2, kBufRsrcWord3);
      constexpr int CH = D / 8, RPI = 64 / CH;
#pragma unroll
      for (int k = 0; k < kBN / RPI / 4; ++k) {
        const int i = k * 4 + w, row = i * RPI + lane / CH;
        const int c = (lane % CH) ^ swz(row, D);
        const unsigned off = (unsigned)((row < last ? row : last) * D + c * 8) * 2u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lvoid_t*)(Bk + i * 512), 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lvoid_t*)(Bv + i * 512), 16, off, 0, 0, 0);
      }
    };

    // Carried between phases: the scores S^T of the tile after a matrix phase; P^T (bf16, packed
    // into s[0]) after a vector phase.
    f32x16 s[2] = {f32x16{}, f32x16{}};
    // One phase for tile t (0-based within the pair's tiles from kt0): the matrix phase (mph: the
    // P V contraction of tile t - 1 if pv, the scores of tile t if sc) or the vector phase.  Kc is
    // the K tile of tile t, Vo the V tile of tile t - 1; Kn, Vn receive tile t + 2 (first team,
    // matrix phase).
    auto phase = [&](bool mph, bool pv, bool sc, int t, u16* __restrict__ Kn, u16* __restrict__ Vn,
                     const u16* __restrict__ Vo, const u16* __restrict__ Kc) {
      const int64_t kbase = (kt0 + t) * kBN;
      if (mph) {
        __builtin_amdgcn_s_setprio(1);  // the matrix phase's MFMAs go ahead of the other wavefront's vector work
        if (team == 0 && t + 2 < niter) load(kt0 + t + 2, Kn, Vn);
        if (pv) {
          // O^T += V^T P^T of tile t - 1: P^T for key step c is registers 8 (c & 1) .. of block c >> 1,
          // packed as bf16 into s[0]
          bf16x8 pb[4];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            pb[c] = __builtin_bit_cast(
                bf16x8, c == 0 ? __builtin_shufflevector(s[0], s[0], 0, 1, 2, 3)
                               : c == 1 ? __builtin_shufflevector(s[0], s[0], 4, 5, 6, 7)
                                        : c == 2 ? __builtin_shufflevector(s[0], s[0], 8, 9, 10, 11)
                                                 : __builtin_shufflevector(s[0], s[0], 12, 13, 14, 15));
          __builtin_amdgcn_sched_barrier(0);
          // the 16 MFMAs in the order (c, db) (consecutive ones into different accumulators), the A
          // operand V^T(c, db) read kWin - 1 MFMAs ahead
          constexpr int kWin = 8;
          bf16x8 A[kWin];
          auto load_op = [&](int i) {
            const int c = i / C::DB, db = i % C::DB;
            const char* const t0 = reinterpret_cast<const char*>(Vo) - 8 * C::TILE + 32 * c * D;
            const v4i16 lo = ds_read_tr16(reinterpret_cast<const u16*>(t0 + vb[db][0]));
            const v4i16 hi = ds_read_tr16(reinterpret_cast<const u16*>(t0 + vb[db][1]));
            A[i % kWin] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          };
#pragma unroll
          for (int i = 0; i < kWin - 1; ++i) load_op(i);
#pragma unroll
          for (int i = 0; i < 4 * C::DB; ++i) {
            if (i + kWin - 1 < 4 * C::DB) load_op(i + kWin - 1);
            __builtin_amdgcn_sched_barrier(0);
            oacc[i % C::DB] = mfma32(A[i % kWin], pb[i / C::DB], oacc[i % C::DB]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (sc) {
          // S^T = K Q^T of tile t for its two 32-key blocks; K rows read two kk ahead
          bf16x8 k0o[3], k1o[3];
          auto load_k = [&](int kk) {
            const char* const a = reinterpret_cast<const char*>(Kc) + kb[kk];
            k0o[kk % 3] = *reinterpret_cast<const bf16x8*>(a);
            k1o[kk % 3] = *reinterpret_cast<const bf16x8*>(a + 64 * D);
          };
          load_k(0);
          load_k(1);
          s[0] = f32x16{};
          s[1] = f32x16{};
#pragma unroll
          for (int kk = 0; kk < C::KK; ++kk) {
            if (kk + 2 < C::KK) load_k(kk + 2);
            __builtin_amdgcn_sched_barrier(0);
            s[0] = mfma32(k0o[kk % 3], qreg[kk], s[0]);
            s[1] = mfma32(k1o[kk % 3], qreg[kk], s[1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
      } else {
        // the first team's loads of tile t + 1 (issued two phases ago) are in LDS before the
        // barrier that ends this phase; its only memory operations in flight are its direct loads,
        // which complete in order (8 instructions per tile)
        if (team == 0) {
          if (t + 2 < niter)
            __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
          else
            wait_vmem();
        }
        // keys past the pair, after this lane's query (diagonal pair) or below its lowest visible
        // key get -inf (edge tiles only)
        if (t >= t_hi || t < t_lo) {
          const int64_t lim = diag ? (iq < pr.kv_len - 1 ? iq : pr.kv_len - 1) : pr.kv_len - 1;
          const int kmax = (int)(lim - kbase < -1 ? -1 : (lim - kbase > kBN - 1 ? kBN - 1 : lim - kbase));
          const int kmin = has_lo ? (int)(lo - kbase < 0 ? 0 : (lo - kbase > kBN ? kBN : lo - kbase)) : 0;
          const int kmh = kmax - 8 * hh, kml = kmin - 8 * hh;
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = b * 32 + perm_reg_row(r, 0);
              if (key > kmh || key < kml) s[b][r] = -__builtin_inff();
            }
        }
        float mx = -__builtin_inff();
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
        mx = xor32_max(mx) * p.scale_log2;
        const bool grow = mx > m2 + kLazyLog2;
        if (__ballot(grow)) {
          const float mnew = grow ? mx : m2;
          const float alpha = mnew == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m2 - mnew);
          lsum *= alpha;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
          m2 = mnew;
        }
        const float nbase = m2 == -__builtin_inff() ? 0.f : -m2;
        float rs = 0.f;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(fmaf(s[b][r], p.scale_log2, nbase));
            s[b][r] = e;
            rs += e;
          }
        rs = xor32_sum(rs);
        lsum += rs;
        bf16x8 pb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[c][e] = (__bf16)s[c >> 1][8 * (c & 1) + e];
        }
        const f32x4 w0 = __builtin_bit_cast(f32x4, pb[0]), w1 = __builtin_bit_cast(f32x4, pb[1]);
        const f32x4 w2 = __builtin_bit_cast(f32x4, pb[2]), w3 = __builtin_bit_cast(f32x4, pb[3]);
        s[0] = f32x16{w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3],
                      w2[0], w2[1], w2[2], w2[3], w3[0], w3[1], w3[2], w3[3]};
      }
    };
    // A phase of tile t, whose buffer index t & 3 is the compile-time P.
    auto run = [&](auto P, bool mph, bool pv, bool sc, int t) {
      constexpr int b = decltype(P)::value;
      phase(mph, pv, sc, t, lds + ((b + 2) & 3) * C::TILE, lds + (4 + ((b + 2) & 3)) * C::TILE,
            lds + (4 + ((b + 3) & 3)) * C::TILE, lds + b * C::TILE);
      phase_barrier();
    };

    if (team == 0) {
      load(kt0, lds, lds + 4 * C::TILE);
      if (niter > 1) load(kt0 + 1, lds + C::TILE, lds + 5 * C::TILE);
    }
    wait_vmem();
    __syncthreads();
    // Each loop step is the vector phase of tile t and the matrix phase of tile t + 1 (the first M
    // has no P V, the last no scores).  The second team runs one phase behind the first.
    // (the vector phase reads no tile: its buffer index is immaterial)
    auto step = [&](auto P, int t) {  // P: the buffer of tile t + 1
      if (t >= 0) run(P, false, false, false, t);
      else phase_barrier();
      run(P, true, t >= 0, t + 1 < niter, t + 1);
    };
    if (team == 1) phase_barrier();
    for (int t = -1; t < niter; t += 4) {
      step(Step<0>{}, t);
      if (t + 1 >= niter) break;
      step(Step<1>{}, t + 1);
      if (t + 2 >= niter) break;
      step(Step<2>{}, t + 2);
      if (t + 3 >= niter) break;
      step(Step<3>{}, t + 3);
    }
    if (team == 0) phase_barrier();
  }

  if (qvalid) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = oacc[db][4 * j + i];
        *reinterpret_cast<f32x4*>(p.U + qrow * D + 32 * db + 8 * j + 4 * hh) = u;
      }
    if (hh == 0) {
      p.m[qrow] = m2 * kLn2;
      p.l[qrow] = lsum;
    }
  }
}

template <int D>
int launch_fwd(const KParams& kp, void* stream) {
  const int64_t nblk = (int64_t)kp.B * kp.Hq * kp.tiles_per_head;
  if (nblk == 0) return 0;
  if (D == 128)
    hipLaunchKernelGGL(chunk_fwd_pp_kernel<D>, dim3((unsigned)nblk), dim3(kPPNT), 0, (hipStream_t)stream, kp);
  else
    hipLaunchKernelGGL(chunk_fwd_bf16_kernel<D>, dim3((unsigned)nblk), dim3(kNT), 0, (hipStream_t)stream, kp);
  return (int)hipGetLastError();
}

}  // namespace

int launch_chunk_fwd_bf16(const KParams& kp, void* stream) {
  return kp.D == 128 ? launch_fwd<128>(kp, stream) : launch_fwd<64>(kp, stream);
}

}  // namespace ra
