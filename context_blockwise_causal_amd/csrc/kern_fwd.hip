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

template <int D>
int launch_fwd(const KParams& kp, void* stream) {
  const int64_t nblk = (int64_t)kp.B * kp.Hq * kp.tiles_per_head;
  if (nblk == 0) return 0;
  hipLaunchKernelGGL(chunk_fwd_bf16_kernel<D>, dim3((unsigned)nblk), dim3(kNT), 0, (hipStream_t)stream, kp);
  return (int)hipGetLastError();
}

}  // namespace

int launch_chunk_fwd_bf16(const KParams& kp, void* stream) {
  return kp.D == 128 ? launch_fwd<128>(kp, stream) : launch_fwd<64>(kp, stream);
}

}  // namespace ra
