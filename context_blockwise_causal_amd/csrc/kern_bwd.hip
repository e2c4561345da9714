// Chunk backward on bf16 MFMA (gfx950) with probability recompute.
//
// Method: InfiniTrain pull request "Feat: Context Parallel", section 主要改动, p2p mode: the
// backward recomputes the probabilities from the saved log-sum-exp and returns the K/V
// gradients to the chunk's owner.  Per query row t and key j (scale = softmax scale):
//   P = exp(scale q.k - lse),  dP = dO.v,  dS = P (dP - delta),  delta = <dO, O>,
//   dV += P^T dO,  dK += scale dS^T Q,  dQ += scale dS K.
//
// Layout of the work (one workgroup = 4 wavefronts = 128 keys of one (batch, query head)):
//  * Each wavefront owns 32 keys and keeps their K and V rows in registers as MFMA operands,
//    plus its dK^T and dV^T accumulators (fp32, 32 keys x head_dim each).
//  * The workgroup walks the query rows of every pair that reads its keys, 64 rows at a time;
//    the Q / dO tiles, lse and delta are staged in LDS (double buffered, prefetched one tile
//    ahead with 16-byte loads).
//  * S = Q K^T and dP = dO V^T come out with the key index across lanes and the query index in
//    registers (queries fed in perm32 order), which is exactly the B-operand layout that
//    dV^T += dO^T P and dK^T += Q^T dS need; no register shuffles.
//  * Operands that the contraction needs transposed (Q^T, dO^T, dS, K for dQ) are read with
//    ds_read_b64_tr_b16 out of row-major LDS tiles: two reads per 8-element operand.  All LDS
//    tiles are unpadded and chunk-swizzled (conflict-free row reads, transposed reads, writes).
//  * dS is scaled by the softmax scale once, so dK and dQ need no further multiplies.
//  * dS goes to LDS once, as dS^T (bf16, 16-byte row writes), so that dQ = dS K (contraction
//    over the workgroup's 128 keys) can be formed by all wavefronts, each for a 32-column slice
//    of the head dim, and added to the fp32 dQ accumulator with coalesced 128-byte atomics.
//  * dK / dV of one key/value head receive the contributions of all heads_q / heads_kv query
//    heads through fp32 atomics at the end of each workgroup (the GQA group sum in-kernel).
#include "kern_common.h"

namespace ra {
namespace {

constexpr int kNT = 256;
constexpr int kBN = 128;  // keys per workgroup
constexpr int kBQ = 64;   // query rows per iteration

template <int D>
struct BwdCfg {
  static constexpr int KK = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int VROW = D / 8;
  static constexpr int LOADS = kBQ * VROW / kNT;   // 16-byte chunks per thread per tile, per tensor
  static constexpr int QT = kBQ * D;               // elements of one Q (or dO) tile
  // [Q buf0 | Q buf1 | dO buf0 | dO buf1 | dS^T (kBN x kBQ)] u16, then [lse2 x2 | delta x2] fp32
  static constexpr int OFF_DO = 2 * QT;
  static constexpr int OFF_DS = 4 * QT;
  static constexpr int U16_ELEMS = 4 * QT + kBN * kBQ;
  static constexpr size_t LDS_BYTES = U16_ELEMS * sizeof(u16) + 4 * kBQ * sizeof(float);
  static_assert(2 * QT >= kBN * D, "the K tile used to build the dQ operand must fit in the Q buffers");
};

template <int D>
__device__ __forceinline__ void load_qdo(const u16* __restrict__ Qp, const u16* __restrict__ dOp,
                                         const float* __restrict__ lse, const float* __restrict__ dlt,
                                         int64_t q0, int64_t q_len, bool full, u32x4* qr, u32x4* dr,
                                         float* extra) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int u = threadIdx.x + kNT * i;
    const int row = u / C::VROW, col = (u % C::VROW) * 8;
    const int64_t q = q0 + row;
    if (full || q < q_len) {
      qr[i] = *reinterpret_cast<const u32x4*>(Qp + q * D + col);
      dr[i] = *reinterpret_cast<const u32x4*>(dOp + q * D + col);
    } else {
      qr[i] = u32x4{0u, 0u, 0u, 0u};
      dr[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  // threads 0..63 fetch lse (pre-scaled to base 2; +inf for rows outside the pair so that
  // their probabilities are 0), threads 64..127 fetch delta.
  const int t = threadIdx.x;
  if (t < 2 * kBQ) {
    const int row = t & (kBQ - 1);
    const int64_t q = q0 + row;
    if (t < kBQ) *extra = q < q_len ? lse[q] * kLog2e : __builtin_inff();
    else *extra = q < q_len ? dlt[q] : 0.f;
  }
}

template <int D>
__device__ __forceinline__ void store_qdo(u16* __restrict__ lds, float* __restrict__ ldsf, int buf,
                                          const u32x4* qr, const u32x4* dr, float extra) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int u = threadIdx.x + kNT * i;
    const int row = u / C::VROW, col = (u % C::VROW) * 8;
    const int off = swz_off(row, col, D);
    *reinterpret_cast<u32x4*>(lds + buf * C::QT + off) = qr[i];
    *reinterpret_cast<u32x4*>(lds + C::OFF_DO + buf * C::QT + off) = dr[i];
  }
  const int t = threadIdx.x;
  if (t < 2 * kBQ) {
    const int row = t & (kBQ - 1);
    ldsf[(t < kBQ ? 0 : 2 * kBQ) + buf * kBQ + row] = extra;
  }
}

template <int D>
__global__ __launch_bounds__(kNT, 1) void chunk_bwd_bf16_kernel(const KParams p) {
  using C = BwdCfg<D>;
  extern __shared__ __attribute__((aligned(16))) u16 lds[];
  float* ldsf = reinterpret_cast<float*>(lds + C::U16_ELEMS);  // [lse2 buf0|buf1][delta buf0|buf1]

  const TileRef tr = map_tile(p, kBN);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int kl = 32 * w + lq;  // this lane's key within the tile
  const bool kvalid = kl < tr.nrows;
  const int64_t kvhead = ((int64_t)tr.b * p.Hkv + tr.g) * p.kv_head_rows;
  const int64_t qhead = ((int64_t)tr.b * p.Hq + tr.hq) * p.q_head_rows;
  const int64_t dkvhead = ((int64_t)tr.b * p.Hkv + tr.g) * p.dkv_head_rows;
  const u16* __restrict__ Kg = reinterpret_cast<const u16*>(p.k) + kvhead * D;
  const u16* __restrict__ Vg = reinterpret_cast<const u16*>(p.v) + kvhead * D;

  // B operands of S = Q K^T and dP = dO V^T: lane holds K/V[key][kk*16 + 8*hh .. +8].
  bf16x8 kreg[C::KK], vreg[C::KK];
  {
    const int64_t krow = tr.row0 + kl;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      if (kvalid) {
        kreg[kk] = *reinterpret_cast<const bf16x8*>(Kg + krow * D + kk * 16 + 8 * hh);
        vreg[kk] = *reinterpret_cast<const bf16x8*>(Vg + krow * D + kk * 16 + 8 * hh);
      } else {
        kreg[kk] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        vreg[kk] = kreg[kk];
      }
    }
  }

  // dQ task of this wavefront: head-dim block `dblk` for query blocks [qb_lo, qb_hi).
  constexpr int NDB = D / 32;
  const int dblk = w % NDB;
  const int qb_lo = NDB >= 4 ? 0 : w / NDB;
  const int qb_hi = NDB >= 4 ? 2 : qb_lo + 1;
  // B operand of dQ = dS K: lane holds K[16c + 8hh + e][32*dblk + lq] for c = 0..7, read once
  // (transposed) from the workgroup's K tile staged in the Q buffers.
  bf16x8 ktreg[kBN / 16];
  {
    constexpr int KV = kBN * (D / 8);
#pragma unroll
    for (int i = 0; i < KV / kNT; ++i) {
      const int u = tid + kNT * i;
      const int row = u / (D / 8), col = (u % (D / 8)) * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (row < tr.nrows) v = *reinterpret_cast<const u32x4*>(Kg + (tr.row0 + row) * D + col);
      *reinterpret_cast<u32x4*>(lds + swz_off(row, col, D)) = v;
    }
    __syncthreads();
    const TrAddr ka = make_tr_addr(lane, D);
#pragma unroll
    for (int c = 0; c < kBN / 16; ++c) ktreg[c] = tr_operand(lds, ka, D, c, dblk);
    __syncthreads();
  }

  f32x16 dk_acc[C::DB], dv_acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }

  // Query row fed to A-operand row lq of each 32-query block (perm32), and operand addresses.
  const RowAddr qa0 = make_row_addr(perm32(lq), hh, D);
  const RowAddr qa1 = make_row_addr(32 + perm32(lq), hh, D);
  const TrAddr ta = make_tr_addr(lane, D);       // Q^T, dO^T out of the [query][d] tiles
  const TrAddr sa = make_tr_addr(lane, kBQ);     // dS out of the dS^T [key][query] tile
  const KRange& R = p.ranges[tr.range];
  for (int pi = 0; pi < R.npairs; ++pi) {
    const KPair pr = p.pairs[R.pair[pi]];
    const bool diag = pr.mask == RA_MASK_DIAG;
    const int64_t kloc0 = tr.row0 - pr.kv_row0;  // pair-local index of the tile's first key
    const int64_t kj = kloc0 + kl;              // pair-local index of this lane's key
    const int64_t q_begin = diag ? (kloc0 / kBQ) * kBQ : 0;
    const int niter = (int)((pr.q_len - q_begin + kBQ - 1) / kBQ);
    if (niter <= 0) continue;
    const u16* Qp = reinterpret_cast<const u16*>(p.q) + (qhead + pr.q_row0) * D;
    const u16* dOp = reinterpret_cast<const u16*>(p.dO) + (qhead + pr.q_row0) * D;
    const float* lsep = p.lse + qhead + pr.q_row0;
    const float* dltp = p.delta + qhead + pr.q_row0;
    float* dqp = p.U + (qhead + pr.q_row0) * D;

    u32x4 qr[C::LOADS], dr[C::LOADS];
    float extra = 0.f;
    load_qdo<D>(Qp, dOp, lsep, dltp, q_begin, pr.q_len, q_begin + kBQ <= pr.q_len, qr, dr, &extra);
    store_qdo<D>(lds, ldsf, 0, qr, dr, extra);
    __syncthreads();

    for (int it = 0; it < niter; ++it) {
      const int buf = it & 1;
      const int64_t qbase = q_begin + (int64_t)it * kBQ;
      if (it + 1 < niter)
        load_qdo<D>(Qp, dOp, lsep, dltp, qbase + kBQ, pr.q_len, qbase + 2 * kBQ <= pr.q_len, qr, dr,
                    &extra);
      const u16* Qs = lds + buf * C::QT;
      const u16* dOs = lds + C::OFF_DO + buf * C::QT;
      const float* lse2s = ldsf + buf * kBQ;
      const float* dlts = ldsf + 2 * kBQ + buf * kBQ;
      u16* dSt = lds + C::OFF_DS;  // dS^T [key][query], swizzled rows of kBQ

      // Whole wavefront in the future of every query of this tile (diagonal pairs only).
      const bool active = !(diag && kloc0 + 32 * w > qbase + kBQ - 1);
      if (active) {
        f32x16 s[2], dp[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          s[qb] = f32x16{};
          dp[qb] = f32x16{};
#pragma unroll
          for (int kk = 0; kk < C::KK; ++kk) {
            s[qb] = mfma32(row_operand(Qs, qb ? qa1 : qa0, kk), kreg[kk], s[qb]);
            dp[qb] = mfma32(row_operand(dOs, qb ? qa1 : qa0, kk), vreg[kk], dp[qb]);
          }
        }
        const bool edge = !kvalid || (diag && kloc0 + 32 * w + 31 > qbase);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // registers 4j..4j+3 hold queries qb*32 + perm_reg_row(4j+i, hh): 4 consecutive rows
            const int r0 = qb * 32 + perm_reg_row(4 * j, hh);
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + r0);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(dlts + r0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 4 * j + i;
              float pv = __builtin_amdgcn_exp2f(fmaf(s[qb][r], p.scale_log2, -l4[i]));
              if (edge) {
                const int64_t qj = qbase + r0 + i;
                if (!kvalid || (diag && kj > qj)) pv = 0.f;
              }
              s[qb][r] = pv;
              dp[qb][r] = (pv * p.scale) * (dp[qb][r] - d4[i]);  // scale * dS
            }
          }
        bf16x8 pb[4], dsb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          bf16x8 a, b;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            a[e] = (__bf16)s[c >> 1][8 * (c & 1) + e];
            b[e] = (__bf16)dp[c >> 1][8 * (c & 1) + e];
          }
          pb[c] = a;
          dsb[c] = b;
        }
        // dV^T += dO^T P and dK^T += Q^T dS; A operands read transposed out of the Q / dO tiles.
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            dv_acc[db] = mfma32(tr_operand(dOs, ta, D, c, db), pb[c], dv_acc[db]);
            dk_acc[db] = mfma32(tr_operand(Qs, ta, D, c, db), dsb[c], dk_acc[db]);
          }
        // dS^T to LDS: register block c holds queries 16c + 8hh + 0..7 of this lane's key, one
        // 16-byte chunk of dS^T[key][query].
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *reinterpret_cast<bf16x8*>(dSt + swz_off(kl, 16 * c + 8 * hh, kBQ)) = dsb[c];
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *reinterpret_cast<u32x4*>(dSt + swz_off(kl, 16 * c + 8 * hh, kBQ)) = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();

      // dQ[query][32*dblk + lq] += sum over the tile's 128 keys of (scale dS) * K; the A operand
      // dS (query x key) is read transposed out of dS^T.
      for (int qb = qb_lo; qb < qb_hi; ++qb) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int c = 0; c < kBN / 16; ++c)
          acc = mfma32(tr_operand(dSt, sa, kBQ, c, qb), ktreg[c], acc);
        const int64_t q0 = qbase + qb * 32;
        float* dst = dqp + (q0 + 4 * hh) * D + 32 * dblk + lq;
        if (q0 + 32 <= pr.q_len) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            unsafeAtomicAdd(dst + ((r >> 2) * 8 + (r & 3)) * D, acc[r]);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (q0 + out_row(r, hh) < pr.q_len) unsafeAtomicAdd(dst + ((r >> 2) * 8 + (r & 3)) * D, acc[r]);
        }
      }
      if (it + 1 < niter) store_qdo<D>(lds, ldsf, buf ^ 1, qr, dr, extra);
      __syncthreads();
    }
  }

  if (kvalid) {
    float* dk = p.dk + (dkvhead + tr.row0 + kl) * D;
    float* dv = p.dv + (dkvhead + tr.row0 + kl) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * db + out_row(r, hh);
        unsafeAtomicAdd(dk + d, dk_acc[db][r]);
        unsafeAtomicAdd(dv + d, dv_acc[db][r]);
      }
  }
}

template <int D>
int launch_bwd(const KParams& kp, void* stream) {
  static bool attr_done = false;
  const size_t lds = BwdCfg<D>::LDS_BYTES;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)chunk_bwd_bf16_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    attr_done = true;
  }
  const int64_t nblk = (int64_t)kp.B * kp.Hq * kp.tiles_per_head;
  if (nblk == 0) return 0;
  hipLaunchKernelGGL(chunk_bwd_bf16_kernel<D>, dim3((unsigned)nblk), dim3(kNT), lds,
                     (hipStream_t)stream, kp);
  return (int)hipGetLastError();
}

}  // namespace

int launch_chunk_bwd_bf16(const KParams& kp, void* stream) {
  return kp.D == 128 ? launch_bwd<128>(kp, stream) : launch_bwd<64>(kp, stream);
}

}  // namespace ra
