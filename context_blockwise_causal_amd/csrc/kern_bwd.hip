// Chunk backward on bf16 MFMA (gfx950) with probability recompute, as two kernels.
//
// Method: InfiniTrain pull request "Feat: Context Parallel", section 主要改动, p2p mode: the
// backward recomputes the probabilities from the saved log-sum-exp and returns the K/V
// gradients to the chunk's owner.  Per query row t and key j (scale = softmax scale):
//   P = exp(scale q.k - lse),  dP = dO.v,  dS = P (dP - delta),  delta = <dO, O>,
//   dV += P^T dO,  dK += scale dS^T Q,  dQ += scale dS K.
//
// Split: a key-major kernel forms dK and dV (each workgroup owns 128 keys and walks the query
// rows that see them), and a query-major kernel forms dQ (each workgroup owns 128 query rows
// and walks the keys they see).  Both recompute S and dP, which costs two extra contractions
// over a fused kernel, but each holds at most ~230 live registers: two wavefronts per SIMD, no
// dQ atomics, no LDS round trip of dS and one barrier per step.
//
// Both kernels use v_mfma_f32_32x32x16_bf16 with fp32 accumulation, LDS tiles that are
// unpadded and chunk-swizzled (conflict-free row reads, ds_read_b64_tr_b16 transposed reads and
// tile writes), double buffering filled by direct global->LDS loads issued one step ahead, and
// the softmax scale folded into dS so that dK and dQ need no further multiplies.
#include "kern_common.h"

namespace ra {
namespace {

constexpr int kNT = 256;

// ======================================================================= dK / dV, key-major
//
// One workgroup = 4 wavefronts = 128 keys of one (batch, query head).  Wavefront w owns keys
// 32w..32w+31: their K rows are in registers (B operand of S = Q K^T), their V rows come from
// the workgroup's V tile in LDS (B operand of dP = dO V^T), and their dK^T / dV^T accumulators
// (fp32, 32 keys x D) live in registers until the end, where they are added to dk / dv with
// fp32 atomics (the query heads of one key/value head add into the same rows).
//
// S and dP come out with the key across lanes and 32 queries in registers (queries fed in
// perm32 order), which is directly the B-operand layout of dV^T += dO^T P and dK^T += Q^T dS.

constexpr int kKvBN = 128;  // keys per workgroup
constexpr int kKvBQ = 32;   // query rows per step

// Stored scale * dS^T (bf16) of one pair and (batch, query head): ds_rows keys x ds_ld queries
// in blocks of 32 keys x 32 queries, each 2 KB and contiguous; block (key / 32, query / 32) at
// element (key / 32) * 32 ds_ld + (query / 32) * 1024, and inside a block key k, query
// 16 c + 8 h + e at 512 c + 16 k + 8 h + e.  A dK/dV wavefront's step (32 keys x 32 queries; lane
// (k, h) holds queries 16 c + 8 h .. +7 of key k for c = 0, 1) is then two fully coalesced 1 KB
// stores, and 8 queries of one key are 16 contiguous bytes for the dQ pass.
__device__ __forceinline__ int64_t ds_block_off(int64_t key, int64_t q, int64_t ld) {
  return (key >> 5) * 32 * ld + (q >> 5) * 1024 + ((q >> 4) & 1) * 512 + (key & 31) * 16 + ((q >> 3) & 1) * 8 +
         (q & 7);
}

template <int D>
struct KvCfg {
  static constexpr int KK = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int QT = kKvBQ * D;  // elements of one Q (or dO) tile
};

// The V tile of a dK/dV workgroup, loaded once through registers into padded rows of D + 8
// elements: logical 16-byte chunk L = 2 kk + hh of a row sits at position KK hh + kk, so a lane's
// B operands of dP (kk = 0 .. KK-1, its lane half hh) are consecutive chunks at immediate offsets
// from one address, and the 16-byte row padding puts 16 consecutive rows on distinct banks
// (conflict-free reads).  Rows past the range repeat the last valid row (masked later).
template <int D, int ROWS, int NT>
__device__ __forceinline__ void load_v_padded(const u16* __restrict__ g, int64_t valid_rows, u16* vt) {
  constexpr int CH = D / 8, KK = D / 16;
  const int last = (int)(valid_rows < ROWS ? valid_rows : ROWS) - 1;
#pragma unroll
  for (int i = 0; i < ROWS * CH / NT; ++i) {
    const int idx = i * NT + (int)threadIdx.x, r = idx / CH, L = idx % CH;
    const u32x4 v = *reinterpret_cast<const u32x4*>(g + (r < last ? r : last) * D + 8 * L);
    *reinterpret_cast<u32x4*>(vt + r * (D + 8) + 8 * (KK * (L & 1) + (L >> 1))) = v;
  }
}

// Raw lse and delta of the step row that accumulator register (lane & 15) holds in this lane's
// half (row index clamped into the pair): lanes 16 c .. 16 c + 15 of each 16-lane DPP row hold
// the 16 values its lanes need, handed out per register by a row broadcast.
__device__ __forceinline__ void kv_load_rows(const float* __restrict__ lse, const float* __restrict__ dlt,
                                             int64_t q0, int64_t q_len, float& a, float& d) {
  const int l = threadIdx.x & 63;
  const int64_t q = q0 + perm_reg_row(l & 15, l >> 5);
  const int64_t qc = q < q_len ? q : q_len - 1;
  a = lse[qc];
  d = dlt[qc];
}

// Value of lane 16 (lane / 16) + r: DPP row_newbcast.
__device__ __forceinline__ float row_bcast(float x, int r) {
  const int v = __builtin_bit_cast(int, x);
  int o;
  switch (r) {
    case 0: o = __builtin_amdgcn_mov_dpp(v, 0x150, 0xF, 0xF, false); break;
    case 1: o = __builtin_amdgcn_mov_dpp(v, 0x151, 0xF, 0xF, false); break;
    case 2: o = __builtin_amdgcn_mov_dpp(v, 0x152, 0xF, 0xF, false); break;
    case 3: o = __builtin_amdgcn_mov_dpp(v, 0x153, 0xF, 0xF, false); break;
    case 4: o = __builtin_amdgcn_mov_dpp(v, 0x154, 0xF, 0xF, false); break;
    case 5: o = __builtin_amdgcn_mov_dpp(v, 0x155, 0xF, 0xF, false); break;
    case 6: o = __builtin_amdgcn_mov_dpp(v, 0x156, 0xF, 0xF, false); break;
    case 7: o = __builtin_amdgcn_mov_dpp(v, 0x157, 0xF, 0xF, false); break;
    case 8: o = __builtin_amdgcn_mov_dpp(v, 0x158, 0xF, 0xF, false); break;
    case 9: o = __builtin_amdgcn_mov_dpp(v, 0x159, 0xF, 0xF, false); break;
    case 10: o = __builtin_amdgcn_mov_dpp(v, 0x15A, 0xF, 0xF, false); break;
    case 11: o = __builtin_amdgcn_mov_dpp(v, 0x15B, 0xF, 0xF, false); break;
    case 12: o = __builtin_amdgcn_mov_dpp(v, 0x15C, 0xF, 0xF, false); break;
    case 13: o = __builtin_amdgcn_mov_dpp(v, 0x15D, 0xF, 0xF, false); break;
    case 14: o = __builtin_amdgcn_mov_dpp(v, 0x15E, 0xF, 0xF, false); break;
    default: o = __builtin_amdgcn_mov_dpp(v, 0x15F, 0xF, 0xF, false); break;
  }
  return __builtin_bit_cast(float, o);
}

template <int D, bool DS>
__global__ __launch_bounds__(kNT, 2) void chunk_bwd_kv_kernel(const KParams p) {
  using C = KvCfg<D>;
  // The V tile and two buffers of (Q, dO), carved out of one LDS array (lse and delta travel in
  // registers and reach their lanes by DPP row broadcasts, see kv_load_rows).  Each step
  // reads one buffer while direct loads fill the other; the step takes every LDS pointer as a
  // __restrict__ parameter, which lets the compiler prove that those loads do not alias its reads
  // (so it does not wait for them before the step's LDS reads).  One array, not several: with
  // several LDS variables the compiler's LDS lowering replaces the pointer-based alias scopes.
  __shared__ __attribute__((aligned(16))) u16 lds[kKvBN * (D + 8) + 4 * C::QT];
  u16* const vt = lds;
  u16* const qdbuf = lds + kKvBN * (D + 8);

  const TileRef tr = map_tile(p, kKvBN);
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int kl = 32 * w + lq;  // this lane's key within the tile
  const bool kvalid = kl < tr.nrows;
  const int64_t kvhead = ((int64_t)tr.b * p.Hkv + tr.g) * p.kv_head_rows;
  const int64_t qhead = ((int64_t)tr.b * p.Hq + tr.hq) * p.q_head_rows;
  const int64_t dkvhead = ((int64_t)tr.b * p.Hkv + tr.g) * p.dkv_head_rows;
  const u16* __restrict__ Kg = reinterpret_cast<const u16*>(p.k) + (kvhead + tr.row0) * D;
  const u16* __restrict__ Vg = reinterpret_cast<const u16*>(p.v) + (kvhead + tr.row0) * D;

  // The workgroup's V tile, resident in LDS for the whole kernel (rows past the range repeat the
  // last key; those keys are masked).
  load_v_padded<D, kKvBN, kNT>(Vg, tr.nrows, vt);
  // B operand of S = Q K^T: lane holds K[key][kk*16 + 8*hh .. +8].
  bf16x8 kreg[C::KK];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk)
    kreg[kk] = kvalid ? *reinterpret_cast<const bf16x8*>(Kg + kl * D + kk * 16 + 8 * hh)
                      : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});

  f32x16 dk_acc[C::DB], dv_acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }

  const RowAddr qa = make_row_addr(perm32(lq), hh, D);  // Q / dO rows in perm32 order
  const int vrow = kl * (D + 8) + 8 * C::KK * hh;        // this lane's V row (padded layout)
  const TrAddr ta = make_tr_addr(lane, D);              // Q^T, dO^T out of the [query][d] tiles
  const KRange& R = p.ranges[tr.range];
  for (int pi = 0; pi < R.npairs; ++pi) {
    const KPair pr = p.pairs[R.pair[pi]];
    const bool diag = pr.mask == RA_MASK_DIAG;
    const int64_t kloc0 = tr.row0 - pr.kv_row0;  // pair-local index of the tile's first key
    const int64_t kj = kloc0 + kl;              // pair-local index of this lane's key
    const int64_t q_begin = diag ? (kloc0 / kKvBQ) * kKvBQ : 0;
    // Window / attention-chunk restriction: pair-local index of the highest query that sees
    // this lane's key (non-decreasing in the key), over the wavefront, and the last query step.
    const bool has_hi = p.window > 0 || p.attn_chunk > 0;
    int64_t wave_hi_min = 0, wave_hi_max = 0, q_end = pr.q_len;
    int hi32 = 1 << 30;  // this lane's highest visible query, clamped to [-1, q_len]
    if (has_hi) {
      const int64_t hi = highest_query(pr.kv_pos0 + kj, p.window, p.attn_chunk) - pr.q_pos0;
      hi32 = (int)(hi < -1 ? -1 : (hi > pr.q_len ? pr.q_len : hi));
      wave_hi_min = highest_query(pr.kv_pos0 + kloc0 + 32 * w, p.window, p.attn_chunk) - pr.q_pos0;
      wave_hi_max = highest_query(pr.kv_pos0 + kloc0 + 32 * w + 31, p.window, p.attn_chunk) - pr.q_pos0;
      const int64_t wg_hi = highest_query(pr.kv_pos0 + kloc0 + tr.nrows - 1, p.window, p.attn_chunk) - pr.q_pos0;
      if (wg_hi + 1 < q_end) q_end = wg_hi + 1;
    }
    const int niter = (int)((q_end - q_begin + kKvBQ - 1) / kKvBQ);
    if (niter <= 0) continue;
    const u16* Qp = reinterpret_cast<const u16*>(p.q) + (qhead + pr.q_row0) * D;
    const u16* dOp = reinterpret_cast<const u16*>(p.dO) + (qhead + pr.q_row0) * D;
    const float* lsep = p.lse + qhead + pr.q_row0;
    const float* dltp = p.delta + qhead + pr.q_row0;
    // Stored scale * dS^T (bf16, 32 x 32 blocks, see ds_block_off) of this (batch, query head)
    // and pair: the block row of this wavefront's 32 keys, and this lane's place in a block.
    u16* const dsp = DS ? reinterpret_cast<u16*>(p.ds) + pr.ds_off +
                              (((int64_t)tr.b * p.Hq + tr.hq) * pr.ds_rows + kloc0 + 32 * w) * pr.ds_ld +
                              16 * lq + 8 * hh
                        : nullptr;
    // One query step on (Qs, dOs); the next step's rows go into (nQ, ndO).
    // (la, ld): raw lse / delta of this step's rows, loaded one step ahead.
    float la, ld;
    auto step = [&](const u16* __restrict__ Vs, const u16* __restrict__ Qs, const u16* __restrict__ dOs,
                    u16* __restrict__ nQ, u16* __restrict__ ndO, int it) {
      const int64_t qbase = q_begin + (int64_t)it * kKvBQ;
      // this lane's broadcast values: lse in base 2 (+inf past the pair, so that P vanishes) and
      // delta (0 past the pair)
      const bool rv = qbase + perm_reg_row(lane & 15, hh) < pr.q_len;
      const float lse2 = rv ? la * kLog2e : __builtin_inff(), dlt = rv ? ld : 0.f;
      if (it + 1 < niter) {
        issue_tile<D, kKvBQ, 4>(Qp + (qbase + kKvBQ) * D, pr.q_len - qbase - kKvBQ, nQ);
        issue_tile<D, kKvBQ, 4>(dOp + (qbase + kKvBQ) * D, pr.q_len - qbase - kKvBQ, ndO);
        kv_load_rows(lsep, dltp, qbase + kKvBQ, pr.q_len, la, ld);
      }
      // The whole wavefront lies in the future of every query of this step (diagonal pairs).  A
      // wavefront that the step does not reach stores no dS: its entries are excluded, and the
      // dQ pass masks them.
      const bool active = !(diag && kloc0 + 32 * w > qbase + kKvBQ - 1) && !(has_hi && qbase > wave_hi_max);
      if (active) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) {
          s = mfma32(row_operand(Qs, qa, kk), kreg[kk], s);
          dp = mfma32(row_operand(dOs, qa, kk), *reinterpret_cast<const bf16x8*>(Vs + vrow + 8 * kk), dp);
        }
        // Excluded (key, query) pairs: keys past the range, and keys after the query in a
        // diagonal pair.  Only steps on an edge take the masked path.
        const bool edge = !kvalid || (diag && kloc0 + 32 * w + 31 > qbase) ||
                          (has_hi && qbase + kKvBQ - 1 > wave_hi_min);
        // first and last visible query of this lane's key in the step
        const int qmin = !edge ? -1 : (!kvalid ? 1 << 20 : (diag ? (int)(kj - qbase) : -1));
        const int qmax = edge ? hi32 - (int)qbase : 1 << 20;  // last visible query of the step
        // query of register 4j+i is perm_reg_row(4j+i, 0) + 8 hh: compare the compile-time part
        // against the bounds shifted by 8 hh
        const int qml = qmin - 8 * hh, qmh = qmax - 8 * hh;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[r], p.scale_log2, -row_bcast(lse2, r)));
          s[r] = pv;
          dp[r] = (pv * p.scale) * (dp[r] - row_bcast(dlt, r));  // scale * dS
        }
        if (edge) {  // excluded (key, query) pairs get P = dS = 0
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qr = perm_reg_row(r, 0);
            if (qr < qml || qr > qmh) {
              s[r] = 0.f;
              dp[r] = 0.f;
            }
          }
        }
        bf16x8 pb[2], dsb[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          bf16x8 a, b;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            a[e] = (__bf16)s[8 * c + e];
            b[e] = (__bf16)dp[8 * c + e];
          }
          pb[c] = a;
          dsb[c] = b;
        }
        // scale * dS (bf16, exactly the operand of dK) for the dQ pass: registers 8c .. 8c+7 of
        // this lane are queries 16 c + 8 hh .. +7 of the step at its key, so the wavefront's step
        // is one 32 x 32 block, two 1 KB stores.  Key rows past the range (the block has 128-row
        // granules) and query columns past the pair (up to ds_ld) get values that nothing reads.
        // The stores go out ahead of the dV / dK contractions, which give them time to complete
        // before the wait that ends the step.
        if (DS) {
#pragma unroll
          for (int c = 0; c < 2; ++c)
            *reinterpret_cast<bf16x8*>(dsp + qbase * 32 + 512 * c) = dsb[c];
          __builtin_amdgcn_sched_barrier(0);
        }
        // dV^T += dO^T P and dK^T += Q^T dS; A operands read transposed out of the tiles.
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            dv_acc[db] = mfma32(tr_operand(dOs, ta, D, c, db), pb[c], dv_acc[db]);
            dk_acc[db] = mfma32(tr_operand(Qs, ta, D, c, db), dsb[c], dk_acc[db]);
          }
      }
      wait_vmem();
      __syncthreads();
    };

    issue_tile<D, kKvBQ, 4>(Qp + q_begin * D, pr.q_len - q_begin, qdbuf);
    issue_tile<D, kKvBQ, 4>(dOp + q_begin * D, pr.q_len - q_begin, qdbuf + C::QT);
    kv_load_rows(lsep, dltp, q_begin, pr.q_len, la, ld);
    wait_vmem();
    __syncthreads();
    for (int it = 0; it < niter; ++it) {
      u16* cur = qdbuf + (it & 1) * 2 * C::QT;
      u16* nxt = qdbuf + ((it + 1) & 1) * 2 * C::QT;
      step(vt, cur, cur + C::QT, nxt, nxt + C::QT, it);
    }
  }

  // The query heads of one key/value head add into the same dK/dV rows, so the sums go out as
  // fp32 atomics.  The accumulators hold one key per lane; written as they are, every atomic
  // instruction would touch 64 rows.  Each wavefront therefore stages its 32 x D block in LDS
  // (16-byte chunks XOR-swizzled by row, conflict-free both ways) and adds it back row by row,
  // 64 consecutive floats per instruction.
  wait_vmem();
  __syncthreads();
  float* const st = reinterpret_cast<float*>(lds) + w * (32 * D);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const f32x16* acc = t ? dv_acc : dk_acc;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // registers 4j..4j+3 hold d = 32 db + 8 j + 4 hh + (0..3): chunk 8 db + 2 j + hh
        const int c = 8 * db + 2 * j + hh;
        *reinterpret_cast<f32x4*>(st + lq * D + ((c ^ (lq & 15)) << 2)) =
            f32x4{acc[db][4 * j], acc[db][4 * j + 1], acc[db][4 * j + 2], acc[db][4 * j + 3]};
      }
    float* const g = (t ? p.dv : p.dk) + (dkvhead + tr.row0 + 32 * w) * D;
    for (int k = 0; k < 32; ++k) {
      if (32 * w + k >= tr.nrows) break;
#pragma unroll
      for (int h = 0; h < D / 64; ++h) {
        const int d = 64 * h + lane;
        unsafeAtomicAdd(g + k * D + d, st[k * D + (((d >> 2) ^ (k & 15)) << 2) + (d & 3)]);
      }
    }
  }
}

// ======================================================================= dK / dV, ping-pong
//
// The same computation with two teams of 4 wavefronts per workgroup (8 wavefronts, two per
// SIMD, one of each team), each team owning 128 keys; both teams walk the same query steps and
// share their Q / dO / lse / delta tiles.  A wavefront's step is split into a matrix phase (the
// dV / dK contractions of the previous step and the S / dP contractions of this step) and a
// vector phase (P and dS of this step).  The teams run these phases half a step apart, separated
// by workgroup barriers, so that on every SIMD one wavefront issues MFMAs while the other does its
// exponentials and conversions: the matrix core does not wait for the vector work of the
// wavefront it serves.  The tiles rotate through three LDS buffers; the first team loads step
// t + 1 during its matrix phase of step t, and its vector phase waits for those loads.

constexpr int kPPKeys = 256;  // keys per workgroup (two teams of 128)
constexpr int kPPNT = 512;    // threads per workgroup

template <int D, bool DS>
__global__ __launch_bounds__(kPPNT, 2) void chunk_bwd_kv_pp_kernel(const KParams p) {
  using C = KvCfg<D>;
  constexpr int BUF = 2 * C::QT + 128;  // Q tile, dO tile, then 32 lse and 32 delta values (fp32)
  constexpr int VP = D + 8;             // padded V row
  constexpr int STG = 4 * 1024;         // the first team's scale * dS of one step (4 x 64 lanes x 32 B)
  __shared__ __attribute__((aligned(16))) u16 lds[kPPKeys * VP + 4 * BUF + (DS ? STG : 0)];
  u16* const vt = lds;
  u16* const tiles = lds + kPPKeys * VP;
  u16* const stg = tiles + 4 * BUF;

  // q_per_wg query heads of one key/value group in turn: one prologue (K, V) and one epilogue (the
  // dK/dV atomics) for all of them
  const int qgroup = p.q_per_wg > 1 ? p.q_per_wg : 1;
  const TileRef tr = map_tile(p, kPPKeys, qgroup);
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int team = w >> 2, kw = 32 * w;  // kw: the wavefront's first key within the tile
  const int kl = kw + lq;                // this lane's key within the tile
  const bool kvalid = kl < tr.nrows, wvalid = kw < tr.nrows;
  const int64_t kvhead = ((int64_t)tr.b * p.Hkv + tr.g) * p.kv_head_rows;
  const int64_t dkvhead = ((int64_t)tr.b * p.Hkv + tr.g) * p.dkv_head_rows;
  const u16* __restrict__ Kg = reinterpret_cast<const u16*>(p.k) + (kvhead + tr.row0) * D;
  const u16* __restrict__ Vg = reinterpret_cast<const u16*>(p.v) + (kvhead + tr.row0) * D;

  load_v_padded<D, kPPKeys, kPPNT>(Vg, tr.nrows, vt);
  bf16x8 kreg[C::KK];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk)
    kreg[kk] = kvalid ? *reinterpret_cast<const bf16x8*>(Kg + kl * D + kk * 16 + 8 * hh)
                      : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  f32x16 dk_acc[C::DB], dv_acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }
  const RowAddr qa = make_row_addr(perm32(lq), hh, D);
  const int vrow = kl * VP + 8 * C::KK * hh;
  const TrAddr ta = make_tr_addr(lane, D);
  // log2(scale), wave-uniform (kept in a scalar register)
  const float l2s = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, __builtin_amdgcn_logf(p.scale))));

  const KRange& R = p.ranges[tr.range];
  for (int gi = 0; gi < qgroup; ++gi) {
  const int hq = tr.hq + gi;
  const int64_t qhead = ((int64_t)tr.b * p.Hq + hq) * p.q_head_rows;
  for (int pi = 0; pi < R.npairs; ++pi) {
    const KPair pr = p.pairs[R.pair[pi]];
    const bool diag = pr.mask == RA_MASK_DIAG;
    const int64_t kloc0 = tr.row0 - pr.kv_row0;
    const int64_t kwave = kloc0 + kw;  // pair-local index of the wavefront's first key
    const int64_t kj = kwave + lq;
    const int64_t q_begin = diag ? (kloc0 / kKvBQ) * kKvBQ : 0;
    const bool has_hi = p.window > 0 || p.attn_chunk > 0;
    int64_t wave_hi_min = 0, q_end = pr.q_len;
    int hi32 = 1 << 30;
    if (has_hi) {
      const int64_t hi = highest_query(pr.kv_pos0 + kj, p.window, p.attn_chunk) - pr.q_pos0;
      hi32 = (int)(hi < -1 ? -1 : (hi > pr.q_len ? pr.q_len : hi));
      wave_hi_min = highest_query(pr.kv_pos0 + kwave, p.window, p.attn_chunk) - pr.q_pos0;
      const int64_t wg_hi = highest_query(pr.kv_pos0 + kloc0 + tr.nrows - 1, p.window, p.attn_chunk) - pr.q_pos0;
      if (wg_hi + 1 < q_end) q_end = wg_hi + 1;
    }
    const int niter = (int)((q_end - q_begin + kKvBQ - 1) / kKvBQ);
    if (niter <= 0) continue;
    // Steps that take the mask, as bounds on the step index t (scalar): all of them when some key
    // of the wavefront lies past the tile; t < t_lo while a step reaches a key of the wavefront
    // after its query (diagonal pair); t >= t_hi once a step reaches past the window / attention
    // chunk of the wavefront's first key.
    const bool wpart = kw + 32 > tr.nrows;
    int t_lo = 0, t_hi = niter;
    if (diag) {
      const int64_t x = kwave + 31 - q_begin;  // steps with 32 t < x
      t_lo = x <= 0 ? 0 : (int)((x + kKvBQ - 1) / kKvBQ);
    }
    if (has_hi) {
      const int64_t y = wave_hi_min - (kKvBQ - 1) - q_begin;  // steps with 32 t > y
      const int64_t th = y < 0 ? 0 : y / kKvBQ + 1;
      t_hi = (int)(th < niter ? th : niter);
    }
    const u16* Qp = reinterpret_cast<const u16*>(p.q) + (qhead + pr.q_row0) * D;
    const u16* dOp = reinterpret_cast<const u16*>(p.dO) + (qhead + pr.q_row0) * D;
    const float* lsep = p.lse + qhead + pr.q_row0;
    const float* dltp = p.delta + qhead + pr.q_row0;
    // stored scale * dS^T: the block row of the wavefront's 32 keys (see ds_block_off); only rows
    // of wavefronts holding a valid key are stored (they lie inside the pair's 128-row granules)
    char* const dsw = DS ? reinterpret_cast<char*>(reinterpret_cast<u16*>(p.ds) + pr.ds_off +
                                                   (((int64_t)tr.b * p.Hq + hq) * pr.ds_rows + kwave) * pr.ds_ld)
                         : nullptr;

    // Carried from one phase to the next: S and dP after a matrix phase; P and scale * dS (bf16,
    // packed into s) after a vector phase.  One pair of register blocks for both keeps the
    // values live at the loop head to 32 registers.
    f32x16 s = f32x16{}, dp = f32x16{};
    // The first team loads the tiles of the step at row q0 (Q, dO, lse and delta; rows past the
    // pair repeat its last row) with direct buffer loads: unlike the global form, a buffer load to
    // LDS in flight leaves the compiler's waits for LDS reads exact.  Each buffer resource spans
    // the step's rows only.
    auto load = [&](int64_t q0, u16* __restrict__ B) {
      const int last = (int)(pr.q_len - q0 < kKvBQ ? pr.q_len - q0 : kKvBQ) - 1;
      const auto rq = __builtin_amdgcn_make_buffer_rsrc((void*)(Qp + q0 * D), 0, kKvBQ * D * 2, kBufRsrcWord3);
      const auto ro = __builtin_amdgcn_make_buffer_rsrc((void*)(dOp + q0 * D), 0, kKvBQ * D * 2, kBufRsrcWord3);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int i = k * 4 + w, row = i * 4 + lane / 16;
        const int c = (lane % 16) ^ swz(row, D);
        const unsigned off = (unsigned)((row < last ? row : last) * D + c * 8) * 2u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lvoid_t*)(B + i * 512), 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, (lvoid_t*)(B + C::QT + i * 512), 16, off, 0, 0, 0);
      }
      if (w == 0) {  // lanes 0-31: lse, 32-63: delta of the step's rows
        const unsigned off = (unsigned)(lq < last ? lq : last) * 4u;
        // two instructions, each with one half of the lanes active (one resource each)
        const auto rl = __builtin_amdgcn_make_buffer_rsrc((void*)(lsep + q0), 0, kKvBQ * 4, kBufRsrcWord3);
        const auto rd = __builtin_amdgcn_make_buffer_rsrc((void*)(dltp + q0), 0, kKvBQ * 4, kBufRsrcWord3);
        if (hh == 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lvoid_t*)(B + 2 * C::QT), 4, off, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (hh == 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lvoid_t*)(B + 2 * C::QT), 4, off, 0, 0, 0);
      }
    };
    // One phase of this wavefront for step t: the matrix phase (mph: the dV / dK contractions of
    // step t - 1 if dvdk, the S / dP contractions of step t if sdp) or the vector phase.  Bc holds
    // step t's tiles, Bo step t - 1's, B1 step t + 1's and Bn receives step t + 2's (first team,
    // matrix phase); Sg is the staging area of the first team's dS.
    auto phase = [&](bool mph, bool dvdk, bool sdp, int t, u16* __restrict__ Bn, const u16* __restrict__ Bo,
                     const u16* __restrict__ Bc, u16* __restrict__ B1, const u16* __restrict__ Vs,
                     u16* __restrict__ Sg) {
      const int64_t qbase = q_begin + (int64_t)t * kKvBQ;
      if (mph) {
        __builtin_amdgcn_s_setprio(1);  // the matrix phase's MFMAs go ahead of the other wavefront's vector work
        if (team == 0 && t + 2 < niter) load(qbase + 2 * kKvBQ, Bn);
        if (dvdk) {
          // the per-db addresses are formed here, not kept live across the loop
          TrAddr tq = ta;
          asm volatile("" : "+v"(tq.lo), "+v"(tq.hi));
          const bf16x8 pb[2] = {__builtin_bit_cast(bf16x8, __builtin_shufflevector(s, s, 0, 1, 2, 3)),
                                __builtin_bit_cast(bf16x8, __builtin_shufflevector(s, s, 4, 5, 6, 7))};
          const bf16x8 dsb[2] = {__builtin_bit_cast(bf16x8, __builtin_shufflevector(s, s, 8, 9, 10, 11)),
                                 __builtin_bit_cast(bf16x8, __builtin_shufflevector(s, s, 12, 13, 14, 15))};
          __builtin_amdgcn_sched_barrier(0);
          // dV^T += dO^T P and dK^T += Q^T dS of step t - 1.  The operands are read well ahead of
          // their MFMAs (the other wavefront of the SIMD is in its vector phase and cannot fill the
          // matrix core's gaps).
          // The 16 MFMAs in the order (db, c): dV += dO^T(c, db) P(c), dK += Q^T(c, db) dS(c); the
          // A operand of MFMA i is read kWin - 1 MFMAs ahead into a rolling window of registers.
          constexpr int kWin = 8;
          bf16x8 A[kWin];
          auto load_op = [&](int i) {
            const int db = i >> 2, c = (i >> 1) & 1;
            A[i % kWin] = tr_operand((i & 1) ? Bo : Bo + C::QT, tq, D, c, db);
          };
#pragma unroll
          for (int i = 0; i < kWin - 1; ++i) load_op(i);
#pragma unroll
          for (int i = 0; i < 4 * C::DB; ++i) {
            if (i + kWin - 1 < 4 * C::DB) load_op(i + kWin - 1);
            __builtin_amdgcn_sched_barrier(0);
            const int db = i >> 2, c = (i >> 1) & 1;
            if (i & 1)
              dk_acc[db] = mfma32(A[i % kWin], dsb[c], dk_acc[db]);
            else
              dv_acc[db] = mfma32(A[i % kWin], pb[c], dv_acc[db]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // the previous step's operands are dead before this step's S and dP accumulators start
        __builtin_amdgcn_sched_barrier(0);
        if (sdp) {
          // S = Q K^T and dP = dO V^T; the Q and dO operands are read two kk ahead, V one ahead
          bf16x8 qo[3], oo[3], vo[2];
          RowAddr rq = qa;  // the per-kk addresses are formed here, not kept live across the loop
          asm volatile("" : "+v"(rq.base), "+v"(rq.g8));
          auto load_qo = [&](int kk) {
            qo[kk % 3] = row_operand(Bc, rq, kk);
            oo[kk % 3] = row_operand(Bc + C::QT, rq, kk);
          };
          auto load_v = [&](int kk) { vo[kk & 1] = *reinterpret_cast<const bf16x8*>(Vs + vrow + 8 * kk); };
          load_qo(0);
          load_v(0);
          load_qo(1);
          s = f32x16{};
          dp = f32x16{};
#pragma unroll
          for (int kk = 0; kk < C::KK; ++kk) {
            if (kk + 2 < C::KK) load_qo(kk + 2);
            if (kk + 1 < C::KK) load_v(kk + 1);
            __builtin_amdgcn_sched_barrier(0);
            s = mfma32(qo[kk % 3], kreg[kk], s);
            dp = mfma32(oo[kk % 3], vo[kk & 1], dp);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
      } else {
        // Reads whose latency the phase's arithmetic hides: the first team waits for step t + 1's
        // tiles (loaded two phases ago) and wavefront 0 reads their raw lse; the second team reads
        // its partner's staged dS (see the end of the phase).
        const bool conv = team == 0 && w == 0 && t + 1 < niter;
        float* const lnext = reinterpret_cast<float*>(B1 + 2 * C::QT);
        const bool pstore = DS && team == 1 && kw - 128 < tr.nrows;
        float lraw = 0.f;
        f32x4 x2 = f32x4{}, x3 = f32x4{};
        if (team == 0) {
          // The first team's only memory operations in flight are its direct loads, which
          // complete in order: after the loads of step t + 2 (4 instructions; 6 for wavefront 0)
          // leave the wait, those of step t + 1 are done.
          if (t + 2 < niter)
            __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
          else
            wait_vmem();
          if (conv && lane < 32) lraw = lnext[lane];
        } else if (pstore) {
          const u16* const sp = Sg + (w - 4) * 1024 + lane * 8;
          x2 = *reinterpret_cast<const f32x4*>(sp);
          x3 = *reinterpret_cast<const f32x4*>(sp + 512);
        }
        // P' = scale P = exp2(scale log2(e) S - L) with L = log2(e) lse - log2(scale) per row
        // (converted in LDS, +inf past the pair), and scale dS = P' (dP - delta).  Registers
        // 4j .. 4j+3 of a lane hold 4 consecutive rows: their L and delta are one 16-byte LDS read
        // each, the same for all lanes of a half.
        const float* const lf = reinterpret_cast<const float*>(Bc + 2 * C::QT);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rb = ((j >> 1) << 4) | (hh << 3) | ((j & 1) << 2);
          const f32x4 L = *reinterpret_cast<const f32x4*>(lf + rb);
          const f32x4 dl = *reinterpret_cast<const f32x4*>(lf + 32 + rb);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * j + i;
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[r], p.scale_log2, -L[i]));
            s[r] = pv;
            dp[r] = pv * (dp[r] - dl[i]);
          }
        }
        // excluded (key, query) pairs: keys past the range, keys after the query (diagonal pair),
        // queries past the window / attention chunk of the key
        if (wpart || t < t_lo || t >= t_hi) {
          const int qmin = !kvalid ? 1 << 20 : (diag ? (int)(kwave - qbase) + lq : -1);
          const int qml = qmin - 8 * hh, qmh = hi32 - (int)qbase - 8 * hh;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qr = perm_reg_row(r, 0);
            if (qr < qml || qr > qmh) {
              s[r] = 0.f;
              dp[r] = 0.f;
            }
          }
        }
        bf16x8 pb[2], dsb[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pb[c][e] = (__bf16)s[8 * c + e];
            dsb[c][e] = (__bf16)dp[8 * c + e];
          }
        }
        const f32x4 w0 = __builtin_bit_cast(f32x4, pb[0]), w1 = __builtin_bit_cast(f32x4, pb[1]);
        const f32x4 w2 = __builtin_bit_cast(f32x4, dsb[0]), w3 = __builtin_bit_cast(f32x4, dsb[1]);
        s = f32x16{w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3],
                   w2[0], w2[1], w2[2], w2[3], w3[0], w3[1], w3[2], w3[3]};
        if (team == 0) {
          // step t + 1's L (see above), and this wavefront's scale * dS, which its partner in the
          // second team stores
          if (conv && lane < 32)
            lnext[lane] = lane < (int)(pr.q_len - qbase - kKvBQ) ? fmaf(lraw, kLog2e, -l2s) : __builtin_inff();
          if (DS) {
            u16* const sp = Sg + w * 1024 + lane * 8;
            *reinterpret_cast<f32x4*>(sp) = w2;
            *reinterpret_cast<f32x4*>(sp + 512) = w3;
          }
        } else if (DS) {
          // The second team stores scale * dS for the dQ pass: its own and that of its partner in
          // the first team (keys 128 lower), staged in LDS in the previous phase.  Registers
          // 8c .. 8c+7 of a lane are queries 16 c + 8 hh .. +7 of the step at its key: a
          // wavefront's step is one 32 x 32 block (see ds_block_off), two 1 KB stores.  Nothing
          // waits for these stores.
          int ln = lane;  // the lane's byte offset in the block is formed here, not kept live
          asm volatile("" : "+v"(ln));
          const unsigned dslane = (unsigned)((ln & 31) * 32 + 16 * (ln >> 5));
          char* const row = dsw + qbase * 64 + dslane;
          if (wvalid) {
            *reinterpret_cast<f32x4*>(row) = w2;
            *reinterpret_cast<f32x4*>(row + 1024) = w3;
          }
          if (pstore) {
            char* const prow = row - 128 * pr.ds_ld * 2;
            *reinterpret_cast<f32x4*>(prow) = x2;
            *reinterpret_cast<f32x4*>(prow + 1024) = x3;
          }
        }
      }
    };

    if (team == 0) {
      load(q_begin, tiles);
      if (niter > 1) load(q_begin + kKvBQ, tiles + BUF);
    }
    wait_vmem();
    if (w == 0 && lane < 32) {  // L of step 0 (see the vector phase; step t + 1's is formed in step t's)
      float* const ln = reinterpret_cast<float*>(tiles + 2 * C::QT);
      ln[lane] = q_begin + lane < pr.q_len ? fmaf(ln[lane], kLog2e, -l2s) : __builtin_inff();
    }
    __syncthreads();
    auto run = [&](bool mph, bool dvdk, bool sdp, int t) {
      u16* const Bc = tiles + (t & 3) * BUF;
      u16* const Bn = tiles + ((t + 2) & 3) * BUF;
      u16* const Bo = tiles + ((t + 3) & 3) * BUF;
      u16* const B1 = tiles + ((t + 1) & 3) * BUF;
      phase(mph, dvdk, sdp, t, Bn, Bo, Bc, B1, vt, stg);
      phase_barrier();
    };
    // Each loop step is the vector phase of step t and the matrix phase of step t + 1 (the first
    // M has no dV / dK, the last no S / dP).  The second team runs one phase behind the first.
    if (team == 1) phase_barrier();
    for (int t = -1; t < niter; ++t) {
      if (t >= 0) run(false, false, false, t);
      else phase_barrier();
      run(true, t >= 0, t + 1 < niter, t + 1);
    }
    if (team == 0) phase_barrier();
  }

  }  // query heads of the group

  // Epilogue: the teams in turn; each wavefront stages its 32 x D block in LDS and adds it to dk /
  // dv row by row with fp32 atomics (the query heads of a key/value head add into the same rows).
  wait_vmem();
  __syncthreads();
  float* const st = reinterpret_cast<float*>(lds) + (w & 3) * (32 * D);
  for (int turn = 0; turn < 2; ++turn) {
    if (team == turn) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const f32x16* acc = t ? dv_acc : dk_acc;
        const float f = t ? 1.f / p.scale : 1.f;  // dV was accumulated with scale P
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int c = 8 * db + 2 * j + hh;
            *reinterpret_cast<f32x4*>(st + lq * D + ((c ^ (lq & 15)) << 2)) =
                f32x4{acc[db][4 * j] * f, acc[db][4 * j + 1] * f, acc[db][4 * j + 2] * f, acc[db][4 * j + 3] * f};
          }
        float* const g = (t ? p.dv : p.dk) + (dkvhead + tr.row0 + kw) * D;
        for (int k = 0; k < 32; ++k) {
          if (kw + k >= tr.nrows) break;
#pragma unroll
          for (int h = 0; h < D / 64; ++h) {
            const int d = 64 * h + lane;
            unsafeAtomicAdd(g + k * D + d, st[k * D + (((d >> 2) ^ (k & 15)) << 2) + (d & 3)]);
          }
        }
      }
    }
    __syncthreads();
  }
}

// ======================================================================= dQ, query-major
//
// One workgroup = 4 wavefronts = 128 query rows of one (batch, head); wavefront w owns 32 rows,
// a lane one query (the forward's transposed orientation).  Per K/V tile of 64 keys:
//   S^T = K Q^T and dP^T = V dO^T (A = K / V rows in perm32 order from LDS, B = Q / dO rows in
//   registers), P^T = exp2(S^T scale log2e - lse2) and dS^T = scale P^T (dP^T - delta) with one
//   lse and one delta per lane, then dQ^T += K^T dS^T (A = K^T by transposed reads, B = dS^T
//   straight from the registers it was computed in).  The row's dQ accumulator is added to
//   dq_acc once at the end (each row belongs to one workgroup per launch: no atomics).

constexpr int kQBM = 128;  // query rows per workgroup
constexpr int kQBN = 64;   // keys per K/V tile

template <int D>
struct QCfg {
  static constexpr int KK = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int TILE = kQBN * D;
};

template <int D>
__global__ __launch_bounds__(kNT, 2) void chunk_bwd_q_kernel(const KParams p) {
  using C = QCfg<D>;
  // Two K/V buffers, read and filled through __restrict__ pointers (see the dK/dV kernel).
  __shared__ __attribute__((aligned(16))) u16 kvbuf[4 * C::TILE];

  const TileRef tr = map_tile(p, kQBM);
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int qi = 32 * w + lq;
  const bool qvalid = qi < tr.nrows;
  const int64_t qrow = (((int64_t)tr.b * p.Hq + tr.hq) * p.q_head_rows) + tr.row0 + qi;
  const int64_t kvhead = ((int64_t)tr.b * p.Hkv + tr.g) * p.kv_head_rows;
  const u16* __restrict__ Q = reinterpret_cast<const u16*>(p.q);
  const u16* __restrict__ dO = reinterpret_cast<const u16*>(p.dO);

  // B operands: lane holds Q / dO[query][kk*16 + 8*hh .. +8]; one lse and delta per lane.
  bf16x8 qreg[C::KK], doreg[C::KK];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk) {
    if (qvalid) {
      qreg[kk] = *reinterpret_cast<const bf16x8*>(Q + qrow * D + kk * 16 + 8 * hh);
      doreg[kk] = *reinterpret_cast<const bf16x8*>(dO + qrow * D + kk * 16 + 8 * hh);
    } else {
      qreg[kk] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      doreg[kk] = qreg[kk];
    }
  }
  const float nlse2 = qvalid ? -p.lse[qrow] * kLog2e : -__builtin_inff();
  const float dl = qvalid ? p.delta[qrow] : 0.f;

  // dQ^T accumulator: dq[db][4j+i] holds dQ[query][32*db + 8*j + 4*hh + i].
  f32x16 dq[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dq[db] = f32x16{};

  const RowAddr ka0 = make_row_addr(perm32(lq), hh, D);
  const RowAddr ka1 = make_row_addr(32 + perm32(lq), hh, D);
  const TrAddr kt = make_tr_addr(lane, D);
  const u16* Kg = reinterpret_cast<const u16*>(p.k);
  const u16* Vg = reinterpret_cast<const u16*>(p.v);
  const KRange& R = p.ranges[tr.range];
  for (int pi = 0; pi < R.npairs; ++pi) {
    const KPair pr = p.pairs[R.pair[pi]];
    const bool diag = pr.mask == RA_MASK_DIAG;
    const int64_t qloc0 = tr.row0 - pr.q_row0;
    const int64_t iq = qloc0 + qi;
    int64_t key_end = pr.kv_len;
    if (diag && qloc0 + tr.nrows < key_end) key_end = qloc0 + tr.nrows;
    const int nkt = (int)((key_end + kQBN - 1) / kQBN);
    const u16* Kp = Kg + (kvhead + pr.kv_row0) * D;
    const u16* Vp = Vg + (kvhead + pr.kv_row0) * D;
    const int64_t wq_first = qloc0 + 32 * w;
    const bool wave_has_rows = 32 * w < tr.nrows;
    // Window / attention-chunk restriction: pair-local index of the lowest key this lane's
    // query sees (non-decreasing in the query), over the wavefront, and the first key tile.
    const bool has_lo = p.window > 0 || p.attn_chunk > 0;
    int64_t lo = 0, wave_lo = 0, wave_lo_max = 0, kt0 = 0;
    if (has_lo) {
      lo = lowest_key(pr.q_pos0 + iq, p.window, p.attn_chunk) - pr.kv_pos0;
      wave_lo = lowest_key(pr.q_pos0 + wq_first, p.window, p.attn_chunk) - pr.kv_pos0;
      wave_lo_max = lowest_key(pr.q_pos0 + wq_first + 31, p.window, p.attn_chunk) - pr.kv_pos0;
      const int64_t tile_lo = lowest_key(pr.q_pos0 + qloc0, p.window, p.attn_chunk) - pr.kv_pos0;
      kt0 = tile_lo > 0 ? tile_lo / kQBN : 0;
    }

    auto step = [&](const u16* __restrict__ kb, const u16* __restrict__ vb, u16* __restrict__ nk,
                    u16* __restrict__ nv, int t) {
      const int64_t kbase = (int64_t)t * kQBN;
      if (t + 1 < nkt) {
        issue_tile<D, kQBN, 4>(Kp + (kbase + kQBN) * D, pr.kv_len - kbase - kQBN, nk);
        issue_tile<D, kQBN, 4>(Vp + (kbase + kQBN) * D, pr.kv_len - kbase - kQBN, nv);
      }
      const bool active = wave_has_rows && !(diag && kbase > wq_first + 31) &&
                          !(has_lo && kbase + kQBN - 1 < wave_lo);
      if (active) {
        f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            s[b] = mfma32(row_operand(kb, b ? ka1 : ka0, kk), qreg[kk], s[b]);
            dp[b] = mfma32(row_operand(vb, b ? ka1 : ka0, kk), doreg[kk], dp[b]);
          }
        // Keys past the pair, or after this lane's query in a diagonal pair, are excluded;
        // kmax is the last visible key of the tile (only edge tiles need it).
        const bool edge = (kbase + kQBN > pr.kv_len) || (diag && kbase + kQBN - 1 > wq_first) ||
                          (has_lo && kbase < wave_lo_max);
        int kmax = kQBN - 1, kmin = 0;
        if (edge) {
          const int64_t lim = diag ? (iq < pr.kv_len - 1 ? iq : pr.kv_len - 1) : pr.kv_len - 1;
          kmax = (int)(lim - kbase < -1 ? -1 : (lim - kbase > kQBN - 1 ? kQBN - 1 : lim - kbase));
          if (has_lo) kmin = (int)(lo - kbase < 0 ? 0 : (lo - kbase > kQBN ? kQBN : lo - kbase));
        }
        // key of register r in block b is 32 b + perm_reg_row(r, 0) + 8 hh: compare the
        // compile-time part against the bounds shifted by 8 hh
        const int kmh = kmax - 8 * hh, kml = kmin - 8 * hh;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[b][r], p.scale_log2, nlse2));
            dp[b][r] = (pv * p.scale) * (dp[b][r] - dl);  // scale * dS^T
          }
        if (edge) {  // excluded keys get dS = 0
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = b * 32 + perm_reg_row(r, 0);
              if (key > kmh || key < kml) dp[b][r] = 0.f;
            }
        }
        // B operand dS^T for key step c: registers 8*(c&1) .. +8 of block c>>1.
        bf16x8 dsb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          bf16x8 tt;
#pragma unroll
          for (int e = 0; e < 8; ++e) tt[e] = (__bf16)dp[c >> 1][8 * (c & 1) + e];
          dsb[c] = tt;
        }
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int c = 0; c < 4; ++c) dq[db] = mfma32(tr_operand(kb, kt, D, c, db), dsb[c], dq[db]);
      }
      wait_vmem();
      __syncthreads();
    };

    if (kt0 >= nkt) continue;  // uniform over the workgroup
    issue_tile<D, kQBN, 4>(Kp + kt0 * kQBN * D, pr.kv_len - kt0 * kQBN, kvbuf);
    issue_tile<D, kQBN, 4>(Vp + kt0 * kQBN * D, pr.kv_len - kt0 * kQBN, kvbuf + C::TILE);
    wait_vmem();
    __syncthreads();
    for (int t = (int)kt0; t < nkt; ++t) {
      u16* cur = kvbuf + ((t - (int)kt0) & 1) * 2 * C::TILE;
      u16* nxt = kvbuf + ((t - (int)kt0 + 1) & 1) * 2 * C::TILE;
      step(cur, cur + C::TILE, nxt, nxt + C::TILE, t);
    }
  }

  if (qvalid) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4* dst = reinterpret_cast<f32x4*>(p.U + qrow * D + 32 * db + 8 * j + 4 * hh);
        f32x4 u = *dst;
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] += dq[db][4 * j + i];
        *dst = u;
      }
  }
}

// ======================================================================= dQ from stored dS
//
// The dK/dV kernel writes scale * dS^T (bf16, the operand it feeds to dK) in 32 x 32 blocks (see
// ds_block_off).  dQ is then the plain contraction dQ += (scale dS) K: one workgroup = 4
// wavefronts = 128 query rows of one (batch, head), a lane one query; per tile of 64 keys the K
// tile and the workgroup's 64 x 128 block of dS^T are staged in LDS (direct loads, one tile
// ahead) and dQ^T += K^T dS^T, with both operands read transposed out of their [key][..] tiles
// (ds_read_b64_tr_b16).  The kernel is bound by reading dS from HBM (two bytes per (query, key)
// pair against 2 D FLOPs).
//
// Entries of dS^T that no query of a pair sees may never have been written, or hold stale values
// (the dK/dV kernel skips query steps that lie wholly before its keys or past their window, and
// wavefronts whose keys a step does not reach store nothing), so tiles that straddle a mask bound
// zero the excluded entries of the operand before the MFMA; interior tiles are fully visible and
// were written.

// A workgroup of the dQ kernel takes QB query blocks of 32 per wavefront (128 QB queries) and
// steps over 64 / QB keys at a time, so that every step is 16 MFMAs per wavefront either way; with
// QB = 2 each K^T operand read from LDS feeds two MFMAs.
template <int QB> constexpr int ds_bm() { return 128 * QB; }  // query rows per workgroup
template <int QB> constexpr int ds_bn() { return 64 / QB; }   // keys per tile

// A workgroup's dS^T tile in LDS: its 16 half-blocks (32 keys x 16 queries, 1 KB: key block kb,
// query block qs of the workgroup, half c; wavefront w reads query blocks QB w .. QB w + QB - 1)
// at half-block h = (4 QB kb + qs) * 2 + c, each in the global layout (key k, query 8 hh + e at
// 16 k + 8 hh + e) and padded to 1152 bytes, so that the two query halves a transposed read takes
// at once sit 32 banks apart.
constexpr int kDsHalf = 576;  // elements per padded half-block

// Issues the direct loads of one dS^T tile (keys key0 .., queries q0 .. of the slab S of one
// (batch, head), leading dimension ld; key0 and q0 multiples of 32): each instruction copies one
// contiguous 1 KB half-block, lane i its 16-byte chunk i, past the caches (read once).  The buffer
// resource spans the tile's key-block rows, so with QB = 2 query blocks past the slab's width (the
// last tile of a pair can reach past its 128-column granule) read as out of range rather than
// another row's data; they feed only query columns past the pair, which are never stored.  Keys
// past the pair (up to the slab's 128-row granule) hold values the masks exclude.
template <int QB>
__device__ __forceinline__ void issue_ds_tile(const u16* S, int64_t ld, int64_t key0, int64_t q0, u16* tile) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)(S + (key0 >> 5) * 32 * ld), 0,
                                                     (int)(ds_bn<QB>() * ld * 2), kBufRsrcWord3);
  const unsigned base = (unsigned)((q0 >> 5) * 1024 * 2) + 16u * lane;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int h = 4 * k + w, c = h & 1, q = h >> 1, kb = q / (4 * QB), qs = q % (4 * QB);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lvoid_t*)(tile + h * kDsHalf), 16,
        base + (unsigned)(kb * 32 * ld * 2) + (unsigned)(qs * 2048 + c * 1024), 0, 0, 2);
  }
}

template <int D, int QB>
__global__ __launch_bounds__(kNT, 2) void chunk_bwd_dq_ds_kernel(const KParams p) {
  constexpr int DB = D / 32;
  constexpr int BM = ds_bm<QB>(), BN = ds_bn<QB>();
  constexpr int KS = BN / 16;         // 16-key MFMA steps per tile
  constexpr int KT = BN * D;          // elements of one K tile
  constexpr int ST = 16 * kDsHalf;    // elements of one dS^T tile (BN keys x BM queries, padded)
  // two buffers of (K tile, dS^T tile), read and filled through __restrict__ pointers
  __shared__ __attribute__((aligned(16))) u16 buf[2 * (KT + ST)];

  const TileRef tr = map_tile(p, BM);
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  // the lane's query in each of the wavefront's query blocks: qi0 + 32 j
  const int qi0 = 32 * QB * w + lq;
  const int64_t qrow0 = (((int64_t)tr.b * p.Hq + tr.hq) * p.q_head_rows) + tr.row0 + qi0;
  const int64_t kvhead = ((int64_t)tr.b * p.Hkv + tr.g) * p.kv_head_rows;
  const int64_t head = (int64_t)tr.b * p.Hq + tr.hq;

  // dQ^T accumulators: dq[j][db] holds query block j's dQ^T rows 32 db .. 32 db + 31
  f32x16 dq[QB][DB];
#pragma unroll
  for (int j = 0; j < QB; ++j)
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[j][db] = f32x16{};

  const TrAddr kt = make_tr_addr(lane, D);      // K^T out of the [key][d] tile
  // dS^T columns out of the half-blocks: lane j of 16-lane group g addresses key 8 (g >> 1) + j / 4
  // (+4 for the second read, +16 per odd key step, + one key block per two steps) and queries
  // 16 (g & 1) + 4 (j % 4) .. +3 of its query block
  const int dsg = lane >> 4, dsj = lane & 15;
  const int dsaddr = (2 * QB * w + (dsg & 1)) * kDsHalf + (8 * (dsg >> 1) + (dsj >> 2)) * 16 +
                     ((dsj & 3) >> 1) * 8 + (dsj & 1) * 4;
  const u16* Kg = reinterpret_cast<const u16*>(p.k);
  const KRange& R = p.ranges[tr.range];
  for (int pi = 0; pi < R.npairs; ++pi) {
    const KPair pr = p.pairs[R.pair[pi]];
    const bool diag = pr.mask == RA_MASK_DIAG;
    const int64_t qloc0 = tr.row0 - pr.q_row0;
    int64_t key_end = pr.kv_len;
    if (diag && qloc0 + tr.nrows < key_end) key_end = qloc0 + tr.nrows;
    const int nkt = (int)((key_end + BN - 1) / BN);
    const u16* Kp = Kg + (kvhead + pr.kv_row0) * D;
    // the pair's dS^T slab of this (batch, head); this workgroup reads its BM query columns
    const u16* Sp = reinterpret_cast<const u16*>(p.ds) + pr.ds_off + head * pr.ds_rows * pr.ds_ld;
    const int64_t wq_first = qloc0 + 32 * QB * w;   // the wavefront's first query (pair-local)
    const bool wave_has_rows = 32 * QB * w < tr.nrows;
    const bool has_lo = p.window > 0 || p.attn_chunk > 0;
    int64_t lo[QB] = {}, wave_lo = 0, wave_lo_max = 0, kt0 = 0;
    if (has_lo) {
#pragma unroll
      for (int j = 0; j < QB; ++j)
        lo[j] = lowest_key(pr.q_pos0 + qloc0 + qi0 + 32 * j, p.window, p.attn_chunk) - pr.kv_pos0;
      wave_lo = lowest_key(pr.q_pos0 + wq_first, p.window, p.attn_chunk) - pr.kv_pos0;
      wave_lo_max = lowest_key(pr.q_pos0 + wq_first + 32 * QB - 1, p.window, p.attn_chunk) - pr.kv_pos0;
      const int64_t tile_lo = lowest_key(pr.q_pos0 + qloc0, p.window, p.attn_chunk) - pr.kv_pos0;
      kt0 = tile_lo > 0 ? tile_lo / BN : 0;
    }

    auto step = [&](const u16* __restrict__ kb, const u16* __restrict__ sb, u16* __restrict__ nk,
                    u16* __restrict__ ns, int t) {
      const int64_t kbase = (int64_t)t * BN;
      if (t + 1 < nkt) {
        issue_tile<D, BN, 4>(Kp + (kbase + BN) * D, pr.kv_len - kbase - BN, nk);
        issue_ds_tile<QB>(Sp, pr.ds_ld, kbase + BN, qloc0, ns);
      }
      const bool active = wave_has_rows && !(diag && kbase > wq_first + 32 * QB - 1) &&
                          !(has_lo && kbase + BN - 1 < wave_lo);
      if (active) {
        // B operands dS^T for query block j and key step c: lane holds
        // dS^T[16c + 8hh + e][its query of block j], e = 0..7
        bf16x8 dsb[QB][KS];
#pragma unroll
        for (int j = 0; j < QB; ++j)
#pragma unroll
          for (int c = 0; c < KS; ++c) {
            const int off = dsaddr + ((c >> 1) * 8 * QB + 2 * j) * kDsHalf + (c & 1) * 256;
            const v4i16 lo4 = ds_read_tr16(sb + off), hi4 = ds_read_tr16(sb + off + 64);
            dsb[j][c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        const bool edge = (kbase + BN > pr.kv_len) || (diag && kbase + BN - 1 > wq_first) ||
                          (has_lo && kbase < wave_lo_max);
        if (edge) {
#pragma unroll
          for (int j = 0; j < QB; ++j) {
            // visible keys of this lane's query in block j, as tile offsets [kmin, kmax]
            const int64_t iq = qloc0 + qi0 + 32 * j;
            const int64_t lim = diag ? (iq < pr.kv_len - 1 ? iq : pr.kv_len - 1) : pr.kv_len - 1;
            const int kmax = (int)(lim - kbase < -1 ? -1 : (lim - kbase > BN - 1 ? BN - 1 : lim - kbase));
            const int kmin = has_lo ? (int)(lo[j] - kbase < 0 ? 0 : (lo[j] - kbase > BN ? BN : lo[j] - kbase)) : 0;
            // element e of step c is key 16 c + 8 hh + e: compare the compile-time part against
            // the bounds shifted by 8 hh; bf16 element 2 i + b is half b of 32-bit word i
            const int kmh = kmax - 8 * hh, kml = kmin - 8 * hh;
#pragma unroll
            for (int c = 0; c < KS; ++c) {
              u32x4 wv = __builtin_bit_cast(u32x4, dsb[j][c]);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int k0 = 16 * c + 2 * i;
                const unsigned lo16 = (k0 >= kml && k0 <= kmh) ? 0xFFFFu : 0u;
                const unsigned hi16 = (k0 + 1 >= kml && k0 + 1 <= kmh) ? 0xFFFF0000u : 0u;
                wv[i] &= lo16 | hi16;
              }
              dsb[j][c] = __builtin_bit_cast(bf16x8, wv);
            }
          }
        }
        // each K^T operand feeds the wavefront's QB query blocks
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int c = 0; c < KS; ++c) {
            const bf16x8 a = tr_operand(kb, kt, D, c, db);
#pragma unroll
            for (int j = 0; j < QB; ++j) dq[j][db] = mfma32(a, dsb[j][c], dq[j][db]);
          }
      }
      wait_vmem();
      __syncthreads();
    };

    if (kt0 >= nkt) continue;  // uniform over the workgroup
    issue_tile<D, BN, 4>(Kp + kt0 * BN * D, pr.kv_len - kt0 * BN, buf);
    issue_ds_tile<QB>(Sp, pr.ds_ld, kt0 * BN, qloc0, buf + KT);
    wait_vmem();
    __syncthreads();
    for (int t = (int)kt0; t < nkt; ++t) {
      u16* cur = buf + ((t - (int)kt0) & 1) * (KT + ST);
      u16* nxt = buf + ((t - (int)kt0 + 1) & 1) * (KT + ST);
      step(cur, cur + KT, nxt, nxt + KT, t);
    }
  }

#pragma unroll
  for (int jq = 0; jq < QB; ++jq) {
    if (qi0 + 32 * jq >= tr.nrows) continue;
    const int64_t qrow = qrow0 + 32 * jq;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4* dst = reinterpret_cast<f32x4*>(p.U + qrow * D + 32 * db + 8 * j + 4 * hh);
        f32x4 u = *dst;
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] += dq[jq][db][4 * j + i];
        *dst = u;
      }
  }
}

template <int D>
int launch_bwd_ds(const KParams& kv, const KParams& q, void* stream, const BwdFork* fork) {
  int e;
  const int64_t nkv = kv.dk ? (int64_t)kv.B * kv.Hq * kv.tiles_per_head : 0;
  const int64_t nq = q.U ? (int64_t)q.B * q.Hq * q.tiles_per_head : 0;
  if (nkv > 0) {
    if (D == 128) {
      const int64_t G = kv.q_per_wg > 1 ? kv.q_per_wg : 1;
      hipLaunchKernelGGL((chunk_bwd_kv_pp_kernel<D, true>), dim3((unsigned)(nkv / G)), dim3(kPPNT), 0,
                         (hipStream_t)stream, kv);
    } else
      hipLaunchKernelGGL((chunk_bwd_kv_kernel<D, true>), dim3((unsigned)nkv), dim3(kNT), 0, (hipStream_t)stream, kv);
    if ((e = (int)hipGetLastError())) return e;
  }
  if (nq == 0) return 0;
  // the dQ kernel reads what the dK/dV kernel wrote: with a side stream it starts after it
  hipStream_t qs = (hipStream_t)stream;
  if (fork) {
    if ((e = (int)hipEventRecord((hipEvent_t)fork->fork, (hipStream_t)stream))) return e;
    if ((e = (int)hipStreamWaitEvent((hipStream_t)fork->side, (hipEvent_t)fork->fork, 0))) return e;
    qs = (hipStream_t)fork->side;
  }
  if (q.dq_qblocks == 2)
    hipLaunchKernelGGL((chunk_bwd_dq_ds_kernel<D, 2>), dim3((unsigned)nq), dim3(kNT), 0, qs, q);
  else
    hipLaunchKernelGGL((chunk_bwd_dq_ds_kernel<D, 1>), dim3((unsigned)nq), dim3(kNT), 0, qs, q);
  if ((e = (int)hipGetLastError())) return e;
  if (qs != (hipStream_t)stream && fork->join) {
    if ((e = (int)hipEventRecord((hipEvent_t)fork->join, qs))) return e;
    if ((e = (int)hipStreamWaitEvent((hipStream_t)stream, (hipEvent_t)fork->join, 0))) return e;
  }
  return 0;
}

template <int D>
int launch_bwd(const KParams& kv, const KParams& q, void* stream, const BwdFork* fork) {
  int e;
  const int64_t nkv = (int64_t)kv.B * kv.Hq * kv.tiles_per_head;
  const int64_t nq = (int64_t)q.B * q.Hq * q.tiles_per_head;
  const bool do_kv = nkv > 0 && kv.dk, do_q = nq > 0 && q.U;
  // The two kernels are independent (dK/dV and dQ); with a side stream the dQ kernel runs
  // beside the dK/dV kernel and the caller's stream waits for both.
  hipStream_t qs = (hipStream_t)stream;
  if (fork && do_kv && do_q) {
    if ((e = (int)hipEventRecord((hipEvent_t)fork->fork, (hipStream_t)stream))) return e;
    if ((e = (int)hipStreamWaitEvent((hipStream_t)fork->side, (hipEvent_t)fork->fork, 0))) return e;
    qs = (hipStream_t)fork->side;
  }
  if (do_kv) {
    if (D == 128) {
      const int64_t G = kv.q_per_wg > 1 ? kv.q_per_wg : 1;
      hipLaunchKernelGGL((chunk_bwd_kv_pp_kernel<D, false>), dim3((unsigned)(nkv / G)), dim3(kPPNT), 0,
                         (hipStream_t)stream, kv);
    } else
      hipLaunchKernelGGL((chunk_bwd_kv_kernel<D, false>), dim3((unsigned)nkv), dim3(kNT), 0, (hipStream_t)stream, kv);
    if ((e = (int)hipGetLastError())) return e;
  }
  if (do_q) {
    hipLaunchKernelGGL(chunk_bwd_q_kernel<D>, dim3((unsigned)nq), dim3(kNT), 0, qs, q);
    if ((e = (int)hipGetLastError())) return e;
  }
  if (qs != (hipStream_t)stream && fork->join) {
    if ((e = (int)hipEventRecord((hipEvent_t)fork->join, qs))) return e;
    if ((e = (int)hipStreamWaitEvent((hipStream_t)stream, (hipEvent_t)fork->join, 0))) return e;
  }
  return 0;
}

}  // namespace

int launch_chunk_bwd_bf16(const KParams& kv, const KParams& q, void* stream, const BwdFork* fork) {
  return kv.D == 128 ? launch_bwd<128>(kv, q, stream, fork) : launch_bwd<64>(kv, q, stream, fork);
}

int launch_chunk_bwd_ds_bf16(const KParams& kv, const KParams& q, void* stream, const BwdFork* fork) {
  return kv.D == 128 ? launch_bwd_ds<128>(kv, q, stream, fork) : launch_bwd_ds<64>(kv, q, stream, fork);
}

}  // namespace ra
