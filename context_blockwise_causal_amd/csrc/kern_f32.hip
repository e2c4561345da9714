// fp32 chunk kernels: the correctness path for fp32 inputs (small problems), fp32 end to
// end with accurate expf.  One wavefront per query row; a lane owns one key of each 64-key
// block for the scores and one or two head-dim columns of the row's output.
//
// Same method as the bf16 kernels (lecture note "上下文并行", "朴素 Ring Attention": safe
// softmax with the per-block online update; "Feat: Context Parallel" 主要改动: recompute
// backward), without MFMA.
#include "kern_common.h"

namespace ra {
namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int D>
__global__ __launch_bounds__(64) void chunk_fwd_f32_kernel(const KParams p) {
  constexpr int PER = D / 64;
  __shared__ float qs[D];
  const TileRef tr = map_tile(p, 1);
  const int lane = threadIdx.x;
  const int64_t qrow = ((int64_t)tr.b * p.Hq + tr.hq) * p.q_head_rows + tr.row0;
  const int64_t kvhead = ((int64_t)tr.b * p.Hkv + tr.g) * p.kv_head_rows;
  const float* Q = reinterpret_cast<const float*>(p.q);
  const float* K = reinterpret_cast<const float*>(p.k) + kvhead * D;
  const float* V = reinterpret_cast<const float*>(p.v) + kvhead * D;
  for (int d = lane; d < D; d += 64) qs[d] = Q[qrow * D + d];
  __syncthreads();

  float m = -__builtin_inff(), l = 0.f;
  float o[PER];
#pragma unroll
  for (int t = 0; t < PER; ++t) o[t] = 0.f;
  if (!p.fresh) {
    m = p.m[qrow];
    l = p.l[qrow];
#pragma unroll
    for (int t = 0; t < PER; ++t) o[t] = p.U[qrow * D + lane + 64 * t];
  }

  const KRange& R = p.ranges[tr.range];
  for (int pi = 0; pi < R.npairs; ++pi) {
    const KPair pr = p.pairs[R.pair[pi]];
    const int64_t iq = tr.row0 - pr.q_row0;
    int64_t key_end = pr.kv_len;
    if (pr.mask == RA_MASK_DIAG && iq + 1 < key_end) key_end = iq + 1;
    const float* Kp = K + pr.kv_row0 * D;
    const float* Vp = V + pr.kv_row0 * D;
    // window / attention chunk: the row's lowest visible key (pair-local)
    int64_t key_begin = 0;
    if (p.window > 0 || p.attn_chunk > 0) {
      const int64_t lo = lowest_key(pr.q_pos0 + iq, p.window, p.attn_chunk) - pr.kv_pos0;
      key_begin = lo > 0 ? lo : 0;
    }
    for (int64_t k0 = key_begin; k0 < key_end; k0 += 64) {
      const int64_t j = k0 + lane;
      float s = -__builtin_inff();
      if (j < key_end) {
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc = fmaf(qs[d], Kp[j * D + d], acc);
        s = acc * p.scale;
      }
      const float mt = wave_max(s);
      const float mn = fmaxf(m, mt);
      const float alpha = m == -__builtin_inff() ? 0.f : expf(m - mn);
      const float pj = j < key_end ? expf(s - mn) : 0.f;
      l = l * alpha + wave_sum(pj);
#pragma unroll
      for (int t = 0; t < PER; ++t) o[t] *= alpha;
      const int nk = (int)(key_end - k0 < 64 ? key_end - k0 : 64);
      for (int jj = 0; jj < nk; ++jj) {
        const float pv = __shfl(pj, jj);
#pragma unroll
        for (int t = 0; t < PER; ++t) o[t] = fmaf(pv, Vp[(k0 + jj) * D + lane + 64 * t], o[t]);
      }
      m = mn;
    }
  }
#pragma unroll
  for (int t = 0; t < PER; ++t) p.U[qrow * D + lane + 64 * t] = o[t];
  if (lane == 0) {
    p.m[qrow] = m;
    p.l[qrow] = l;
  }
}

// Backward, one wavefront per query row: dq of the row is owned by the wavefront (added to
// the accumulator once); dk/dv rows are shared by every query row and head of the group and
// are added with fp32 atomics.
template <int D>
__global__ __launch_bounds__(64) void chunk_bwd_f32_kernel(const KParams p) {
  constexpr int PER = D / 64;
  __shared__ float qs[D], dos[D];
  const TileRef tr = map_tile(p, 1);
  const int lane = threadIdx.x;
  const int64_t qrow = ((int64_t)tr.b * p.Hq + tr.hq) * p.q_head_rows + tr.row0;
  const int64_t kvhead = ((int64_t)tr.b * p.Hkv + tr.g) * p.kv_head_rows;
  const int64_t dkvhead = ((int64_t)tr.b * p.Hkv + tr.g) * p.dkv_head_rows;
  const float* Q = reinterpret_cast<const float*>(p.q);
  const float* dO = reinterpret_cast<const float*>(p.dO);
  const float* K = reinterpret_cast<const float*>(p.k) + kvhead * D;
  const float* V = reinterpret_cast<const float*>(p.v) + kvhead * D;
  for (int d = lane; d < D; d += 64) {
    qs[d] = Q[qrow * D + d];
    dos[d] = dO[qrow * D + d];
  }
  __syncthreads();
  const float lse = p.lse[qrow], dl = p.delta[qrow];
  float dq[PER];
#pragma unroll
  for (int t = 0; t < PER; ++t) dq[t] = 0.f;

  const KRange& R = p.ranges[tr.range];
  for (int pi = 0; pi < R.npairs; ++pi) {
    const KPair pr = p.pairs[R.pair[pi]];
    const int64_t iq = tr.row0 - pr.q_row0;
    int64_t key_end = pr.kv_len;
    if (pr.mask == RA_MASK_DIAG && iq + 1 < key_end) key_end = iq + 1;
    const float* Kp = K + pr.kv_row0 * D;
    const float* Vp = V + pr.kv_row0 * D;
    float* dKp = p.dk + (dkvhead + pr.kv_row0) * D;
    float* dVp = p.dv + (dkvhead + pr.kv_row0) * D;
    int64_t key_begin = 0;
    if (p.window > 0 || p.attn_chunk > 0) {
      const int64_t lo = lowest_key(pr.q_pos0 + iq, p.window, p.attn_chunk) - pr.kv_pos0;
      key_begin = lo > 0 ? lo : 0;
    }
    for (int64_t k0 = key_begin; k0 < key_end; k0 += 64) {
      const int64_t j = k0 + lane;
      float pj = 0.f, dsj = 0.f;
      if (j < key_end) {
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
          s = fmaf(qs[d], Kp[j * D + d], s);
          dp = fmaf(dos[d], Vp[j * D + d], dp);
        }
        pj = expf(s * p.scale - lse);
        dsj = pj * (dp - dl);
        if (p.dk) {
          for (int d = 0; d < D; ++d) {
            atomicAdd(dKp + j * D + d, p.scale * dsj * qs[d]);
            atomicAdd(dVp + j * D + d, pj * dos[d]);
          }
        }
      }
      const int nk = (int)(key_end - k0 < 64 ? key_end - k0 : 64);
      for (int jj = 0; jj < nk; ++jj) {
        const float dsv = __shfl(dsj, jj);
#pragma unroll
        for (int t = 0; t < PER; ++t) dq[t] = fmaf(dsv, Kp[(k0 + jj) * D + lane + 64 * t], dq[t]);
      }
    }
  }
  if (p.U) {
#pragma unroll
    for (int t = 0; t < PER; ++t) p.U[qrow * D + lane + 64 * t] += p.scale * dq[t];
  }
}

template <int D>
int launch_f32(const KParams& kp, bool bwd, void* stream) {
  const int64_t nblk = (int64_t)kp.B * kp.Hq * kp.tiles_per_head;
  if (nblk == 0) return 0;
  if (bwd)
    hipLaunchKernelGGL(chunk_bwd_f32_kernel<D>, dim3((unsigned)nblk), dim3(64), 0,
                       (hipStream_t)stream, kp);
  else
    hipLaunchKernelGGL(chunk_fwd_f32_kernel<D>, dim3((unsigned)nblk), dim3(64), 0,
                       (hipStream_t)stream, kp);
  return (int)hipGetLastError();
}

}  // namespace

int launch_chunk_fwd_f32(const KParams& kp, void* stream) {
  return kp.D == 128 ? launch_f32<128>(kp, false, stream) : launch_f32<64>(kp, false, stream);
}

int launch_chunk_bwd_f32(const KParams& kp, void* stream) {
  return kp.D == 128 ? launch_f32<128>(kp, true, stream) : launch_f32<64>(kp, true, stream);
}

}  // namespace ra
