// Memory-bound kernels of the rank view: layout permutation, state init / merge / finalize,
// the backward's delta pre-pass, casts, fills and the staging copy.  All are HBM-bound
// streaming kernels: 16-byte vector loads/stores, one pass, no reuse.
#include "kern_common.h"

namespace ra {
namespace {

constexpr int kThreads = 256;

// ---- layout permutation ---------------------------------------------------------------------
// Row lr of the gathered tensor (ranks [rank_begin, rank_begin + rank_count), owner after
// owner) maps to a global row of the full tensor: contiguous slice r is rows
// [r*chunk, (r+1)*chunk); a zigzag slice is chunk r then chunk 2cp-1-r of 2cp equal chunks.
__global__ __launch_bounds__(kThreads) void layout_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, int zigzag,
                                                          unsigned cp, unsigned rank_begin,
                                                          unsigned chunk, unsigned crow,
                                                          unsigned rows_out, unsigned vec_shift,
                                                          unsigned long long S, int gather) {
  const unsigned idx = blockIdx.x * kThreads + threadIdx.x;
  const unsigned vecs = rows_out << vec_shift;
  if (idx >= vecs) return;
  const unsigned lr = idx >> vec_shift;
  const unsigned vec = idx & ((1u << vec_shift) - 1);
  const unsigned rank = rank_begin + lr / chunk;
  const unsigned w = lr % chunk;
  unsigned long long grow;
  if (zigzag) {
    const unsigned which = w / crow, off = w % crow;
    const unsigned c = which == 0 ? rank : 2 * cp - 1 - rank;
    grow = (unsigned long long)c * crow + off;
  } else {
    grow = (unsigned long long)rank * chunk + w;
  }
  const unsigned long long head = blockIdx.y;
  const unsigned long long full_i = ((head * S + grow) << vec_shift) + vec;
  const unsigned long long part_i = ((head * rows_out + lr) << vec_shift) + vec;
  if (gather) dst[part_i] = src[full_i];
  else dst[full_i] = src[part_i];
}

// ---- Ulysses re-shard ---------------------------------------------------------------------------
// Rows are indexed by (j, b, h', s): j < cp the shard, h' < Hh = heads / cp, s < Sc = S / cp.
// Layout 0, a sequence shard (B, heads, Sc): row ((b cp + j) Hh + h') Sc + s, i.e. head j Hh + h'.
// Layout 1, the all-to-all buffer (cp, B, Hh, Sc): row ((j B + b) Hh + h') Sc + s.
// Layout 2, a head shard (B, Hh, S): row ((b Hh + h') cp + j) Sc + s, i.e. position j Sc + s.
// In every layout the Sc rows of one (j, b, h') are contiguous, so the re-shard is a copy of
// B cp Hh blocks of Sc rows: blockIdx.y picks the block (in destination order), x runs over it.
__device__ __forceinline__ unsigned long long block_row(int layout, unsigned cp, unsigned B, unsigned Hh,
                                                        unsigned Sc, unsigned j, unsigned b, unsigned h) {
  unsigned long long r;
  if (layout == 0) r = ((unsigned long long)b * cp + j) * Hh + h;
  else if (layout == 1) r = ((unsigned long long)j * B + b) * Hh + h;
  else r = ((unsigned long long)b * Hh + h) * cp + j;
  return r * Sc;
}

__global__ __launch_bounds__(kThreads) void reshard_kernel(const u32x4* __restrict__ src,
                                                           u32x4* __restrict__ dst, int src_layout,
                                                           int dst_layout, unsigned cp, unsigned B,
                                                           unsigned Hh, unsigned Sc, unsigned vec_shift) {
  // destination block index -> (j, b, h')
  unsigned y = blockIdx.y, j, b, h;
  if (dst_layout == 0) { h = y % Hh; y /= Hh; j = y % cp; b = y / cp; }
  else if (dst_layout == 1) { h = y % Hh; y /= Hh; b = y % B; j = y / B; }
  else { j = y % cp; y /= cp; h = y % Hh; b = y / Hh; }
  const unsigned long long so = block_row(src_layout, cp, B, Hh, Sc, j, b, h) << vec_shift;
  const unsigned long long dO = block_row(dst_layout, cp, B, Hh, Sc, j, b, h) << vec_shift;
  const unsigned n = Sc << vec_shift;
  for (unsigned i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads)
    dst[dO + i] = src[so + i];
}

// ---- online-softmax state ---------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void state_init_kernel(f32x4* __restrict__ U, float* __restrict__ m,
                                                              float* __restrict__ l, long long nrows,
                                                              int vec_per_row) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i < nrows * vec_per_row) U[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (i < nrows) {
    m[i] = -__builtin_inff();
    l[i] = 0.f;
  }
}

// exp(a - b) with an empty left side (a = -inf) giving 0 and no NaN when b = -inf too.
__device__ __forceinline__ float rescale(float a, float b) {
  if (a == -__builtin_inff()) return 0.f;
  return __expf(a - b);
}

// One thread per 4 floats of a row; all threads of a row recompute the row's two factors.
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(const f32x4* __restrict__ o_part,
                                                             const float* __restrict__ lse_part,
                                                             f32x4* __restrict__ U, float* __restrict__ m,
                                                             float* __restrict__ l, long long nrows,
                                                             int vec_shift) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (nrows << vec_shift)) return;
  const long long row = i >> vec_shift;
  const float mo = m[row], lp = lse_part[row];
  const float mn = fmaxf(mo, lp);
  const float a = rescale(mo, mn), b = rescale(lp, mn);
  const f32x4 u = U[i], o = o_part[i];
  U[i] = a * u + b * o;
  // the row's scalars are updated only after every vector of the row has read them: the
  // scalar writer is the row's last vector, and the row's vectors live in one wavefront for
  // head_dim <= 256, which executes the reads above before this write.
  if ((i & ((1ll << vec_shift) - 1)) == ((1ll << vec_shift) - 1)) {
    m[row] = mn;
    l[row] = a * l[row] + b;
  }
}

// Partial state (Up, mp, lp) folded into (U, m, l); same row scheme as lse_merge_kernel.
__global__ __launch_bounds__(kThreads) void state_merge_kernel(const f32x4* __restrict__ Up,
                                                               const float* __restrict__ mp,
                                                               const float* __restrict__ lp,
                                                               f32x4* __restrict__ U, float* __restrict__ m,
                                                               float* __restrict__ l, long long nrows,
                                                               int vec_shift) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (nrows << vec_shift)) return;
  const long long row = i >> vec_shift;
  const float mo = m[row], mq = mp[row];
  const float mn = fmaxf(mo, mq);
  const float a = rescale(mo, mn), b = rescale(mq, mn);
  U[i] = a * U[i] + b * Up[i];
  if ((i & ((1ll << vec_shift) - 1)) == ((1ll << vec_shift) - 1)) {
    m[row] = mn;
    l[row] = a * l[row] + b * lp[row];
  }
}


__device__ __forceinline__ u16 f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(u16, (__bf16)f);
}

// Two running states of the same rows (from steps that ran on different streams) merged and
// finalized in one pass: the merge of state_merge_kernel followed by the division and the LSE
// of finalize_kernel, without writing the merged state back.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void merge_finalize_kernel(const f32x4* __restrict__ Ub,
                                                                  const float* __restrict__ mb,
                                                                  const float* __restrict__ lb,
                                                                  const f32x4* __restrict__ Ua,
                                                                  const float* __restrict__ ma,
                                                                  const float* __restrict__ la,
                                                                  void* __restrict__ o,
                                                                  float* __restrict__ lse,
                                                                  long long nrows, int vec_shift) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (nrows << vec_shift)) return;
  const long long row = i >> vec_shift;
  const float mo = ma[row], mq = mb[row];
  const float mn = fmaxf(mo, mq);
  const float a = rescale(mo, mn), b = rescale(mq, mn);
  const f32x4 u = a * Ua[i] + b * Ub[i];
  const float lr = a * la[row] + b * lb[row];
  const float inv = lr > 0.f ? 1.0f / lr : 0.f;
  const f32x4 v = u * inv;
  if (BF16) {
    const unsigned lo = (unsigned)f32_to_bf16_rne(v[0]) | ((unsigned)f32_to_bf16_rne(v[1]) << 16);
    const unsigned hi = (unsigned)f32_to_bf16_rne(v[2]) | ((unsigned)f32_to_bf16_rne(v[3]) << 16);
    reinterpret_cast<uint2*>(o)[i] = make_uint2(lo, hi);
  } else {
    reinterpret_cast<f32x4*>(o)[i] = v;
  }
  if ((i & ((1ll << vec_shift) - 1)) == 0) lse[row] = lr > 0.f ? mn + logf(lr) : -__builtin_inff();
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void finalize_kernel(const f32x4* __restrict__ U,
                                                            const float* __restrict__ m,
                                                            const float* __restrict__ l,
                                                            void* __restrict__ o,
                                                            float* __restrict__ lse, long long nrows,
                                                            int vec_shift) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (nrows << vec_shift)) return;
  const long long row = i >> vec_shift;
  const float lr = l[row];
  const float inv = lr > 0.f ? 1.0f / lr : 0.f;
  const f32x4 v = U[i] * inv;
  if (BF16) {
    const unsigned lo = (unsigned)f32_to_bf16_rne(v[0]) | ((unsigned)f32_to_bf16_rne(v[1]) << 16);
    const unsigned hi = (unsigned)f32_to_bf16_rne(v[2]) | ((unsigned)f32_to_bf16_rne(v[3]) << 16);
    reinterpret_cast<uint2*>(o)[i] = make_uint2(lo, hi);
  } else {
    reinterpret_cast<f32x4*>(o)[i] = v;
  }
  if ((i & ((1ll << vec_shift) - 1)) == 0)
    lse[row] = lr > 0.f ? m[row] + logf(lr) : -__builtin_inff();
}

// delta = rowsum(dO * O): 16 lanes per row, each summing D/16 products, then a 16-lane
// butterfly.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void preprocess_kernel(const void* __restrict__ o,
                                                              const void* __restrict__ dO,
                                                              float* __restrict__ delta,
                                                              long long nrows, int D) {
  const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long row = t >> 4;
  const int sub = (int)(t & 15);
  float acc = 0.f;
  if (row < nrows) {
    // D / 16 = 4 or 8 elements per lane, read as one or two 16-byte vectors (8 bytes for bf16
    // at D = 64); the tensors are 16-byte aligned and rows are D elements.
    const int per = D / 16;
    const long long base = row * D + sub * per;
    if (BF16) {
      // bf16 widens to fp32 exactly: the high half of a 32-bit word as is, the low one shifted
      const unsigned* a = reinterpret_cast<const unsigned*>(reinterpret_cast<const u16*>(o) + base);
      const unsigned* b = reinterpret_cast<const unsigned*>(reinterpret_cast<const u16*>(dO) + base);
      auto dot2 = [&](unsigned x, unsigned y) {
        acc = fmaf(__builtin_bit_cast(float, x << 16), __builtin_bit_cast(float, y << 16), acc);
        acc = fmaf(__builtin_bit_cast(float, x & 0xFFFF0000u), __builtin_bit_cast(float, y & 0xFFFF0000u), acc);
      };
      if (per == 8) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(a), y = *reinterpret_cast<const u32x4*>(b);
#pragma unroll
        for (int e = 0; e < 4; ++e) dot2(x[e], y[e]);
      } else {
        const u32x2 x = *reinterpret_cast<const u32x2*>(a), y = *reinterpret_cast<const u32x2*>(b);
        dot2(x[0], y[0]);
        dot2(x[1], y[1]);
      }
    } else {
      const f32x4* a = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(o) + base);
      const f32x4* b = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(dO) + base);
      for (int v = 0; v < per / 4; ++v) {
        const f32x4 x = a[v], y = b[v];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf(x[e], y[e], acc);
      }
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (row < nrows && sub == 0) delta[row] = acc;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void cast_kernel(const f32x4* __restrict__ src,
                                                        void* __restrict__ dst, long long nvec) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= nvec) return;
  const f32x4 v = src[i];
  if (BF16) {
    const unsigned lo = (unsigned)f32_to_bf16_rne(v[0]) | ((unsigned)f32_to_bf16_rne(v[1]) << 16);
    const unsigned hi = (unsigned)f32_to_bf16_rne(v[2]) | ((unsigned)f32_to_bf16_rne(v[3]) << 16);
    reinterpret_cast<uint2*>(dst)[i] = make_uint2(lo, hi);
  } else {
    reinterpret_cast<f32x4*>(dst)[i] = v;
  }
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(f32x4* __restrict__ dst, long long nvec) {
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride)
    dst[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Zeroes blocks x nvec 16-byte vectors spaced pitch_vec apart; grid.y walks the blocks.
__global__ __launch_bounds__(kThreads) void zero2d_kernel(u32x4* __restrict__ dst, long long pitch_vec,
                                                          long long nvec) {
  const long long b = blockIdx.y;
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride)
    dst[b * pitch_vec + i] = u32x4{0u, 0u, 0u, 0u};
}

// Fills blocks x nvec 16-byte vectors spaced pitch_vec apart with one 32-bit word.
__global__ __launch_bounds__(kThreads) void fill2d_kernel(u32x4* __restrict__ dst, long long pitch_vec,
                                                          long long nvec, unsigned word) {
  const long long b = blockIdx.y;
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride)
    dst[b * pitch_vec + i] = u32x4{word, word, word, word};
}

// Casts blocks x nvec groups of 4 fp32 values to the output dtype; source and destination
// blocks are pitch4 groups of 4 elements apart.  grid.y walks the blocks.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void cast2d_kernel(const f32x4* __restrict__ src, void* __restrict__ dst,
                                                          long long pitch4, long long nvec) {
  const long long b = blockIdx.y;
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
    const long long j = b * pitch4 + i;
    const f32x4 v = src[j];
    if (BF16) {
      const unsigned lo = (unsigned)f32_to_bf16_rne(v[0]) | ((unsigned)f32_to_bf16_rne(v[1]) << 16);
      const unsigned hi = (unsigned)f32_to_bf16_rne(v[2]) | ((unsigned)f32_to_bf16_rne(v[3]) << 16);
      reinterpret_cast<uint2*>(dst)[j] = make_uint2(lo, hi);
    } else {
      reinterpret_cast<f32x4*>(dst)[j] = v;
    }
  }
}

// blocks x (block_bytes / 16) vectors; grid.y walks the blocks.
__global__ __launch_bounds__(kThreads) void copy2d_kernel(const u32x4* __restrict__ src,
                                                          long long src_pitch_vec,
                                                          u32x4* __restrict__ dst,
                                                          long long dst_pitch_vec, long long nvec) {
  const long long b = blockIdx.y;
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride)
    dst[b * dst_pitch_vec + i] = src[b * src_pitch_vec + i];
}

inline unsigned blocks_for(long long n) { return (unsigned)((n + kThreads - 1) / kThreads); }

inline int log2i(long long v) {
  int s = 0;
  while ((1ll << s) < v) ++s;
  return s;
}

}  // namespace

int launch_layout(const Shape& s, int32_t rank_begin, int32_t rank_count, int64_t heads,
                  const void* src, void* dst, bool gather, void* stream) {
  const long long row_vec = s.D * s.esize / 16;  // power of two (D in {64,128}, esize in {2,4})
  const unsigned rows_out = (unsigned)(rank_count * s.chunk);
  const long long total = (long long)rows_out * row_vec;
  const long long bh = s.B * heads;
  if (total == 0 || bh == 0) return 0;
  dim3 grid(blocks_for(total), (unsigned)bh);
  hipLaunchKernelGGL(layout_kernel, grid, dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst, s.layout == RA_ZIGZAG ? 1 : 0,
                     (unsigned)s.cp, (unsigned)rank_begin, (unsigned)s.chunk, (unsigned)s.crow,
                     rows_out, (unsigned)log2i(row_vec), (unsigned long long)s.S, gather ? 1 : 0);
  return (int)hipGetLastError();
}

int launch_state_merge(int64_t nrows, int64_t D, const float* Up, const float* mp, const float* lp,
                       float* U, float* m, float* l, void* stream) {
  const int vs = log2i(D / 4);
  const long long n = (long long)nrows << vs;
  if (n == 0) return 0;
  hipLaunchKernelGGL(state_merge_kernel, dim3(blocks_for(n)), dim3(kThreads), 0, (hipStream_t)stream,
                     (const f32x4*)Up, mp, lp, (f32x4*)U, m, l, (long long)nrows, vs);
  return (int)hipGetLastError();
}

int launch_reshard(const Shape& s, int32_t step, int64_t heads, const void* src, void* dst, void* stream) {
  static const int kSrc[4] = {0, 1, 2, 1}, kDst[4] = {1, 2, 1, 0};
  const long long row_vec = s.D * s.esize / 16;
  const long long Sc = s.S / s.cp, Hh = heads / s.cp;
  const long long nblk = s.B * s.cp * Hh;
  const long long per = Sc * row_vec;
  if (nblk == 0 || per == 0) return 0;
  long long gx = (per + kThreads - 1) / kThreads;
  const long long cap = nblk >= 512 ? 4 : 2048 / nblk;  // enough workgroups to fill the chip
  if (gx > cap) gx = cap < 1 ? 1 : cap;
  hipLaunchKernelGGL(reshard_kernel, dim3((unsigned)gx, (unsigned)nblk), dim3(kThreads), 0,
                     (hipStream_t)stream, (const u32x4*)src, (u32x4*)dst, kSrc[step], kDst[step],
                     (unsigned)s.cp, (unsigned)s.B, (unsigned)Hh, (unsigned)Sc, (unsigned)log2i(row_vec));
  return (int)hipGetLastError();
}

int launch_state_init(int64_t nrows, int64_t D, float* U, float* m, float* l, void* stream) {
  const long long nvec = nrows * (D / 4);
  if (nvec == 0) return 0;
  hipLaunchKernelGGL(state_init_kernel, dim3(blocks_for(nvec)), dim3(kThreads), 0,
                     (hipStream_t)stream, (f32x4*)U, m, l, (long long)nrows, (int)(D / 4));
  return (int)hipGetLastError();
}

int launch_lse_merge(int64_t nrows, int64_t D, const float* o_part, const float* lse_part,
                     float* U, float* m, float* l, void* stream) {
  const int vs = log2i(D / 4);
  const long long n = (long long)nrows << vs;
  if (n == 0) return 0;
  hipLaunchKernelGGL(lse_merge_kernel, dim3(blocks_for(n)), dim3(kThreads), 0, (hipStream_t)stream,
                     (const f32x4*)o_part, lse_part, (f32x4*)U, m, l, (long long)nrows, vs);
  return (int)hipGetLastError();
}

int launch_fwd_finalize(int64_t nrows, int64_t D, int32_t dtype, const float* U, const float* m,
                        const float* l, void* o, float* lse, void* stream) {
  const int vs = log2i(D / 4);
  const long long n = (long long)nrows << vs;
  if (n == 0) return 0;
  if (dtype == RA_BF16)
    hipLaunchKernelGGL(finalize_kernel<true>, dim3(blocks_for(n)), dim3(kThreads), 0,
                       (hipStream_t)stream, (const f32x4*)U, m, l, o, lse, (long long)nrows, vs);
  else
    hipLaunchKernelGGL(finalize_kernel<false>, dim3(blocks_for(n)), dim3(kThreads), 0,
                       (hipStream_t)stream, (const f32x4*)U, m, l, o, lse, (long long)nrows, vs);
  return (int)hipGetLastError();
}

int launch_merge_finalize(int64_t nrows, int64_t D, int32_t dtype, const float* Ub, const float* mb,
                          const float* lb, const float* Ua, const float* ma, const float* la, void* o,
                          float* lse, void* stream) {
  const int vs = log2i(D / 4);
  const long long n = (long long)nrows << vs;
  if (n == 0) return 0;
  if (dtype == RA_BF16)
    hipLaunchKernelGGL(merge_finalize_kernel<true>, dim3(blocks_for(n)), dim3(kThreads), 0, (hipStream_t)stream,
                       (const f32x4*)Ub, mb, lb, (const f32x4*)Ua, ma, la, o, lse, (long long)nrows, vs);
  else
    hipLaunchKernelGGL(merge_finalize_kernel<false>, dim3(blocks_for(n)), dim3(kThreads), 0, (hipStream_t)stream,
                       (const f32x4*)Ub, mb, lb, (const f32x4*)Ua, ma, la, o, lse, (long long)nrows, vs);
  return (int)hipGetLastError();
}

int launch_bwd_preprocess(int64_t nrows, int64_t D, int32_t dtype, const void* o, const void* dO,
                          float* delta, void* stream) {
  const long long n = nrows * 16;
  if (n == 0) return 0;
  if (dtype == RA_BF16)
    hipLaunchKernelGGL(preprocess_kernel<true>, dim3(blocks_for(n)), dim3(kThreads), 0,
                       (hipStream_t)stream, o, dO, delta, (long long)nrows, (int)D);
  else
    hipLaunchKernelGGL(preprocess_kernel<false>, dim3(blocks_for(n)), dim3(kThreads), 0,
                       (hipStream_t)stream, o, dO, delta, (long long)nrows, (int)D);
  return (int)hipGetLastError();
}

int launch_cast_from_f32(int64_t n, int32_t dtype, const float* src, void* dst, void* stream) {
  const long long nvec = n / 4;
  if (nvec == 0) return 0;
  if (dtype == RA_BF16)
    hipLaunchKernelGGL(cast_kernel<true>, dim3(blocks_for(nvec)), dim3(kThreads), 0,
                       (hipStream_t)stream, (const f32x4*)src, dst, nvec);
  else
    hipLaunchKernelGGL(cast_kernel<false>, dim3(blocks_for(nvec)), dim3(kThreads), 0,
                       (hipStream_t)stream, (const f32x4*)src, dst, nvec);
  return (int)hipGetLastError();
}

// Grid width for a blocks x nvec 2-D pass: enough workgroups to fill the chip in total.
inline long long grid2d_x(long long nvec, long long blocks) {
  long long gx = (nvec + kThreads - 1) / kThreads;
  const long long cap = blocks >= 2048 ? 1 : 2048 / blocks;
  return gx > cap ? cap : gx;
}

int launch_zero2d(void* dst, int64_t pitch_bytes, int64_t block_bytes, int64_t blocks, void* stream) {
  const long long nvec = block_bytes / 16;
  if (nvec == 0 || blocks == 0) return 0;
  hipLaunchKernelGGL(zero2d_kernel, dim3((unsigned)grid2d_x(nvec, blocks), (unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, (u32x4*)dst, (long long)(pitch_bytes / 16), nvec);
  return (int)hipGetLastError();
}

int launch_fill2d(void* dst, int64_t pitch_bytes, int64_t block_bytes, int64_t blocks, uint32_t word,
                  void* stream) {
  const long long nvec = block_bytes / 16;
  if (nvec == 0 || blocks == 0) return 0;
  hipLaunchKernelGGL(fill2d_kernel, dim3((unsigned)grid2d_x(nvec, blocks), (unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, (u32x4*)dst, (long long)(pitch_bytes / 16), nvec, (unsigned)word);
  return (int)hipGetLastError();
}

int launch_cast2d(const float* src, void* dst, int64_t pitch, int64_t block, int64_t blocks, int32_t dtype,
                  void* stream) {
  const long long nvec = block / 4;
  if (nvec == 0 || blocks == 0) return 0;
  const dim3 grid((unsigned)grid2d_x(nvec, blocks), (unsigned)blocks);
  if (dtype == RA_BF16)
    hipLaunchKernelGGL(cast2d_kernel<true>, grid, dim3(kThreads), 0, (hipStream_t)stream, (const f32x4*)src, dst,
                       (long long)(pitch / 4), nvec);
  else
    hipLaunchKernelGGL(cast2d_kernel<false>, grid, dim3(kThreads), 0, (hipStream_t)stream, (const f32x4*)src, dst,
                       (long long)(pitch / 4), nvec);
  return (int)hipGetLastError();
}

int launch_fill_zero(int64_t n_floats, float* dst, void* stream) {
  const long long nvec = n_floats / 4;
  if (nvec == 0) return 0;
  long long nb = (nvec + kThreads - 1) / kThreads;
  if (nb > 8192) nb = 8192;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)nb), dim3(kThreads), 0, (hipStream_t)stream,
                     (f32x4*)dst, nvec);
  return (int)hipGetLastError();
}

int launch_copy2d(const void* src, int64_t src_pitch, void* dst, int64_t dst_pitch,
                  int64_t block_bytes, int64_t blocks, void* stream) {
  const long long nvec = block_bytes / 16;
  if (nvec == 0 || blocks == 0) return 0;
  long long gx = (nvec + kThreads - 1) / kThreads;
  const long long cap = blocks >= 256 ? 1 : 2048 / blocks;
  if (gx > cap) gx = cap < 1 ? 1 : cap;
  hipLaunchKernelGGL(copy2d_kernel, dim3((unsigned)gx, (unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, (const u32x4*)src, (long long)(src_pitch / 16),
                     (u32x4*)dst, (long long)(dst_pitch / 16), nvec);
  return (int)hipGetLastError();
}

}  // namespace ra
