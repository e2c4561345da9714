// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "ra_internal.h"

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v_mfma_f32_32x32x16_bf16: A is 32(M) x 16(K), B is 16(K) x 32(N), C/D 32 x 32 fp32.
// Lane l supplies A row (l % 32) and B column (l % 32), 8 K-values each (the K index of
// element e in lane half h = l / 32 is the same for A and B, so the contraction is correct
// for any consistent K order).  The accumulator register r = 4*j + i (j, i in 0..3) of lane l
// holds C[8*j + 4*(l/32) + i][l % 32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row order used when an MFMA *output* row index must become a K index of a following
// MFMA.  Output row rho = 8j + 4h + i lives in lane half h, register 4j + i.  Feeding A row
// rho with source row perm32(rho) makes lane half h hold source rows 16*c + 8*h + e
// (e = 0..7) in registers 8*c + e, c = 0, 1: exactly the 8-consecutive K rows that a
// 32x32x16 operand wants from that lane half.
__device__ __forceinline__ int perm32(int rho) {
  const int j = rho >> 3, h = (rho >> 2) & 1, i = rho & 3;
  return ((j >> 1) << 4) | (h << 3) | ((j & 1) << 2) | i;
}

// Source row (0..31) held in accumulator register r of lane half h after perm32.
__device__ __forceinline__ int perm_reg_row(int r, int h) {
  const int j = r >> 2, i = r & 3;
  return ((j >> 1) << 4) | (h << 3) | ((j & 1) << 2) | i;
}

// Plain (unpermuted) output row of accumulator register r in lane half h.
__device__ __forceinline__ int out_row(int r, int h) { return ((r >> 2) << 3) | (h << 2) | (r & 3); }

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
  return r;
}

// Gathers 8 bf16 values at stride `pitch` elements (one column of 8 consecutive rows).
__device__ __forceinline__ bf16x8 gather8(const u16* p, int pitch) {
  u32x4 w;
  w[0] = (unsigned)p[0] | ((unsigned)p[pitch] << 16);
  w[1] = (unsigned)p[2 * pitch] | ((unsigned)p[3 * pitch] << 16);
  w[2] = (unsigned)p[4 * pitch] | ((unsigned)p[5 * pitch] << 16);
  w[3] = (unsigned)p[6 * pitch] | ((unsigned)p[7 * pitch] << 16);
  return __builtin_bit_cast(bf16x8, w);
}

// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, output lane i, element e is
// element (i % 4) of the 8-byte chunk addressed by lane 4*e + i/4 of the group.  Pointing lane
// j of a group at row (k0 + j/4), column (m0 + 4*(j%4)) of a row-major tile therefore hands
// lane i the column entries T[k0 + e][m0 + i], e = 0..3: a transposed read.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;
typedef __attribute__((address_space(3))) u16 lds_u16_t;

__device__ __forceinline__ v4i16 ds_read_tr16(const u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)((lds_u16_t*)(p)));
}

// LDS tiles are stored unpadded with their 16-byte chunks XOR-swizzled per row: chunk c of
// row r lives at chunk position c ^ swz(r).  The LDS has 64 banks of 4 bytes; a 16-byte read
// serves 16 lanes per clock and an 8-byte read 32 lanes per clock (both measured).  The swizzle
// below keeps three patterns conflict-free at once: 16 lanes reading one chunk of 16 different
// rows (row operands, in perm32 or natural order), 32 lanes doing ds_read_b64_tr_b16 over 4
// aligned rows x 4 chunks, and lane-linear 16-byte writes (direct global -> LDS loads).  Rows
// hold 128 bf16 (16 chunks) or 64 bf16 (8 chunks).
__device__ __forceinline__ int swz(int r, int rowlen) {
  return rowlen == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

__device__ __forceinline__ int swz_off(int r, int col, int rowlen) {
  return r * rowlen + (((col >> 3) ^ swz(r, rowlen)) << 3) + (col & 7);
}

// Row operands: lane reads T[r][16*kk + 8*hh .. +8] (r fixed per lane).  The chunk is
// 2*kk + hh = (2*kk) ^ hh, so its position is (2*kk) ^ (hh ^ swz(r)): one XOR-add per read.
struct RowAddr {
  int base, g8;
};

__device__ __forceinline__ RowAddr make_row_addr(int r, int hh, int rowlen) {
  RowAddr a;
  a.base = r * rowlen;
  a.g8 = (hh ^ swz(r, rowlen)) << 3;
  return a;
}

__device__ __forceinline__ bf16x8 row_operand(const u16* T, const RowAddr& a, int kk) {
  return *reinterpret_cast<const bf16x8*>(T + a.base + ((16 * kk) ^ a.g8));
}

// Transposed operands (ds_read_b64_tr_b16): lane l receives T[k0 + 8*(l/32) + e][m0 + l%32],
// e = 0..7, with k0 = 16*c and m0 = 32*db.  Lane j of 16-lane group g addresses row
// 16c + 8*(g>>1) + (j>>2) (+4 for the second read), column 32*db + 16*(g&1) + 4*(j&3).  The
// swizzle of those rows does not depend on c, so one address per (db, half) is precomputed and
// c enters as an immediate offset.
struct TrAddr {
  int lo, hi;  // addresses for db = 0; db enters by XOR into element bits 5..6
};

__device__ __forceinline__ TrAddr make_tr_addr(int lane, int rowlen) {
  TrAddr a;
  const int j = lane & 15, g = lane >> 4;
  const int r = 8 * (g >> 1) + (j >> 2);
  const int t = 2 * (g & 1) + ((j & 3) >> 1);
  const int within = 4 * (j & 1);
  a.lo = r * rowlen + ((t ^ swz(r, rowlen)) << 3) + within;
  a.hi = (r + 4) * rowlen + ((t ^ swz(r + 4, rowlen)) << 3) + within;
  return a;
}

__device__ __forceinline__ bf16x8 tr_operand(const u16* T, const TrAddr& a, int rowlen, int c, int db) {
  const int off = 16 * c * rowlen;
  const v4i16 lo = ds_read_tr16(T + (a.lo ^ (db << 5)) + off);
  const v4i16 hi = ds_read_tr16(T + (a.hi ^ (db << 5)) + off);
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, w);
}

// Index of the calling wavefront in its workgroup, as a wave-uniform (scalar) value: derived
// from threadIdx it would be treated as per-lane, and everything computed from it would take
// vector registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Sum / max of a value and its partner 32 lanes away, every lane getting the result, without
// going through LDS: v_permlane32_swap (gfx950) leaves, in each lane, v of lane l and of lane
// l ^ 32 in its two outputs.
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Direct global -> LDS loads (global_load_lds_dwordx4): every lane copies 16 bytes from its own
// global address to LDS at dst + 16 * lane, where dst must be wave-uniform.  The data does not
// pass through VGPRs; completion is counted by vmcnt, so wait_vmem() followed by a barrier makes
// a tile visible to the workgroup.
typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

__device__ __forceinline__ void g2lds16(const void* src, void* dst_wave) {
  __builtin_amdgcn_global_load_lds((gvoid_t*)src, (lvoid_t*)dst_wave, 16, 0, 0);
}

// The same with the non-temporal cache policy, for data read once (streamed past the caches).
__device__ __forceinline__ void g2lds16_nt(const void* src, void* dst_wave) {
  __builtin_amdgcn_global_load_lds((gvoid_t*)src, (lvoid_t*)dst_wave, 16, 0, 2);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Issues the loads of a swizzled ROWS x D bf16 tile whose row r comes from global row
// g + min(r, valid_rows - 1) (valid_rows >= 1): rows past the end repeat the last valid row, so
// every value is finite and the caller masks them out.  One wave instruction fills 1 KB of LDS,
// i.e. 64/(D/8) whole rows; lane i lands at physical chunk i % (D/8) of its row and therefore
// fetches the logical chunk stored there, (i % (D/8)) ^ swz(row).
template <int D, int ROWS, int NWAVES>
__device__ __forceinline__ void issue_tile(const u16* __restrict__ g, int64_t valid_rows, u16* tile) {
  constexpr int CH = D / 8;
  constexpr int RPI = 64 / CH;
  constexpr int NI = ROWS / RPI;
  const int lane = threadIdx.x & 63, w = wave_id();
  static_assert(NI % NWAVES == 0, "tile rows must split evenly over the wavefronts");
  const int last = (int)(valid_rows < ROWS ? valid_rows : ROWS) - 1;
#pragma unroll
  for (int k = 0; k < NI / NWAVES; ++k) {
    const int i = k * NWAVES + w;
    const int row = i * RPI + lane / CH;
    const int c = (lane % CH) ^ swz(row, D);
    const unsigned off = (unsigned)((row < last ? row : last) * D + c * 8) * 2u;  // bytes
    g2lds16(reinterpret_cast<const char*>(g) + off, tile + i * 512);
  }
}

constexpr int kBufRsrcWord3 = 0x00020000;  // buffer resource word 3 (gfx9 family): raw 32-bit data

// Barrier between two phases of a ping-pong kernel (two teams of wavefronts alternating matrix
// and vector phases).  The only data the wavefronts share inside the phase loop are LDS tiles
// written by direct loads whose issuer waits for them (vmcnt) before the barrier that publishes
// them, LDS values written by ds stores, and LDS tiles read by operand loads that must be done
// before a later phase overwrites them: this waits for the wavefront's LDS operations only, not for
// its global stores or the direct loads it has in flight (which a fence-carrying barrier would).
// The empty asm with a memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

struct TileRef {
  int b, hq, g, range;
  int64_t row0;  // first outer row of the tile (in the operand's rows)
  int nrows;     // rows of the tile inside its range (<= tile rows)
};

// Maps the hardware workgroup index to (batch, head, tile).  The logical order is batch, head
// (kv-head major), then tiles heaviest first.  Workgroup i is dispatched to XCD i % 8.  When the
// heads split evenly over the 8 XCDs, each XCD is given one contiguous run of the logical order
// (whole heads), so that the query heads sharing a key/value head meet in the same L2.
// Otherwise a run would end inside a head, and with a causal diagonal the XCD holding a head's
// heavy tiles would work far longer than the one holding its light tiles: the logical order is
// then dealt out round-robin (logical index = hardware index), which gives every XCD every
// eighth tile of each head.
// With group > 1 a workgroup takes `group` consecutive query heads (which share a key/value
// head): the heads counted here are the groups, and r.hq is the group's first query head.
__device__ __forceinline__ TileRef map_tile(const KParams& p, int64_t tile_rows, int group = 1) {
  const int64_t nblk = (int64_t)gridDim.x;
  const int64_t bid = (int64_t)blockIdx.x;
  const int heads = p.Hq / group;
  int64_t logical = bid;
  if ((((int64_t)p.B * heads) & 7) == 0) {
    const int64_t x = bid & 7, k = bid >> 3;
    const int64_t q = nblk >> 3, rem = nblk & 7;
    logical = x * q + (x < rem ? x : rem) + k;
  }
  const int64_t head = logical / p.tiles_per_head;
  int64_t t = logical - head * p.tiles_per_head;
  TileRef r;
  r.b = (int)(head / heads);
  r.hq = (int)(head - (int64_t)r.b * heads) * group;
  r.g = r.hq / p.n_rep;
  int ri = 0;
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (i < p.nranges && t >= p.ranges[i].tile0) ri = i;
  const KRange& R = p.ranges[ri];
  t -= R.tile0;
  if (R.reverse) t = R.ntiles - 1 - t;
  r.range = ri;
  r.row0 = R.row0 + t * tile_rows;
  const int64_t left = R.len - t * tile_rows;
  r.nrows = (int)(left < tile_rows ? left : tile_rows);
  return r;
}

}  // namespace ra
