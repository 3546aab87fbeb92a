// Device helpers shared by the MFMA kernels of k_gemm2.hip and k_block.hip:
// buffer resources, vmcnt waits, direct-to-LDS tile loaders with their XOR
// swizzles, and the fragment reads that match them.  Internal to libpoetx.
#pragma once

#include <type_traits>

#include "kernels.h"

namespace poetx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) void lds_void;

namespace {

constexpr uint32_t RSRC_DW3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  uint32_t n = bytes > 0x7fffffff ? 0x7fffffffu : (uint32_t)(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, (int)RSRC_DW3);
}

// s_waitcnt with vmcnt = N (expcnt, lgkmcnt left at their maxima); gfx9 encoding.
template <int N>
__device__ inline void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// k-contiguous tile [R][BKT] bf16 (BKT = 32, 64 or more -> 64-, 128-, ...-byte rows).  The
// 16-byte chunk c of row r sits at c ^ kc_key(r).  The LDS serves a ds_read_b128 sixteen
// lanes at a time from 64 four-byte banks (256 bytes); a fragment read puts 16 consecutive
// rows in those lanes, one chunk each, so the key spreads them over all sixteen 16-byte
// bank groups: rows of 128 bytes share a 256-byte window in pairs and are keyed by their
// row index halved, rows of 64 bytes in fours (index quartered), rows of 256 bytes and
// more one to a window (keyed by the row index itself).  Measured with fragment-shaped
// reads: keyed for 32 banks instead (r & 7), 16-row reads lost 5% and 32-row reads 28%
// of the LDS rate.  One wave instruction (64 lanes x 16 B) fills 1 KB = 64 / (BKT/8) rows.
#ifndef POETX_KC_KEY32
template <int BKT>
__device__ inline int kc_key(int r) { return BKT >= 128 ? (r & 15) : BKT == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
#else
template <int BKT>
__device__ inline int kc_key(int r) { return BKT >= 64 ? (r & 7) : ((r >> 1) & 3); }
#endif

template <int R, int NW, int BKT, int WOFF = 0>
struct LoaderKC {
  static constexpr int CR = BKT / 8;        // chunks per row
  static constexpr int RPI = 64 / CR;       // rows per wave instruction
  static constexpr int INSTR = R / RPI / NW;
  int voff[INSTR];  // per-lane byte offset of its 16-byte chunk at k0 = 0
  __device__ void init(int64_t ld, int64_t row0) {
    const int w = (threadIdx.x >> 6) - WOFF, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      const int row = (w * INSTR + i) * RPI + l / CR;
      const int lchunk = (l % CR) ^ kc_key<BKT>(row);
      voff[i] = (int)(((row0 + row) * ld + lchunk * 8) * 2);
    }
  }
  // k0 is added to the per-lane offset: the raw-buffer range check covers only the
  // lane offset (not soffset), and rows past the valid extent must read as zero.
  // the wave index through readfirstlane: the LDS destination (M0) is then known to be
  // uniform, and no operand of the loads needs a waterfall loop
  __device__ void issue(__amdgpu_buffer_rsrc_t rs, int64_t k0, int64_t ld, bf16_t *tile) const {
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) - WOFF;
    const int kb = (int)(k0 * 2);
#pragma unroll
    for (int i = 0; i < INSTR; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(tile + (w * INSTR + i) * RPI * BKT), 16,
                                               voff[i] + kb, 0, 0, 0);
  }
  // the i-th of the INSTR loads alone (a wave index the compiler knows to be uniform)
  __device__ void issue_one(__amdgpu_buffer_rsrc_t rs, int64_t k0, bf16_t *tile, int i) const {
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) - WOFF;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(tile + (w * INSTR + i) * RPI * BKT), 16,
                                             voff[i] + (int)(k0 * 2), 0, 0, 0);
  }
};

// k-major tile [BKT][C] bf16 = 2C-byte rows; chunk c of row r sits at c ^ (km_key(r) << 1):
// 32-byte blocks rotate with row bits {0, 1, 3}, so the 8 rows that two 16-lane groups of
// one ds_read_b64_tr_b16 touch (k .. k+3 and k+8 .. k+11) land in 8 different 32-byte
// bank groups.  One wave instruction fills 1 KB.
__device__ inline int km_key(int r) { return (r & 3) | ((r >> 1) & 4); }
// chunk XOR for a k-major tile of C columns (C/8 chunks per row; narrow tiles keep
// only the bits that stay inside the row)
template <int C>
__device__ inline int km_xor(int r) { return (km_key(r) << 1) & (C / 8 - 1); }
// int8 k-major tiles are read 8 consecutive rows at a time (ds_read_b64_tr_b8), one
// 16-byte chunk per row: rotating the chunk by the row's low three bits puts those 8
// chunks on 8 different 16-byte bank groups.
template <int C, bool I8>
__device__ inline int km_xor_sel(int r) { return I8 ? (r & 7) : km_xor<C>(r); }

// I8: the tile holds int8 rows of 2C bytes, loaded as if they were C bf16 values.
template <int C, int NW, int BKT, int WOFF = 0, bool I8 = false>
struct LoaderKM {
  static constexpr int CH = C / 8;     // 16-byte chunks per row
  static constexpr int RPI = 64 / CH;  // rows per wave instruction
  static constexpr int INSTR = BKT / RPI / NW;
  int voff[INSTR];
  __device__ void init(int64_t ld, int64_t col0) {
    const int w = (threadIdx.x >> 6) - WOFF, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      const int row = (w * INSTR + i) * RPI + l / CH;
      const int lchunk = (l % CH) ^ km_xor_sel<C, I8>(row);
      voff[i] = (int)((row * ld + col0 + lchunk * 8) * 2);
    }
  }
  __device__ void issue(__amdgpu_buffer_rsrc_t rs, int64_t k0, int64_t ld, bf16_t *tile) const {
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) - WOFF;
    const int kb = (int)(k0 * ld * 2);
#pragma unroll
    for (int i = 0; i < INSTR; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(tile + (w * INSTR + i) * RPI * C), 16,
                                               voff[i] + kb, 0, 0, 0);
  }
};

// MFMA operand fragment (lane l: 8 consecutive k of row/column l % 16).
template <int BKT>
__device__ inline bf16x8 frag_kc(const bf16_t *t, int r0, int ks) {
  const int l = threadIdx.x & 63, row = r0 + (l & 15);
  const int pchunk = ((ks >> 3) + (l >> 4)) ^ kc_key<BKT>(row);
  s16x8 v = *(const s16x8 *)(t + row * BKT + pchunk * 8);
  return __builtin_bit_cast(bf16x8, v);
}
// From a k-major tile through ds_read_b64_tr_b16: within each 16-lane group, lane i
// receives element i%4 of the 8-byte chunk that lane 4e + i/4 addressed (e = 0..3);
// lane j addressing row kb + j/4, columns c0 + 4(j%4) .. +3 gives lane i the four
// k values kb .. kb+3 of column c0 + i.
template <int C>
__device__ inline bf16x8 frag_km(const bf16_t *t, int c0, int ks) {
  const int l = threadIdx.x & 63, g = l >> 4, j = l & 15;
  const int col = c0 + 4 * (j & 3);
  const int r0 = ks + 8 * g + (j >> 2), r1 = r0 + 4;
  const int p0 = ((col >> 3) ^ km_xor<C>(r0)) * 8 + (col & 7);
  const int p1 = ((col >> 3) ^ km_xor<C>(r1)) * 8 + (col & 7);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(t + r0 * C + p0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(t + r1 * C + p1));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Eight signed bytes (|q| <= 127) widened to bf16; every such integer is exact in bf16,
// so the float's upper half is the bf16 value.
__device__ inline bf16x8 widen_i8x8(uint32_t lo, uint32_t hi) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t src = e < 2 ? lo : hi;
    const int sh = (e & 1) * 16;
    const float x0 = (float)(int)(int8_t)(src >> sh), x1 = (float)(int)(int8_t)(src >> (sh + 8));
    w[e] = __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x07060302u);
  }
  const u32x4v v = {w[0], w[1], w[2], w[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// MFMA operand fragment from a k-major int8 tile of CB-byte rows (chunks rotated by
// km_xor_sel<., true>), through ds_read_b64_tr_b8: within each 16-lane group, lane i
// receives byte i%8 of the 8-byte pieces that lanes 2e + i/8 addressed (e = 0..7); lane
// j addressing row kb + j/2, columns c0 + 8(j%2) .. +7 therefore gives lane i the eight
// k values kb .. kb+7 of column c0 + i.  c0 is a multiple of 16.
template <int CB>
__device__ inline bf16x8 frag_km8(const bf16_t *t, int c0, int ks) {
  const int l = threadIdx.x & 63, g = l >> 4, j = l & 15;
  const int r = ks + 8 * g + (j >> 1);
  const int p = (((c0 >> 4) ^ (r & 7)) << 4) + 8 * (j & 1);
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)((const char *)t + r * CB + p));
  return widen_i8x8((uint32_t)v[0], (uint32_t)v[1]);
}

template <int LX, int K>
__device__ inline void wait_tiles(int later) {  // vmcnt <= later * LX, later clamped to K
  if constexpr (K == 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= K) wait_vmcnt<K * LX>();
    else wait_tiles<LX, K - 1>(later);
  }
}

}  // namespace
}  // namespace poetx
