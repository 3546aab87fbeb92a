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
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
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
// 16-byte chunk c of row r sits at c ^ kc_key(r), which spreads the rows one
// 8-lane ds_read_b128 phase touches over all 128 bytes of a bank sweep.  One wave
// instruction (64 lanes x 16 B) fills 1 KB = 64 / (BKT/8) rows.
template <int BKT>
__device__ inline int kc_key(int r) { return BKT >= 64 ? (r & 7) : ((r >> 1) & 3); }

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
  __device__ void issue(__amdgpu_buffer_rsrc_t rs, int64_t k0, int64_t ld, bf16_t *tile) const {
    const int w = (threadIdx.x >> 6) - WOFF;
    const int kb = (int)(k0 * 2);
#pragma unroll
    for (int i = 0; i < INSTR; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(tile + (w * INSTR + i) * RPI * BKT), 16,
                                               voff[i] + kb, 0, 0, 0);
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

template <int C, int NW, int BKT, int WOFF = 0>
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
      const int lchunk = (l % CH) ^ km_xor<C>(row);
      voff[i] = (int)((row * ld + col0 + lchunk * 8) * 2);
    }
  }
  __device__ void issue(__amdgpu_buffer_rsrc_t rs, int64_t k0, int64_t ld, bf16_t *tile) const {
    const int w = (threadIdx.x >> 6) - WOFF;
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
