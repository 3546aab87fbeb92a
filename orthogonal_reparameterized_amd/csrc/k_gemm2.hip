// bf16 MFMA products, second generation: operands go global -> LDS directly
// (buffer_load ... lds, 16 bytes per lane) into XOR-swizzled tiles, two LDS stages,
// one barrier per 64-deep k step, and an XCD-aware mapping of output tiles.
//
// Tile shapes:
//   BM x BN = 256 x 256 with 8 waves (2 x 4, 128 x 64 per wave)  -- the W' products
//   BM x BN = 128 x 128 with 4 waves (2 x 2,  64 x 64 per wave)  -- block products
// Operand layouts as in kernels.h (MfmaDesc): "k-contiguous" tiles [rows][64 k] are
// read with ds_read_b128, "k-major" tiles [64 k][cols] with ds_read_b64_tr_b16.
// Buffer resources clip every operand to its valid rows, so rows past M (token
// tails) and past the k range of a split read as zero without a branch.
#include <type_traits>

#include "kernels.h"

namespace poetx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// kernel argument block (external linkage: kernel templates are instantiated with it)
struct G2Args {
  int64_t M, N, K, Kc;
  int splits;
  int tiles_m, tiles_n;
  const bf16_t *A; int64_t lda, sAb;
  const bf16_t *B; int64_t ldb, sBb;
  void *C; int64_t ldc, sCb, sCsplit;
  const float *scaleN; int64_t sSNb;
};

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


}  // namespace

// ROLE separates instantiations per use.  WGM x WGN waves, each computing a
// (BM/WGM) x (BN/WGN) patch; k advances BKT per step through NST LDS stages with
// NST-1 steps of prefetch in flight.
template <int ROLE, int BM, int BN, int WGM, int WGN, int BKT, int NST, bool AKM, bool BKM, bool OUTF32>
__global__ __launch_bounds__(64 * WGM * WGN) void k_gemm2(G2Args a) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN, FM = WTM / 16, FN = WTN / 16;
  constexpr int A_ELEMS = BM * BKT, B_ELEMS = BN * BKT;
  constexpr int PF = NST - 1;
  extern __shared__ __align__(16) bf16_t smem[];
  // stage s: A tile at smem + s*A_ELEMS, B tile at smem + NST*A_ELEMS + s*B_ELEMS

  // ---- tile mapping: batch/split in z; (m, n) from an XCD-aware order of blockIdx.x
  const int64_t z = blockIdx.z, bidx = z / a.splits, kz = z % a.splits;
  const int T = a.tiles_m * a.tiles_n;
  int L = blockIdx.x;
  if (T % 8 == 0) L = (L % 8) * (T / 8) + L / 8;  // consecutive ids land on one XCD
  const int GM = a.tiles_m < 4 ? a.tiles_m : 4;   // 4 m-tiles share each sweep over n
  const int grp_size = GM * a.tiles_n;
  const int grp = L / grp_size, first_m = grp * GM;
  const int gm = (a.tiles_m - first_m) < GM ? (a.tiles_m - first_m) : GM;
  const int local = L % grp_size;
  const int tm = first_m + local % gm, tn = local / gm;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int64_t kbeg = kz * a.Kc;
  const int64_t kend = (kbeg + a.Kc < a.K) ? kbeg + a.Kc : a.K;
  const bf16_t *A = a.A + bidx * a.sAb;
  const bf16_t *B = a.B + bidx * a.sBb;
  // valid extents: k-contiguous operands end at their last row, k-major at kend
  const __amdgpu_buffer_rsrc_t ra = AKM ? make_rsrc(A, kend * a.lda * 2) : make_rsrc(A, a.M * a.lda * 2);
  const __amdgpu_buffer_rsrc_t rb = BKM ? make_rsrc(B, kend * a.ldb * 2) : make_rsrc(B, a.N * a.ldb * 2);

  const int wave = threadIdx.x >> 6;
  const int wm = (wave / WGN) * WTM, wn = (wave % WGN) * WTN;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  using LA = typename std::conditional<AKM, LoaderKM<BM, NW, BKT>, LoaderKC<BM, NW, BKT>>::type;
  using LB = typename std::conditional<BKM, LoaderKM<BN, NW, BKT>, LoaderKC<BN, NW, BKT>>::type;
  constexpr int LPS = LA::INSTR + LB::INSTR;  // loads per wave per stage
  LA la;
  LB lb;
  la.init(a.lda, m0);
  lb.init(a.ldb, n0);
  auto issue = [&](int buf, int64_t k0) {
    la.issue(ra, k0, a.lda, smem + buf * A_ELEMS);
    lb.issue(rb, k0, a.ldb, smem + NST * A_ELEMS + buf * B_ELEMS);
  };

  const int nk = (int)((kend - kbeg + BKT - 1) / BKT);
#pragma unroll
  for (int s = 0; s < PF; ++s)
    if (s < nk) issue(s, kbeg + (int64_t)s * BKT);
  for (int t = 0; t < nk; ++t) {
    // stage t has landed for this wave once at most (PF-1) newer stages are outstanding
    if (t + PF <= nk) wait_vmcnt<(PF - 1) * LPS>();
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // everyone's stage t is in LDS; stage t-1 is no longer read
    if (t + PF < nk) issue((t + PF) % NST, kbeg + (int64_t)(t + PF) * BKT);
    const int cur = t % NST;
    const bf16_t *ta = smem + cur * A_ELEMS, *tb = smem + NST * A_ELEMS + cur * B_ELEMS;
    // All fragments of the step are requested before the first MFMA (a scheduling
    // barrier keeps the compiler from sinking the second half's reads into the MFMA
    // chain), so LDS latency is paid once per step instead of once per fragment pair.
    constexpr int KH = BKT / 32;
    bf16x8 fa[KH][FM], fb[KH][FN];
#pragma unroll
    for (int h = 0; h < KH; ++h) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[h][i] = AKM ? frag_km<BM>(ta, wm + 16 * i, 32 * h) : frag_kc<BKT>(ta, wm + 16 * i, 32 * h);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[h][j] = BKM ? frag_km<BN>(tb, wn + 16 * j, 32 * h) : frag_kc<BKT>(tb, wn + 16 * j, 32 * h);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < KH; ++h)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          // operands swapped: lane l then holds C[m = l%16][n = 4*(l/16) + 0..3]
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[h][j], fa[h][i], acc[i][j], 0, 0, 0);
  }

  const int l = threadIdx.x & 63;
  char *Cb = (char *)a.C + (bidx * a.sCb + kz * a.sCsplit) * (OUTF32 ? 4 : 2);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wm + 16 * i + (l & 15);
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn + 16 * j + 4 * (l >> 4);
      f32x4 v = acc[i][j];
      if (a.scaleN) {
        float4 sc = *(const float4 *)(a.scaleN + bidx * a.sSNb + n);
        v[0] *= sc.x; v[1] *= sc.y; v[2] *= sc.z; v[3] *= sc.w;
      }
      if constexpr (OUTF32) {
        *(float4 *)(Cb + (m * a.ldc + n) * 4) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        uint2 p;
        p.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        p.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *(uint2 *)(Cb + (m * a.ldc + n) * 2) = p;
      }
    }
  }
}


// Ping-pong schedule for the W' products (256 x 256 tile, 8 waves, BK = 64, 2 LDS
// stages).  The waves form two groups of four, one wave of each group per SIMD.
// Group 1 runs one phase behind group 0, so in every phase one group issues MFMAs
// while the other reads its next fragments from LDS; a wave loads all fragments of a
// k step into registers before its MFMA phase, so an LDS stage is free as soon as
// both groups have read it.  Group 0 also issues the global->LDS loads of the next
// stage at the start of its read phase and waits for them before the barrier that
// ends its MFMA phase (two phases of latency cover).
//   phase A of step t: group 0 reads stage t (and issues stage t+1); group 1 multiplies step t-1
//   phase B of step t: group 0 multiplies step t;                     group 1 reads stage t
template <int ROLE, bool AKM, bool BKM, bool OUTF32>
__global__ __launch_bounds__(512) void k_gemm_pp(G2Args a) {
  constexpr int BM = 256, BN = 256, BKT = 64, WGN = 4;
  constexpr int WTM = 128, WTN = 64, FM = WTM / 16, FN = WTN / 16;
  constexpr int A_ELEMS = BM * BKT, B_ELEMS = BN * BKT;
  extern __shared__ __align__(16) bf16_t smem[];

  const int64_t z = blockIdx.z, bidx = z / a.splits, kz = z % a.splits;
  const int T = a.tiles_m * a.tiles_n;
  int L = blockIdx.x;
  if (T % 8 == 0) L = (L % 8) * (T / 8) + L / 8;
  const int GM = a.tiles_m < 4 ? a.tiles_m : 4;
  const int grp_size = GM * a.tiles_n;
  const int grp = L / grp_size, first_m = grp * GM;
  const int gm = (a.tiles_m - first_m) < GM ? (a.tiles_m - first_m) : GM;
  const int local = L % grp_size;
  const int tm = first_m + local % gm, tn = local / gm;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int64_t kbeg = kz * a.Kc;
  const int64_t kend = (kbeg + a.Kc < a.K) ? kbeg + a.Kc : a.K;
  const bf16_t *A = a.A + bidx * a.sAb;
  const bf16_t *B = a.B + bidx * a.sBb;
  const __amdgpu_buffer_rsrc_t ra = AKM ? make_rsrc(A, kend * a.lda * 2) : make_rsrc(A, a.M * a.lda * 2);
  const __amdgpu_buffer_rsrc_t rb = BKM ? make_rsrc(B, kend * a.ldb * 2) : make_rsrc(B, a.N * a.ldb * 2);

  const int wave = threadIdx.x >> 6, group = wave >> 2;
  const int wm = (wave / WGN) * WTM, wn = (wave % WGN) * WTN;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  using LA = typename std::conditional<AKM, LoaderKM<BM, 4, BKT>, LoaderKC<BM, 4, BKT>>::type;
  using LB = typename std::conditional<BKM, LoaderKM<BN, 4, BKT>, LoaderKC<BN, 4, BKT>>::type;
  LA la;
  LB lb;
  if (group == 0) {
    la.init(a.lda, m0);
    lb.init(a.ldb, n0);
  }
  auto issue = [&](int buf, int64_t k0) {
    la.issue(ra, k0, a.lda, smem + buf * A_ELEMS);
    lb.issue(rb, k0, a.ldb, smem + 2 * A_ELEMS + buf * B_ELEMS);
  };
  bf16x8 fa[FM], fb[FN];  // fragments of one 32-deep half step
  auto read_frags = [&](int buf, int h) {
    const bf16_t *ta = smem + buf * A_ELEMS, *tb = smem + 2 * A_ELEMS + buf * B_ELEMS;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[i] = AKM ? frag_km<BM>(ta, wm + 16 * i, 32 * h) : frag_kc<BKT>(ta, wm + 16 * i, 32 * h);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[j] = BKM ? frag_km<BN>(tb, wn + 16 * j, 32 * h) : frag_kc<BKT>(tb, wn + 16 * j, 32 * h);
  };
  auto multiply = [&]() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };

  const int nk = (int)((kend - kbeg + BKT - 1) / BKT);
  if (group == 0) {
    if (nk > 0) issue(0, kbeg);
    if (nk > 1) issue(1, kbeg + BKT);
    wait_vmcnt<LA::INSTR + LB::INSTR>();  // stage 0 landed (stage 1 may still be in flight)
    if (nk <= 1) __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // phase A: group 0 reads half h of stage t; group 1 multiplies the half before
      if (group == 0) read_frags(t & 1, h);
      else if (t > 0 || h > 0) multiply();
      __syncthreads();
      // phase B: group 0 multiplies half h; group 1 reads it
      if (group == 0) {
        multiply();
        if (h == 1) __builtin_amdgcn_s_waitcnt(0);  // stage t+1 has landed
      } else {
        read_frags(t & 1, h);
      }
      __syncthreads();
    }
    // both groups are done with stage t: its buffer takes stage t+2
    if (group == 0 && t + 2 < nk) issue(t & 1, kbeg + (int64_t)(t + 2) * BKT);
  }
  if (group == 1 && nk > 0) multiply();

  const int l = threadIdx.x & 63;
  char *Cb = (char *)a.C + (bidx * a.sCb + kz * a.sCsplit) * (OUTF32 ? 4 : 2);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wm + 16 * i + (l & 15);
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn + 16 * j + 4 * (l >> 4);
      f32x4 v = acc[i][j];
      if (a.scaleN) {
        float4 sc = *(const float4 *)(a.scaleN + bidx * a.sSNb + n);
        v[0] *= sc.x; v[1] *= sc.y; v[2] *= sc.z; v[3] *= sc.w;
      }
      if constexpr (OUTF32) {
        *(float4 *)(Cb + (m * a.ldc + n) * 4) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        uint2 p;
        p.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        p.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *(uint2 *)(Cb + (m * a.ldc + n) * 2) = p;
      }
    }
  }
}


// Streaming block-diagonal product: Y_j = X_j . G_j (TRANS = false) or X_j . G_j^T
// (TRANS = true) for every b x b block j, where X_j, Y_j are columns [jb, (j+1)b) of
// token-major activations.  The op is HBM-bound (about 130 flop per byte at b = 256),
// so each workgroup keeps one SW-wide slice of G_j resident in LDS and streams
// T-token tiles of X_j through a 3-stage ring (prefetch distance 2), writing the
// T x SW output tile straight from the accumulators.  A tile is read by the b/SW
// slice workgroups of its block; their ids are 8 apart so they share an XCD (and its L2).
struct BSArgs {
  int64_t N, d;           // tokens, row stride (elements) of X and Y
  int nb, P;              // blocks; workgroups per (block, slice)
  const bf16_t *X; const bf16_t *G; bf16_t *Y;
  const float *scaleN;    // per output column (length d) or null
};

template <int B, int SW, int T, bool TRANS>
__global__ __launch_bounds__(384) void k_block_stream(BSArgs a) {
  // waves 0-3 multiply and store; waves 4-5 only issue the global->LDS loads, so the
  // producers' vmcnt waits track loads alone and the consumers' stores never stall
  // the ring
  constexpr int NCW = 4, NPW = 2;
  constexpr int NSL = B / SW, NST = 3;
  constexpr int WTM = T / 2, WTN = SW / 2, FM = WTM / 16, FN = WTN / 16;
  constexpr int G_ELEMS = B * SW, A_ELEMS = T * B;
  extern __shared__ __align__(16) bf16_t smem[];
  bf16_t *sG = smem;

  // blockIdx.x = (u / 8) * (8 * NSL) + h * 8 + u % 8 with u = j * P + p
  const int x = blockIdx.x;
  const int h = (x / 8) % NSL;
  const int u = (x / (8 * NSL)) * 8 + x % 8;
  if (u >= a.nb * a.P) return;
  const int j = u / a.P, p = u % a.P;
  const int64_t ntile = (a.N + T - 1) / T;

  const int wave = threadIdx.x >> 6;
  const bool producer = wave >= NCW;
  const int wm = ((wave & 3) >> 1) * WTM, wn = (wave & 1) * WTN;
  const int l = threadIdx.x & 63;

  using LG = typename std::conditional<TRANS, LoaderKC<SW, NPW, B, NCW>, LoaderKM<SW, NPW, B, NCW>>::type;
  using LXT = LoaderKC<T, NPW, B, NCW>;
  constexpr int LX = LXT::INSTR;
  LXT lx;
  const bf16_t *Xj = a.X + (int64_t)j * B;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(Xj, a.N * a.d * 2);
  if (producer) {
    const bf16_t *Gs = TRANS ? a.G + (int64_t)j * B * B + (int64_t)h * SW * B : a.G + (int64_t)j * B * B + h * SW;
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(Gs, (int64_t)B * B * 2);
    LG lg;
    lg.init(B, 0);
    lx.init(a.d, 0);
    lg.issue(rg, 0, B, sG);
    if (p < ntile) lx.issue(rx, (int64_t)p * T * a.d, a.d, smem + G_ELEMS);
    if (p + a.P < ntile) lx.issue(rx, (int64_t)(p + a.P) * T * a.d, a.d, smem + G_ELEMS + A_ELEMS);
  }
  int64_t tile = p;
  for (int it = 0; tile < ntile; ++it, tile += a.P) {
    if (producer) {
      if (tile + a.P < ntile) wait_vmcnt<LX>();  // this tile (and G) landed; the next may fly
      else __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();  // the tile is in LDS; the stage of tile it-1 is no longer read
    if (producer) {
      if (tile + 2 * a.P < ntile)
        lx.issue(rx, (tile + 2 * a.P) * T * a.d, a.d, smem + G_ELEMS + ((it + 2) % NST) * A_ELEMS);
      continue;
    }
    const bf16_t *ta = smem + G_ELEMS + (it % NST) * A_ELEMS;
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jj = 0; jj < FN; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < B; k2 += 64) {
      bf16x8 fa[2][FM], fb[2][FN];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int ks = k2 + 32 * hh;
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[hh][i] = frag_kc<B>(ta, wm + 16 * i, ks);
#pragma unroll
        for (int jj = 0; jj < FN; ++jj)
          fb[hh][jj] = TRANS ? frag_kc<B>(sG, wn + 16 * jj, ks) : frag_km<SW>(sG, wn + 16 * jj, ks);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int jj = 0; jj < FN; ++jj)
            acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[hh][jj], fa[hh][i], acc[i][jj], 0, 0, 0);
    }
    // epilogue: lane holds Y[m = l%16][n = 4*(l/16) + 0..3] of each 16 x 16 patch
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = tile * T + wm + 16 * i + (l & 15);
      if (m >= a.N) continue;
#pragma unroll
      for (int jj = 0; jj < FN; ++jj) {
        const int64_t n = (int64_t)j * B + h * SW + wn + 16 * jj + 4 * (l >> 4);
        f32x4 v = acc[i][jj];
        if (a.scaleN) {
          float4 sc = *(const float4 *)(a.scaleN + n);
          v[0] *= sc.x; v[1] *= sc.y; v[2] *= sc.z; v[3] *= sc.w;
        }
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *(uint2 *)(a.Y + m * a.d + n) = pk;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load into LDS may outlive the workgroup
}

#define POETX_BS_INST(Bv, SWv, Tv)                                       \
  template __global__ void k_block_stream<Bv, SWv, Tv, false>(BSArgs); \
  template __global__ void k_block_stream<Bv, SWv, Tv, true>(BSArgs);
POETX_BS_INST(128, 128, 64)
POETX_BS_INST(256, 128, 64)
POETX_BS_INST(512, 64, 32)
#undef POETX_BS_INST

// Register-resident variant for b = 128 and 256: each of the 4 consumer waves keeps
// its b x (b/4) share of G_j (or G_j^T) as MFMA operand fragments in registers for
// the whole kernel (b = 256: 128 VGPRs), so one workgroup covers the block's full
// width -- every token tile of X_j is read once -- and the whole LDS is a 4-stage
// ring of T-token tiles (more bytes in flight per CU than with G held in LDS).
// G is staged once through the ring's LDS at the start.  Workgroup u covers block
// j = u % nb and token tiles p, p + P, ... with p = u / nb, so the blocks of the
// same token rows run side by side.
template <int LX, int K>
__device__ inline void wait_tiles(int later) {  // vmcnt <= later * LX, later clamped to K
  if constexpr (K == 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= K) wait_vmcnt<K * LX>();
    else wait_tiles<LX, K - 1>(later);
  }
}

template <int B, int T, int NST, bool TRANS>
__global__ __launch_bounds__(384) void k_block_reg(BSArgs a) {
  constexpr int NCW = 4, NPW = 2;
  constexpr int NTW = B / 64, NKS = B / 32, FM = T / 16;
  constexpr int A_ELEMS = T * B;
  static_assert(NST * A_ELEMS >= B * B, "G is staged in the ring");
  extern __shared__ __align__(16) bf16_t smem[];
  const int u = blockIdx.x;
  if (u >= a.nb * a.P) return;
  const int p = u / a.nb, j = u % a.nb;
  const int64_t ntile = (a.N + T - 1) / T;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const bool producer = wave >= NCW;
  const int n0 = wave * (B / 4);  // a consumer's first output column within the block

  // ---- this wave's columns of the block operand, into registers
  bf16x8 gf[NTW][NKS];
  if (!producer) {
    const bf16_t *Gj = a.G + (int64_t)j * B * B;
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(Gj, (int64_t)B * B * 2);
    if constexpr (TRANS) {
      LoaderKC<B, NCW, B, 0> lg;  // rows n, k contiguous: G_j^T fragments via frag_kc
      lg.init(B, 0);
      lg.issue(rg, 0, B, smem);
    } else {
      LoaderKM<B, NCW, B, 0> lg;  // rows k, n contiguous: G_j fragments via frag_km
      lg.init(B, 0);
      lg.issue(rg, 0, B, smem);
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  if (!producer) {
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        gf[t][s] = TRANS ? frag_kc<B>(smem, n0 + 16 * t, 32 * s) : frag_km<B>(smem, n0 + 16 * t, 32 * s);
  }
  __syncthreads();  // the ring may now overwrite the staged block

  using LXT = LoaderKC<T, NPW, B, NCW>;
  constexpr int LX = LXT::INSTR;
  LXT lx;
  const bf16_t *Xj = a.X + (int64_t)j * B;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(Xj, a.N * a.d * 2);
  if (producer) {
    lx.init(a.d, 0);
#pragma unroll
    for (int s = 0; s < NST - 1; ++s) {
      const int64_t tl = p + (int64_t)s * a.P;
      if (tl < ntile) lx.issue(rx, tl * T * a.d, a.d, smem + s * A_ELEMS);
    }
  }
  int64_t tile = p;
  for (int it = 0; tile < ntile; ++it, tile += a.P) {
    if (producer) {
      // tiles it .. it + NST - 2 may be in flight (loads complete in order): wait for
      // tile it only
      const int64_t later = (ntile - 1 - tile) / a.P;
      wait_tiles<LX, NST - 2>((int)(later < NST - 2 ? later : NST - 2));
    }
    __syncthreads();  // tile it is in LDS; the stage read in iteration it-1 is free
    if (producer) {
      const int64_t nx = tile + (int64_t)(NST - 1) * a.P;
      if (nx < ntile) lx.issue(rx, nx * T * a.d, a.d, smem + ((it + NST - 1) % NST) * A_ELEMS);
      continue;
    }
    const bf16_t *ta = smem + (it % NST) * A_ELEMS;
    f32x4 acc[FM][NTW];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int t = 0; t < NTW; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < NKS; s2 += 2) {
      bf16x8 fa[2][FM];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[h][i] = frag_kc<B>(ta, 16 * i, 32 * (s2 + h));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int t = 0; t < NTW; ++t)
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gf[t][s2 + h], fa[h][i], acc[i][t], 0, 0, 0);
    }
    // epilogue: lane holds Y[m = l%16][n = 4*(l/16) + 0..3] of each 16 x 16 patch
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = tile * T + 16 * i + (l & 15);
      if (m >= a.N) continue;
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int64_t n = (int64_t)j * B + n0 + 16 * t + 4 * (l >> 4);
        f32x4 v = acc[i][t];
        if (a.scaleN) {
          float4 sc = *(const float4 *)(a.scaleN + n);
          v[0] *= sc.x; v[1] *= sc.y; v[2] *= sc.z; v[3] *= sc.w;
        }
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *(uint2 *)(a.Y + m * a.d + n) = pk;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load into LDS may outlive the workgroup
}
// b = 256 uses 32-token tiles (the 128 registers of G leave room for 2 x 4 patches of
// accumulators), b = 128 64-token tiles; both rings hold 128 or 64 KB
template __global__ void k_block_reg<128, 64, 4, false>(BSArgs);
template __global__ void k_block_reg<128, 64, 4, true>(BSArgs);
template __global__ void k_block_reg<256, 32, 8, false>(BSArgs);
template __global__ void k_block_reg<256, 32, 8, true>(BSArgs);

template <int B, int T, int NST, bool TRANS>
static int run_br(const BSArgs &a, const char *name, hipStream_t s) {
  const size_t lds = (size_t)NST * T * B * 2;
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&k_block_reg<B, T, NST, TRANS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return POETX_ERR_HIP;
    attr = true;
  }
  const dim3 grid((unsigned)(a.nb * a.P));
  return launch(name, s, [&] { k_block_reg<B, T, NST, TRANS><<<grid, 384, lds, s>>>(a); });
}

template <int B, int SW, int T, bool TRANS>
static int run_bs(const BSArgs &a, const char *name, hipStream_t s) {
  const size_t lds = ((size_t)B * SW + 3 * (size_t)T * B) * 2;
  constexpr int NSL = B / SW;
  const int64_t units = (int64_t)a.nb * a.P;
  dim3 grid((unsigned)(((units + 7) / 8) * 8 * NSL));
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&k_block_stream<B, SW, T, TRANS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return POETX_ERR_HIP;
    attr = true;
  }
  return launch(name, s, [&] { k_block_stream<B, SW, T, TRANS><<<grid, 384, lds, s>>>(a); });
}

bool block_stream_supported(int64_t b, int64_t d, int64_t n_tokens) {
  if (b != 128 && b != 256 && b != 512) return false;
  if (d % b) return false;
  return (n_tokens + 64) * d * 2 < 0x7fffffff;
}

int block_stream(const bf16_t *X, const bf16_t *G, bf16_t *Y, int64_t n_tokens, int64_t d, int64_t b,
                 bool transposed, const float *scaleN, const char *name, hipStream_t s) {
  if (n_tokens <= 0) return POETX_OK;
  if (!block_stream_supported(b, d, n_tokens)) return POETX_ERR_UNSUPPORTED;
  BSArgs a;
  a.N = n_tokens; a.d = d; a.nb = (int)(d / b);
  a.X = X; a.G = G; a.Y = Y; a.scaleN = scaleN;
  if (b == 128 || b == 256) {
    // one workgroup per (token partition, block), about one per CU in total
    const int tt = b == 256 ? 32 : 64;
    const int64_t ntile = (n_tokens + tt - 1) / tt;
    int64_t P = 256 / a.nb;
    if (P > ntile) P = ntile;
    a.P = (int)(P < 1 ? 1 : P);
    if (b == 128) return transposed ? run_br<128, 64, 4, true>(a, name, s) : run_br<128, 64, 4, false>(a, name, s);
    return transposed ? run_br<256, 32, 8, true>(a, name, s) : run_br<256, 32, 8, false>(a, name, s);
  }
  const int sw = b == 512 ? 64 : 128, t = b == 512 ? 32 : 64;
  const int64_t slices = (int64_t)a.nb * (b / sw);
  const int64_t ntile = (n_tokens + t - 1) / t;
  int64_t P = (256 + slices - 1) / slices;  // about one workgroup per CU in total
  if (P > ntile) P = ntile;
  a.P = (int)(P < 1 ? 1 : P);
  if (b == 128) return transposed ? run_bs<128, 128, 64, true>(a, name, s) : run_bs<128, 128, 64, false>(a, name, s);
  if (b == 256) return transposed ? run_bs<256, 128, 64, true>(a, name, s) : run_bs<256, 128, 64, false>(a, name, s);
  return transposed ? run_bs<512, 64, 32, true>(a, name, s) : run_bs<512, 64, 32, false>(a, name, s);
}


// Streaming block gradient: parts[p][j][r][c] = sum over the token tiles t = p, p+P, ...
// of Xs_j[t]^T dY_j[t], for every b x b block j (r indexes columns of Xs_j, c of dY_j).
// Each workgroup owns one 128 x 128 slice (rs, cs) of one block's gradient and keeps it
// in registers while T-token tiles of both operands stream through a 4-stage LDS ring
// (producer waves as in k_block_stream).  The P partials per block are summed later in
// a fixed order.
struct BGArgs {
  int64_t N, d;
  int nb, P;
  const bf16_t *Xs; const bf16_t *dY; float *parts;  // parts: [P][nb][b][b]
};

template <int B>
__global__ __launch_bounds__(384) void k_block_grad_stream(BGArgs a) {
  constexpr int NCW = 4, NPW = 2, S = 128, T = 64, NST = 4;
  constexpr int NSL = (B / S) * (B / S);
  constexpr int WT = S / 2, F = WT / 16;  // 2 x 2 waves of 64 x 64
  constexpr int TILE = T * S;             // elements per operand tile
  extern __shared__ __align__(16) bf16_t smem[];

  const int x = blockIdx.x;
  const int sl = (x / 8) % NSL;
  const int u = (x / (8 * NSL)) * 8 + x % 8;
  if (u >= a.nb * a.P) return;
  const int j = u / a.P, p = u % a.P;
  const int rs = sl / (B / S), cs = sl % (B / S);
  const int64_t ntile = (a.N + T - 1) / T;

  const int wave = threadIdx.x >> 6;
  const bool producer = wave >= NCW;
  const int wm = ((wave & 3) >> 1) * WT, wn = (wave & 1) * WT;
  const int l = threadIdx.x & 63;

  using LT = LoaderKM<S, NPW, T, NCW>;
  constexpr int LPT = 2 * LT::INSTR;  // loads per producer wave per token tile
  LT la, lb;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.Xs + (int64_t)j * B + rs * S, a.N * a.d * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.dY + (int64_t)j * B + cs * S, a.N * a.d * 2);
  auto issue = [&](int64_t t, int stage) {
    la.issue(ra, t * T, a.d, smem + (2 * stage) * TILE);
    lb.issue(rb, t * T, a.d, smem + (2 * stage + 1) * TILE);
  };
  if (producer) {
    la.init(a.d, 0);
    lb.init(a.d, 0);
    for (int s = 0; s < NST - 1; ++s)
      if (p + (int64_t)s * a.P < ntile) issue(p + (int64_t)s * a.P, s);
  }
  f32x4 acc[F][F];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int jj = 0; jj < F; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  int64_t tile = p;
  for (int it = 0; tile < ntile; ++it, tile += a.P) {
    if (producer) {
      if (tile + 2 * a.P < ntile) wait_vmcnt<2 * LPT>();
      else if (tile + a.P < ntile) wait_vmcnt<LPT>();
      else __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    if (producer) {
      if (tile + 3 * a.P < ntile) issue(tile + 3 * a.P, (it + 3) % NST);
      continue;
    }
    const bf16_t *ta = smem + (2 * (it % NST)) * TILE, *tb = ta + TILE;
    bf16x8 fa[2][F], fb[2][F];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int i = 0; i < F; ++i) fa[hh][i] = frag_km<S>(ta, wm + 16 * i, 32 * hh);
#pragma unroll
      for (int jj = 0; jj < F; ++jj) fb[hh][jj] = frag_km<S>(tb, wn + 16 * jj, 32 * hh);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int jj = 0; jj < F; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[hh][jj], fa[hh][i], acc[i][jj], 0, 0, 0);
  }
  if (!producer) {
    float *out = a.parts + ((int64_t)p * a.nb + j) * B * B;
#pragma unroll
    for (int i = 0; i < F; ++i) {
      const int r = rs * S + wm + 16 * i + (l & 15);
#pragma unroll
      for (int jj = 0; jj < F; ++jj) {
        const int c = cs * S + wn + 16 * jj + 4 * (l >> 4);
        *(float4 *)(out + (int64_t)r * B + c) = make_float4(acc[i][jj][0], acc[i][jj][1], acc[i][jj][2], acc[i][jj][3]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load into LDS may outlive the workgroup
}
template __global__ void k_block_grad_stream<128>(BGArgs);
template __global__ void k_block_grad_stream<256>(BGArgs);
template __global__ void k_block_grad_stream<512>(BGArgs);

template <int B>
static int run_bg(const BGArgs &a, hipStream_t s) {
  constexpr int NSL = (B / 128) * (B / 128);
  const size_t lds = (size_t)4 * 2 * 64 * 128 * 2;
  const int64_t units = (int64_t)a.nb * a.P;
  dim3 grid((unsigned)(((units + 7) / 8) * 8 * NSL));
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&k_block_grad_stream<B>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return POETX_ERR_HIP;
    attr = true;
  }
  return launch("block_grad", s, [&] { k_block_grad_stream<B><<<grid, 384, lds, s>>>(a); });
}

int64_t block_grad_stream_parts(int64_t b, int64_t d, int64_t n_tokens) {
  const int64_t slices = (d / b) * (b / 128) * (b / 128);
  int64_t P = (256 + slices - 1) / slices;
  const int64_t ntile = (n_tokens + 63) / 64;
  if (P > ntile) P = ntile;
  return P < 1 ? 1 : P;
}

int block_grad_stream(const bf16_t *Xs, const bf16_t *dY, float *parts, int64_t n_tokens, int64_t d, int64_t b,
                      hipStream_t s) {
  if (!block_stream_supported(b, d, n_tokens)) return POETX_ERR_UNSUPPORTED;
  BGArgs a;
  a.N = n_tokens; a.d = d; a.nb = (int)(d / b);
  a.P = (int)block_grad_stream_parts(b, d, n_tokens);
  a.Xs = Xs; a.dY = dY; a.parts = parts;
  if (b == 128) return run_bg<128>(a, s);
  if (b == 256) return run_bg<256>(a, s);
  return run_bg<512>(a, s);
}

// explicit instantiations (every configuration the dispatcher below launches)
#define POETX_G2_INST(R, BMv, BNv, WM, WN, BKv, NS, AK, BKm)                                     \
  template __global__ void k_gemm2<R, BMv, BNv, WM, WN, BKv, NS, AK, BKm, true>(G2Args);       \
  template __global__ void k_gemm2<R, BMv, BNv, WM, WN, BKv, NS, AK, BKm, false>(G2Args);
POETX_G2_INST(MFMA_GEMM_NT, 256, 256, 2, 4, 64, 2, false, false)
POETX_G2_INST(MFMA_BLOCK_APPLY, 128, 128, 2, 2, 64, 2, false, true)
POETX_G2_INST(MFMA_BLOCK_APPLY_T, 128, 128, 2, 2, 64, 2, false, false)
POETX_G2_INST(MFMA_BLOCK_GRAD, 128, 128, 2, 2, 64, 2, true, true)
#undef POETX_G2_INST
template __global__ void k_gemm_pp<MFMA_GEMM_NN, false, true, false>(G2Args);
template __global__ void k_gemm_pp<MFMA_GEMM_NN, false, true, true>(G2Args);

template <int ROLE, bool AKM, bool BKM>
static int run_pp(const G2Args &k, const MfmaDesc &d, hipStream_t s) {
  const size_t lds = (size_t)2 * 512 * 64 * 2;
  if (d.M <= 0 || d.N % 256 || d.K % 64) return POETX_ERR_UNSUPPORTED;
  G2Args a = k;
  a.tiles_m = (int)cdiv(d.M, 256);
  a.tiles_n = (int)(d.N / 256);
  dim3 grid((unsigned)(a.tiles_m * a.tiles_n), 1, (unsigned)(d.batch * d.splits));
  if (d.c_dt == POETX_F32) {
    static bool attr = false;
    if (!attr) {
      if (hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm_pp<ROLE, AKM, BKM, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return POETX_ERR_HIP;
      attr = true;
    }
    return launch(d.name, s, [&] { k_gemm_pp<ROLE, AKM, BKM, true><<<grid, 512, lds, s>>>(a); });
  }
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm_pp<ROLE, AKM, BKM, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return POETX_ERR_HIP;
    attr = true;
  }
  return launch(d.name, s, [&] { k_gemm_pp<ROLE, AKM, BKM, false><<<grid, 512, lds, s>>>(a); });
}

template <int ROLE, int BM, int BN, int WGM, int WGN, int BKT, int NST, bool AKM, bool BKM, bool OUTF32>
static int run2o(const G2Args &a, const char *name, dim3 grid, size_t lds, hipStream_t s) {
  constexpr int NT = 64 * WGM * WGN;
  auto kern = &k_gemm2<ROLE, BM, BN, WGM, WGN, BKT, NST, AKM, BKM, OUTF32>;
  static bool attr = false;  // raise the dynamic-LDS limit once per instantiation
  if (!attr) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
      return POETX_ERR_HIP;
    attr = true;
  }
  return launch(name, s, [&] { k_gemm2<ROLE, BM, BN, WGM, WGN, BKT, NST, AKM, BKM, OUTF32><<<grid, NT, lds, s>>>(a); });
}

template <int ROLE, int BM, int BN, int WGM, int WGN, int BKT, int NST, bool AKM, bool BKM>
static int run2(const G2Args &k, const MfmaDesc &d, hipStream_t s) {
  const size_t lds = (size_t)NST * (BM + BN) * BKT * 2;
  if (d.M <= 0 || d.N % BN || d.K % BKT && (!AKM || !BKM)) return POETX_ERR_UNSUPPORTED;
  G2Args a = k;
  a.tiles_m = (int)cdiv(d.M, BM);
  a.tiles_n = (int)(d.N / BN);
  dim3 grid((unsigned)(a.tiles_m * a.tiles_n), 1, (unsigned)(d.batch * d.splits));
  if (d.c_dt == POETX_F32) return run2o<ROLE, BM, BN, WGM, WGN, BKT, NST, AKM, BKM, true>(a, d.name, grid, lds, s);
  return run2o<ROLE, BM, BN, WGM, WGN, BKT, NST, AKM, BKM, false>(a, d.name, grid, lds, s);
}

bool mfma2_supported(const MfmaDesc &d) {
  if (d.b_dt != POETX_BF16) return false;  // int8 weights keep the register-staged kernel
  if (d.c_dt != POETX_BF16 && d.c_dt != POETX_F32) return false;
  if (d.splits < 1 || d.batch * d.splits > 65535) return false;
  if (d.splits > 1 && (d.kchunk <= 0 || d.kchunk % 64 || cdiv(d.K, d.kchunk) != d.splits)) return false;
  if ((!d.a_km || !d.b_km) && d.K % 64) return false;
  // 32-bit buffer offsets, with room for the rows a last partial tile addresses
  const int64_t a_ext = ((d.a_km ? d.K : d.M) + 256) * d.lda * 2, b_ext = ((d.b_km ? d.K : d.N) + 256) * d.ldb * 2;
  if (a_ext > 0x7fffffff || b_ext > 0x7fffffff) return false;
  switch (d.role) {
    case MFMA_GEMM_NT: case MFMA_GEMM_NN: return d.N % 256 == 0 && cdiv(d.M, 256) * (d.N / 256) < (1 << 30);
    default: return d.N % 128 == 0 && (!d.a_km || d.M % 128 == 0);
  }
}

int gemm_mfma2(const MfmaDesc &d, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0 || d.batch <= 0) return POETX_OK;
  if (!mfma2_supported(d)) return POETX_ERR_UNSUPPORTED;
  G2Args k;
  k.M = d.M; k.N = d.N; k.K = d.K;
  k.splits = (int)d.splits;
  k.Kc = d.splits > 1 ? d.kchunk : d.K;
  k.A = (const bf16_t *)d.A; k.lda = d.lda; k.sAb = d.sAb;
  k.B = (const bf16_t *)d.B; k.ldb = d.ldb; k.sBb = d.sBb;
  k.C = d.C; k.ldc = d.ldc; k.sCb = d.sCb; k.sCsplit = d.sCsplit;
  k.scaleN = d.scaleN; k.sSNb = d.sSNb;
  k.tiles_m = k.tiles_n = 0;
  switch (d.role) {
    case MFMA_GEMM_NT:
      if (d.a_km || d.b_km) return POETX_ERR_UNSUPPORTED;
      return run2<MFMA_GEMM_NT, 256, 256, 2, 4, 64, 2, false, false>(k, d, s);
    case MFMA_GEMM_NN:
      if (d.a_km || !d.b_km) return POETX_ERR_UNSUPPORTED;
      // the k-major W' operand goes through the transposing LDS reads; the ping-pong
      // schedule hides their extra latency best (measured against the plain schedule)
      return run_pp<MFMA_GEMM_NN, false, true>(k, d, s);
    case MFMA_BLOCK_APPLY:
      if (d.a_km || !d.b_km) return POETX_ERR_UNSUPPORTED;
      return run2<MFMA_BLOCK_APPLY, 128, 128, 2, 2, 64, 2, false, true>(k, d, s);
    case MFMA_BLOCK_APPLY_T:
      if (d.a_km || d.b_km) return POETX_ERR_UNSUPPORTED;
      return run2<MFMA_BLOCK_APPLY_T, 128, 128, 2, 2, 64, 2, false, false>(k, d, s);
    case MFMA_BLOCK_GRAD:
      if (!d.a_km || !d.b_km) return POETX_ERR_UNSUPPORTED;
      return run2<MFMA_BLOCK_GRAD, 128, 128, 2, 2, 64, 2, true, true>(k, d, s);
    default:
      return POETX_ERR_UNSUPPORTED;
  }
}

}  // namespace poetx
