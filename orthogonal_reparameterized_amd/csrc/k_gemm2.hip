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

namespace {

constexpr int BK = 64;
constexpr uint32_t RSRC_DW3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

struct G2Args {
  int64_t M, N, K, Kc;
  int splits;
  int tiles_m, tiles_n;
  const bf16_t *A; int64_t lda, sAb;
  const bf16_t *B; int64_t ldb, sBb;
  void *C; int64_t ldc, sCb, sCsplit;
  const float *scaleN; int64_t sSNb;
};

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  uint32_t n = bytes > 0x7fffffff ? 0x7fffffffu : (uint32_t)(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, (int)RSRC_DW3);
}

// k-contiguous tile [R][64] bf16 = 128-byte rows; 16-byte chunk c of row r sits at
// chunk c ^ (r & 7).  One wave instruction fills 8 rows (1 KB).
template <int R, int NW>
__device__ inline void load_kc(__amdgpu_buffer_rsrc_t rs, int64_t ld, int64_t row0, int64_t k0,
                               bf16_t *tile) {
  constexpr int INSTR = R / 8 / NW;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < INSTR; ++i) {
    const int grp = w * INSTR + i;
    const int row = grp * 8 + (l >> 3);
    const int lchunk = (l & 7) ^ (row & 7);
    const int64_t off = ((row0 + row) * ld + k0 + lchunk * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(tile + grp * 8 * BK), 16, (int)off, 0, 0, 0);
  }
}

// k-major tile [64][C] bf16 = 2C-byte rows; chunk c of row r sits at c ^ ((r & 3) << 1)
// (32-byte blocks rotate with the row so the 4 rows one ds_read_b64_tr_b16 group reads
// fall in different banks).  One wave instruction fills 1 KB.
template <int C, int NW>
__device__ inline void load_km(__amdgpu_buffer_rsrc_t rs, int64_t ld, int64_t col0, int64_t k0,
                               bf16_t *tile) {
  constexpr int CH = C / 8;               // 16-byte chunks per row
  constexpr int RPI = 64 / CH;            // rows per wave instruction
  constexpr int INSTR = BK / RPI / NW;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < INSTR; ++i) {
    const int grp = w * INSTR + i;
    const int row = grp * RPI + l / CH;
    const int lchunk = (l % CH) ^ ((row & 3) << 1);
    const int64_t off = ((k0 + row) * ld + col0 + lchunk * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(tile + grp * RPI * C), 16, (int)off, 0, 0, 0);
  }
}

// MFMA operand fragment (lane l: 8 consecutive k of row/column l % 16).
__device__ inline bf16x8 frag_kc(const bf16_t *t, int r0, int ks) {
  const int l = threadIdx.x & 63, row = r0 + (l & 15);
  const int pchunk = ((ks >> 3) + (l >> 4)) ^ (row & 7);
  s16x8 v = *(const s16x8 *)(t + row * BK + pchunk * 8);
  return __builtin_bit_cast(bf16x8, v);
}
template <int C>
__device__ inline bf16x8 frag_km(const bf16_t *t, int c0, int ks) {
  const int l = threadIdx.x & 63, g = l >> 4, j = l & 15;
  const int col = c0 + 4 * (j & 3);
  const int r0 = ks + 8 * g + (j >> 2), r1 = r0 + 4;
  const int p0 = ((col >> 3) ^ ((r0 & 3) << 1)) * 8 + (col & 7);
  const int p1 = ((col >> 3) ^ ((r1 & 3) << 1)) * 8 + (col & 7);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(t + r0 * C + p0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(t + r1 * C + p1));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace

// ROLE separates instantiations per use; WGM x WGN waves, each computing a
// (BM/WGM) x (BN/WGN) patch.
template <int ROLE, int BM, int BN, int WGM, int WGN, bool AKM, bool BKM, bool OUTF32>
__global__ __launch_bounds__(64 * WGM * WGN) void k_gemm2(G2Args a) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN, FM = WTM / 16, FN = WTN / 16;
  constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
  extern __shared__ __align__(16) bf16_t smem[];
  // stage s: A tile at smem + s*A_ELEMS, B tile at smem + 2*A_ELEMS + s*B_ELEMS

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

  auto issue = [&](int buf, int64_t k0) {
    bf16_t *ta = smem + buf * A_ELEMS, *tb = smem + 2 * A_ELEMS + buf * B_ELEMS;
    if constexpr (AKM) load_km<BM, NW>(ra, a.lda, m0, k0, ta);
    else load_kc<BM, NW>(ra, a.lda, m0, k0, ta);
    if constexpr (BKM) load_km<BN, NW>(rb, a.ldb, n0, k0, tb);
    else load_kc<BN, NW>(rb, a.ldb, n0, k0, tb);
  };

  int cur = 0;
  if (kbeg < kend) issue(0, kbeg);
  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of stage `cur` have landed
    __syncthreads();                // ... and everyone's; stage cur^1 is free again
    if (k0 + BK < kend) issue(cur ^ 1, k0 + BK);
    const bf16_t *ta = smem + cur * A_ELEMS, *tb = smem + 2 * A_ELEMS + cur * B_ELEMS;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      bf16x8 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = AKM ? frag_km<BM>(ta, wm + 16 * i, ks) : frag_kc(ta, wm + 16 * i, ks);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = BKM ? frag_km<BN>(tb, wn + 16 * j, ks) : frag_kc(tb, wn + 16 * j, ks);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          // operands swapped: lane l then holds C[m = l%16][n = 4*(l/16) + 0..3]
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
    cur ^= 1;
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
        float4 s = *(const float4 *)(a.scaleN + bidx * a.sSNb + n);
        v[0] *= s.x; v[1] *= s.y; v[2] *= s.z; v[3] *= s.w;
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

template <int ROLE, int BM, int BN, int WGM, int WGN, bool AKM, bool BKM>
static int run2(const G2Args &k, const MfmaDesc &d, hipStream_t s) {
  const size_t lds = (size_t)2 * (BM + BN) * BK * 2;
  if (d.M <= 0 || d.N % BN) return POETX_ERR_UNSUPPORTED;
  G2Args a = k;
  a.tiles_m = (int)cdiv(d.M, BM);
  a.tiles_n = (int)(d.N / BN);
  dim3 grid((unsigned)(a.tiles_m * a.tiles_n), 1, (unsigned)(d.batch * d.splits));
  constexpr int NT = 64 * WGM * WGN;
  if (d.c_dt == POETX_F32) {
    auto kern = k_gemm2<ROLE, BM, BN, WGM, WGN, AKM, BKM, true>;
    static bool attr = false;  // raise the dynamic-LDS limit once per instantiation
    if (!attr) {
      if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return POETX_ERR_HIP;
      attr = true;
    }
    return launch(d.name, s, [&] { kern<<<grid, NT, lds, s>>>(a); });
  }
  auto kern = k_gemm2<ROLE, BM, BN, WGM, WGN, AKM, BKM, false>;
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return POETX_ERR_HIP;
    attr = true;
  }
  return launch(d.name, s, [&] { kern<<<grid, NT, lds, s>>>(a); });
}

bool mfma2_supported(const MfmaDesc &d) {
  if (d.b_dt != POETX_BF16) return false;  // int8 weights keep the register-staged kernel
  if (d.c_dt != POETX_BF16 && d.c_dt != POETX_F32) return false;
  if (d.splits < 1 || d.batch * d.splits > 65535) return false;
  if (d.splits > 1 && (d.kchunk <= 0 || d.kchunk % BK || cdiv(d.K, d.kchunk) != d.splits)) return false;
  if ((!d.a_km || !d.b_km) && d.K % BK) return false;
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
      return run2<MFMA_GEMM_NT, 256, 256, 2, 4, false, false>(k, d, s);
    case MFMA_GEMM_NN:
      if (d.a_km || !d.b_km) return POETX_ERR_UNSUPPORTED;
      return run2<MFMA_GEMM_NN, 256, 256, 2, 4, false, true>(k, d, s);
    case MFMA_BLOCK_APPLY:
      if (d.a_km || !d.b_km) return POETX_ERR_UNSUPPORTED;
      return run2<MFMA_BLOCK_APPLY, 128, 128, 2, 2, false, true>(k, d, s);
    case MFMA_BLOCK_APPLY_T:
      if (d.a_km || d.b_km) return POETX_ERR_UNSUPPORTED;
      return run2<MFMA_BLOCK_APPLY_T, 128, 128, 2, 2, false, false>(k, d, s);
    case MFMA_BLOCK_GRAD:
      if (!d.a_km || !d.b_km) return POETX_ERR_UNSUPPORTED;
      return run2<MFMA_BLOCK_GRAD, 128, 128, 2, 2, true, true>(k, d, s);
    default:
      return POETX_ERR_UNSUPPORTED;
  }
}

}  // namespace poetx
