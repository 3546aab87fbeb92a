// bf16 MFMA products for gfx950 (v_mfma_f32_16x16x32_bf16, float32 accumulation).
//
// One kernel template covers every dense contraction of the layer:
//   forward  B = A . W'^T       (A k-contiguous, W' k-contiguous)
//   backward dA = dB . W'       (W' n-contiguous: "k-major" operand)
//   block apply  X_j . G_j      (G_j k-major),   dY_j . G_j^T (G_j k-contiguous)
//   block gradient X_j^T dY_j   (both operands k-major: the token index is k)
// Operands are staged through LDS in their memory layout; k-contiguous tiles are
// read with 16-byte ds_read_b128, k-major tiles with the gfx950 transposing
// ds_read_b64_tr_b16, so no operand is ever transposed in global memory.
#include <type_traits>

#include "kernels.h"

namespace poetx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;
constexpr int KC_LD = BK + 8;      // k-contiguous tile row (elements): 144 B rows
constexpr int KM_LD = 128 + 16;    // k-major tile row (elements): 288 B rows
constexpr int TILE_ELEMS = (BM * KC_LD > BK * KM_LD) ? BM * KC_LD : BK * KM_LD;

struct KArgs {
  int64_t M, N, K, Kc;  // Kc: k extent per split (multiple of BK)
  int splits;
  const bf16_t *A; int64_t lda, sAb;
  const void *B; int64_t ldb, sBb;
  void *C; int64_t ldc, sCb, sCsplit;
  const float *scaleN;
  int64_t sSNb;
};

__device__ inline uint32_t i8pair_to_bf16x2(int8_t lo, int8_t hi) {
  uint32_t a = __float_as_uint((float)lo) >> 16, b = __float_as_uint((float)hi) >> 16;
  return a | (b << 16);
}

// ---- tile loaders: global -> registers -> LDS -------------------------------
// k-contiguous bf16 tile: 128 rows x 64 k, 8 chunks of 16 B per row, 4 chunks per thread.
struct LoadKC {
  uint4 r[4];
  __device__ void load(const bf16_t *base, int64_t ld, int64_t row0, int64_t rows, int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = threadIdx.x + NT * i, row = q >> 3, kc = q & 7;
      int64_t gr = row0 + row;
      r[i] = gr < rows ? *(const uint4 *)(base + gr * ld + k0 + kc * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ void store(bf16_t *t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = threadIdx.x + NT * i, row = q >> 3, kc = q & 7;
      *(uint4 *)(t + row * KC_LD + kc * 8) = r[i];
    }
  }
};
// k-major bf16 tile: 64 k-rows x 128 columns, 16 chunks per row; rows past kend read as 0.
struct LoadKM {
  uint4 r[4];
  __device__ void load(const bf16_t *base, int64_t ld, int64_t col0, int64_t k0, int64_t kend) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = threadIdx.x + NT * i, kr = q >> 4, c = q & 15;
      int64_t gk = k0 + kr;
      r[i] = gk < kend ? *(const uint4 *)(base + gk * ld + col0 + c * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ void store(bf16_t *t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = threadIdx.x + NT * i, kr = q >> 4, c = q & 15;
      *(uint4 *)(t + kr * KM_LD + c * 8) = r[i];
    }
  }
};
// int8 tiles, widened exactly to bf16 on the way into LDS.
struct LoadKC8 {
  uint4 r[2];
  __device__ void load(const int8_t *base, int64_t ld, int64_t row0, int64_t rows, int64_t k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int q = threadIdx.x + NT * i, row = q >> 2, kc = q & 3;
      int64_t gr = row0 + row;
      r[i] = gr < rows ? *(const uint4 *)(base + gr * ld + k0 + kc * 16) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ void store(bf16_t *t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int q = threadIdx.x + NT * i, row = q >> 2, kc = q & 3;
      const int8_t *v = (const int8_t *)&r[i];
      uint4 lo, hi;
      lo.x = i8pair_to_bf16x2(v[0], v[1]);   lo.y = i8pair_to_bf16x2(v[2], v[3]);
      lo.z = i8pair_to_bf16x2(v[4], v[5]);   lo.w = i8pair_to_bf16x2(v[6], v[7]);
      hi.x = i8pair_to_bf16x2(v[8], v[9]);   hi.y = i8pair_to_bf16x2(v[10], v[11]);
      hi.z = i8pair_to_bf16x2(v[12], v[13]); hi.w = i8pair_to_bf16x2(v[14], v[15]);
      *(uint4 *)(t + row * KC_LD + kc * 16) = lo;
      *(uint4 *)(t + row * KC_LD + kc * 16 + 8) = hi;
    }
  }
};
struct LoadKM8 {
  uint4 r[2];
  __device__ void load(const int8_t *base, int64_t ld, int64_t col0, int64_t k0, int64_t kend) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int q = threadIdx.x + NT * i, kr = q >> 3, c = q & 7;
      int64_t gk = k0 + kr;
      r[i] = gk < kend ? *(const uint4 *)(base + gk * ld + col0 + c * 16) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ void store(bf16_t *t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int q = threadIdx.x + NT * i, kr = q >> 3, c = q & 7;
      const int8_t *v = (const int8_t *)&r[i];
      uint4 lo, hi;
      lo.x = i8pair_to_bf16x2(v[0], v[1]);   lo.y = i8pair_to_bf16x2(v[2], v[3]);
      lo.z = i8pair_to_bf16x2(v[4], v[5]);   lo.w = i8pair_to_bf16x2(v[6], v[7]);
      hi.x = i8pair_to_bf16x2(v[8], v[9]);   hi.y = i8pair_to_bf16x2(v[10], v[11]);
      hi.z = i8pair_to_bf16x2(v[12], v[13]); hi.w = i8pair_to_bf16x2(v[14], v[15]);
      *(uint4 *)(t + kr * KM_LD + c * 16) = lo;
      *(uint4 *)(t + kr * KM_LD + c * 16 + 8) = hi;
    }
  }
};

// ---- fragment reads ---------------------------------------------------------
// Operand fragment of v_mfma_f32_16x16x32_bf16: lane l holds 8 consecutive k
// (k = 8*(l/16) .. +7) of row/column (l % 16) of a 16-wide slab.
__device__ inline bf16x8 frag_kc(const bf16_t *t, int r0, int ks) {
  int l = threadIdx.x & 63;
  s16x8 v = *(const s16x8 *)(t + (r0 + (l & 15)) * KC_LD + ks + 8 * (l >> 4));
  return __builtin_bit_cast(bf16x8, v);
}
// Same fragment from a k-major tile: ds_read_b64_tr_b16 hands lane i of a 16-lane
// group element i%4 of the 8-byte chunk read by lane 4e + i/4, for e = 0..3; with
// lane j reading row kb + j/4, columns c0 + 4*(j%4) .. +3, lane i receives the four
// k values kb..kb+3 of column c0 + i.
__device__ inline bf16x8 frag_km(const bf16_t *t, int c0, int ks) {
  int l = threadIdx.x & 63, g = l >> 4, j = l & 15;
  const bf16_t *p0 = t + (ks + 8 * g + (j >> 2)) * KM_LD + c0 + 4 * (j & 3);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + 4 * KM_LD));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// ROLE only separates the instantiations per use (distinct kernel symbols in traces).
template <int ROLE, bool AKM, bool BKM, bool BI8, bool OUTF32>
__global__ __launch_bounds__(NT) void k_mfma_gemm(KArgs a) {
  __shared__ __align__(16) bf16_t sA[2][TILE_ELEMS];
  __shared__ __align__(16) bf16_t sB[2][TILE_ELEMS];
  const int64_t z = blockIdx.z, bidx = z / a.splits, kz = z % a.splits;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t kbeg = kz * a.Kc;
  const int64_t kend = (kbeg + a.Kc < a.K) ? kbeg + a.Kc : a.K;
  const bf16_t *A = a.A + bidx * a.sAb;
  const int wave = threadIdx.x >> 6, wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  using LA = typename std::conditional<AKM, LoadKM, LoadKC>::type;
  using LB = typename std::conditional<BI8, typename std::conditional<BKM, LoadKM8, LoadKC8>::type,
                                       typename std::conditional<BKM, LoadKM, LoadKC>::type>::type;
  using TB = typename std::conditional<BI8, int8_t, bf16_t>::type;
  const TB *B = (const TB *)a.B + bidx * a.sBb;
  LA la;
  LB lb;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto gload = [&](int64_t k0) {
    if constexpr (AKM) la.load(A, a.lda, m0, k0, kend);
    else la.load(A, a.lda, m0, a.M, k0);
    if constexpr (BKM) lb.load(B, a.ldb, n0, k0, kend);
    else lb.load(B, a.ldb, n0, a.N, k0);
  };

  if (kbeg < kend) {
    gload(kbeg);
    la.store(sA[0]);
    lb.store(sB[0]);
    __syncthreads();
  }
  int cur = 0;
  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    const bool more = k0 + BK < kend;
    if (more) gload(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = AKM ? frag_km(sA[cur], wm + 16 * i, ks) : frag_kc(sA[cur], wm + 16 * i, ks);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = BKM ? frag_km(sB[cur], wn + 16 * j, ks) : frag_kc(sB[cur], wn + 16 * j, ks);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          // operands swapped: lane l then holds C[m = l%16][n = 4*(l/16) + 0..3]
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      la.store(sA[cur ^ 1]);
      lb.store(sB[cur ^ 1]);
    }
    __syncthreads();
    cur ^= 1;
  }

  // epilogue
  const int l = threadIdx.x & 63;
  char *Cb = (char *)a.C + (bidx * a.sCb + kz * a.sCsplit) * (OUTF32 ? 4 : 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t m = m0 + wm + 16 * i + (l & 15);
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t n = n0 + wn + 16 * j + 4 * (l >> 4);
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

bool mfma_supported(const MfmaDesc &d) {
  if (d.N % BN) return false;
  if (d.a_km && d.M % BM) return false;
  if (d.splits < 1) return false;
  if (!d.a_km || !d.b_km) {  // a k-contiguous operand needs whole 64-wide k slices
    if (d.K % BK) return false;
  }
  if (d.splits > 1 && (d.kchunk <= 0 || d.kchunk % BK || cdiv(d.K, d.kchunk) != d.splits)) return false;
  if (d.b_dt != POETX_BF16 && d.b_dt != POETX_I8) return false;
  if (d.c_dt != POETX_BF16 && d.c_dt != POETX_F32) return false;
  if (cdiv(d.M, BM) > 65535 || d.batch * d.splits > 65535) return false;
  return true;
}

template <int ROLE, bool AKM, bool BKM, bool BI8>
static int run_c(const KArgs &k, const MfmaDesc &d, dim3 grid, hipStream_t s) {
  if (d.c_dt == POETX_F32)
    return launch_k(d.name, s, k_mfma_gemm<ROLE, AKM, BKM, BI8, true>, grid, NT, 0, k);
  return launch_k(d.name, s, k_mfma_gemm<ROLE, AKM, BKM, BI8, false>, grid, NT, 0, k);
}

int gemm_mfma(const MfmaDesc &d, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0 || d.batch <= 0) return POETX_OK;
  if (!mfma_supported(d)) return POETX_ERR_UNSUPPORTED;
  KArgs k;
  k.M = d.M; k.N = d.N; k.K = d.K;
  k.splits = (int)d.splits;
  k.Kc = d.splits > 1 ? d.kchunk : d.K;
  k.A = (const bf16_t *)d.A; k.lda = d.lda; k.sAb = d.sAb;
  k.B = d.B; k.ldb = d.ldb; k.sBb = d.sBb;
  k.C = d.C; k.ldc = d.ldc; k.sCb = d.sCb; k.sCsplit = d.sCsplit;
  k.scaleN = d.scaleN;
  k.sSNb = d.sSNb;
  dim3 grid((unsigned)(d.N / BN), (unsigned)cdiv(d.M, BM), (unsigned)(d.batch * d.splits));
  const bool i8 = d.b_dt == POETX_I8;
  // the operand layouts each use needs; anything else is rejected
  switch (d.role) {
    case MFMA_GEMM_NT:
      if (d.a_km || d.b_km) return POETX_ERR_UNSUPPORTED;
      return i8 ? run_c<MFMA_GEMM_NT, false, false, true>(k, d, grid, s)
                : run_c<MFMA_GEMM_NT, false, false, false>(k, d, grid, s);
    case MFMA_GEMM_NN:
      if (d.a_km || !d.b_km) return POETX_ERR_UNSUPPORTED;
      return i8 ? run_c<MFMA_GEMM_NN, false, true, true>(k, d, grid, s)
                : run_c<MFMA_GEMM_NN, false, true, false>(k, d, grid, s);
    case MFMA_BLOCK_APPLY:
      if (d.a_km || !d.b_km || i8) return POETX_ERR_UNSUPPORTED;
      return run_c<MFMA_BLOCK_APPLY, false, true, false>(k, d, grid, s);
    case MFMA_BLOCK_APPLY_T:
      if (d.a_km || d.b_km || i8) return POETX_ERR_UNSUPPORTED;
      return run_c<MFMA_BLOCK_APPLY_T, false, false, false>(k, d, grid, s);
    case MFMA_BLOCK_GRAD:
      if (!d.a_km || !d.b_km || i8) return POETX_ERR_UNSUPPORTED;
      return run_c<MFMA_BLOCK_GRAD, true, true, false>(k, d, grid, s);
    default:
      return POETX_ERR_UNSUPPORTED;
  }
}

}  // namespace poetx
