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
#include "lds_tiles.h"

namespace poetx {

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
