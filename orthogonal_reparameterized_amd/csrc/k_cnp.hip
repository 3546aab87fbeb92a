// Float32-accurate b x b products for the Cayley-Neumann steps, on bf16 MFMA.
//
// Every float32 operand x is split on its way into LDS as x = hi + lo with
// hi = bf16(x) and lo = bf16(x - hi) (both round-to-nearest-even), and
//     A.B ~= Ahi.Bhi + Ahi.Blo + Alo.Bhi
// accumulates in float32 (three v_mfma_f32_16x16x32_bf16 passes).  The dropped
// Alo.Blo term and the residual of the split are about 2^-16 of |A||B| per
// product, well inside float32-level accuracy for the CNP outputs.
//
// One launch computes, for every block z of up to two segments (the R and the
// P side of a layer) and every 64 x 64 output tile, up to two outputs
//     out_o[z] = alpha_o * A[z] . B[z] + sum_i ce_o[i] * E_i[z] + cI_o * I      (o = 0, 1)
// with A, B, E_i dense row-major float32 [b][b]; out_0 is written as float32 (C)
// and/or bf16 (Cb), out_1 as float32 (C2).  The k loop runs in 32-deep steps
// through two LDS stages (small footprint, so several workgroups share a CU).
#include "kernels.h"

namespace poetx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

namespace {
constexpr int TM = 64, TK = 32, NTH = 256;
constexpr int A_LD = TK + 8;   // [64][40] bf16: 80-byte rows
constexpr int B_LD = TM + 16;  // [32][80] bf16: 160-byte rows

__device__ inline void split2(float x, uint16_t &hi, uint16_t &lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}
// The same split of two floats at once, packed (element 0 in the low half): gfx950's
// v_cvt_pk_bf16_f32 rounds to nearest even like f32_to_bf16 (checked over every finite
// float), in one instruction per pair where the integer rounding takes three per value.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
#ifndef POETX_CVT_PK
#define POETX_CVT_PK 1
#endif
__device__ inline void split_pk(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  if constexpr (POETX_CVT_PK) {
    const f32x2 v = {x0, x1};
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    const f32x2 r = {x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xffff0000u)};
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
  } else {
    uint16_t h0, l0, h1, l1;
    split2(x0, h0, l0);
    split2(x1, h1, l1);
    hi = h0 | (uint32_t)h1 << 16;
    lo = l0 | (uint32_t)l1 << 16;
  }
}

__device__ inline bf16x8 frag_a(const bf16_t *t, int r0, int ks) {
  int l = threadIdx.x & 63;
  s16x8 v = *(const s16x8 *)(t + (r0 + (l & 15)) * A_LD + ks + 8 * (l >> 4));
  return __builtin_bit_cast(bf16x8, v);
}
// k-major tile fragment through ds_read_b64_tr_b16 (see the layout note in k_mfma.hip)
__device__ inline bf16x8 frag_b(const bf16_t *t, int c0, int ks) {
  int l = threadIdx.x & 63, g = l >> 4, j = l & 15;
  const bf16_t *p0 = t + (ks + 8 * g + (j >> 2)) * B_LD + c0 + 4 * (j & 3);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + 4 * B_LD));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}
}  // namespace

// NKS = b / 32 when known at compile time (the k loop is then fully unrolled, so the
// register ring has static slots); NKS = 0 handles any b % 64 == 0 with no ring.
template <int NKS>
__global__ __launch_bounds__(NTH) void k_cnp_mm(CnpMMArgs a) {
  __shared__ __align__(16) bf16_t sAh[2][TM * A_LD], sAl[2][TM * A_LD];
  __shared__ __align__(16) bf16_t sBh[2][TK * B_LD], sBl[2][TK * B_LD];
  const int b = a.b;
  // 1-D grid; workgroup L runs on XCD L % 8.  All tiles of one b x b block go to the
  // same XCD (block = xcd + 8 * (slot / T)), so each block's operands are fetched
  // into one L2 only; blocks past the last full group of 8 keep the plain order.
  const int tpr = b / TM, T = tpr * tpr;
  const int64_t nz = a.seg[0].nblk + a.seg[1].nblk, nz8 = nz & ~(int64_t)7;
  const int64_t L = blockIdx.x;
  int64_t z, t;
  if (L < nz8 * T) {
    const int64_t slot = L >> 3;
    z = (L & 7) + 8 * (slot / T);
    t = slot % T;
  } else {
    z = L / T;
    t = L % T;
  }
  int sg = 0;
  if (z >= a.seg[0].nblk) { z -= a.seg[0].nblk; sg = 1; }
  const CnpMMSeg &S = a.seg[sg];
  const int64_t off = z * (int64_t)b * b;
  const float *A = S.A + off, *B = S.B + off;
  const int m0 = (int)(t / tpr) * TM, n0 = (int)(t % tpr) * TM;
  const int tid = threadIdx.x, wave = tid >> 6, wm = (wave >> 1) * 32, wn = (wave & 1) * 32;

  // register ring of RD k-steps in flight: the small per-step MFMA work cannot cover a
  // global round trip, so loads are issued RD-1 steps ahead of their LDS store
  constexpr int RD = NKS ? 3 : 1;
  float4 ra[RD][2], rb[RD][2];
  auto gload = [&](int slot, int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int q = tid + NTH * i;                 // 512 float4 per operand tile
      int ar = q >> 3, ac = (q & 7) * 4;     // A tile: 64 rows x 32 k
      ra[slot][i] = *(const float4 *)(A + (int64_t)(m0 + ar) * b + k0 + ac);
      int br = q >> 4, bc = (q & 15) * 4;    // B tile: 32 k-rows x 64 columns
      rb[slot][i] = *(const float4 *)(B + (int64_t)(k0 + br) * b + n0 + bc);
    }
  };
  auto lstore = [&](int slot, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int q = tid + NTH * i;
      int ar = q >> 3, ac = (q & 7) * 4;
      int br = q >> 4, bc = (q & 15) * 4;
      uint16_t h[4], l[4];
      split2(ra[slot][i].x, h[0], l[0]); split2(ra[slot][i].y, h[1], l[1]);
      split2(ra[slot][i].z, h[2], l[2]); split2(ra[slot][i].w, h[3], l[3]);
      *(uint2 *)(sAh[buf] + ar * A_LD + ac) = make_uint2(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16);
      *(uint2 *)(sAl[buf] + ar * A_LD + ac) = make_uint2(l[0] | (uint32_t)l[1] << 16, l[2] | (uint32_t)l[3] << 16);
      split2(rb[slot][i].x, h[0], l[0]); split2(rb[slot][i].y, h[1], l[1]);
      split2(rb[slot][i].z, h[2], l[2]); split2(rb[slot][i].w, h[3], l[3]);
      *(uint2 *)(sBh[buf] + br * B_LD + bc) = make_uint2(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16);
      *(uint2 *)(sBl[buf] + br * B_LD + bc) = make_uint2(l[0] | (uint32_t)l[1] << 16, l[2] | (uint32_t)l[3] << 16);
    }
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = NKS ? NKS : b / TK;
#pragma unroll
  for (int s = 0; s < RD; ++s)
    if (s < nk) gload(s, s * TK);
  lstore(0, 0);
  __syncthreads();
#pragma unroll
  for (int st = 0; st < (NKS ? NKS : nk); ++st) {
    const int cur = st & 1;
    if (st + RD < nk) gload(st % RD, (st + RD) * TK);  // slot st%RD was stored at step st-1
    bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ah[i] = frag_a(sAh[cur], wm + 16 * i, 0);
      al[i] = frag_a(sAl[cur], wm + 16 * i, 0);
      bh[i] = frag_b(sBh[cur], wn + 16 * i, 0);
      bl[i] = frag_b(sBl[cur], wn + 16 * i, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // operands swapped: lane l holds C[m = l%16][n = 4*(l/16) + 0..3]
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bl[j], ah[i], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh[j], al[i], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh[j], ah[i], acc[i][j], 0, 0, 0);
      }
    if (st + 1 < nk) lstore((st + 1) % RD, cur ^ 1);
    __syncthreads();
  }

  const int l = tid & 63;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + wm + 16 * i + (l & 15);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 16 * j + 4 * (l >> 4);
      const int64_t e = off + (int64_t)m * b + n;
      float4 ex[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        ex[t] = S.E[t] ? *(const float4 *)(S.E[t] + e) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        if (o == 1 && !S.C2) continue;
        f32x4 v = acc[i][j] * a.alpha[o];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float c = a.ce[o][t];
          v[0] += c * ex[t].x; v[1] += c * ex[t].y; v[2] += c * ex[t].z; v[3] += c * ex[t].w;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (m == n + c) v[c] += a.cI[o];
        if (o == 1) {
          *(float4 *)(S.C2 + e) = make_float4(v[0], v[1], v[2], v[3]);
          continue;
        }
        if (S.C) *(float4 *)(S.C + e) = make_float4(v[0], v[1], v[2], v[3]);
        if (S.Cb) {
          uint2 p;
          p.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
          p.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
          *(uint2 *)(S.Cb + e) = p;
        }
      }
    }
  }
}

template __global__ void k_cnp_mm<0>(CnpMMArgs);
template __global__ void k_cnp_mm<2>(CnpMMArgs);
template __global__ void k_cnp_mm<4>(CnpMMArgs);
template __global__ void k_cnp_mm<8>(CnpMMArgs);
template __global__ void k_cnp_mm<16>(CnpMMArgs);

int cnp_mm(const CnpMMArgs &a, hipStream_t s) {
  const int64_t nz = a.seg[0].nblk + a.seg[1].nblk;
  if (nz <= 0) return POETX_OK;
  const int64_t nwg = nz * (a.b / TM) * (a.b / TM);
  if (a.b % TM || nwg > 0x7fffffff) return POETX_ERR_UNSUPPORTED;
  dim3 grid((unsigned)nwg);
  switch (a.b) {
    case 64: return launch_k(a.name, s, k_cnp_mm<2>, grid, NTH, 0, a);
    case 128: return launch_k(a.name, s, k_cnp_mm<4>, grid, NTH, 0, a);
    case 256: return launch_k(a.name, s, k_cnp_mm<8>, grid, NTH, 0, a);
    case 512: return launch_k(a.name, s, k_cnp_mm<16>, grid, NTH, 0, a);
    default: return launch_k(a.name, s, k_cnp_mm<0>, grid, NTH, 0, a);
  }
}



// ================================================================ chains ====
// The forward is a chain of products by the same Q,
//   G = (((Q + 2I) Q + 2I) Q + 2I) Q + I                 (eq. 9, Horner in Q),
// and a row panel of X.Q needs only the same rows of X, so one workgroup runs the whole
// chain on a panel of rows, which stays in LDS as split planes.  Q never goes through LDS:
// the unpack stores its bf16 planes in MFMA fragment order (see cnp_frag_off), so each
// wave streams its own B fragments from L2 straight into registers with 16-byte
// coalesced loads, several k steps ahead, and the waves only meet at the end of each
// product, when the panel is replaced.  The backward (k_cnp_bwd5 below) is built the same
// way.
namespace {
constexpr int CTK = 32, CNTH = 512;

// RP: rows per panel (one workgroup).  32 fills the GPU from few blocks; 64 halves the
// streaming of Q (every panel workgroup streams all of Q once per product) when there
// are blocks enough for 4 workgroups per CU (b = 128 and 256).
// b = 512 panel height: 32 (two workgroups per CU) or 64 (one; half the Q streamed per row,
// but 288 workgroups for workload 4's 36 blocks and spills in the backward's first half:
// 122 / 165 / 157 against 102 / 158 / 132 us for the three chains)
#ifndef POETX_CHAIN512_RP
#define POETX_CHAIN512_RP 32
#endif

// NW: waves per workgroup.  16 waves split a 128-row panel into two 64-row halves, wave w
// and w + 8 taking the same columns: their streams of Q fragments are the same, so the
// second read of each can hit the CU's vector L1 and the panel asks L2 for half the bytes
// of two 64-row workgroups (same waves per SIMD, one workgroup per CU).  Measured slower
// at 4096 blocks of 256 (forward 1.75 against 1.64 ms), so it is off (POETX_CHAIN16).
template <int B, int RP, int NW = 8>
struct ChainCfg {
  static_assert(RP == 32 || (RP == 64 && B >= 128) || (RP == 128 && NW == 16 && B >= 128 && B <= 256),
                "panel height");
  static_assert(NW == 8 || RP == 128, "16 waves only for 128-row panels");
  static constexpr int NTH = 64 * NW;
  static constexpr int RW = RP / (NW / 8);            // rows of one wave's patch
  static constexpr int NK = B / CTK;                  // k steps per product
  static constexpr int NT = B / 16;                   // 16-column tiles of Q
  static constexpr int WM = B >= 128 ? RW / 16 : 1;   // 16-row tiles per wave
  static constexpr int WN = B >= 128 ? B / 128 : 1;   // 16-column tiles per wave
  // k steps of B fragments in flight per wave: enough bytes in flight to cover the
  // latency of the first product, whose fragments are not in L2 yet (a 64-row panel
  // spends twice the MFMAs on each fragment)
  static constexpr int D = B >= 512 ? 2 : RW == 64 ? 4 : (3 * NK < 8 ? 3 * NK : 8);
  static constexpr int A_LD = B + 8;
  static constexpr int NP = B / RP;                   // panels per block
};

__device__ inline bf16x8 frag_a_ld(const bf16_t *t, int ld, int r0, int k0) {
  int l = threadIdx.x & 63;
  s16x8 v = *(const s16x8 *)(t + (r0 + (l & 15)) * ld + k0 + 8 * (l >> 4));
  return __builtin_bit_cast(bf16x8, v);
}
__device__ inline void put_split4(bf16_t *h, bf16_t *lo, float4 v) {
  uint32_t a0, a1, c0, c1;
  split_pk(v.x, v.y, a0, c0);
  split_pk(v.z, v.w, a1, c1);
  *(uint2 *)h = make_uint2(a0, a1);
  *(uint2 *)lo = make_uint2(c0, c1);
}
}  // namespace

// QL: Q's planes carry a lo part.  With bf16 theta, Q is exact in bf16 (lo = 0): the lo
// plane is neither written nor read and the pass with Q_lo is dropped, which changes nothing
// but the work (two MFMA passes per product instead of three, half the Q bytes).
template <int B, int RP, int NW, bool QL>
__global__ __launch_bounds__(64 * NW) void k_cnp_chain(CnpChainArgs a) {
  using C = ChainCfg<B, RP, NW>;
  constexpr int NPL = QL ? 2 : 1;  // Q planes streamed
  extern __shared__ __align__(16) bf16_t smem[];
  bf16_t *sAh = smem, *sAl = smem + RP * C::A_LD;

  // 1-D grid, all panels of one block on one XCD (workgroup L runs on XCD L % 8)
  const int64_t nz = a.seg[0].nblk + a.seg[1].nblk, nz8 = nz & ~(int64_t)7;
  const int64_t L = blockIdx.x;
  int64_t z, pnl;
  if (L < nz8 * C::NP) {
    const int64_t slot = L >> 3;
    z = (L & 7) + 8 * (slot / C::NP);
    pnl = slot % C::NP;
  } else {
    z = L / C::NP;
    pnl = L % C::NP;
  }
  int sg = 0;
  if (z >= a.seg[0].nblk) { z -= a.seg[0].nblk; sg = 1; }
  const CnpChainSeg &S = a.seg[sg];
  const int64_t off = z * (int64_t)B * B;
  const int r0 = (int)pnl * RP;
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int mb = B >= 128 ? C::RW * (wave >> 3) : 16 * (wave >> 2);
  const int nb = B >= 128 ? (wave & 7) * (B / 8) : 16 * (wave & 3);

  // ---- B fragments of Q: chunk (k, t, plane) of 1 KB holds what lane l needs for
  // k step k and column tile t; this wave reads tiles nb/16 .. nb/16 + WN - 1.
  const bf16_t *qf = S.qp + 2 * off;
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(qf), (short)0, 4 * B * B, 0x00020000);
  const int voff = l * 16 + (nb / 16) * 2048;
  u32x4 fb[C::D][C::WN][NPL];
  auto fload = [&](int slot, int k) {
#pragma unroll
    for (int j = 0; j < C::WN; ++j)
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl)
        fb[slot][j][pl] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, voff, (k * C::NT + j) * 2048 + pl * 1024, 0));
  };
#pragma unroll
  for (int s = 0; s < C::D; ++s) fload(s, s % C::NK);

  // ---- start panel
  // X = Q[rows] + 2I: rows r0.. are k steps pnl * RP/32 .. of the fragment-ordered planes
  for (int q = tid; q < (RP / 32) * C::NT * 2 * 64; q += C::NTH) {
    const int ln = q & 63, pl = (q >> 6) & 1, t = (q >> 7) % C::NT, ks = (q >> 7) / C::NT;
    const u32x4 v = (QL || !pl) ? *(const u32x4 *)(qf + (((pnl * (RP / 32) + ks) * C::NT + t) * 2 + pl) * 512 + ln * 8)
                                : u32x4{0u, 0u, 0u, 0u};
    bf16_t *dst = (pl ? sAl : sAh) + (32 * ks + 8 * (ln >> 4)) * C::A_LD + 16 * t + (ln & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e * C::A_LD] = (bf16_t)(v[e >> 1] >> (16 * (e & 1)));
  }
  __syncthreads();
  if (tid < RP) sAh[tid * C::A_LD + r0 + tid] = 0x4000;  // bf16(2.0); Q has a zero diagonal
  __syncthreads();

  f32x4 acc[C::WM][C::WN];
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int NS = 3 * C::NK;
  // one k step of product p; st is always a compile-time value, p is one too for
  // b <= 256 (everything unrolled: every wait on the loads in flight is exact) and a
  // loop variable for b = 512 (three unrolled products would not fit the registers)
  auto step = [&](const int st, const int p) {
    const int g = p * C::NK + st;
    const int u = C::NK % C::D == 0 ? st % C::D : g % C::D;
    bf16x8 ah[C::WM], al[C::WM], fbh[C::WN], fbl[C::WN];
#pragma unroll
    for (int i = 0; i < C::WM; ++i) {
      ah[i] = frag_a_ld(sAh, C::A_LD, mb + 16 * i, st * CTK);
      al[i] = frag_a_ld(sAl, C::A_LD, mb + 16 * i, st * CTK);
    }
#pragma unroll
    for (int j = 0; j < C::WN; ++j) {
      fbh[j] = __builtin_bit_cast(bf16x8, fb[u][j][0]);
      if constexpr (QL) fbl[j] = __builtin_bit_cast(bf16x8, fb[u][j][NPL - 1]);
    }
    // operands swapped: lane l holds C[m = l%16][n = 4*(l/16) + 0..3]; pass-major
    // order puts the other accumulators between two passes on the same one
    if constexpr (QL) {
#pragma unroll
      for (int i = 0; i < C::WM; ++i)
#pragma unroll
        for (int j = 0; j < C::WN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fbl[j], ah[i], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::WM; ++i)
#pragma unroll
      for (int j = 0; j < C::WN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fbh[j], al[i], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < C::WM; ++i)
#pragma unroll
      for (int j = 0; j < C::WN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fbh[j], ah[i], acc[i][j], 0, 0, 0);
    if (g + C::D < NS) fload(u, (st + C::D) % C::NK);  // refill the slot just consumed

    if (st == C::NK - 1) {
      // ---- end of product p: every wave is done with the panel before it is replaced
      if (p < 2) __syncthreads();
#pragma unroll
      for (int i = 0; i < C::WM; ++i)
#pragma unroll
        for (int j = 0; j < C::WN; ++j) {
          const int m = mb + 16 * i + (l & 15), n = nb + 16 * j + 4 * (l >> 4);
          const int gm = r0 + m;  // row within the block
          f32x4 v = acc[i][j];
          const float d = p < 2 ? 2.f : 1.f;
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (gm == n + c) v[c] += d;
          if (p == 2) {
            const int64_t e = off + (int64_t)gm * B + n;
            if (S.out) *(float4 *)(S.out + e) = make_float4(v[0], v[1], v[2], v[3]);
            if (S.outb) {
              uint2 pk;
              pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
              pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
              *(uint2 *)(S.outb + e) = pk;
            }
          }
          if (p < 2)
            put_split4(sAh + m * C::A_LD + n, sAl + m * C::A_LD + n, make_float4(v[0], v[1], v[2], v[3]));
          acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      if (p < 2) __syncthreads();
    }
  };
  if constexpr (B >= 512) {
    static_assert(C::NK % C::D == 0, "slots must not depend on p");
#pragma unroll 1
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int st = 0; st < C::NK; ++st) step(st, p);
  } else {
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int st = 0; st < C::NK; ++st) step(st, p);
  }
}

#define POETX_CHAIN_INST(B, R, W)                                      \
  template __global__ void k_cnp_chain<B, R, W, true>(CnpChainArgs);  \
  template __global__ void k_cnp_chain<B, R, W, false>(CnpChainArgs);
POETX_CHAIN_INST(64, 32, 8)
POETX_CHAIN_INST(128, 32, 8)
POETX_CHAIN_INST(256, 32, 8)
POETX_CHAIN_INST(512, 32, 8)
POETX_CHAIN_INST(128, 64, 8)
POETX_CHAIN_INST(256, 64, 8)
#if POETX_CHAIN512_RP == 64
POETX_CHAIN_INST(512, 64, 8)
#endif
POETX_CHAIN_INST(128, 128, 16)
POETX_CHAIN_INST(256, 128, 16)
#undef POETX_CHAIN_INST

// ===================================================== five-product backward ====
// dtheta reads only the skew part D = Qbar - Qbar^T of the adjoint of eq. 9.  The adjoint
// is sum_k c_k sum_{i+j=k-1} Q^i A_k Q^j with A_k = Gb - Gb^T (k odd) or -(Gb + Gb^T)
// (k even), and the terms Q^i A_k Q^j and Q^j A_k Q^i are minus each other's transposes,
// so D = E - E^T where E keeps one term of each such pair (and half of each Q^i A Q^i):
//     E = K - 2HQ + 2KQ^2 - HQ^3 + QKQ - QHQ^2,   K = Gb - Gb^T,  H = Gb + Gb^T.
// Grouped by Horner,
//     J = 2K - HQ - QH,   F = -2H + QK + JQ,   E = K + FQ,
// every product of which a row panel C computes from rows C alone:
//   1a  Q[C] H and Q[C] K  (A: Q[C] in LDS; B: H and K, whose fragments are eight
//                           consecutive elements of a row of Gb and of a column of Gb)
//   1b  H[C] Q             (A: H[C] in LDS; B: Q's fragment-ordered planes)
//   2   J[C] Q             (J[C] replaces Q[C] in LDS)
//   3   F[C] Q             (F[C] replaces H[C]); E[C] = K[C] + F[C] Q is stored row-major.
// The pack reads E as it reads Qbar (dtheta_rc = E_rc - E_cr).  Five products in four
// passes over k: 15 MFMAs per 16 x 16 tile and k step (10 when Q is exact in bf16).  A
// regrouping that keeps Qbar itself needs eight (each row panel then also has to form
// Q^j[C,:] for j = 2, 3), and two launches with the six products of Horner in Q send three
// b x b intermediates through HBM.
#ifndef POETX_BWD5_DG
#define POETX_BWD5_DG 2
#endif
#ifndef POETX_BWD5_DQ
#define POETX_BWD5_DQ 4
#endif
#ifndef POETX_BWD5_ROLL256
#define POETX_BWD5_ROLL256 0
#endif
template <int B, int RP>
struct Bwd5Cfg {
  static_assert(RP == 32 || (RP == 64 && B >= 128 && B <= 256), "panel height");
  static constexpr int NK = B / CTK;
  static constexpr int NT = B / 16;
  static constexpr int WM = B >= 128 ? RP / 16 : 1;
  static constexpr int WN = B >= 128 ? B / 128 : 1;
  static constexpr int DG = B >= 512 ? 1 : POETX_BWD5_DG;  // k steps of Gb in flight (1a)
  static constexpr int DQ = B >= 512 ? 2 : (3 * NK < POETX_BWD5_DQ ? 3 * NK : POETX_BWD5_DQ);  // of Q
  static constexpr int A_LD = B + 8;
  static constexpr int NP = B / RP;
  static constexpr int MR = RP * B / CNTH;  // prologue: rows of H[C] per thread, one column each
  static_assert(CNTH % B == 0 && MR % 4 == 0, "prologue layout");
};

template <int B, int RP, bool QL>
__global__ __launch_bounds__(CNTH) void k_cnp_bwd5(CnpChainArgs a) {
  using C = Bwd5Cfg<B, RP>;
  constexpr int NPL = QL ? 2 : 1;  // Q planes streamed (see k_cnp_chain)
  constexpr int NK = C::NK, WM = C::WM, WN = C::WN, DQ = C::DQ, DG = C::DG, LD = C::A_LD;
  // ROLL: the k loops are rolled (one round of slots unrolled) instead of fully unrolled, so
  // that the kernel's code fits the instruction cache (b = 512: 2600 instructions against
  // 8900, 283 -> 263 us at workload 4)
  constexpr bool ROLL = B >= 512 ? true : (B >= 256 && POETX_BWD5_ROLL256);
  extern __shared__ __align__(16) bf16_t smem[];
  // slot A: Q[C], then J[C]; slot B: H[C], then F[C] (hi and lo planes, RP rows each)
  bf16_t *sAh = smem, *sAl = smem + RP * LD;
  bf16_t *sBh = smem + 2 * RP * LD, *sBl = smem + 3 * RP * LD;

  // 1-D grid, all panels of one block on one XCD (workgroup L runs on XCD L % 8)
  const int64_t nz = a.seg[0].nblk + a.seg[1].nblk, nz8 = nz & ~(int64_t)7;
  const int64_t L = blockIdx.x;
  int64_t z, pnl;
  if (L < nz8 * C::NP) {
    const int64_t slot = L >> 3;
    z = (L & 7) + 8 * (slot / C::NP);
    pnl = slot % C::NP;
  } else {
    z = L / C::NP;
    pnl = L % C::NP;
  }
  int sg = 0;
  if (z >= a.seg[0].nblk) { z -= a.seg[0].nblk; sg = 1; }
  const CnpChainSeg &S = a.seg[sg];
  const int64_t off = z * (int64_t)B * B;
  const int r0 = (int)pnl * RP;
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int mb = B >= 128 ? 0 : 16 * (wave >> 2);
  const int nb = B >= 128 ? wave * (B / 8) : 16 * (wave & 3);

  const bf16_t *qf = S.qp + 2 * off;
  const float *G = S.dg + off;
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(qf), (short)0, 4 * B * B, 0x00020000);
  const __amdgpu_buffer_rsrc_t rg =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(G), (short)0, 4 * B * B, 0x00020000);

  // ---- 1a operands: for k step kk and column tile j (n = nb + 16 j + l%16, k = 32 kk +
  // 8 (l/16) + e) lane l needs Gb[n][k] (32 contiguous bytes of row n) and Gb[k][n] (eight
  // rows, one element each; sixteen lanes read 64 contiguous bytes of each row)
  u32x4 grw[DG][WN][2];
  float gcl[DG][WN][8];
  const int goff = ((nb + (l & 15)) * B + 8 * (l >> 4)) * 4;
  const int coff = (8 * (l >> 4) * B + nb + (l & 15)) * 4;
  auto gload = [&](int slot, int kk) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        grw[slot][j][h] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, goff, (16 * j * B + kk * CTK) * 4 + 16 * h, 0));
#pragma unroll
      for (int e = 0; e < 8; ++e)
        gcl[slot][j][e] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rg, coff, ((kk * CTK + e) * B + 16 * j) * 4, 0));
    }
  };
  // ---- 1b, 2, 3 operand: Q's planes, chunk (k, t, plane) of 1 KB per k step and column tile
  u32x4 fq[DQ][WN][NPL];
  const int voff = l * 16 + (nb / 16) * 2048;
  auto qload = [&](int slot, int k) {
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl)
        fq[slot][j][pl] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, voff, (k * C::NT + j) * 2048 + pl * 1024, 0));
  };
#pragma unroll
  for (int s = 0; s < DG; ++s) gload(s, s);

  // ---- start panels: Q[C] (k steps pnl * RP/32 .. of the planes) into slot A, H[C] into slot B
  for (int q = tid; q < (RP / 32) * C::NT * 2 * 64; q += CNTH) {
    const int ln = q & 63, pl = (q >> 6) & 1, t = (q >> 7) % C::NT, ks = (q >> 7) / C::NT;
    const u32x4 v = (QL || !pl) ? *(const u32x4 *)(qf + (((pnl * (RP / 32) + ks) * C::NT + t) * 2 + pl) * 512 + ln * 8)
                                : u32x4{0u, 0u, 0u, 0u};
    bf16_t *dst = (pl ? sAl : sAh) + (32 * ks + 8 * (ln >> 4)) * LD + 16 * t + (ln & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e * LD] = (bf16_t)(v[e >> 1] >> (16 * (e & 1)));
  }
  {
    // thread: column kc of H[C], rows m0 .. m0 + MR - 1: H[m][kc] = Gb[r0 + m][kc] + Gb[kc][r0 + m]
    const int kc = tid % B, m0 = (tid / B) * C::MR;
    float tcol[C::MR];
#pragma unroll
    for (int c = 0; c < C::MR / 4; ++c) {
      const float4 v = *(const float4 *)(G + (int64_t)kc * B + r0 + m0 + 4 * c);
      tcol[4 * c] = v.x; tcol[4 * c + 1] = v.y; tcol[4 * c + 2] = v.z; tcol[4 * c + 3] = v.w;
    }
#pragma unroll
    for (int mm = 0; mm < C::MR; ++mm) {
      const int m = m0 + mm;
      uint16_t h, lo;
      split2(G[(int64_t)(r0 + m) * B + kc] + tcol[mm], h, lo);
      sBh[m * LD + kc] = h;
      sBl[m * LD + kc] = lo;
    }
  }
  __syncthreads();

  // H[C] and K[C] at the accumulator positions of patch (i, j): rows r0 + m, columns n .. n+3
  auto hk_at = [&](int i, int j, f32x4 &hv, f32x4 &kv) {
    const int m = mb + 16 * i + (l & 15), n = nb + 16 * j + 4 * (l >> 4);
    const float4 rw = *(const float4 *)(G + (int64_t)(r0 + m) * B + n);
    const float rr[4] = {rw.x, rw.y, rw.z, rw.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float cl = G[(int64_t)(n + c) * B + r0 + m];
      hv[c] = rr[c] + cl;
      kv[c] = rr[c] - cl;
    }
  };

  // the terms of J and F that are not products start in the accumulators of 1a:
  // accQH = -2K + Q[C]H (so that J = -(HQ + accQH)), accQK = -2H + Q[C]K = F - JQ
  f32x4 accQH[WM][WN], accQK[WM][WN], acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      f32x4 hv, kv;
      hk_at(i, j, hv, kv);
      accQH[i][j] = -2.f * kv;
      accQK[i][j] = -2.f * hv;
      acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // ---- 1a: Q[C] H and Q[C] K; the first DQ k steps of Q go out over the last steps (after
  // 1a when its loop is rolled)
  constexpr int QS0 = NK >= DQ ? NK - DQ : 0;
  auto step1a = [&](const int kk, const int u) {
    bf16x8 hh[WN], hl[WN], kh[WN], kl[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      // whole vectors are reinterpreted, then indexed: a bit cast of one element of a
      // vector (bit_cast(float, v[i])) reads element 0 whatever i is with this compiler
      const f32x4 g0 = __builtin_bit_cast(f32x4, grw[u][j][0]), g1 = __builtin_bit_cast(f32x4, grw[u][j][1]);
      u32x4 vh, vl, wh, wl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float r0v = e < 2 ? g0[2 * e] : g1[2 * e - 4], r1v = e < 2 ? g0[2 * e + 1] : g1[2 * e - 3];
        const float c0v = gcl[u][j][2 * e], c1v = gcl[u][j][2 * e + 1];
        uint32_t a0, a1, b0, b1;
        split_pk(c0v + r0v, c1v + r1v, a0, a1);  // H[k][n] = Gb[k][n] + Gb[n][k]
        split_pk(c0v - r0v, c1v - r1v, b0, b1);  // K[k][n] = Gb[k][n] - Gb[n][k]
        vh[e] = a0; vl[e] = a1; wh[e] = b0; wl[e] = b1;
      }
      hh[j] = __builtin_bit_cast(bf16x8, vh); hl[j] = __builtin_bit_cast(bf16x8, vl);
      kh[j] = __builtin_bit_cast(bf16x8, wh); kl[j] = __builtin_bit_cast(bf16x8, wl);
    }
    bf16x8 qh[WM], ql[WM];
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      qh[i] = frag_a_ld(sAh, LD, mb + 16 * i, kk * CTK);
      if constexpr (QL) ql[i] = frag_a_ld(sAl, LD, mb + 16 * i, kk * CTK);
    }
    if (kk + DG < NK) gload(u, kk + DG);
    if constexpr (!ROLL) {
#pragma unroll
      for (int s = 0; s < DQ; ++s)
        if (NK >= DQ ? kk == QS0 + s : kk == 0) qload(s, s % NK);
    }
    // operands swapped: lane l holds C[m = l%16][n = 4*(l/16) + 0..3]
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        accQH[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hl[j], qh[i], accQH[i][j], 0, 0, 0);
        accQK[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl[j], qh[i], accQK[i][j], 0, 0, 0);
      }
    if constexpr (QL) {
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          accQH[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hh[j], ql[i], accQH[i][j], 0, 0, 0);
          accQK[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh[j], ql[i], accQK[i][j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        accQH[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hh[j], qh[i], accQH[i][j], 0, 0, 0);
        accQK[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh[j], qh[i], accQK[i][j], 0, 0, 0);
      }
  };
  if constexpr (ROLL) {
    // a loop over rounds of the DG slots (one k step per slot), each round unrolled
    static_assert(NK % DG == 0 && NK % DQ == 0, "rolled loops need whole rounds of slots");
    constexpr int U1 = DG == 1 ? 2 : DG;
#pragma unroll 1
    for (int kb = 0; kb < NK; kb += U1)
#pragma unroll
      for (int c = 0; c < U1; ++c) step1a(kb + c, c % DG);
#pragma unroll
    for (int s = 0; s < DQ; ++s) qload(s, s % NK);
  } else {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) step1a(kk, kk % DG);
  }

  // ---- 1b, 2, 3: X Q for X = H[C], J[C], F[C], one k step at a time
  constexpr int NS = 3 * NK;
  auto qstep = [&](const int st, const int p, const int u) {
    const int g = p * NK + st;
    const bf16_t *xh = p == 1 ? sAh : sBh, *xl = p == 1 ? sAl : sBl;
    bf16x8 ah[WM], al[WM], fbh[WN], fbl[WN];
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      ah[i] = frag_a_ld(xh, LD, mb + 16 * i, st * CTK);
      al[i] = frag_a_ld(xl, LD, mb + 16 * i, st * CTK);
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      fbh[j] = __builtin_bit_cast(bf16x8, fq[u][j][0]);
      if constexpr (QL) fbl[j] = __builtin_bit_cast(bf16x8, fq[u][j][NPL - 1]);
    }
    if constexpr (QL) {
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fbl[j], ah[i], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fbh[j], al[i], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fbh[j], ah[i], acc[i][j], 0, 0, 0);
    if (g + DQ < NS) qload(u, (st + DQ) % NK);  // refill the slot just consumed

    if (st == NK - 1) {
      if (p == 0) {
        // J = 2K - HQ - QH into slot A (every wave is past 1a, the last reader of Q[C])
        __syncthreads();
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            const int m = mb + 16 * i + (l & 15), n = nb + 16 * j + 4 * (l >> 4);
            const f32x4 jv = -(acc[i][j] + accQH[i][j]);
            put_split4(sAh + m * LD + n, sAl + m * LD + n, make_float4(jv[0], jv[1], jv[2], jv[3]));
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        __syncthreads();
      } else if (p == 1) {
        // F = -2H + QK + JQ into slot B (H[C] was last read in 1b, before the barrier above);
        // the last product accumulates onto K[C]
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            const int m = mb + 16 * i + (l & 15), n = nb + 16 * j + 4 * (l >> 4);
            const f32x4 fv = accQK[i][j] + acc[i][j];
            put_split4(sBh + m * LD + n, sBl + m * LD + n, make_float4(fv[0], fv[1], fv[2], fv[3]));
            f32x4 hv, kv;
            hk_at(i, j, hv, kv);
            acc[i][j] = kv;
          }
        __syncthreads();
      } else {
        // E = K + FQ, row-major
        float *O = S.out + off;
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            const int m = mb + 16 * i + (l & 15), n = nb + 16 * j + 4 * (l >> 4);
            const f32x4 ev = acc[i][j];
            *(float4 *)(O + (int64_t)(r0 + m) * B + n) = make_float4(ev[0], ev[1], ev[2], ev[3]);
          }
      }
    }
  };
  if constexpr (ROLL) {
    // slot u of k step st is st % DQ: the inner loop over one round of slots is unrolled
#pragma unroll 1
    for (int p = 0; p < 3; ++p)
#pragma unroll 1
      for (int sb = 0; sb < NK; sb += DQ)
#pragma unroll
        for (int su = 0; su < DQ; ++su) qstep(sb + su, p, su);
  } else {
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int st = 0; st < NK; ++st) qstep(st, p, NK % DQ == 0 ? st % DQ : (p * NK + st) % DQ);
  }
}
#define POETX_BWD5_INST(B, R)                                              \
  template __global__ void k_cnp_bwd5<B, R, true>(CnpChainArgs);           \
  template __global__ void k_cnp_bwd5<B, R, false>(CnpChainArgs);
POETX_BWD5_INST(64, 32)
POETX_BWD5_INST(128, 32)
POETX_BWD5_INST(128, 64)
POETX_BWD5_INST(256, 32)
POETX_BWD5_INST(256, 64)
POETX_BWD5_INST(512, 32)
#undef POETX_BWD5_INST

// b = 512 on the row-panel chains; off, it takes the per-product launches (k_cnp_mm, two
// forward, six backward): measured slower at workload 4 (115 against 104 us forward, 345
// against 277 us backward)
#ifndef POETX_CHAIN512
#define POETX_CHAIN512 1
#endif
bool cnp_chain_supported(int64_t b) { return b == 64 || b == 128 || b == 256 || (POETX_CHAIN512 && b == 512); }
namespace {
template <int B, int RP, int NW = 8>
int chain_run(const CnpChainArgs &a, hipStream_t s) {
  using C = ChainCfg<B, RP, NW>;
  const int64_t nz = a.seg[0].nblk + a.seg[1].nblk;
  const int64_t nwg = nz * C::NP;
  if (nwg > 0x7fffffff) return POETX_ERR_UNSUPPORTED;
  const size_t lds = (size_t)2 * RP * C::A_LD * sizeof(bf16_t);
  static std::atomic<uint64_t> attr[2];  // dynamic LDS above 64 KB, per kernel and device
  auto go = [&](void (*kern)(CnpChainArgs), int id) -> int {
    POETX_TRY(lds_limit((const void *)kern, lds, attr[id]));
    return launch_k(a.name, s, kern, dim3((unsigned)nwg), C::NTH, lds, a);
  };
  return a.qlo ? go(k_cnp_chain<B, RP, NW, true>, 0) : go(k_cnp_chain<B, RP, NW, false>, 1);
}
}  // namespace

bool cnp_bwd5_supported(int64_t b) { return b == 64 || b == 128 || b == 256 || b == 512; }

namespace {
template <int B, int RP>
int bwd5_run(const CnpChainArgs &a, hipStream_t s) {
  using C = Bwd5Cfg<B, RP>;
  const int64_t nz = a.seg[0].nblk + a.seg[1].nblk;
  const int64_t nwg = nz * C::NP;
  if (nwg > 0x7fffffff) return POETX_ERR_UNSUPPORTED;
  const size_t lds = (size_t)4 * RP * C::A_LD * sizeof(bf16_t);
  static std::atomic<uint64_t> attr[2];  // dynamic LDS above 64 KB, per kernel and device
  if (a.qlo) {
    POETX_TRY(lds_limit((const void *)k_cnp_bwd5<B, RP, true>, lds, attr[0]));
    return launch_k(a.name, s, k_cnp_bwd5<B, RP, true>, dim3((unsigned)nwg), CNTH, lds, a);
  }
  POETX_TRY(lds_limit((const void *)k_cnp_bwd5<B, RP, false>, lds, attr[1]));
  return launch_k(a.name, s, k_cnp_bwd5<B, RP, false>, dim3((unsigned)nwg), CNTH, lds, a);
}
}  // namespace

int cnp_bwd5(const CnpChainArgs &a, hipStream_t s) {
  const int64_t nz = a.seg[0].nblk + a.seg[1].nblk;
  if (nz <= 0) return POETX_OK;
  // 64-row panels (half the streaming of Q per row) once they still give 4 workgroups per CU
  const int cus = device_cus() > 0 ? device_cus() : 256;
  const bool tall = nz * (a.b / 64) >= 4 * (int64_t)cus;
  switch (a.b) {
    case 64: return bwd5_run<64, 32>(a, s);
    case 128: return tall ? bwd5_run<128, 64>(a, s) : bwd5_run<128, 32>(a, s);
    case 256: return tall ? bwd5_run<256, 64>(a, s) : bwd5_run<256, 32>(a, s);
    case 512: return bwd5_run<512, 32>(a, s);
    default: return POETX_ERR_UNSUPPORTED;
  }
}

int cnp_chain(const CnpChainArgs &a, hipStream_t s) {
  const int64_t nz = a.seg[0].nblk + a.seg[1].nblk;
  if (nz <= 0) return POETX_OK;
  // 64-row panels once they still give 4 workgroups per CU
  const int cus = device_cus() > 0 ? device_cus() : 256;
  const bool tall = nz * (a.b / 64) >= 4 * (int64_t)cus;
#ifndef POETX_CHAIN16
#define POETX_CHAIN16 0
#endif
  // 128-row panels of 16 waves once they still give 2 workgroups per CU
  const bool tall2 = POETX_CHAIN16 && nz * (a.b / 128) >= 2 * (int64_t)cus;
  switch (a.b) {
    case 64: return chain_run<64, 32>(a, s);
    case 128: return tall2 ? chain_run<128, 128, 16>(a, s) : tall ? chain_run<128, 64>(a, s) : chain_run<128, 32>(a, s);
    case 256: return tall2 ? chain_run<256, 128, 16>(a, s) : tall ? chain_run<256, 64>(a, s) : chain_run<256, 32>(a, s);
    case 512: return POETX_CHAIN512_RP == 64 ? chain_run<512, 64>(a, s) : chain_run<512, 32>(a, s);
    default: return POETX_ERR_UNSUPPORTED;
  }
}

}  // namespace poetx
