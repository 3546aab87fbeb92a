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
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

namespace {
constexpr int TM = 64, TK = 32, NTH = 256;
constexpr int A_LD = TK + 8;   // [64][40] bf16: 80-byte rows
constexpr int B_LD = TM + 16;  // [32][80] bf16: 160-byte rows

__device__ inline void split2(float x, uint16_t &hi, uint16_t &lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
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
  int64_t z = blockIdx.z;
  int sg = 0;
  if (z >= a.seg[0].nblk) { z -= a.seg[0].nblk; sg = 1; }
  const CnpMMSeg &S = a.seg[sg];
  const int64_t off = z * (int64_t)b * b;
  const float *A = S.A + off, *B = S.B + off;
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TM;
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
  if (a.b % TM || nz > 65535) return POETX_ERR_UNSUPPORTED;
  dim3 grid(a.b / TM, a.b / TM, (unsigned)nz);
  switch (a.b) {
    case 64: return launch(a.name, s, [&] { k_cnp_mm<2><<<grid, NTH, 0, s>>>(a); });
    case 128: return launch(a.name, s, [&] { k_cnp_mm<4><<<grid, NTH, 0, s>>>(a); });
    case 256: return launch(a.name, s, [&] { k_cnp_mm<8><<<grid, NTH, 0, s>>>(a); });
    case 512: return launch(a.name, s, [&] { k_cnp_mm<16><<<grid, NTH, 0, s>>>(a); });
    default: return launch(a.name, s, [&] { k_cnp_mm<0><<<grid, NTH, 0, s>>>(a); });
  }
}

}  // namespace poetx
