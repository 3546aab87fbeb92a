// Block-diagonal products on token-major activations (Method §3: one b x b block per
// group of b features, batched over the blocks): the streaming apply Y_j = X_j G_j or
// X_j G_j^T and the per-block gradients X_j^T dY_j.  HBM-bound at the layer's shapes.
#include "lds_tiles.h"

namespace poetx {

// Block-diagonal product arguments: Y_j = X_j . G_j (TRANS = false) or X_j . G_j^T
// (TRANS = true) for every b x b block j, where X_j, Y_j are columns [jb, (j+1)b) of
// token-major activations.
struct BSArgs {
  int64_t N, d;           // tokens, row stride (elements) of X and Y
  int nb, P;              // blocks; workgroups per (block, slice)
  const bf16_t *X; const bf16_t *G; bf16_t *Y;
  const float *scaleN;    // per output column (length d) or null
};


// Register-resident variant for b = 128 and 256: each of the NCW consumer waves keeps
// its b x (b/NCW) share of G_j (or G_j^T) as MFMA operand fragments in registers for
// the whole kernel, so one workgroup covers the block's full width -- every token tile
// of X_j is read once -- and the whole LDS is a ring of T-token tiles (more bytes in
// flight per CU than with G held in LDS).  At b = 256 the 8 consumers (64 VGPRs of G
// each) put two MFMA-issuing waves on every SIMD: a lone wave issues MFMAs at about
// two thirds of the SIMD's rate (measured on bare MFMAs), and with 4 consumers the
// kernel was bound by exactly that.
// G is staged once through the ring's LDS at the start.  Workgroup u covers block
// j = u % nb and token tiles p, p + P, ... with p = u / nb, so the blocks of the
// same token rows run side by side.
// b = 256 block products: tokens per ring stage and ring stages
#ifndef POETX_BR256_T
#define POETX_BR256_T 32
#define POETX_BR256_NST 7
#endif
template <int B, int T, int NST, bool TRANS, int NCW = 4>
__global__ __launch_bounds__(64 * (NCW + 2)) void k_block_reg(BSArgs a) {
  constexpr int NPW = 2;
  constexpr int NTW = B / (16 * NCW), NKS = B / 32, FM = T / 16;
  constexpr int A_ELEMS = T * B;
  // per consumer wave, its T x (B/NCW) output tile is restaged in LDS so that the
  // global stores are 16 bytes per lane along rows
  constexpr int OW = B / NCW, OCH = OW / 8, O_ELEMS = T * OW;
  static_assert(NST * A_ELEMS + NCW * O_ELEMS >= B * B, "G is staged in the ring");
  extern __shared__ __align__(16) bf16_t smem[];
  const int u = blockIdx.x;
  if (u >= a.nb * a.P) return;
  const int p = u / a.nb, j = u % a.nb;
  const int64_t ntile = (a.N + T - 1) / T;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const bool producer = wave >= NCW;
  const int n0 = wave * (B / NCW);  // a consumer's first output column within the block

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
  // this workgroup's tile count, once: the tiles after tile `it` are then cnt - 1 - it
  const int cnt = tile < ntile ? (int)((ntile - 1 - tile) / a.P) + 1 : 0;
  for (int it = 0; tile < ntile; ++it, tile += a.P) {
    if (producer) {
      // tiles it .. it + NST - 2 may be in flight (loads complete in order): wait for
      // tile it only
      const int later = cnt - 1 - it;
      wait_tiles<LX, NST - 2>(later < NST - 2 ? later : NST - 2);
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
    // A fragments double-buffered per pair of k steps: the next pair's LDS reads are
    // in flight while this pair's MFMAs issue
    bf16x8 fa[2][2][FM];
    auto read_pair = [&](int q, int s2) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[q][h][i] = frag_kc<B>(ta, 16 * i, 32 * (s2 + h));
    };
    read_pair(0, 0);
#pragma unroll
    for (int s2 = 0; s2 < NKS; s2 += 2) {
      const int q = (s2 / 2) & 1;
      if (s2 + 2 < NKS) read_pair(q ^ 1, s2 + 2);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int t = 0; t < NTW; ++t)
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gf[t][s2 + h], fa[q][h][i], acc[i][t], 0, 0, 0);
    }
    // epilogue: lane holds Y[m = l%16][n = 4*(l/16) + 0..3] of each 16 x 16 patch; the
    // bf16 tile goes to this wave's staging rows (16-byte chunks XOR-swizzled by row),
    // then back out 16 bytes per lane, 8 (b = 256) or 4 (b = 128) lanes per row
    bf16_t *so = smem + NST * A_ELEMS + wave * O_ELEMS;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int row = 16 * i + (l & 15), col = 16 * t + 4 * (l >> 4);
        f32x4 v = acc[i][t];
        if (a.scaleN) {
          float4 sc = *(const float4 *)(a.scaleN + (int64_t)j * B + n0 + col);
          v[0] *= sc.x; v[1] *= sc.y; v[2] *= sc.z; v[3] *= sc.w;
        }
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        const int pch = (col >> 3) ^ (row & (OCH - 1));
        *(uint2 *)(so + row * OW + pch * 8 + (col & 7)) = pk;
      }
    __builtin_amdgcn_wave_barrier();  // the wave's LDS writes precede its reads (in order)
#pragma unroll
    for (int k = 0; k < T * OCH / 64; ++k) {
      const int q = l + 64 * k, row = q / OCH, c = q % OCH;
      const int64_t m = tile * T + row;
      const uint4 v = *(const uint4 *)(so + row * OW + ((c ^ (row & (OCH - 1))) * 8));
      if (m < a.N) *(uint4 *)(a.Y + m * a.d + (int64_t)j * B + n0 + c * 8) = v;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load into LDS may outlive the workgroup
}
// b = 256 uses 8 consumers (64 registers of G each, 2 x 2 accumulator patches), 32-token
// tiles and a 7-stage ring; b = 128 and 64 4 consumers, 64-token tiles and 4 stages.  With
// the output staging that is 128, 80 or 40 KB of LDS.
template __global__ void k_block_reg<64, 64, 4, false>(BSArgs);
template __global__ void k_block_reg<64, 64, 4, true>(BSArgs);
template __global__ void k_block_reg<128, 64, 4, false>(BSArgs);
template __global__ void k_block_reg<128, 64, 4, true>(BSArgs);
template __global__ void k_block_reg<256, POETX_BR256_T, POETX_BR256_NST, false, 8>(BSArgs);
template __global__ void k_block_reg<256, POETX_BR256_T, POETX_BR256_NST, true, 8>(BSArgs);

// b = 512: a block's G (512 KB) is more than the registers of one CU hold, so a workgroup covers
// one 256-column half of block j's output.  Its eight waves keep that half of G_j (or G_j^T)
// as MFMA operand fragments in registers, 512 x 32 each (128 VGPRs), and issue their own
// direct-to-LDS loads of T-token tiles of X_j (all 512 input columns) into an NST-stage
// ring.  The two halves of a block read the same token tiles in the same order on the
// same XCD (workgroups u and u ^ 8), so the second read of a tile is an L2 hit and X is
// read from HBM about once.  G's half is staged through LDS in two k halves at the start.
template <int T, int NST, bool TRANS>
__global__ __launch_bounds__(512) void k_block_half512(BSArgs a) {
  constexpr int B = 512, CS = 256, NW = 8, KH = 256;
  constexpr int NTW = CS / (16 * NW), NKS = B / 32, FM = T / 16;
  constexpr int A_ELEMS = T * B;
  constexpr int OW = CS / NW, OCH = OW / 8, O_ELEMS = T * OW;
  static_assert(NTW == 2 && NKS % 2 == 0, "wave layout");
  extern __shared__ __align__(16) bf16_t smem[];
  // workgroup u: half = bit 3, (token partition, block) from the other bits
  const int u = blockIdx.x;
  const int half = (u >> 3) & 1, q = (u & 7) | ((u >> 4) << 3);
  if (q >= a.nb * a.P) return;
  const int p = q / a.nb, j = q % a.nb;
  const int64_t ntile = (a.N + T - 1) / T;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int c0 = half * CS, n0 = wave * OW;  // the half's first column; the wave's within it

  // ---- this wave's 32 columns of the half, all 512 k, into registers (two k halves)
  bf16x8 gf[NTW][NKS];
  {
    const bf16_t *Gj = a.G + (int64_t)j * B * B;
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(Gj, (int64_t)B * B * 2);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      if constexpr (TRANS) {
        LoaderKC<CS, NW, KH> lg;  // rows n of G_j (k contiguous): G_j^T fragments via frag_kc
        lg.init(B, c0);
        lg.issue(rg, kh * KH, B, smem);
      } else {
        LoaderKM<CS, NW, KH> lg;  // rows k of G_j, the half's columns: G_j fragments via frag_km
        lg.init(B, c0);
        lg.issue(rg, kh * KH, B, smem);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int s = 0; s < NKS / 2; ++s)
          gf[t][kh * (NKS / 2) + s] = TRANS ? frag_kc<KH>(smem, n0 + 16 * t, 32 * s) : frag_km<CS>(smem, n0 + 16 * t, 32 * s);
      __syncthreads();  // the next k half (or the ring) may now overwrite the staging
    }
  }

  using LXT = LoaderKC<T, NW, B>;
  constexpr int LX = LXT::INSTR;
  LXT lx;
  const bf16_t *Xj = a.X + (int64_t)j * B;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(Xj, a.N * a.d * 2);
  lx.init(a.d, 0);
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) {
    const int64_t tl = p + (int64_t)s * a.P;
    if (tl < ntile) lx.issue(rx, tl * T * a.d, a.d, smem + s * A_ELEMS);
  }
  bf16_t *so = smem + NST * A_ELEMS + wave * O_ELEMS;
  int64_t tile = p;
  // this workgroup's tile count, once: the tiles after tile `it` are then cnt - 1 - it
  const int cnt = tile < ntile ? (int)((ntile - 1 - tile) / a.P) + 1 : 0;
  for (int it = 0; tile < ntile; ++it, tile += a.P) {
    // tiles it+1 .. it+NST-2 may still be in flight behind tile it (loads complete in order;
    // the epilogue's stores, also counted, only make the wait longer)
    const int later = cnt - 1 - it;
    wait_tiles<LX, NST - 2>(later < NST - 2 ? later : NST - 2);
    __syncthreads();  // every wave's share of tile it is in LDS; tile it-1's stage is free
    const int64_t nx = tile + (int64_t)(NST - 1) * a.P;
    if (nx < ntile) lx.issue(rx, nx * T * a.d, a.d, smem + ((it + NST - 1) % NST) * A_ELEMS);
    const bf16_t *ta = smem + (it % NST) * A_ELEMS;
    f32x4 acc[FM][NTW];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int t = 0; t < NTW; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 fa[2][2][FM];
    auto read_pair = [&](int qq, int s2) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[qq][h][i] = frag_kc<B>(ta, 16 * i, 32 * (s2 + h));
    };
    read_pair(0, 0);
#pragma unroll
    for (int s2 = 0; s2 < NKS; s2 += 2) {
      const int qq = (s2 / 2) & 1;
      if (s2 + 2 < NKS) read_pair(qq ^ 1, s2 + 2);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int t = 0; t < NTW; ++t)
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gf[t][s2 + h], fa[qq][h][i], acc[i][t], 0, 0, 0);
    }
    // epilogue as in k_block_reg: lane holds Y[m = l%16][n = 4*(l/16) + 0..3] of each patch;
    // the wave's T x 32 tile is restaged (chunks XOR-swizzled by row) and leaves 16 bytes per lane
    const int64_t col0 = (int64_t)j * B + c0 + n0;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int row = 16 * i + (l & 15), col = 16 * t + 4 * (l >> 4);
        f32x4 v = acc[i][t];
        if (a.scaleN) {
          float4 sc = *(const float4 *)(a.scaleN + col0 + col);
          v[0] *= sc.x; v[1] *= sc.y; v[2] *= sc.z; v[3] *= sc.w;
        }
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        const int pch = (col >> 3) ^ (row & (OCH - 1));
        *(uint2 *)(so + row * OW + pch * 8 + (col & 7)) = pk;
      }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int k = 0; k < T * OCH / 64; ++k) {
      const int qr = l + 64 * k, row = qr / OCH, c = qr % OCH;
      const int64_t m = tile * T + row;
      const uint4 v = *(const uint4 *)(so + row * OW + ((c ^ (row & (OCH - 1))) * 8));
      if (m < a.N) *(uint4 *)(a.Y + m * a.d + col0 + c * 8) = v;
    }
    __builtin_amdgcn_wave_barrier();  // the staging rows are rewritten next iteration
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load into LDS may outlive the workgroup
}
// 32-token tiles and a 4-stage ring (144 KB of LDS with the output staging): at workload 4's
// P side (28 blocks, 8192 tokens) 142 us, against 179 us with 16-token tiles and 6 stages
// and 163 us for the batched 256 x 256 GEMM tiles
#ifndef POETX_H512_T
#define POETX_H512_T 32
#endif
#ifndef POETX_H512_NST
#define POETX_H512_NST 4
#endif
template __global__ void k_block_half512<POETX_H512_T, POETX_H512_NST, false>(BSArgs);
template __global__ void k_block_half512<POETX_H512_T, POETX_H512_NST, true>(BSArgs);

template <bool TRANS>
static int run_h512(BSArgs a, const char *name, hipStream_t s) {
  constexpr int T = POETX_H512_T, NST = POETX_H512_NST;
  const size_t ring = (size_t)NST * T * 512 * 2 + (size_t)8 * T * 32 * 2, stage_g = (size_t)256 * 256 * 2;
  const size_t lds = ring > stage_g ? ring : stage_g;
  static std::atomic<uint64_t> attr{0};
  POETX_TRY(lds_limit(reinterpret_cast<const void *>(&k_block_half512<T, NST, TRANS>), lds, attr));
  // one workgroup per CU: (token partition, block) pairs times two halves, in groups of 16
  const int cus = device_cus() > 0 ? device_cus() : 256;
  const int64_t ntile = (a.N + T - 1) / T;
  int64_t P = cus / (2 * a.nb);
  if (P > ntile) P = ntile;
  a.P = (int)(P < 1 ? 1 : P);
  const int64_t q = (int64_t)a.nb * a.P;
  const dim3 grid((unsigned)(16 * ((q + 7) / 8)));
  return launch_k(name, s, k_block_half512<T, NST, TRANS>, grid, 512, lds, a);
}

template <int B, int T, int NST, bool TRANS, int NCW = 4>
static int run_br(const BSArgs &a, const char *name, hipStream_t s) {
  const size_t lds = (size_t)(NST + 1) * T * B * 2;  // ring + NCW output staging tiles
  static std::atomic<uint64_t> attr{0};
  POETX_TRY(lds_limit(reinterpret_cast<const void *>(&k_block_reg<B, T, NST, TRANS, NCW>), lds, attr));
  const dim3 grid((unsigned)(a.nb * a.P));
  return launch_k(name, s, k_block_reg<B, T, NST, TRANS, NCW>, grid, 64 * (NCW + 2), lds, a);
}

bool block_stream_supported(int64_t b, int64_t ld, int64_t nb, int64_t n_tokens) {
  if (b != 64 && b != 128 && b != 256 && b != 512) return false;
  if (nb < 1 || nb * b > ld || ld % 8) return false;
  return (n_tokens + 64) * ld * 2 < 0x7fffffff;
}

int block_stream(const bf16_t *X, const bf16_t *G, bf16_t *Y, int64_t n_tokens, int64_t ld, int64_t nb,
                 int64_t b, bool transposed, const float *scaleN, const char *name, hipStream_t s) {
  if (n_tokens <= 0) return POETX_OK;
  if (!block_stream_supported(b, ld, nb, n_tokens)) return POETX_ERR_UNSUPPORTED;
  BSArgs a;
  a.N = n_tokens; a.d = ld; a.nb = (int)nb;
  a.X = X; a.G = G; a.Y = Y; a.scaleN = scaleN;
  if (b == 512) return transposed ? run_h512<true>(a, name, s) : run_h512<false>(a, name, s);
  const int cus = device_cus() > 0 ? device_cus() : 256;
  if (b == 64 || b == 128 || b == 256) {
    // one workgroup per (token partition, block), about one per CU in total
    const int tt = b == 256 ? 32 : 64;
    const int64_t ntile = (n_tokens + tt - 1) / tt;
    int64_t P = cus / a.nb;
    if (P > ntile) P = ntile;
    a.P = (int)(P < 1 ? 1 : P);
    if (b == 64) return transposed ? run_br<64, 64, 4, true>(a, name, s) : run_br<64, 64, 4, false>(a, name, s);
    if (b == 128) return transposed ? run_br<128, 64, 4, true>(a, name, s) : run_br<128, 64, 4, false>(a, name, s);
    return transposed ? run_br<256, POETX_BR256_T, POETX_BR256_NST, true, 8>(a, name, s)
                      : run_br<256, POETX_BR256_T, POETX_BR256_NST, false, 8>(a, name, s);
  }
  return POETX_ERR_UNSUPPORTED;
}


// Streaming block gradient: parts[p][j][r][c] = sum over the token tiles t = p, p+P, ...
// of Xs_j[t]^T dY_j[t], for every b x b block j (r indexes columns of Xs_j, c of dY_j).
// Each workgroup owns one S x S slice (rs, cs) of one block's gradient, S = min(b, 128),
// and keeps it in registers while T-token tiles of both operands stream through an NST-stage
// LDS ring (two producer waves that only issue the global->LDS loads).  The P partials per
// block are summed later in a fixed order; with P = 1 the slices are the gradient itself.
// The (b/S)^2 slices of a block run on one XCD, so that an operand column slice, which b/S
// workgroups read, can come from HBM once.
struct BGArgs {
  int64_t N, d;
  int nb, P;
  const bf16_t *Xs; const bf16_t *dY; float *parts;  // parts: [P][nb][b][b]
};

template <int B, int S, int NST, int T, int NPW>
__global__ __launch_bounds__(64 * (4 + NPW)) void k_block_grad_stream(BGArgs a) {
  static_assert(S == 64 || S == 128, "slice width");
  static_assert(B % S == 0, "whole slices");
  constexpr int NCW = 4, KH = T / 32;
  constexpr int NSL = (B / S) * (B / S);
  constexpr int WT = S / 2, F = WT / 16;  // 2 x 2 waves of S/2 x S/2
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
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
      if (p + (int64_t)s * a.P < ntile) issue(p + (int64_t)s * a.P, s);
  }
  f32x4 acc[F][F];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int jj = 0; jj < F; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  int64_t tile = p;
  // this workgroup's tile count, once: the tiles after tile `it` are then cnt - 1 - it
  const int cnt = tile < ntile ? (int)((ntile - 1 - tile) / a.P) + 1 : 0;
  for (int it = 0; tile < ntile; ++it, tile += a.P) {
    if (producer) {
      // tiles it .. it + NST - 2 may be in flight (loads complete in order): wait for
      // tile it only
      const int later = cnt - 1 - it;
      wait_tiles<LPT, NST - 2>(later < NST - 2 ? later : NST - 2);
    }
    __syncthreads();
    if (producer) {
      const int64_t nx = tile + (int64_t)(NST - 1) * a.P;
      if (nx < ntile) issue(nx, (it + NST - 1) % NST);
      continue;
    }
    const bf16_t *ta = smem + (2 * (it % NST)) * TILE, *tb = ta + TILE;
    // per 32-token half: its fragments, then its MFMAs (the compiler overlaps the second
    // half's LDS reads with the first half's MFMAs)
    bf16x8 fa[KH][F], fb[KH][F];
#pragma unroll
    for (int hh = 0; hh < KH; ++hh) {
#pragma unroll
      for (int i = 0; i < F; ++i) fa[hh][i] = frag_km<S>(ta, wm + 16 * i, 32 * hh);
#pragma unroll
      for (int jj = 0; jj < F; ++jj) fb[hh][jj] = frag_km<S>(tb, wn + 16 * jj, 32 * hh);
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int jj = 0; jj < F; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[hh][jj], fa[hh][i], acc[i][jj], 0, 0, 0);
    }
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
// ring of BG_NST stages of two BG_T-token operand tiles, BG_NPW producer waves
#ifndef POETX_BG_NST
#define POETX_BG_NST 4
#endif
#ifndef POETX_BG_T
#define POETX_BG_T 64
#endif
#ifndef POETX_BG_NPW
#define POETX_BG_NPW 2
#endif
constexpr int BG_NST = POETX_BG_NST, BG_T = POETX_BG_T, BG_NPW = POETX_BG_NPW;
#define POETX_BG_INST(B, S) template __global__ void k_block_grad_stream<B, S, BG_NST, BG_T, BG_NPW>(BGArgs);
POETX_BG_INST(64, 64)
POETX_BG_INST(128, 128)
POETX_BG_INST(256, 128)
POETX_BG_INST(512, 128)
#undef POETX_BG_INST

template <int B>
static int run_bg(const BGArgs &a, hipStream_t s) {
  constexpr int S = B < 128 ? B : 128, NSL = (B / S) * (B / S);
  const size_t lds = (size_t)BG_NST * 2 * BG_T * S * 2;
  const int64_t units = (int64_t)a.nb * a.P;
  dim3 grid((unsigned)(((units + 7) / 8) * 8 * NSL));
  static std::atomic<uint64_t> attr{0};
  POETX_TRY(lds_limit(reinterpret_cast<const void *>(&k_block_grad_stream<B, S, BG_NST, BG_T, BG_NPW>), lds, attr));
  return launch_k("block_grad", s, k_block_grad_stream<B, S, BG_NST, BG_T, BG_NPW>, grid, 64 * (4 + BG_NPW), lds, a);
}

bool block_grad_stream_supported(int64_t b, int64_t ld, int64_t nb, int64_t n_tokens) {
  if (b != 64 && b != 128 && b != 256 && b != 512) return false;
  if (nb < 1 || nb * b > ld || ld % 8) return false;
  return (n_tokens + 64) * ld * 2 < 0x7fffffff;
}

int64_t block_grad_stream_parts(int64_t b, int64_t nb, int64_t n_tokens) {
  // about one workgroup per CU in a single round: rounding the partition count up would
  // start a second, mostly idle round
  const int64_t sl = b < 128 ? b : 128, slices = nb * (b / sl) * (b / sl);
  const int cus = device_cus() > 0 ? device_cus() : 256;
  int64_t P = cus / slices;
  // more partitions past kMaxChain tokens each: a float32 accumulation over millions of
  // tokens in one chain loses digits
  if (P < cdiv(n_tokens, kMaxChain)) P = cdiv(n_tokens, kMaxChain);
  const int64_t ntile = (n_tokens + BG_T - 1) / BG_T;
  if (P > ntile) P = ntile;
  return P < 1 ? 1 : P;
}

int block_grad_stream(const bf16_t *Xs, const bf16_t *dY, float *parts, int64_t n_tokens, int64_t ld, int64_t nb,
                      int64_t b, hipStream_t s) {
  if (!block_grad_stream_supported(b, ld, nb, n_tokens)) return POETX_ERR_UNSUPPORTED;
  BGArgs a;
  a.N = n_tokens; a.d = ld; a.nb = (int)nb;
  a.P = (int)block_grad_stream_parts(b, nb, n_tokens);
  a.Xs = Xs; a.dY = dY; a.parts = parts;
  if (b == 64) return run_bg<64>(a, s);
  if (b == 128) return run_bg<128>(a, s);
  if (b == 256) return run_bg<256>(a, s);
  return run_bg<512>(a, s);
}

}  // namespace poetx
