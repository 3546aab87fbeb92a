// Host-side launchers of the HIP kernels (internal to libpoetx).
#pragma once

#include "common.h"

namespace poetx {

// ---------------------------------------------------------------------------
// Strided batched product on the vector ALUs with float32 accumulation:
//   C[z][m][n] = alpha * scaleN[z*sSNb + n] * sum_k (A[z][m][k] * scaleK[k]) * B[z][k][n]
//                + beta * D[z][m][n]
// Any strides; A/B dtypes F32, BF16 or I8; C dtype F32 or BF16; D float32 (optional).
// Used for float32 layers, for shapes outside the MFMA kernels' tiling, and as
// the building block of the float32 Cayley-Neumann steps.
// ---------------------------------------------------------------------------
struct GemmDesc {
  int64_t M = 0, N = 0, K = 0, batch = 1;
  const void *A = nullptr; int a_dt = POETX_F32; int64_t sAb = 0, sAm = 0, sAk = 0;
  const void *B = nullptr; int b_dt = POETX_F32; int64_t sBb = 0, sBk = 0, sBn = 0;
  void *C = nullptr;       int c_dt = POETX_F32; int64_t sCb = 0, sCm = 0, sCn = 0;
  const float *D = nullptr; int64_t sDb = 0, sDm = 0, sDn = 0;
  float alpha = 1.f, beta = 0.f;
  const float *scaleN = nullptr, *scaleK = nullptr;
  int64_t sSNb = 0;  // batch stride of scaleN
  const char *name = "gemm_generic";  // label for the measurement hooks
};
int gemm_generic(const GemmDesc &g, hipStream_t s);

// Column permutation of a row-major [rows][cols] matrix of esize-byte elements:
//   gather : out[r][i] = in[rperm ? rperm[r] : r][cperm[i]]
//   scatter: out[r][cperm[i]] = in[r][i]
int permute_cols(const void *in, void *out, int64_t rows, int64_t cols, int esize,
                 const int32_t *rperm, const int32_t *cperm, bool scatter, hipStream_t s);
// out[c][r] = in[r][c] ([rows][cols] -> [cols][rows]) for esize-byte elements
int transpose(const void *in, void *out, int64_t rows, int64_t cols, int esize, hipStream_t s);
// the same for each of batch contiguous bf16 matrices (rows, cols multiples of 8, 16-byte
// aligned pointers)
int transpose_batched(const void *in, void *out, int64_t batch, int64_t rows, int64_t cols, hipStream_t s);
// out[i] = src[perm[i]] for float32 vectors
int gather_f32(const float *src, float *out, int64_t n, const int32_t *perm, hipStream_t s);

// Packed skew helpers (Method §4 storage), over up to two segments of blocks:
//   unpack: dst = Q[n][b][b] from src = theta[n][b(b-1)/2]
//   pack  : dst = dtheta[k(i,j)] = M[i][j] - M[j][i] from src = M[n][b][b]
//   unpack with planes[0] set (b % 32 == 0): Q as bf16 planes hi = bf16(Q) and
//   lo = bf16(Q - hi) in MFMA fragment order (cnp_frag_off), instead of dst
// Element offset of Q[r][c] (hi plane; the lo plane is 512 further) within one
// block's 2 b^2 fragment-ordered planes: 1 KB chunks (k step kk = r / 32, column
// tile t = c / 16, plane), each the B operand of a v_mfma_f32_16x16x32_bf16 for
// that k step and tile, lane l holding Q[32 kk + 8 (l / 16) + e][16 t + l % 16]
// as element e = 0..7.
__host__ __device__ inline int64_t cnp_frag_off(int64_t r, int64_t c, int64_t b) {
  const int64_t kk = r >> 5, kr = r & 31, t = c >> 4;
  const int64_t lane = 16 * (kr >> 3) + (c & 15);
  return (kk * (b >> 4) + t) * 1024 + lane * 8 + (kr & 7);
}
// src: theta (unpack; float32, or bf16 when src_bf16) or M (pack; float32).
struct SkewSegs {
  const void *src[2] = {nullptr, nullptr};
  float *dst[2] = {nullptr, nullptr};
  bf16_t *planes[2] = {nullptr, nullptr};
  int64_t n[2] = {0, 0};
  int src_bf16 = 0;  // theta in bf16: Q is exact in bf16, and the planes' lo part (all zero) is not written
};
// Adam hyperparameters (step_size and rs2 carry the bias corrections) and, for the update
// fused into the pack of dtheta, the parameter and state buffers of up to two segments.
struct AdamEpi {
  const void *theta_in[2] = {nullptr, nullptr};
  void *theta_out[2] = {nullptr, nullptr};
  float *m[2] = {nullptr, nullptr}, *v[2] = {nullptr, nullptr};
  int theta_bf16 = 0;
  float step_size = 0.f, b1 = 0.f, b2 = 0.f, rs2 = 1.f, eps = 1.f;
};
// fused Adam pass on packed parameters (theta float32 or bf16)
int adam_step(int64_t n, void *theta, int theta_dt, const float *g, float *m, float *v, const AdamEpi &h,
              hipStream_t s);
// inv[perm[i]] = i for a permutation of 0 .. n-1
int invert_perm(const int32_t *perm, int32_t *inv, int64_t n, hipStream_t s);
int unpack_skew2(const SkewSegs &sg, int64_t b, hipStream_t s);
// with ad: the Adam update of theta fused into the same pass (dtheta written where sg.dst is set)
int pack_skew_grad2(const SkewSegs &sg, int64_t b, hipStream_t s, const AdamEpi *ad = nullptr);
int unpack_skew(const float *theta, float *Q, int64_t n, int64_t b, hipStream_t s);
int pack_skew_grad(const float *M, float *dtheta, int64_t n, int64_t b, hipStream_t s);
// out = c0*X0 + c1*X1 + c2*X2 + c3*X3 + cI*I over n blocks of b x b (null X_i skipped)
int lincomb(float *out, int64_t n, int64_t b, float cI, const float *X0, float c0,
            const float *X1, float c1, const float *X2, float c2, const float *X3, float c3,
            hipStream_t s);
// out[e] = sum_{p < parts} in[p * stride + e], in a fixed order (deterministic)
int fill_one(void *out, int64_t n, int dt, hipStream_t s);  // n values 1 (F32 or BF16)
// n blocks of size b embedded in blocks of size bp > b, zeros elsewhere, and back (the
// CNP of a block size without MFMA kernels runs at bp): modes below, esize 4 or 2 for the
// theta and G copies, 4 for dG and dtheta.
enum { CNP_PAD_THETA = 0, CNP_CUT_G = 1, CNP_PAD_DG = 2, CNP_CUT_DTHETA = 3 };
int cnp_pad(int mode, int64_t n, int64_t b, int64_t bp, int esize, const void *in, void *out, hipStream_t s);

int reduce_parts(const float *in, float *out, int64_t elems, int64_t parts, int64_t stride,
                 hipStream_t s);

// ---------------------------------------------------------------------------
// bf16 MFMA products (gfx950 v_mfma_f32_16x16x32_bf16), float32 accumulation.
//   C[z][m][n] = scaleN[z*sSNb + n] * sum_k A[z][m][k] * B[z][k][n]
// Operand layouts in memory:
//   A: a_km == false -> element (m, k) at A + z*sAb + m*lda + k      (k contiguous)
//      a_km == true  -> element (m, k) at A + z*sAb + k*lda + m      (m contiguous)
//   B: b_km == false -> element (k, n) at B + z*sBb + n*ldb + k      (k contiguous)
//      b_km == true  -> element (k, n) at B + z*sBb + k*ldb + n      (n contiguous)
//   C: element (m, n) at C + z*sCb + m*ldc + n, bf16 or float32
// Split-K: k range [kz*kchunk, (kz+1)*kchunk) of split kz goes to C + kz*sCsplit
// (kchunk a multiple of 64, splits == ceil(K / kchunk)).
// Requirements (checked): N % 64 == 0, K % 64 == 0 (per split), M any (masked).
// B may be I8 (converted exactly to bf16 in the kernel).
// ---------------------------------------------------------------------------
enum MfmaRole { MFMA_GEMM_NT = 0, MFMA_GEMM_NN, MFMA_BLOCK_APPLY, MFMA_BLOCK_APPLY_T, MFMA_BLOCK_GRAD };
struct MfmaDesc {
  int role = MFMA_GEMM_NT;
  int64_t M = 0, N = 0, K = 0, batch = 1, splits = 1, kchunk = 0;
  const void *A = nullptr; bool a_km = false; int64_t lda = 0, sAb = 0;
  const void *B = nullptr; bool b_km = false; int b_dt = POETX_BF16; int64_t ldb = 0, sBb = 0;
  void *C = nullptr; int c_dt = POETX_BF16; int64_t ldc = 0, sCb = 0, sCsplit = 0;
  const float *scaleN = nullptr;
  int64_t sSNb = 0;  // batch stride of scaleN
  const char *name = "mfma_gemm";  // label for the measurement hooks
  // Workspace of gemm_tail_ws_bytes(M, N, K) bytes for the W' products (batch 1, no
  // split): lets the last round's leftover tiles be split along k.  Optional.
  void *tail_ws = nullptr;
  size_t tail_ws_bytes = 0;
};
bool mfma_supported(const MfmaDesc &d);
int gemm_mfma(const MfmaDesc &d, hipStream_t s);    // register-staged kernel (any operand dtype)
bool mfma2_supported(const MfmaDesc &d);
size_t gemm_tail_ws_bytes(int64_t M, int64_t N, int64_t K);  // 0: no tile would be split
int device_cus();  // compute units of the current device, 0 if unknown
int gemm_mfma2(const MfmaDesc &d, hipStream_t s);   // direct-to-LDS kernel (bf16 operands)
// Streaming block-diagonal product over the first nb blocks (b in {64, 128, 256, 512}; G in
// registers, at b = 512 one 256-column half of a block per workgroup):
//   Y[:, jb:(j+1)b] = X[:, jb:(j+1)b] . G[j]  (transposed: . G[j]^T), times scaleN[col],
// j < nb.  X, Y token-major with row stride ld (>= nb*b, a multiple of 8) bf16,
// G [nb][b][b] bf16.
bool block_stream_supported(int64_t b, int64_t ld, int64_t nb, int64_t n_tokens);
int block_stream(const bf16_t *X, const bf16_t *G, bf16_t *Y, int64_t n_tokens, int64_t ld, int64_t nb,
                 int64_t b, bool transposed, const float *scaleN, const char *name, hipStream_t s);
// Streaming block gradient (b in {64, 128, 256, 512}, shape limits as block_stream): P partials
//   parts[p][j] = sum_{t in token tiles p, p+P, ...} Xs_j[t]^T dY_j[t],  parts [P][nb][b][b] fp32,
// with P = block_grad_stream_parts(b, nb, n_tokens); n_tokens >= 1.
bool block_grad_stream_supported(int64_t b, int64_t ld, int64_t nb, int64_t n_tokens);
int64_t block_grad_stream_parts(int64_t b, int64_t nb, int64_t n_tokens);
// most tokens one float32 accumulator of a block gradient sums before its partial is
// written (the partials are then summed in a fixed order)
constexpr int64_t kMaxChain = 65536;
int block_grad_stream(const bf16_t *Xs, const bf16_t *dY, float *parts, int64_t n_tokens, int64_t ld, int64_t nb,
                      int64_t b, hipStream_t s);
// the direct-to-LDS kernel where it applies, else the register-staged one
inline int gemm_mfma_best(const MfmaDesc &d, hipStream_t s) {
  return mfma2_supported(d) ? gemm_mfma2(d, s) : gemm_mfma(d, s);
}

// ---------------------------------------------------------------------------
// Float32-accurate batched b x b products for the CNP steps (split-bf16 MFMA), b % 64 == 0,
// over the blocks of up to two segments, with up to two outputs:
//   out_o[z] = alpha[o] * A[z] . B[z] + sum_i ce[o][i] * E_i[z] + cI[o] * I
// out_0 written as float32 (C) and/or bf16 (Cb); out_1 as float32 (C2, optional).
// ---------------------------------------------------------------------------
struct CnpMMSeg {
  const float *A = nullptr, *B = nullptr;
  float *C = nullptr, *C2 = nullptr;
  bf16_t *Cb = nullptr;
  const float *E[4] = {nullptr, nullptr, nullptr, nullptr};
  int64_t nblk = 0;
};
struct CnpMMArgs {
  int b = 0;
  float alpha[2] = {1.f, 1.f}, cI[2] = {0.f, 0.f};
  float ce[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  CnpMMSeg seg[2];
  const char *name = "cnp_mm";
};
int cnp_mm(const CnpMMArgs &a, hipStream_t s);

// Row-panel chains of products by one b x b matrix Q per block (b in {64, 128, 256,
// 512}), float32-accurate through split-bf16 MFMA, Q given as its hi and lo bf16 planes,
// 2 b^2 values per block in MFMA fragment order (cnp_frag_off, the unpack's planes).
//   cnp_chain (the forward): one workgroup keeps a panel X of rows of its block resident
//     and runs X = Q + 2I; X <- XQ + 2I; X <- XQ + 2I; G = XQ + I -> out (f32) or outb (bf16)
//   cnp_bwd5 (the backward): reads qp and dg (fp32 [b][b] row-major), writes to out a
//     matrix E with E - E^T = Qbar - Qbar^T (all that dtheta needs), fp32 row-major.
struct CnpChainSeg {
  const bf16_t *qp = nullptr;
  const float *dg = nullptr;
  float *out = nullptr;
  bf16_t *outb = nullptr;
  int64_t nblk = 0;
};
struct CnpChainArgs {
  int b = 0;
  int qlo = 1;  // 0: Q's planes have no lo part (bf16 theta: Q is exact in bf16)
  CnpChainSeg seg[2];
  const char *name = "cnp_chain";
};
bool cnp_chain_supported(int64_t b);
int cnp_chain(const CnpChainArgs &a, hipStream_t s);
bool cnp_bwd5_supported(int64_t b);
int cnp_bwd5(const CnpChainArgs &a, hipStream_t s);

}  // namespace poetx
