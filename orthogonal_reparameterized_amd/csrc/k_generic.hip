// Vector-ALU kernels of libpoetx: the strided float32-accumulating product, the
// LDS-staged column permutation, packed-skew helpers and fixed-order reductions.
#include "kernels.h"

namespace poetx {

// ===================================================================== GEMM ====
// 64 x 64 output tile per 256-thread workgroup, 16-deep k slices staged in LDS
// as float; every thread owns a 4 x 4 patch.  Bounds are checked everywhere, so
// any M, N, K and any strides work (this is the correctness path, not the fast one).
template <typename TA, typename TB, typename TC>
__global__ __launch_bounds__(256) void k_gemm_generic(GemmDesc g) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t z = blockIdx.z;
  const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
  const TA *A = (const TA *)g.A + z * g.sAb;
  const TB *B = (const TB *)g.B + z * g.sBb;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < g.K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = tid + 256 * i;
      int mm = e >> 4, kk = e & 15;
      int64_t m = m0 + mm, k = k0 + kk;
      float v = 0.f;
      if (m < g.M && k < g.K) {
        v = ld_f(A + m * g.sAm + k * g.sAk);
        if (g.scaleK) v *= g.scaleK[k];
      }
      As[kk][mm] = v;
      int kb = e >> 6, nn = e & 63;
      int64_t n = n0 + nn, k2 = k0 + kb;
      Bs[kb][nn] = (n < g.N && k2 < g.K) ? ld_f(B + k2 * g.sBk + n * g.sBn) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  TC *C = (TC *)g.C + z * g.sCb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t n = n0 + tx * 4 + j;
      if (n >= g.N) continue;
      float v = g.alpha * acc[i][j];
      if (g.scaleN) v *= g.scaleN[z * g.sSNb + n];
      if (g.D) v += g.beta * g.D[z * g.sDb + m * g.sDm + n * g.sDn];
      st_f(C + m * g.sCm + n * g.sCn, v);
    }
  }
}

template <typename TA, typename TB>
static int gemm_generic_c(const GemmDesc &g, hipStream_t s) {
  dim3 grid((unsigned)cdiv(g.N, 64), (unsigned)cdiv(g.M, 64), (unsigned)g.batch);
  if (g.c_dt == POETX_F32)
    return launch_k(g.name, s, k_gemm_generic<TA, TB, float>, grid, 256, 0, g);
  return launch_k(g.name, s, k_gemm_generic<TA, TB, bf16_t>, grid, 256, 0, g);
}

template <typename TA>
static int gemm_generic_b(const GemmDesc &g, hipStream_t s) {
  switch (g.b_dt) {
    case POETX_F32: return gemm_generic_c<TA, float>(g, s);
    case POETX_BF16: return gemm_generic_c<TA, bf16_t>(g, s);
    default: return gemm_generic_c<TA, int8_t>(g, s);
  }
}

int gemm_generic(const GemmDesc &g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return POETX_OK;
  if (cdiv(g.N, 64) > 0x7fffffff) return POETX_ERR_UNSUPPORTED;
  constexpr int64_t MCH = 65535 * 64;  // rows per launch: 64-row tiles along the grid's y
  if (g.M > MCH) {
    for (int64_t m0 = 0; m0 < g.M; m0 += MCH) {
      GemmDesc c = g;
      c.M = g.M - m0 < MCH ? g.M - m0 : MCH;
      c.A = (const char *)g.A + m0 * g.sAm * (int64_t)dtype_size(g.a_dt);
      c.C = (char *)g.C + m0 * g.sCm * (int64_t)dtype_size(g.c_dt);
      if (g.D) c.D = g.D + m0 * g.sDm;
      POETX_TRY(gemm_generic(c, s));
    }
    return POETX_OK;
  }
  if (g.batch > 65535) {
    // the batch runs along the grid's z (at most 65535): launch it in chunks
    for (int64_t z0 = 0; z0 < g.batch; z0 += 65535) {
      GemmDesc c = g;
      c.batch = g.batch - z0 < 65535 ? g.batch - z0 : 65535;
      c.A = (const char *)g.A + z0 * g.sAb * (int64_t)dtype_size(g.a_dt);
      c.B = (const char *)g.B + z0 * g.sBb * (int64_t)dtype_size(g.b_dt);
      c.C = (char *)g.C + z0 * g.sCb * (int64_t)dtype_size(g.c_dt);
      if (g.D) c.D = g.D + z0 * g.sDb;
      if (g.scaleN) c.scaleN = g.scaleN + z0 * g.sSNb;
      POETX_TRY(gemm_generic(c, s));
    }
    return POETX_OK;
  }
  switch (g.a_dt) {
    case POETX_F32: return gemm_generic_b<float>(g, s);
    case POETX_BF16: return gemm_generic_b<bf16_t>(g, s);
    default: return gemm_generic_b<int8_t>(g, s);
  }
}

// ============================================================== permutation ====
// One token row at a time goes through LDS: the global reads and writes are
// contiguous and only the LDS side is indexed by the permutation.
template <typename T>
__global__ __launch_bounds__(256) void k_permute_cols(const T *__restrict__ in, T *__restrict__ out,
                                                      int64_t rows, int64_t cols,
                                                      const int32_t *__restrict__ rperm,
                                                      const int32_t *__restrict__ cperm, int scatter) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  T *row = (T *)lds_raw;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    if (!scatter) {
      int64_t src = rperm ? rperm[r] : r;
      for (int64_t c = threadIdx.x; c < cols; c += blockDim.x) row[c] = in[src * cols + c];
      __syncthreads();
      for (int64_t c = threadIdx.x; c < cols; c += blockDim.x)
        out[r * cols + c] = row[cperm ? cperm[c] : c];
    } else {
      for (int64_t c = threadIdx.x; c < cols; c += blockDim.x)
        row[cperm ? cperm[c] : c] = in[r * cols + c];
      __syncthreads();
      for (int64_t c = threadIdx.x; c < cols; c += blockDim.x) out[r * cols + c] = row[c];
    }
    __syncthreads();
  }
}

// Vectorized form: 16-byte global accesses, RB rows staged in LDS per pass, and the
// permutation indices a thread needs kept in registers across all of its rows.  Rows are
// streamed with nontemporal loads and stores: the stores then leave no dirty lines in L2
// whose write-back would compete with the next kernels (measured: the block gradient that
// reads a gathered activation runs 42 -> 37 us at 8192 x 4096 bf16).
// Requires cols % (16 / sizeof(T)) == 0 and cols / (16 / sizeof(T)) <= MAXC * blockDim.
// (512 threads and about two workgroups per CU measured fastest; rows per pass and MAXC
// are picked per row width below.)
template <typename T, int RB, int MAXC>
__global__ __launch_bounds__(512) void k_permute_cols_v(const T *__restrict__ in, T *__restrict__ out,
                                                        int64_t rows, int64_t cols,
                                                        const int32_t *__restrict__ rperm,
                                                        const int32_t *__restrict__ cperm, int scatter) {
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte chunk
  extern __shared__ __align__(16) unsigned char lds_raw[];
  T *buf = (T *)lds_raw;
  const int64_t nch = cols / V;
  int idx[MAXC][V];
#pragma unroll
  for (int u = 0; u < MAXC; ++u) {
    const int64_t ch = threadIdx.x + (int64_t)u * blockDim.x;
#pragma unroll
    for (int e = 0; e < V; ++e) idx[u][e] = ch < nch ? (cperm ? cperm[ch * V + e] : (int)(ch * V + e)) : 0;
  }
  // The next RB rows are loaded into registers while the current ones are written,
  // so every workgroup keeps reads in flight across its whole loop.
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 pre[RB][MAXC];
  const int64_t stride = (int64_t)gridDim.x * RB;
  auto load_rows = [&](int64_t r0) {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      if (r0 + rr >= rows) continue;
      const int64_t src = (!scatter && rperm) ? rperm[r0 + rr] : r0 + rr;
#pragma unroll
      for (int u = 0; u < MAXC; ++u) {
        const int64_t ch = threadIdx.x + (int64_t)u * blockDim.x;
        if (ch < nch) pre[rr][u] = __builtin_nontemporal_load((const u32x4 *)(in + src * cols + ch * V));
      }
    }
  };
  int64_t r0 = (int64_t)blockIdx.x * RB;
  if (r0 < rows) load_rows(r0);
  for (; r0 < rows; r0 += stride) {
    const int nr = (int)(rows - r0 < RB ? rows - r0 : RB);
    // rows r0 .. r0 + nr into LDS: as read (gather) or scattered by column (scatter)
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      if (rr >= nr) continue;
#pragma unroll
      for (int u = 0; u < MAXC; ++u) {
        const int64_t ch = threadIdx.x + (int64_t)u * blockDim.x;
        if (ch >= nch) continue;
        if (!scatter) {
          *(u32x4 *)(buf + rr * cols + ch * V) = pre[rr][u];
        } else {
          union { u32x4 q; T v[V]; } o;
          o.q = pre[rr][u];
#pragma unroll
          for (int e = 0; e < V; ++e) buf[rr * cols + idx[u][e]] = o.v[e];
        }
      }
    }
    __syncthreads();
    if (r0 + stride < rows) load_rows(r0 + stride);
    for (int rr = 0; rr < nr; ++rr) {
#pragma unroll
      for (int u = 0; u < MAXC; ++u) {
        const int64_t ch = threadIdx.x + (int64_t)u * blockDim.x;
        if (ch >= nch) continue;
        union { u32x4 q; T v[V]; } o;
        if (!scatter) {
#pragma unroll
          for (int e = 0; e < V; ++e) o.v[e] = buf[rr * cols + idx[u][e]];
        } else {
          o.q = *(const u32x4 *)(buf + rr * cols + ch * V);
        }
        __builtin_nontemporal_store(o.q, (u32x4 *)(out + (r0 + rr) * cols + ch * V));
      }
    }
    __syncthreads();
  }
}

template <typename T, int RB, int MAXC>
static int permute_rbm(const void *in, void *out, int64_t rows, int64_t cols, const int32_t *rperm,
                       const int32_t *cperm, int sc, hipStream_t s) {
  const size_t row_bytes = (size_t)cols * sizeof(T);
  const unsigned grid = (unsigned)(cdiv(rows, RB) < 512 ? cdiv(rows, RB) : 512);
  return launch_k("permute_cols", s, k_permute_cols_v<T, RB, MAXC>, grid, 512, row_bytes * RB, (const T *)in,
                  (T *)out, rows, cols, rperm, cperm, sc);
}

// A thread's chunk slots per row (MAXC) sized to the row: at 4096 bf16 columns one slot
// instead of four frees about half the registers (63 instead of 127 at 2 rows per pass), so
// 4 rows per pass fit at 2 workgroups per CU: 25.7 -> 23.4 us per 8192 x 4096 bf16 pass
// (2 rows per pass, and 256, 384 or 768 workgroups, were slower; 8 rows slower still).
template <typename T, int RB>
static int permute_rb(const void *in, void *out, int64_t rows, int64_t cols, const int32_t *rperm,
                      const int32_t *cperm, int sc, hipStream_t s) {
  const int64_t nch = cols / (16 / sizeof(T));
  if (nch <= 512) return permute_rbm<T, RB, 1>(in, out, rows, cols, rperm, cperm, sc, s);
  if (nch <= 1024) return permute_rbm<T, RB, 2>(in, out, rows, cols, rperm, cperm, sc, s);
  return permute_rbm<T, RB, 4>(in, out, rows, cols, rperm, cperm, sc, s);
}

// 4 rows per pass where they fit the 64 KB of LDS a launch gets without an attribute, else 2
template <typename T>
static int permute_v(const void *in, void *out, int64_t rows, int64_t cols, const int32_t *rperm,
                     const int32_t *cperm, int sc, hipStream_t s) {
  const size_t row_bytes = (size_t)cols * sizeof(T);
  if (row_bytes * 4 <= 65536) return permute_rb<T, 4>(in, out, rows, cols, rperm, cperm, sc, s);
  return permute_rb<T, 2>(in, out, rows, cols, rperm, cperm, sc, s);
}

int permute_cols(const void *in, void *out, int64_t rows, int64_t cols, int esize,
                 const int32_t *rperm, const int32_t *cperm, bool scatter, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return POETX_OK;
  size_t lds = (size_t)cols * esize;
  if (lds > 65536) return POETX_ERR_UNSUPPORTED;
  int sc = scatter ? 1 : 0;
  const int V = 16 / esize;
  const bool vec_ok = cols % V == 0 && cols / V <= 4 * 512 && lds * 2 <= 65536 &&
                      ((uintptr_t)in % 16) == 0 && ((uintptr_t)out % 16) == 0;
  if (vec_ok) {
    switch (esize) {
      case 4: return permute_v<uint32_t>(in, out, rows, cols, rperm, cperm, sc, s);
      case 2: return permute_v<uint16_t>(in, out, rows, cols, rperm, cperm, sc, s);
      default: return permute_v<uint8_t>(in, out, rows, cols, rperm, cperm, sc, s);
    }
  }
  unsigned grid = (unsigned)(rows < 4096 ? rows : 4096);
  switch (esize) {
    case 4:
      return launch_k("permute_cols", s, k_permute_cols<uint32_t>, grid, 256, lds, (const uint32_t *)in, (uint32_t *)out, rows, cols, rperm, cperm, sc);
    case 2:
      return launch_k("permute_cols", s, k_permute_cols<uint16_t>, grid, 256, lds, (const uint16_t *)in, (uint16_t *)out, rows, cols, rperm, cperm, sc);
    default:
      return launch_k("permute_cols", s, k_permute_cols<uint8_t>, grid, 256, lds, (const uint8_t *)in, (uint8_t *)out, rows, cols, rperm, cperm, sc);
  }
}

// inv[perm[i]] = i (perm must be a permutation of 0 .. n-1; not checked).
__global__ void k_invert_perm(const int32_t *__restrict__ perm, int32_t *__restrict__ inv, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) inv[perm[i]] = (int32_t)i;
}

int invert_perm(const int32_t *perm, int32_t *inv, int64_t n, hipStream_t s) {
  if (n <= 0) return POETX_OK;
  return launch_k("invert_perm", s, k_invert_perm, (unsigned)cdiv(n, 256), 256, 0, perm, inv, n);
}

// Adam on packed parameters, one fused pass: m, v, theta updated in place from g.
//   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;  theta -= step_size * m / (sqrt(v) * rs2 + eps)
// with step_size = gamma lr / (1 - b1^t) and rs2 = 1 / sqrt(1 - b2^t) from the host.  A bf16
// theta is widened, updated in float32 and rounded back to nearest even.
__device__ inline float adam_update(float th, float gg, float &mm, float &vv, const AdamEpi &h) {
  mm = h.b1 * mm + (1.f - h.b1) * gg;
  vv = h.b2 * vv + (1.f - h.b2) * gg * gg;
  return th - h.step_size * mm / (sqrtf(vv) * h.rs2 + h.eps);
}

template <typename T>
__global__ void k_adam(int64_t n, T *__restrict__ theta, const float *__restrict__ g, float *__restrict__ m,
                       float *__restrict__ v, AdamEpi h) {
  const int64_t n4 = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    float tp[4];
    if constexpr (sizeof(T) == 4) {
      const float4 t = ((const float4 *)theta)[i];
      tp[0] = t.x; tp[1] = t.y; tp[2] = t.z; tp[3] = t.w;
    } else {
      const uint2 t = ((const uint2 *)theta)[i];
      tp[0] = bf16_to_f32((bf16_t)t.x); tp[1] = bf16_to_f32((bf16_t)(t.x >> 16));
      tp[2] = bf16_to_f32((bf16_t)t.y); tp[3] = bf16_to_f32((bf16_t)(t.y >> 16));
    }
    float4 gg = ((const float4 *)g)[i], mm = ((float4 *)m)[i], vv = ((float4 *)v)[i];
    float *gp = &gg.x, *mp = &mm.x, *vp = &vv.x;
#pragma unroll
    for (int c = 0; c < 4; ++c) tp[c] = adam_update(tp[c], gp[c], mp[c], vp[c], h);
    if constexpr (sizeof(T) == 4) {
      ((float4 *)theta)[i] = make_float4(tp[0], tp[1], tp[2], tp[3]);
    } else {
      ((uint2 *)theta)[i] = make_uint2((uint32_t)f32_to_bf16(tp[0]) | ((uint32_t)f32_to_bf16(tp[1]) << 16),
                                       (uint32_t)f32_to_bf16(tp[2]) | ((uint32_t)f32_to_bf16(tp[3]) << 16));
    }
    ((float4 *)m)[i] = mm; ((float4 *)v)[i] = vv;
  }
  // tail (n % 4 elements), handled by the first threads of the grid
  const int64_t e = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) {
    float mm = m[e], vv = v[e];
    const float t = adam_update(ld_f(theta + e), g[e], mm, vv, h);
    m[e] = mm; v[e] = vv;
    st_f(theta + e, t);
  }
}

int adam_step(int64_t n, void *theta, int theta_dt, const float *g, float *m, float *v, const AdamEpi &h,
              hipStream_t s) {
  if (n <= 0) return POETX_OK;
  const int64_t want = cdiv(n / 4 > 0 ? n / 4 : 1, 256);
  const unsigned grid = (unsigned)(want < 2048 ? want : 2048);
  if (theta_dt == POETX_BF16)
    return launch_k("adam_step", s, k_adam<bf16_t>, grid, 256, 0, n, (bf16_t *)theta, g, m, v, h);
  return launch_k("adam_step", s, k_adam<float>, grid, 256, 0, n, (float *)theta, g, m, v, h);
}

// out[c][r] = in[r][c] for a [rows][cols] matrix, through 64 x 64 LDS tiles.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T *__restrict__ in, T *__restrict__ out, int64_t rows,
                                                   int64_t cols) {
  __shared__ T t[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) t[i][tx] = in[r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) out[c * rows + r] = t[tx][i];
  }
}

// The same with 16-byte global accesses: a tile of TR x TR elements (128-byte tile rows:
// 64 x 64 for 2-byte, 128 x 128 for 1-byte elements) is read along its rows in 16-byte
// chunks into LDS, and written along its columns in 16-byte chunks, each gathered from
// V = 16 / sizeof(T) consecutive tile rows.  A thread reads those V rows a 4-byte word at a
// time (P = 4 / sizeof(T) columns per word) and writes P output chunks, so the LDS is read
// with one instruction per word instead of one per element.  The 16-byte chunk c of tile
// row r sits at chunk c ^ ((r / V) % 8), which puts the eight row groups a wave reads at
// once on different banks.  Needs rows and cols to be multiples of V (whole chunks) and
// 16-byte aligned buffers.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose_v(const T *__restrict__ in, T *__restrict__ out, int64_t rows,
                                                     int64_t cols) {
  constexpr int V = 16 / sizeof(T), TR = 128 / sizeof(T), P = 4 / sizeof(T);
  __shared__ __align__(16) uint32_t t[TR * 32];  // TR rows of 128 bytes
  const int64_t r0 = (int64_t)blockIdx.y * TR, c0 = (int64_t)blockIdx.x * TR;
  in += (int64_t)blockIdx.z * rows * cols;  // matrix z of a batch (z = 0 for one matrix)
  out += (int64_t)blockIdx.z * rows * cols;
  for (int q = threadIdx.x; q < TR * 8; q += 256) {
    const int row = q >> 3, ch = q & 7;
    const int64_t r = r0 + row, c = c0 + ch * V;
    if (r < rows && c < cols)
      *(uint4 *)&t[row * 32 + ((ch ^ ((row / V) & 7)) << 2)] = *(const uint4 *)(in + r * cols + c);
  }
  __syncthreads();
  const int rr = threadIdx.x & 7, cg = threadIdx.x >> 3;  // rows rr*V .., columns cg*P ..
  const int64_t r = r0 + rr * V;
  if (r >= rows) return;
  uint32_t w[V];
#pragma unroll
  for (int j = 0; j < V; ++j) w[j] = t[(rr * V + j) * 32 + ((((cg >> 2) ^ rr) & 7) << 2) + (cg & 3)];
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const int64_t c = c0 + cg * P + e;
    if (c >= cols) break;
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t x = 0;
#pragma unroll
      for (int k = 0; k < P; ++k)  // element e of the words of rows 4i/P*... in order
        x |= ((w[i * P + k] >> (8 * sizeof(T) * e)) & ((1u << (8 * sizeof(T))) - 1)) << (8 * sizeof(T) * k);
      u[i] = x;
    }
    *(uint4 *)(out + c * rows + r) = make_uint4(u[0], u[1], u[2], u[3]);
  }
}

int transpose(const void *in, void *out, int64_t rows, int64_t cols, int esize, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return POETX_OK;
  const int64_t V = 16 / esize, TR = 128 / esize;
  if (esize <= 2 && rows % V == 0 && cols % V == 0 && (((uintptr_t)in | (uintptr_t)out) & 15) == 0 &&
      cdiv(rows, TR) <= 65535) {
    dim3 grid((unsigned)cdiv(cols, TR), (unsigned)cdiv(rows, TR));
    if (esize == 2)
      return launch_k("transpose", s, k_transpose_v<uint16_t>, grid, 256, 0, (const uint16_t *)in, (uint16_t *)out, rows, cols);
    return launch_k("transpose", s, k_transpose_v<uint8_t>, grid, 256, 0, (const uint8_t *)in, (uint8_t *)out, rows, cols);
  }
  if (cdiv(rows, 64) > 65535) return POETX_ERR_UNSUPPORTED;
  dim3 grid((unsigned)cdiv(cols, 64), (unsigned)cdiv(rows, 64));
  switch (esize) {
    case 4: return launch_k("transpose", s, k_transpose<uint32_t>, grid, 256, 0, (const uint32_t *)in, (uint32_t *)out, rows, cols);
    case 2: return launch_k("transpose", s, k_transpose<uint16_t>, grid, 256, 0, (const uint16_t *)in, (uint16_t *)out, rows, cols);
    default: return launch_k("transpose", s, k_transpose<uint8_t>, grid, 256, 0, (const uint8_t *)in, (uint8_t *)out, rows, cols);
  }
}

int transpose_batched(const void *in, void *out, int64_t batch, int64_t rows, int64_t cols, hipStream_t s) {
  if (batch <= 0 || rows <= 0 || cols <= 0) return POETX_OK;
  const int64_t V = 8, TR = 64;  // bf16
  if (rows % V || cols % V || (((uintptr_t)in | (uintptr_t)out) & 15) || batch > 65535 || cdiv(rows, TR) > 65535)
    return POETX_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)cdiv(cols, TR), (unsigned)cdiv(rows, TR), (unsigned)batch);
  return launch_k("transpose", s, k_transpose_v<uint16_t>, grid, 256, 0, (const uint16_t *)in, (uint16_t *)out, rows, cols);
}

__global__ void k_gather_f32(const float *__restrict__ src, float *__restrict__ out, int64_t n,
                             const int32_t *__restrict__ perm) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = src[perm ? perm[i] : i];
}

int gather_f32(const float *src, float *out, int64_t n, const int32_t *perm, hipStream_t s) {
  if (n <= 0) return POETX_OK;
  return launch_k("gather_f32", s, k_gather_f32, (unsigned)cdiv(n, 256), 256, 0, src, out, n, perm);
}

// ============================================================= packed skew ====
// Offset of (r, c), r < c, in the row-major strict upper triangle of a b x b block.
__device__ inline int64_t triu_index(int64_t r, int64_t c, int64_t b) {
  return r * b - r * (r + 1) / 2 + (c - r - 1);
}

// Tile (rb, cb), rb <= cb, of the upper triangle from the linear index of the upper tiles
// of a T x T tile grid (row-major over rb, then cb = rb .. T-1).
__device__ inline void upper_tile(int idx, int T, int &rb, int &cb) {
  rb = 0;
  while (idx >= T - rb) { idx -= T - rb; ++rb; }
  cb = rb + idx;
}

// Block z and upper tile (rb, cb) of 1-D workgroup L over nz blocks of T x T tiles.  All
// tiles of one block run on one XCD (workgroup L runs on XCD L % 8): neighbouring tiles
// share the cache lines at their edges (a row of packed theta runs across them), which
// then meet in one L2 instead of being written back in parts by several.
__device__ inline void block_tile(int64_t L, int64_t nz, int T, int64_t &z, int &rb, int &cb) {
  const int64_t NT = (int64_t)T * (T + 1) / 2, nz8 = nz & ~(int64_t)7;
  int64_t idx;
  if (L < nz8 * NT) {
    const int64_t slot = L >> 3;
    z = (L & 7) + 8 * (slot / NT);
    idx = slot % NT;
  } else {
    z = L / NT;
    idx = L % NT;
  }
  upper_tile((int)idx, T, rb, cb);
}

// Packed parameter e of segment si: float32, or bf16 widened exactly.
__device__ inline float ld_theta(const SkewSegs &sg, int si, int64_t e) {
  return sg.src_bf16 ? bf16_to_f32(((const bf16_t *)sg.src[si])[e]) : ((const float *)sg.src[si])[e];
}

// Both kernels walk 32 x 32 tiles (rb <= cb) of the upper triangle and handle the
// mirrored tile through LDS, so every global access is contiguous along a row.
__global__ __launch_bounds__(256) void k_unpack_skew(SkewSegs sg, int64_t b) {
  __shared__ float t[32][33];
  int rb, cb;
  int64_t z;
  block_tile(blockIdx.x, sg.n[0] + sg.n[1], (int)((b + 31) / 32), z, rb, cb);
  int si = 0;
  if (z >= sg.n[0]) { z -= sg.n[0]; si = 1; }
  const int64_t th0 = z * (b * (b - 1) / 2);
  float *Q = sg.dst[si] + z * b * b;
  const int tc = threadIdx.x & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = (threadIdx.x >> 5) + 8 * i;
    const int64_t r = rb * 32 + tr, c = cb * 32 + tc;
    float v = 0.f;
    if (r < b && c < b) {
      if (r < c) v = ld_theta(sg, si, th0 + triu_index(r, c, b));
      if (r <= c) Q[r * b + c] = v;
    }
    t[tr][tc] = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = (threadIdx.x >> 5) + 8 * i;
    const int64_t r = cb * 32 + tr, c = rb * 32 + tc;  // mirrored element (r > c)
    if (r < b && c < b && r > c) Q[r * b + c] = -t[tc][tr];
  }
}

// Fragment-order planes (b % 32 == 0): workgroup (u, z) reads the upper-triangle tile
// (rb, cb), rb <= cb, of theta along its rows into LDS, then writes the 32 x 32 tile of Q
// at rows 32 rb.., columns 32 cb.. and, off the diagonal, its mirror at (cb, rb) (the
// negated transpose), each as four 1 KB fragment chunks (2 column tiles x 2 planes), 16
// bytes per thread.
__global__ __launch_bounds__(256) void k_unpack_frag(SkewSegs sg, int64_t b) {
  __shared__ float t[32][33];
  int rb, cb;
  int64_t z;
  block_tile(blockIdx.x, sg.n[0] + sg.n[1], (int)((b + 31) / 32), z, rb, cb);
  int si = 0;
  if (z >= sg.n[0]) { z -= sg.n[0]; si = 1; }
  const int64_t th0 = z * (b * (b - 1) / 2);
  const int tid = threadIdx.x, tc = tid & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = (tid >> 5) + 8 * i;
    const int64_t r = rb * 32 + tr, c = cb * 32 + tc;
    t[tr][tc] = r < c ? ld_theta(sg, si, th0 + triu_index(r, c, b)) : 0.f;
  }
  __syncthreads();
  const int tt = tid >> 7, pl = (tid >> 6) & 1, ln = tid & 63;
  if (pl && sg.src_bf16) return;  // bf16 theta: the lo plane is all zero and never read
  const int col = 16 * tt + (ln & 15);
  bf16_t *base = sg.planes[si] + 2 * z * b * b + pl * 512 + ln * 8;
  // mir = 0: the tile at (rb, cb); mir = 1: its mirror at (cb, rb)
  for (int mir = 0; mir < (rb < cb ? 2 : 1); ++mir) {
    uint32_t w[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t h2 = 0;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int row = 8 * (ln >> 4) + 2 * e2 + hf;
        // Q[r][c] = theta(r, c) above the diagonal, -theta(c, r) below, 0 on it
        float v;
        if (mir) v = -t[col][row];
        else if (rb < cb) v = t[row][col];
        else v = row < col ? t[row][col] : (row > col ? -t[col][row] : 0.f);
        const bf16_t hi = f32_to_bf16(v);
        const bf16_t q = pl ? f32_to_bf16(v - bf16_to_f32(hi)) : hi;
        h2 |= (uint32_t)q << (16 * hf);
      }
      w[e2] = h2;
    }
    const int r0 = 32 * (mir ? cb : rb), c0 = 32 * (mir ? rb : cb);
    *(uint4 *)(base + cnp_frag_off(r0, c0 + 16 * tt, b)) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Row-strip form of the fragment-order unpack (b % 32 == 0): workgroup (z, kk) owns the 32
// rows 32 kk .. 32 kk + 31 of the upper triangle, whose packed parameters are one contiguous
// run of theta.  It reads that run once, coalesced, into LDS (row pitch SP floats), then
// writes every 1 KB fragment chunk those parameters determine: the chunks of the strip's
// own rows right of its diagonal tile (and the diagonal tile itself), and the mirrored
// chunks below it (rows 32 kk' > 32 kk, column tiles 2 kk and 2 kk + 1), one chunk per wave
// at a time, both planes at once, 16 bytes per lane and plane.
// A lane's chunk values are a column of the strip (rows 8 g .. 8 g + 7 at one column) for
// the chunks of its own rows, and a row (8 consecutive columns) for the mirrored ones; the
// pitch puts the four row groups g of a column read on four disjoint sets of 16 banks.
constexpr int SP = 258;
__global__ __launch_bounds__(512) void k_unpack_frag_strip(SkewSegs sg, int64_t b) {
  extern __shared__ float strip[];  // [32][SP]: strip[rl][c] = theta(32 kk + rl, c), c > row
  const int64_t NS = b / 32;
  const int64_t L = blockIdx.x;
  int64_t z = L / NS;
  const int kk = (int)(L % NS);
  int si = 0;
  if (z >= sg.n[0]) { z -= sg.n[0]; si = 1; }
  const int64_t th0 = z * (b * (b - 1) / 2);
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  // ---- load: row rl of the strip is the run theta(r, r+1 .. b-1), r = 32 kk + rl; all of a
  // lane's loads (b <= 256: at most 4 per row) are in flight before the first store
  float val[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = 32 * kk + wave + 8 * i;
    const int64_t base = th0 + triu_index(r, r + 1, b);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t c = r + 1 + l + 64 * j;
      val[i][j] = c < b ? ld_theta(sg, si, base + (c - r - 1)) : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = wave + 8 * i, r = 32 * kk + rl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = r + 1 + l + 64 * j;
      if (c < b) strip[rl * SP + c] = val[i][j];
    }
  }
  __syncthreads();
  const int NT = (int)(b / 16), NK = (int)NS;
  const int n_up = NT - 2 * kk, n_mir = 2 * (NK - kk - 1);
  const int g = l >> 4, c16 = l & 15;
  bf16_t *planes = sg.planes[si] + 2 * z * b * b;
  for (int ci = wave; ci < n_up + n_mir; ci += 8) {
    int r0, c0;
    float v[8];
    if (ci < n_up) {
      // chunk (kk, t) of the strip's own rows: Q[32 kk + 8 g + e][16 t + c16]
      const int t = 2 * kk + ci;
      r0 = 32 * kk; c0 = 16 * t;
      const int c = c0 + c16;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int rl = 8 * g + e, r = r0 + rl;
        v[e] = c > r ? strip[rl * SP + c] : (c < r ? -strip[(c - r0) * SP + r] : 0.f);
      }
    } else {
      // mirrored chunk (kk', t), t = 2 kk + (j & 1): Q[32 kk' + 8 g + e][16 t + c16]
      //   = -theta(16 t + c16, 32 kk' + 8 g + e)
      const int j = ci - n_up, kp = kk + 1 + (j >> 1), t = 2 * kk + (j & 1);
      r0 = 32 * kp; c0 = 16 * t;
      const float *src = strip + (c0 + c16 - 32 * kk) * SP + r0 + 8 * g;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = -src[e];
    }
    uint32_t wh[4], wl[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint16_t h0, l0, h1, l1;
      h0 = f32_to_bf16(v[2 * e2]); l0 = f32_to_bf16(v[2 * e2] - bf16_to_f32(h0));
      h1 = f32_to_bf16(v[2 * e2 + 1]); l1 = f32_to_bf16(v[2 * e2 + 1] - bf16_to_f32(h1));
      wh[e2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      wl[e2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    bf16_t *dst = planes + cnp_frag_off(r0, c0, b) + l * 8;
    *(uint4 *)dst = make_uint4(wh[0], wh[1], wh[2], wh[3]);
    if (!sg.src_bf16) *(uint4 *)(dst + 512) = make_uint4(wl[0], wl[1], wl[2], wl[3]);
  }
}

int unpack_skew2(const SkewSegs &sg, int64_t b, hipStream_t s) {
  const int64_t nz = sg.n[0] + sg.n[1];
  if (nz <= 0) return POETX_OK;
  // one workgroup per upper 32 x 32 tile of every block, 1-D (see block_tile)
  const int64_t T = cdiv(b, 32), nwg = nz * (T * (T + 1) / 2);
  if (nwg > 0x7fffffff) return POETX_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)nwg);
  if (sg.planes[0]) {
    if (b % 32) return POETX_ERR_UNSUPPORTED;
#ifndef POETX_UNPACK_TILES
    if (b <= SP) {
      const size_t lds = (size_t)32 * SP * sizeof(float);
      return launch_k("unpack_skew", s, k_unpack_frag_strip, dim3((unsigned)(nz * (b / 32))), 512, lds, sg, b);
    }
#endif
    return launch_k("unpack_skew", s, k_unpack_frag, grid, 256, 0, sg, b);
  }
  return launch_k("unpack_skew", s, k_unpack_skew, grid, 256, 0, sg, b);
}

int unpack_skew(const float *theta, float *Q, int64_t n, int64_t b, hipStream_t s) {
  SkewSegs sg;
  sg.src[0] = theta; sg.dst[0] = Q; sg.n[0] = n;
  return unpack_skew2(sg, b, s);
}

// dtheta[k(r, c)] = M[r][c] - M[c][r]; with ADAM the same pass applies the Adam update to
// theta (read from ad.theta_in, written to ad.theta_out, which may be the same buffer:
// each element is read and written by one thread) and to its state m, v, and writes
// dtheta only where sg.dst is set.
template <bool ADAM>
__global__ __launch_bounds__(256) void k_pack_skew_grad(SkewSegs sg, int64_t b, AdamEpi ad) {
  __shared__ float up[32][33], lo[32][33];
  int rb, cb;
  int64_t z;
  block_tile(blockIdx.x, sg.n[0] + sg.n[1], (int)((b + 31) / 32), z, rb, cb);
  int si = 0;
  if (z >= sg.n[0]) { z -= sg.n[0]; si = 1; }
  const float *M = (const float *)sg.src[si] + z * b * b;
  const int64_t th0 = z * (b * (b - 1) / 2);
  float *dth = sg.dst[si] ? sg.dst[si] + th0 : nullptr;
  const int tc = threadIdx.x & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = (threadIdx.x >> 5) + 8 * i;
    const int64_t r = rb * 32 + tr, c = cb * 32 + tc;
    up[tr][tc] = (r < b && c < b) ? M[r * b + c] : 0.f;
    const int64_t r2 = cb * 32 + tr, c2 = rb * 32 + tc;
    lo[tr][tc] = (r2 < b && c2 < b) ? M[r2 * b + c2] : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = (threadIdx.x >> 5) + 8 * i;
    const int64_t r = rb * 32 + tr, c = cb * 32 + tc;
    if (r < c && c < b) {
      const int64_t k = triu_index(r, c, b);
      const float g = up[tr][tc] - lo[tc][tr];
      if (!ADAM || dth) dth[k] = g;
      if constexpr (ADAM) {
        const int64_t e = th0 + k;
        float mm = ad.m[si][e], vv = ad.v[si][e];
        const float th = ad.theta_bf16 ? bf16_to_f32(((const bf16_t *)ad.theta_in[si])[e])
                                       : ((const float *)ad.theta_in[si])[e];
        const float t = adam_update(th, g, mm, vv, ad);
        ad.m[si][e] = mm; ad.v[si][e] = vv;
        if (ad.theta_bf16) ((bf16_t *)ad.theta_out[si])[e] = f32_to_bf16(t);
        else ((float *)ad.theta_out[si])[e] = t;
      }
    }
  }
}

// Row-strip form of the pack (b <= 256): workgroup (z, kk) writes the packed run of rows
// 32 kk .. 32 kk + 31, one contiguous stretch of dtheta (and of theta, m, v with ADAM).  It
// loads the strip's rows of M right of its diagonal (256-byte row segments) and the
// mirrored columns below it (128-byte row segments) into LDS with every load of a lane in
// flight at once, then writes each output row segment with consecutive lanes.
constexpr int PK_AP = 257;  // A[32][PK_AP]: A[rl][c - r0] = M[r0 + rl][c]
template <bool ADAM>
__global__ __launch_bounds__(512) void k_pack_skew_strip(SkewSegs sg, int64_t b, AdamEpi ad) {
  extern __shared__ float pk_lds[];
  float *A = pk_lds, *Bt = pk_lds + 32 * PK_AP;  // Bt[cl][33]: Bt[cl][rl] = M[r0 + cl][r0 + rl]
  const int64_t NS = (b + 31) / 32;
  const int64_t L = blockIdx.x;
  int64_t z = L / NS;
  const int kk = (int)(L % NS);
  int si = 0;
  if (z >= sg.n[0]) { z -= sg.n[0]; si = 1; }
  const float *M = (const float *)sg.src[si] + z * b * b;
  const int64_t th0 = z * (b * (b - 1) / 2);
  float *dth = sg.dst[si] ? sg.dst[si] + th0 : nullptr;
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int r0 = 32 * kk, w = (int)b - r0;  // columns r0 .. b-1 of the strip
  float va[4][4], vb[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + wave + 8 * i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cl = l + 64 * j;
      va[i][j] = (r < b && cl < w) ? M[(int64_t)r * b + r0 + cl] : 0.f;
    }
  }
  const int rl2 = tid & 31;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int cl = (tid >> 5) + 16 * i;
    vb[i] = (cl < w && r0 + rl2 < b) ? M[(int64_t)(r0 + cl) * b + r0 + rl2] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) A[(wave + 8 * i) * PK_AP + l + 64 * j] = va[i][j];
#pragma unroll
  for (int i = 0; i < 16; ++i) Bt[((tid >> 5) + 16 * i) * 33 + rl2] = vb[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = wave + 8 * i, r = r0 + rl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cl = l + 64 * j, c = r0 + cl;
      if (c > r && c < b) {
        const int64_t k = triu_index(r, c, b);
        const float gr = A[rl * PK_AP + cl] - Bt[cl * 33 + rl];
        if (!ADAM || dth) dth[k] = gr;
        if constexpr (ADAM) {
          const int64_t e = th0 + k;
          float mm = ad.m[si][e], vv = ad.v[si][e];
          const float th = ad.theta_bf16 ? bf16_to_f32(((const bf16_t *)ad.theta_in[si])[e])
                                         : ((const float *)ad.theta_in[si])[e];
          const float t = adam_update(th, gr, mm, vv, ad);
          ad.m[si][e] = mm; ad.v[si][e] = vv;
          if (ad.theta_bf16) ((bf16_t *)ad.theta_out[si])[e] = f32_to_bf16(t);
          else ((float *)ad.theta_out[si])[e] = t;
        }
      }
    }
  }
}

int pack_skew_grad2(const SkewSegs &sg, int64_t b, hipStream_t s, const AdamEpi *ad) {
  const int64_t nz = sg.n[0] + sg.n[1];
  if (nz <= 0) return POETX_OK;
  const int64_t T = cdiv(b, 32), nwg = nz * (T * (T + 1) / 2);
  if (nwg > 0x7fffffff) return POETX_ERR_UNSUPPORTED;
#ifndef POETX_PACK_TILES
  if (b <= 256) {
    const dim3 gs((unsigned)(nz * cdiv(b, 32)));
    const size_t lds = (size_t)(32 * PK_AP + 256 * 33) * sizeof(float);
    static std::atomic<uint64_t> attr[2];  // dynamic LDS above 64 KB, per kernel and device
    if (ad) {
      POETX_TRY(lds_limit((const void *)k_pack_skew_strip<true>, lds, attr[1]));
      return launch_k("pack_skew_grad_adam", s, k_pack_skew_strip<true>, gs, 512, lds, sg, b, *ad);
    }
    POETX_TRY(lds_limit((const void *)k_pack_skew_strip<false>, lds, attr[0]));
    return launch_k("pack_skew_grad", s, k_pack_skew_strip<false>, gs, 512, lds, sg, b, AdamEpi());
  }
#endif
  if (ad) return launch_k("pack_skew_grad_adam", s, k_pack_skew_grad<true>, dim3((unsigned)nwg), 256, 0, sg, b, *ad);
  return launch_k("pack_skew_grad", s, k_pack_skew_grad<false>, dim3((unsigned)nwg), 256, 0, sg, b, AdamEpi());
}

int pack_skew_grad(const float *M, float *dtheta, int64_t n, int64_t b, hipStream_t s) {
  SkewSegs sg;
  sg.src[0] = M; sg.dst[0] = dtheta; sg.n[0] = n;
  return pack_skew_grad2(sg, b, s);
}

__global__ void k_lincomb(float *__restrict__ out, int64_t n, int64_t b, float cI, const float *X0,
                          float c0, const float *X1, float c1, const float *X2, float c2,
                          const float *X3, float c3) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t bb = b * b;
  if (e >= n * bb) return;
  int64_t rc = e % bb;
  float v = (rc / b == rc % b) ? cI : 0.f;
  if (X0) v += c0 * X0[e];
  if (X1) v += c1 * X1[e];
  if (X2) v += c2 * X2[e];
  if (X3) v += c3 * X3[e];
  out[e] = v;
}

int lincomb(float *out, int64_t n, int64_t b, float cI, const float *X0, float c0, const float *X1,
            float c1, const float *X2, float c2, const float *X3, float c3, hipStream_t s) {
  int64_t tot = n * b * b;
  if (tot <= 0) return POETX_OK;
  return launch_k("lincomb", s, k_lincomb, (unsigned)cdiv(tot, 256), 256, 0, out, n, b, cI, X0, c0, X1, c1, X2, c2, X3, c3);
}

__global__ void k_reduce_parts(const float *__restrict__ in, float *__restrict__ out, int64_t elems,
                               int64_t parts, int64_t stride) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= elems) return;
  float acc = 0.f;
  for (int64_t p = 0; p < parts; ++p) acc += in[p * stride + e];
  out[e] = acc;
}

// Same sums, 4 elements per thread, the loads of four partials in flight at a time; the
// additions keep the order p = 0, 1, ... of the scalar kernel.
__global__ void k_reduce_parts4(const float4 *__restrict__ in, float4 *__restrict__ out, int64_t n4,
                                int64_t parts, int64_t stride4) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n4) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](const float4 v) { acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w; };
  int64_t p = 0;
  for (; p + 4 <= parts; p += 4) {
    const float4 v0 = in[p * stride4 + e], v1 = in[(p + 1) * stride4 + e];
    const float4 v2 = in[(p + 2) * stride4 + e], v3 = in[(p + 3) * stride4 + e];
    add(v0); add(v1); add(v2); add(v3);
  }
  for (; p < parts; ++p) add(in[p * stride4 + e]);
  out[e] = acc;
}

int reduce_parts(const float *in, float *out, int64_t elems, int64_t parts, int64_t stride,
                 hipStream_t s) {
  if (elems <= 0) return POETX_OK;
  if (elems % 4 == 0 && stride % 4 == 0 && (uintptr_t)in % 16 == 0 && (uintptr_t)out % 16 == 0) {
    const int64_t n4 = elems / 4;
    return launch_k("reduce_parts", s, k_reduce_parts4, (unsigned)cdiv(n4, 256), 256, 0, (const float4 *)in, (float4 *)out, n4, parts, stride / 4);
  }
  return launch_k("reduce_parts", s, k_reduce_parts, (unsigned)cdiv(elems, 256), 256, 0, in, out, elems, parts, stride);
}

// n elements set to 1 (float32 or bf16): the G of n blocks of size 1.
__global__ void k_fill_one(void *out, int64_t n, int bf) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (bf) ((bf16_t *)out)[i] = (bf16_t)0x3F80;
  else ((float *)out)[i] = 1.f;
}

// ==================================================== padded CNP blocks ====
// A b x b block embedded in a bp x bp one (bp > b) with zeros elsewhere: Q_p = diag(Q, 0),
// so G_p = diag(G, I) and, for dG_p = diag(dG, 0), the packed gradient of Q_p restricted
// to the entries r < c < b is the packed gradient of Q.  One workgroup per row r of a
// padded block z, its lanes over the columns:
//   CNP_PAD_THETA : packed theta (esize 4 or 2) of size b -> of size bp (zeros past b)
//   CNP_CUT_G     : G [b][b] <- G_p [bp][bp] (esize 4 or 2)
//   CNP_PAD_DG    : dG [b][b] fp32 -> dG_p [bp][bp] (zeros past b)
//   CNP_CUT_DTHETA: packed dtheta fp32 of size bp -> of size b
namespace {
__device__ inline int64_t tri_at(int64_t B, int64_t r, int64_t c) { return r * (B - 1) - r * (r - 1) / 2 + (c - r - 1); }
template <typename T>
__global__ __launch_bounds__(64) void k_cnp_pad(int mode, int b, int bp, const T *__restrict__ in,
                                                T *__restrict__ out) {
  const int64_t z = blockIdx.x / bp;
  const int r = (int)(blockIdx.x % bp);
  const int64_t pb = (int64_t)b * (b - 1) / 2, pbp = (int64_t)bp * (bp - 1) / 2;
  switch (mode) {
    case CNP_PAD_THETA:
      for (int c = r + 1 + (int)threadIdx.x; c < bp; c += 64)
        out[z * pbp + tri_at(bp, r, c)] = c < b ? in[z * pb + tri_at(b, r, c)] : (T)0;
      break;
    case CNP_CUT_G:
      if (r < b)
        for (int c = threadIdx.x; c < b; c += 64) out[(z * b + r) * b + c] = in[(z * bp + r) * bp + c];
      break;
    case CNP_PAD_DG:
      for (int c = threadIdx.x; c < bp; c += 64)
        out[(z * bp + r) * bp + c] = r < b && c < b ? in[(z * b + r) * b + c] : (T)0;
      break;
    default:  // CNP_CUT_DTHETA
      if (r < b)
        for (int c = r + 1 + (int)threadIdx.x; c < b; c += 64) out[z * pb + tri_at(b, r, c)] = in[z * pbp + tri_at(bp, r, c)];
      break;
  }
}
}  // namespace

int cnp_pad(int mode, int64_t n, int64_t b, int64_t bp, int esize, const void *in, void *out, hipStream_t s) {
  if (n <= 0) return POETX_OK;
  if (bp <= b || n * bp > 0x7fffffff || (esize != 2 && esize != 4)) return POETX_ERR_UNSUPPORTED;
  const unsigned grid = (unsigned)(n * bp);
  if (esize == 2)
    return launch_k("cnp_pad", s, k_cnp_pad<uint16_t>, grid, 64, 0, mode, (int)b, (int)bp, (const uint16_t *)in,
                    (uint16_t *)out);
  return launch_k("cnp_pad", s, k_cnp_pad<uint32_t>, grid, 64, 0, mode, (int)b, (int)bp, (const uint32_t *)in,
                  (uint32_t *)out);
}

int fill_one(void *out, int64_t n, int dt, hipStream_t s) {
  if (n <= 0) return POETX_OK;
  return launch_k("fill_one", s, k_fill_one, (unsigned)cdiv(n, 256), 256, 0, out, n, dt == POETX_BF16 ? 1 : 0);
}

}  // namespace poetx
