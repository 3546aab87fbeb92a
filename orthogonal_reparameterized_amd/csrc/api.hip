// libpoetx C ABI: argument validation, workspace carving and kernel sequencing
// for the POET-X layer (declarations and contracts in include/poetx.h).
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"

using namespace poetx;

// ============================================================ measurement ====
// Per-thread recorder of kernel durations (poetx_prof_enable / poetx_prof_read): each
// launch made by this thread while it is on carries a start and a stop event bound to
// the dispatch (launch_k in common.h).  Nothing here is shared between threads.
namespace poetx {
namespace {
struct ProfRec {
  const char *name;
  hipEvent_t a, b;
};
struct Recorder {
  bool on = false;
  std::string only;  // record only launches with this label ("" = every launch)
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;  // events are reused, never destroyed (the runtime may be
                                 // gone by the time a thread's storage is torn down)
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    // timing-only events: without the system-scope fence an event would write back and
    // invalidate the caches around every recorded dispatch (idle gaps of several us between
    // kernels, and kernels that start on cold caches)
    hipEvent_t e = nullptr;
    return hipEventCreateWithFlags(&e, hipEventDisableSystemFence) == hipSuccess ? e : nullptr;
  }
};
thread_local Recorder t_rec;
}  // namespace

bool prof_on() { return t_rec.on; }
bool prof_events(const char *name, hipEvent_t *start, hipEvent_t *stop) {
  if (!t_rec.only.empty() && t_rec.only != name) return false;
  *start = t_rec.get();
  *stop = t_rec.get();
  if (*start && *stop) return true;
  if (*start) t_rec.pool.push_back(*start);
  if (*stop) t_rec.pool.push_back(*stop);
  *start = *stop = nullptr;
  return false;
}
void prof_commit(const char *name, hipEvent_t start, hipEvent_t stop) { t_rec.recs.push_back({name, start, stop}); }
}  // namespace poetx

extern "C" int poetx_prof_enable(int32_t on) {
  t_rec.on = on != 0;
  return POETX_OK;
}

extern "C" int poetx_prof_only(const char *label) {
  t_rec.only = label ? label : "";
  return POETX_OK;
}

extern "C" int poetx_prof_read(char *buf, size_t len) {
  struct Acc { std::string name; long n; double ms, mn, mx; };
  std::vector<Acc> acc;
  int st = POETX_OK;
  for (auto &r : t_rec.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      st = POETX_ERR_HIP;
    bool found = false;
    for (auto &a : acc)
      if (a.name == r.name) {
        a.n++; a.ms += ms; a.mn = ms < a.mn ? ms : a.mn; a.mx = ms > a.mx ? ms : a.mx;
        found = true;
        break;
      }
    if (!found) acc.push_back({r.name, 1, (double)ms, (double)ms, (double)ms});
    t_rec.pool.push_back(r.a);
    t_rec.pool.push_back(r.b);
  }
  t_rec.recs.clear();
  std::string out;
  char line[256];
  for (auto &a : acc) {
    snprintf(line, sizeof line, "%s %ld %.6f %.6f %.6f\n", a.name.c_str(), a.n, a.ms, a.mn, a.mx);
    out += line;
  }
  if (buf && len) {
    size_t n = out.size() < len - 1 ? out.size() : len - 1;
    memcpy(buf, out.data(), n);
    buf[n] = 0;
  }
  return st;
}

extern "C" const char *poetx_status_string(int st) {
  switch (st) {
    case POETX_OK: return "POETX_OK";
    case POETX_ERR_INVALID_ARG: return "POETX_ERR_INVALID_ARG";
    case POETX_ERR_SHAPE: return "POETX_ERR_SHAPE";
    case POETX_ERR_UNSUPPORTED: return "POETX_ERR_UNSUPPORTED";
    case POETX_ERR_WORKSPACE: return "POETX_ERR_WORKSPACE";
    case POETX_ERR_HIP: return "POETX_ERR_HIP";
    default: return "POETX_UNKNOWN_STATUS";
  }
}

extern "C" const char *poetx_version(void) { return "0.1.0"; }

// ============================================================ permutation ====
extern "C" int poetx_merge_perm(const void *w, const float *w_scale, int32_t w_dtype,
                                int64_t d_out, int64_t d_in, const int32_t *perm_out,
                                const int32_t *perm_in, void *w_merged, float *w_scale_merged,
                                void *w_merged_t, void *stream) {
  if (!w || !w_merged || d_out < 1 || d_in < 1) return POETX_ERR_INVALID_ARG;
  if (w_dtype != POETX_F32 && w_dtype != POETX_BF16 && w_dtype != POETX_I8) return POETX_ERR_INVALID_ARG;
  if (w_dtype == POETX_I8 && (!w_scale || !w_scale_merged)) return POETX_ERR_INVALID_ARG;
  if ((size_t)d_in * dtype_size(w_dtype) > 65536) return POETX_ERR_UNSUPPORTED;
  if (w_merged_t && (w_merged_t == w || w_merged_t == w_merged)) return POETX_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  POETX_TRY(permute_cols(w, w_merged, d_out, d_in, (int)dtype_size(w_dtype), perm_out, perm_in, false, s));
  if (w_dtype == POETX_I8) POETX_TRY(gather_f32(w_scale, w_scale_merged, d_out, perm_out, s));
  if (w_merged_t) POETX_TRY(transpose(w_merged, w_merged_t, d_out, d_in, (int)dtype_size(w_dtype), s));
  return POETX_OK;
}

// ==================================================================== CNP ====
// Cayley-Neumann map (Method §4, eq. 9) in Horner form
//   G = I + 2Q + S (2I + 2Q + S),  S = Q^2,
// and its adjoint (the page does not print eq. 10; this is the exact adjoint of
// eq. 9).  With P = Q^T = -Q and Gb = dL/dG,
//   Qbar = sum_{j+l<=3} a_{j+l+1} P^j Gb P^l,   a = (2, 2, 2, 1),
// grouped by j and evaluated by Horner in P:
//   K1 = Gb P, K2 = K1 P, K3 = K2 P,
//   H2 = (2Gb + K1) + P Gb, H1 = (2Gb + 2K1 + K2) + P H2, Qbar = (2Gb + 2K1 + 2K2 + K3) + P H1,
// then dtheta[k(i,j)] = Qbar[i][j] - Qbar[j][i].
// For b in {64, 128, 256, 512} both directions run as row-panel chains of products
// (k_cnp.hip): the forward as G = (((Q + 2I)Q + 2I)Q + 2I)Q + I in one launch, the
// backward in one launch of five products that yield E with E - E^T = Qbar - Qbar^T
// (dtheta reads nothing else).  Other b % 64 == 0 run the products above one launch
// each on split-bf16 MFMA; the remaining b use the float32 vector-ALU product.
namespace {

GemmDesc batched_f32(int64_t n, int64_t b, const float *A, const float *B, void *C, int c_dt) {
  GemmDesc g;
  g.name = "cnp_product";
  g.M = g.N = g.K = b;
  g.batch = n;
  g.A = A; g.a_dt = POETX_F32; g.sAb = b * b; g.sAm = b; g.sAk = 1;
  g.B = B; g.b_dt = POETX_F32; g.sBb = b * b; g.sBk = b; g.sBn = 1;
  g.C = C; g.c_dt = c_dt; g.sCb = b * b; g.sCm = b; g.sCn = 1;
  return g;
}

GemmDesc with_terms(GemmDesc g, const float *D, float beta, float alpha) {
  g.D = D; g.sDb = g.sCb; g.sDm = g.sCm; g.sDn = 1; g.beta = beta; g.alpha = alpha;
  return g;
}

bool cnp_use_mfma(int64_t b) { return b % 64 == 0; }

// Block sizes between 64 and 512 that are not multiples of 64 have no MFMA kernels of
// their own: their CNP runs on blocks of the next row-panel size (128, 256 or 512) with Q
// embedded as diag(Q, 0), which gives diag(G, I), and dG as diag(dG, 0), whose packed
// gradient restricted to Q's entries is Q's (a polynomial of a block-diagonal matrix is
// block-diagonal).  0: no padding.
int64_t cnp_pad_to(int64_t b) {
  if (b <= 64 || b >= 512 || b % 64 == 0) return 0;
  return b <= 128 ? 128 : b <= 256 ? 256 : 512;
}

size_t cnp_ws_bytes(int dir, int64_t n, int64_t b) {
  Arena ar(nullptr);
  const int64_t bp = cnp_pad_to(b);
  if (bp) {
    const size_t pk = (size_t)n * (bp * (bp - 1) / 2) * 4, sq = (size_t)n * bp * bp * 4;
    ar.take(pk);                                   // padded theta
    ar.take(sq);                                   // padded G, or padded dG
    if (dir == POETX_CNP_BWD) {
      ar.take(pk);                                 // padded dtheta
      ar.take((size_t)n * (b * (b - 1) / 2) * 4);  // dtheta for a fused update without one
    }
    ar.take(cnp_ws_bytes(dir, n, bp));
    return ar.used;
  }
  size_t blk = (size_t)n * b * b * 4;
  int bufs = dir == POETX_CNP_FWD ? 4 : 6;
  for (int i = 0; i < bufs; ++i) ar.take(blk);
  return ar.used;
}

bool al16(const void *q) { return ((uintptr_t)q & 15) == 0; }

// qsave (optional, chain block sizes): receives Q's fragment-ordered planes for a later backward.
int cnp_fwd_impl(int64_t n, int64_t b, const void *theta, int theta_bf16, void *g, int g_dtype, void *qsave,
                 void *ws, hipStream_t s) {
  Arena ar(ws);
  if (const int64_t bp = cnp_pad_to(b)) {
    void *tp = ar.take((size_t)n * (bp * (bp - 1) / 2) * 4);
    void *gp = ar.take((size_t)n * bp * bp * 4);
    void *inner = ar.take(cnp_ws_bytes(POETX_CNP_FWD, n, bp));
    POETX_TRY(cnp_pad(CNP_PAD_THETA, n, b, bp, theta_bf16 ? 2 : 4, theta, tp, s));
    POETX_TRY(cnp_fwd_impl(n, bp, tp, theta_bf16, gp, g_dtype, nullptr, inner, s));
    return cnp_pad(CNP_CUT_G, n, b, bp, g_dtype == POETX_F32 ? 4 : 2, gp, g, s);
  }
  size_t blk = (size_t)n * b * b * 4;
  // the chain and MFMA paths store G with 8- and 16-byte stores; a G that is only
  // element-aligned takes the vector-ALU path
  const bool vec = al16(g);
  if (vec && cnp_chain_supported(b)) {
    // Q as bf16 planes (straight into qsave when given), then the whole Horner chain in
    // one launch
    SkewSegs un;
    un.src[0] = theta; un.n[0] = n; un.src_bf16 = theta_bf16;
    un.planes[0] = qsave ? (bf16_t *)qsave : (bf16_t *)ar.take(blk);
    POETX_TRY(unpack_skew2(un, b, s));
    CnpChainArgs c;
    c.b = (int)b;
    c.qlo = !theta_bf16;
    c.name = "cnp_fwd_chain";
    c.seg[0].qp = un.planes[0]; c.seg[0].nblk = n;
    if (g_dtype == POETX_F32) c.seg[0].out = (float *)g;
    else c.seg[0].outb = (bf16_t *)g;
    return cnp_chain(c, s);
  }
  if (qsave) {  // the planes a later backward's chains read, in their own pass here
    SkewSegs un;
    un.src[0] = theta; un.n[0] = n; un.src_bf16 = theta_bf16;
    un.planes[0] = (bf16_t *)qsave;
    POETX_TRY(unpack_skew2(un, b, s));
  }
  float *Q = (float *)ar.take(blk), *S = (float *)ar.take(blk);
  float *T = (float *)ar.take(blk), *U = (float *)ar.take(blk);
  {
    SkewSegs un;
    un.src[0] = theta; un.dst[0] = Q; un.n[0] = n; un.src_bf16 = theta_bf16;
    POETX_TRY(unpack_skew2(un, b, s));
  }
  if (vec && cnp_use_mfma(b)) {
    // S = Q Q and, from the same accumulators, T = 2I + 2Q + S
    CnpMMArgs a;
    a.b = (int)b;
    a.name = "cnp_fwd_mm";
    a.ce[1][0] = 2.f; a.cI[1] = 2.f;
    a.seg[0].A = Q; a.seg[0].B = Q; a.seg[0].C = S; a.seg[0].C2 = T; a.seg[0].E[0] = Q; a.seg[0].nblk = n;
    a.ce[0][0] = 0.f;
    POETX_TRY(cnp_mm(a, s));
    // G = I + 2Q + S T
    CnpMMArgs c;
    c.b = (int)b;
    c.name = "cnp_fwd_mm";
    c.cI[0] = 1.f; c.ce[0][0] = 2.f;
    c.seg[0].A = S; c.seg[0].B = T; c.seg[0].E[0] = Q; c.seg[0].nblk = n;
    if (g_dtype == POETX_F32) c.seg[0].C = (float *)g;
    else c.seg[0].Cb = (bf16_t *)g;
    return cnp_mm(c, s);
  }
  POETX_TRY(gemm_generic(batched_f32(n, b, Q, Q, S, POETX_F32), s));
  POETX_TRY(lincomb(T, n, b, 2.f, Q, 2.f, S, 1.f, nullptr, 0.f, nullptr, 0.f, s));
  POETX_TRY(lincomb(U, n, b, 1.f, Q, 2.f, nullptr, 0.f, nullptr, 0.f, nullptr, 0.f, s));
  return gemm_generic(with_terms(batched_f32(n, b, S, T, g, g_dtype), U, 1.f, 1.f), s);
}

// One side's blocks for the CNP backward.  With an Adam epilogue (adam_step or the
// layer's fused update), dtheta may be null: the update then consumes the gradient in the
// pack pass without storing it.
struct CnpBwdSide {
  int64_t n = 0;
  const void *theta = nullptr;
  const void *qsave = nullptr;  // Q's planes from the forward (chain paths), or null: unpack theta
  const float *dg = nullptr;
  float *dtheta = nullptr;
  // fused Adam: new theta, state
  void *theta_out = nullptr;
  float *m = nullptr, *v = nullptr;
};

// the packs of up to two sides, with the Adam epilogue when `h` is given
int pack_sides(SkewSegs &pk, const CnpBwdSide *side, int nside, int64_t b, int theta_bf16, const AdamEpi *h,
               hipStream_t s) {
  if (!h) return pack_skew_grad2(pk, b, s);
  AdamEpi ad = *h;
  ad.theta_bf16 = theta_bf16;
  for (int i = 0; i < nside; ++i) {
    ad.theta_in[i] = side[i].theta; ad.theta_out[i] = side[i].theta_out;
    ad.m[i] = side[i].m; ad.v[i] = side[i].v;
  }
  return pack_skew_grad2(pk, b, s, &ad);
}

// CNP backward of up to two independent sides sharing b (the R and P sides of a layer):
// unpack Q (unless the forward kept its planes), then the five products of every block in
// one launch, then pack dtheta.
int cnp_bwd5_path(int64_t b, const CnpBwdSide *side, int nside, int theta_bf16, const AdamEpi *h, void *ws,
                  hipStream_t s) {
  Arena ar(ws);
  SkewSegs un, pk;
  un.src_bf16 = theta_bf16;
  CnpChainArgs c;
  c.b = (int)b;
  c.qlo = !theta_bf16;
  c.name = "cnp_bwd5";
  for (int i = 0; i < nside; ++i) {
    const size_t blk = (size_t)side[i].n * b * b * 4;
    // a side with saved planes is not unpacked again (its segment is left empty)
    un.src[i] = side[i].theta; un.n[i] = side[i].qsave ? 0 : side[i].n;
    un.planes[i] = side[i].qsave ? (bf16_t *)side[i].qsave : (bf16_t *)ar.take(blk);
    c.seg[i].qp = un.planes[i]; c.seg[i].dg = side[i].dg; c.seg[i].nblk = side[i].n;
    c.seg[i].out = (float *)ar.take(blk);
    pk.src[i] = c.seg[i].out; pk.dst[i] = side[i].dtheta; pk.n[i] = side[i].n;
  }
  POETX_TRY(unpack_skew2(un, b, s));
  POETX_TRY(cnp_bwd5(c, s));
  return pack_sides(pk, side, nside, b, theta_bf16, h, s);
}

int cnp_bwd_impl(int64_t b, const CnpBwdSide *side, int nside, int theta_bf16, const AdamEpi *h, void *ws,
                 hipStream_t s) {
  if (const int64_t bp = cnp_pad_to(b)) {
    // padded blocks; a fused Adam update then runs as its own pass on the cut-out dtheta
    Arena ar(ws);
    CnpBwdSide ps[2];
    float *dt[2] = {nullptr, nullptr};
    int64_t nall = 0;
    for (int i = 0; i < nside; ++i) {
      const int64_t n = side[i].n;
      nall += n;
      void *tp = ar.take((size_t)n * (bp * (bp - 1) / 2) * 4);
      void *dgp = ar.take((size_t)n * bp * bp * 4);
      void *dtp = ar.take((size_t)n * (bp * (bp - 1) / 2) * 4);
      float *own = (float *)ar.take((size_t)n * (b * (b - 1) / 2) * 4);
      dt[i] = side[i].dtheta ? side[i].dtheta : own;
      POETX_TRY(cnp_pad(CNP_PAD_THETA, n, b, bp, theta_bf16 ? 2 : 4, side[i].theta, tp, s));
      POETX_TRY(cnp_pad(CNP_PAD_DG, n, b, bp, 4, side[i].dg, dgp, s));
      ps[i].n = n; ps[i].theta = tp; ps[i].dg = (const float *)dgp; ps[i].dtheta = (float *)dtp;
    }
    POETX_TRY(cnp_bwd_impl(bp, ps, nside, theta_bf16, nullptr, ar.take(cnp_ws_bytes(POETX_CNP_BWD, nall, bp)), s));
    for (int i = 0; i < nside; ++i) {
      POETX_TRY(cnp_pad(CNP_CUT_DTHETA, side[i].n, b, bp, 4, ps[i].dtheta, dt[i], s));
      if (!h) continue;
      const int64_t np = side[i].n * (b * (b - 1) / 2);
      if (side[i].theta_out != side[i].theta &&
          hipMemcpyAsync(side[i].theta_out, side[i].theta, (size_t)np * (theta_bf16 ? 2 : 4), hipMemcpyDeviceToDevice,
                         s) != hipSuccess)
        return POETX_ERR_HIP;
      POETX_TRY(adam_step(np, side[i].theta_out, theta_bf16 ? POETX_BF16 : POETX_F32, dt[i], side[i].m, side[i].v,
                          *h, s));
    }
    return POETX_OK;
  }
  // the chain and MFMA paths read dG with vector loads: an only element-aligned dG
  // takes the vector-ALU path
  bool vec = true;
  for (int i = 0; i < nside; ++i) vec = vec && al16(side[i].dg);
  if (vec && cnp_bwd5_supported(b)) return cnp_bwd5_path(b, side, nside, theta_bf16, h, ws, s);
  Arena ar(ws);
  struct Bufs { float *Q, *K1, *K2, *K3, *Ha, *Hb; } B[2] = {};
  SkewSegs un;
  un.src_bf16 = theta_bf16;
  for (int i = 0; i < nside; ++i) {
    size_t blk = (size_t)side[i].n * b * b * 4;
    B[i] = {(float *)ar.take(blk), (float *)ar.take(blk), (float *)ar.take(blk),
            (float *)ar.take(blk), (float *)ar.take(blk), (float *)ar.take(blk)};
    un.src[i] = side[i].theta; un.dst[i] = B[i].Q; un.n[i] = side[i].n;
  }
  POETX_TRY(unpack_skew2(un, b, s));
  if (vec && cnp_use_mfma(b)) {
    auto run = [&](auto fill, float alpha, float c0, float c1, float c2, float c3) {
      CnpMMArgs a;
      a.b = (int)b;
      a.name = "cnp_bwd_mm";
      a.alpha[0] = alpha;
      a.ce[0][0] = c0; a.ce[0][1] = c1; a.ce[0][2] = c2; a.ce[0][3] = c3;
      for (int i = 0; i < nside; ++i) {
        fill(a.seg[i], side[i], B[i]);
        a.seg[i].nblk = side[i].n;
      }
      return cnp_mm(a, s);
    };
    // K1 = Gb P = -Gb Q ; K2 = -K1 Q ; K3 = -K2 Q
    POETX_TRY(run([](CnpMMSeg &g, const CnpBwdSide &sd, Bufs &u) { g.A = sd.dg; g.B = u.Q; g.C = u.K1; }, -1.f, 0, 0, 0, 0));
    POETX_TRY(run([](CnpMMSeg &g, const CnpBwdSide &sd, Bufs &u) { g.A = u.K1; g.B = u.Q; g.C = u.K2; }, -1.f, 0, 0, 0, 0));
    POETX_TRY(run([](CnpMMSeg &g, const CnpBwdSide &sd, Bufs &u) { g.A = u.K2; g.B = u.Q; g.C = u.K3; }, -1.f, 0, 0, 0, 0));
    // H2 = 2Gb + K1 - Q Gb
    POETX_TRY(run([](CnpMMSeg &g, const CnpBwdSide &sd, Bufs &u) {
      g.A = u.Q; g.B = sd.dg; g.C = u.Ha; g.E[0] = sd.dg; g.E[1] = u.K1; }, -1.f, 2.f, 1.f, 0, 0));
    // H1 = 2Gb + 2K1 + K2 - Q H2
    POETX_TRY(run([](CnpMMSeg &g, const CnpBwdSide &sd, Bufs &u) {
      g.A = u.Q; g.B = u.Ha; g.C = u.Hb; g.E[0] = sd.dg; g.E[1] = u.K1; g.E[2] = u.K2; }, -1.f, 2.f, 2.f, 1.f, 0));
    // Qbar = 2Gb + 2K1 + 2K2 + K3 - Q H1
    POETX_TRY(run([](CnpMMSeg &g, const CnpBwdSide &sd, Bufs &u) {
      g.A = u.Q; g.B = u.Hb; g.C = u.Ha; g.E[0] = sd.dg; g.E[1] = u.K1; g.E[2] = u.K2; g.E[3] = u.K3; },
      -1.f, 2.f, 2.f, 2.f, 1.f));
    SkewSegs pk;
    for (int i = 0; i < nside; ++i) { pk.src[i] = B[i].Ha; pk.dst[i] = side[i].dtheta; pk.n[i] = side[i].n; }
    return pack_sides(pk, side, nside, b, theta_bf16, h, s);
  }
  for (int i = 0; i < nside; ++i) {
    const int64_t n = side[i].n;
    const float *dg = side[i].dg;
    Bufs &u = B[i];
    if (n == 0) continue;
    POETX_TRY(gemm_generic(with_terms(batched_f32(n, b, dg, u.Q, u.K1, POETX_F32), nullptr, 0.f, -1.f), s));
    POETX_TRY(gemm_generic(with_terms(batched_f32(n, b, u.K1, u.Q, u.K2, POETX_F32), nullptr, 0.f, -1.f), s));
    POETX_TRY(gemm_generic(with_terms(batched_f32(n, b, u.K2, u.Q, u.K3, POETX_F32), nullptr, 0.f, -1.f), s));
    POETX_TRY(lincomb(u.Hb, n, b, 0.f, dg, 2.f, u.K1, 1.f, nullptr, 0.f, nullptr, 0.f, s));
    POETX_TRY(gemm_generic(with_terms(batched_f32(n, b, u.Q, dg, u.Ha, POETX_F32), u.Hb, 1.f, -1.f), s));
    POETX_TRY(lincomb(u.K1, n, b, 0.f, dg, 2.f, u.K1, 2.f, u.K2, 1.f, nullptr, 0.f, s));  // R1 (K1 -> 2Gb + 2K1 + K2)
    POETX_TRY(gemm_generic(with_terms(batched_f32(n, b, u.Q, u.Ha, u.Hb, POETX_F32), u.K1, 1.f, -1.f), s));
    // R0 = 2Gb + 2K1 + 2K2 + K3 = R1 + K2 + K3 (u.K1 now holds R1)
    POETX_TRY(lincomb(u.K2, n, b, 0.f, u.K1, 1.f, u.K2, 1.f, u.K3, 1.f, nullptr, 0.f, s));
    POETX_TRY(gemm_generic(with_terms(batched_f32(n, b, u.Q, u.Hb, u.Ha, POETX_F32), u.K2, 1.f, -1.f), s));
    SkewSegs pk;
    pk.src[0] = u.Ha; pk.dst[0] = side[i].dtheta; pk.n[0] = n;
    POETX_TRY(pack_sides(pk, side + i, 1, b, theta_bf16, h, s));
  }
  return POETX_OK;
}

}  // namespace

extern "C" int poetx_cnp(int32_t dir, int64_t nblocks, int64_t b, const void *theta, int32_t theta_dtype,
                         void *g, int32_t g_dtype, void *qsave, const void *dg, int32_t dg_dtype,
                         float *dtheta, void *ws, size_t *ws_bytes, void *stream) {
  if (dir != POETX_CNP_FWD && dir != POETX_CNP_BWD) return POETX_ERR_INVALID_ARG;
  if (theta_dtype != POETX_F32 && theta_dtype != POETX_BF16) return POETX_ERR_INVALID_ARG;
  if (nblocks < 0 || !ws_bytes) return POETX_ERR_INVALID_ARG;
  if (b < 1 || b > 1024) return POETX_ERR_SHAPE;
  if (dir == POETX_CNP_FWD) {
    if (g_dtype != POETX_F32 && g_dtype != POETX_BF16) return POETX_ERR_INVALID_ARG;
  } else {
    if (dg_dtype != POETX_F32) return POETX_ERR_UNSUPPORTED;
  }
  size_t need = cnp_ws_bytes(dir, nblocks, b);
  if (!ws) {
    *ws_bytes = need;
    return POETX_OK;
  }
  // (blocks of size 1 have no parameters: theta and dtheta may then be NULL)
  if (!theta && b > 1) return POETX_ERR_INVALID_ARG;
  if (dir == POETX_CNP_FWD && !g) return POETX_ERR_INVALID_ARG;
  if (dir == POETX_CNP_BWD && (!dg || (!dtheta && b > 1))) return POETX_ERR_INVALID_ARG;
  if (*ws_bytes < need) return POETX_ERR_WORKSPACE;
  if (qsave && !al16(qsave)) return POETX_ERR_INVALID_ARG;
  if (nblocks == 0) return POETX_OK;
  hipStream_t s = (hipStream_t)stream;
  if (b == 1) {  // no parameters: G = [1], nothing to differentiate
    return dir == POETX_CNP_FWD ? fill_one(g, nblocks, g_dtype, s) : POETX_OK;
  }
  const int tb = theta_dtype == POETX_BF16;
  if (!cnp_bwd5_supported(b)) qsave = nullptr;  // only the five-product backward reads the planes
  if (dir == POETX_CNP_FWD) return cnp_fwd_impl(nblocks, b, theta, tb, g, g_dtype, qsave, ws, s);
  CnpBwdSide sd;
  sd.n = nblocks; sd.theta = theta; sd.dg = (const float *)dg; sd.dtheta = dtheta; sd.qsave = qsave;
  return cnp_bwd_impl(b, &sd, 1, tb, nullptr, ws, s);
}

// ================================================================== layer ====
namespace {

// A side of width d has ceil(d/b) diagonal blocks (Method §3): d/b full b x b blocks
// (nr, np) and, when b does not divide d, a last block of size d % b (lr, lp; 0 when
// there is none).  theta and G of a side hold the full blocks, then the last one.
struct Plan {
  int64_t N, din, dout, b, nr, np, lr, lp;
  int act, w, gdt;
  bool mem, mfma;
  size_t ae;  // activation element size
};

// Block products and gradients of blocks of size bs run on MFMA for bf16 activations when
// bs is 64 or a multiple of 128 (the streaming kernels, or the batched MFMA engines for
// other multiples of 128); every other size on the float32 vector-ALU product.
bool blk_mfma(const Plan &p, int64_t bs) { return p.act == POETX_BF16 && (bs == 64 || bs % 128 == 0); }
// A lone bf16 block (a side's last block) of another size that is a multiple of 8: its
// products and gradient take the tail forms of the 128 x 128 MFMA block kernels where the
// operands are 16-byte aligned, else the vector-ALU product.
bool lone_block(const Plan &p, int64_t nb, int64_t bs) {
  return p.act == POETX_BF16 && p.gdt == POETX_BF16 && nb == 1 && !blk_mfma(p, bs) && bs % 8 == 0;
}

int validate(const poetx_layer *L, int64_t n_tokens, Plan &p) {
  if (!L || n_tokens < 0) return POETX_ERR_INVALID_ARG;
  if (L->d_in < 1 || L->d_out < 1) return POETX_ERR_INVALID_ARG;
  if (L->b < 2 || L->b > 1024) return POETX_ERR_SHAPE;
  if (L->act_dtype != POETX_F32 && L->act_dtype != POETX_BF16) return POETX_ERR_INVALID_ARG;
  if (L->w_dtype != POETX_F32 && L->w_dtype != POETX_BF16 && L->w_dtype != POETX_I8) return POETX_ERR_INVALID_ARG;
  if (L->g_dtype != L->act_dtype) return POETX_ERR_UNSUPPORTED;
  if (L->variant != POETX_FAST && L->variant != POETX_MEM) return POETX_ERR_INVALID_ARG;
  if (L->theta_dtype != POETX_F32 && L->theta_dtype != POETX_BF16) return POETX_ERR_INVALID_ARG;
  if (L->w_dtype == POETX_I8) {
    if (L->act_dtype != POETX_BF16) return POETX_ERR_UNSUPPORTED;
    if (L->variant == POETX_FAST) return POETX_ERR_UNSUPPORTED;
    // a kept W'^T is a BF16-only option: the int8 backward transposes W' itself
    if (L->w_merged_t) return POETX_ERR_INVALID_ARG;
  } else if (L->w_dtype != L->act_dtype) {
    return POETX_ERR_UNSUPPORTED;
  }
  if ((size_t)(L->d_in > L->d_out ? L->d_in : L->d_out) * dtype_size(L->act_dtype) > 65536)
    return POETX_ERR_UNSUPPORTED;
  p.N = n_tokens; p.din = L->d_in; p.dout = L->d_out; p.b = L->b;
  p.nr = L->d_in / L->b; p.np = L->d_out / L->b;
  p.lr = L->d_in % L->b; p.lp = L->d_out % L->b;
  p.act = L->act_dtype; p.w = L->w_dtype; p.gdt = L->g_dtype;
  p.mem = L->variant == POETX_MEM;
  p.ae = dtype_size(p.act);
  // the W' products run on MFMA whenever both widths tile by 128, whatever b is, and for
  // bf16 weights whenever both are multiples of 8 (the NT kernel's tail form); each block
  // product picks its own kernel by its block size (blk_mfma)
  const bool tiles128 = p.din % 128 == 0 && p.dout % 128 == 0;
  p.mfma = p.act == POETX_BF16 &&
           (tiles128 || (p.w == POETX_BF16 && p.din % 8 == 0 && p.dout % 8 == 0));
  return POETX_OK;
}

int check_layer_ptrs(const poetx_layer *L) {
  if (!L->w_merged || !L->theta_r || !L->theta_p || !L->g_r || !L->g_p) return POETX_ERR_INVALID_ARG;
  if (L->w_dtype == POETX_I8 && !L->w_scale) return POETX_ERR_INVALID_ARG;
  return POETX_OK;
}

// Y[:, o:o+bs] = X[:, o:o+bs] . G[j]  (transposed: . G[j]^T) for nb blocks of size bs
// at column offsets o = j*bs; X, Y have row stride ld, G is [nb][bs][bs].
// Gt: optional copy of the blocks' transposes (b = 512): the plain product then runs on the
// k-contiguous NT kernel too.
int apply_blocks(const Plan &p, int64_t ld, int64_t nb, int64_t bs, const void *X, const void *G, void *Y,
                 bool transposed, const float *scaleN, hipStream_t s, const void *Gt = nullptr) {
  if (p.N == 0 || nb == 0) return POETX_OK;
  const bool mfma = blk_mfma(p, bs);
  if (mfma && block_stream_supported(bs, ld, nb, p.N))
    return block_stream((const bf16_t *)X, (const bf16_t *)G, (bf16_t *)Y, p.N, ld, nb, bs, transposed, scaleN,
                        transposed ? "block_apply_t" : "block_apply", s);
  if (mfma && bs == 512) {
    // Shapes the streaming kernel does not take: each block product at b = 512 is a
    // K = N = 512 GEMM on the 256 x 256 W' kernels, batched over blocks
    const bool kc = transposed || Gt;  // B k-contiguous: G^T of the blocks, or G itself for the transposed product
    MfmaDesc m;
    m.M = p.N; m.N = bs; m.K = bs; m.batch = nb;
    m.A = X; m.a_km = false; m.lda = ld; m.sAb = bs;
    m.B = transposed ? G : (Gt ? Gt : G); m.b_km = !kc; m.b_dt = POETX_BF16; m.ldb = bs; m.sBb = bs * bs;
    m.C = Y; m.c_dt = p.act; m.ldc = ld; m.sCb = bs;
    m.scaleN = scaleN; m.sSNb = bs;
    m.name = transposed ? "block_apply_t" : "block_apply";
    m.role = kc ? MFMA_GEMM_NT : MFMA_GEMM_NN;
    if (mfma2_supported(m)) return gemm_mfma2(m, s);
  }
  if (mfma && bs % 128 == 0) {
    MfmaDesc m;
    m.M = p.N; m.N = bs; m.K = bs; m.batch = nb;
    m.A = X; m.a_km = false; m.lda = ld; m.sAb = bs;
    m.B = G; m.b_km = !transposed; m.b_dt = POETX_BF16; m.ldb = bs; m.sBb = bs * bs;
    m.C = Y; m.c_dt = p.act; m.ldc = ld; m.sCb = bs;
    m.scaleN = scaleN; m.sSNb = bs;
    m.name = transposed ? "block_apply_t" : "block_apply";
    m.role = transposed ? MFMA_BLOCK_APPLY_T : MFMA_BLOCK_APPLY;
    return gemm_mfma_best(m, s);
  }
  if (lone_block(p, nb, bs)) {
    // a last block of a size with no block kernel: the tail form of the 128 x 128 kernels
    MfmaDesc m;
    m.M = p.N; m.N = bs; m.K = bs;
    m.A = X; m.a_km = false; m.lda = ld;
    m.B = G; m.b_km = !transposed; m.b_dt = POETX_BF16; m.ldb = bs;
    m.C = Y; m.c_dt = p.act; m.ldc = ld;
    m.scaleN = scaleN;
    m.name = transposed ? "block_apply_t" : "block_apply";
    m.role = transposed ? MFMA_BLOCK_APPLY_T : MFMA_BLOCK_APPLY;
    if (mfma2_supported(m)) return gemm_mfma2(m, s);
  }
  GemmDesc g;
  g.M = p.N; g.N = bs; g.K = bs; g.batch = nb;
  g.A = X; g.a_dt = p.act; g.sAb = bs; g.sAm = ld; g.sAk = 1;
  g.B = G; g.b_dt = p.gdt; g.sBb = bs * bs;
  if (transposed) { g.sBk = 1; g.sBn = bs; } else { g.sBk = bs; g.sBn = 1; }
  g.C = Y; g.c_dt = p.act; g.sCb = bs; g.sCm = ld; g.sCn = 1;
  g.scaleN = scaleN; g.sSNb = bs;
  g.name = transposed ? "block_apply_t_generic" : "block_apply_generic";
  return gemm_generic(g, s);
}

// Offsets of a side's last block: its first column and its G.
const void *col_off(const Plan &p, const void *X, int64_t c) { return (const char *)X + c * p.ae; }
void *col_off(const Plan &p, void *X, int64_t c) { return (char *)X + c * p.ae; }
const void *g_last(const Plan &p, const void *G, int64_t nb) {
  return (const char *)G + nb * p.b * p.b * dtype_size(p.gdt);
}

// Y = X . Diag(G) (transposed: . Diag(G)^T) over all ceil(d/b) blocks of a side.  Gt, if
// given, holds the full blocks' transposes (see apply_blocks).
int block_apply(const Plan &p, int64_t d, const void *X, const void *G, void *Y, bool transposed,
                const float *scaleN, hipStream_t s, const void *Gt = nullptr) {
  const int64_t b = p.b, nb = d / b, bl = d % b;
  POETX_TRY(apply_blocks(p, d, nb, b, X, G, Y, transposed, scaleN, s, Gt));
  if (bl == 0) return POETX_OK;
  const int64_t c = nb * b;
  return apply_blocks(p, d, 1, bl, col_off(p, X, c), g_last(p, G, nb), col_off(p, Y, c), transposed,
                      scaleN ? scaleN + c : nullptr, s);
}

// dG[j] = X[:, o:o+bs]^T . Y[:, o:o+bs] (sum over tokens) for nb blocks of size bs, as
// fp32 partials [P][nb][bs][bs] that are summed later in a fixed order;
// grad_parts() is P.
// The streaming kernel owns 128 x 128 slices of a block's gradient: at b = 512 sixteen of
// them, so every operand slice is read by four workgroups; there the MFMA engine's 256 x 256
// tiles (two readers per slice) split over tokens take over.
bool grad_streams(const Plan &p, int64_t ld, int64_t nb, int64_t bs) {
  return blk_mfma(p, bs) && bs < 512 && p.N > 0 && block_grad_stream_supported(bs, ld, nb, p.N);
}

// the batched MFMA engine (256 x 256 or 128 x 128 tiles split over tokens) takes the
// gradients of blocks of a multiple of 128 that the streaming kernel does not
bool grad_engine(const Plan &p, int64_t bs) { return blk_mfma(p, bs) && bs % 128 == 0; }

int64_t grad_chunk(const Plan &p, int64_t nb, int64_t bs) {  // token chunk of the split-k kernel
  if (p.N == 0) return 1;
  if (!grad_engine(p, bs) && !lone_block(p, nb, bs)) {
    // vector-ALU product: chunks of 1024 tokens keep each float32 accumulation short (a sum
    // over millions of tokens in one chain loses digits), with at most 4096 partials and
    // 256 MB of them.  A single block (the last, smaller block of a side) runs all its
    // chunks in one launch, 256 tokens each, so that its few output tiles are spread over
    // many workgroups.
    const int64_t part_bytes = nb * bs * bs * 4, kmin = nb == 1 ? 256 : 1024;
    int64_t pmax = ((int64_t)256 << 20) / (part_bytes > 0 ? part_bytes : 1);
    pmax = pmax < 1 ? 1 : pmax > 4096 ? 4096 : pmax;
    const int64_t kc = cdiv(p.N, pmax);
    return p.N <= kmin ? p.N : kc > kmin ? kc : kmin;
  }
  // about one round of workgroups: 256 x 256 tiles where b allows (fp32 partials of a
  // whole b x b per split, so no more splits than the CUs need)
  const int64_t t = bs % 256 == 0 ? 256 : 128;
  const int64_t tiles = nb * cdiv(bs, t) * cdiv(bs, t);
  const int cus = device_cus() > 0 ? device_cus() : 256;
  const int64_t want = t == 256 ? (cus / tiles > 1 ? cus / tiles : 1) : cdiv(512, tiles);
  int64_t kc = cdiv(cdiv(p.N, want), 64) * 64;
  if (kc > kMaxChain) kc = kMaxChain;  // keep each float32 accumulation chain bounded
  return kc < 256 ? 256 : kc;
}

int64_t grad_parts(const Plan &p, int64_t ld, int64_t nb, int64_t bs) {
  if (p.N == 0 || nb == 0) return 1;
  if (grad_streams(p, ld, nb, bs)) return block_grad_stream_parts(bs, nb, p.N);
  return cdiv(p.N, grad_chunk(p, nb, bs));
}

int grad_blocks(const Plan &p, int64_t ld, int64_t nb, int64_t bs, const void *X, const void *Y, float *parts,
                hipStream_t s) {
  if (nb == 0) return POETX_OK;
  if (grad_streams(p, ld, nb, bs))
    return block_grad_stream((const bf16_t *)X, (const bf16_t *)Y, parts, p.N, ld, nb, bs, s);
  if (grad_engine(p, bs) || lone_block(p, nb, bs)) {
    const int64_t kc = grad_chunk(p, nb, bs);
    MfmaDesc m;
    m.M = bs; m.N = bs; m.K = p.N; m.batch = nb;
    m.splits = cdiv(p.N, kc); m.kchunk = kc;
    m.A = X; m.a_km = true; m.lda = ld; m.sAb = bs;
    m.B = Y; m.b_km = true; m.b_dt = POETX_BF16; m.ldb = ld; m.sBb = bs;
    m.C = parts; m.c_dt = POETX_F32; m.ldc = bs; m.sCb = bs * bs; m.sCsplit = nb * bs * bs;
    m.name = "block_grad";
    m.role = MFMA_BLOCK_GRAD;
    if (grad_engine(p, bs)) return gemm_mfma_best(m, s);
    if (mfma2_supported(m)) return gemm_mfma2(m, s);
    // an unaligned lone block: the vector-ALU product below, with the same token chunks
  }
  // vector-ALU product into partial c of [P][nb][bs][bs]: one launch per token chunk (a
  // batch over the blocks), or for a single block one launch over its whole chunks (a
  // batch over the chunks) and one for a shorter last chunk
  const int64_t kc = grad_chunk(p, nb, bs);
  if (nb == 1 && p.N >= kc) {
    const int64_t whole = p.N / kc;
    GemmDesc g;
    g.M = bs; g.N = bs; g.K = kc; g.batch = whole;
    g.A = X; g.a_dt = p.act; g.sAb = kc * ld; g.sAm = 1; g.sAk = ld;
    g.B = Y; g.b_dt = p.act; g.sBb = kc * ld; g.sBk = ld; g.sBn = 1;
    g.C = parts; g.c_dt = POETX_F32; g.sCb = bs * bs; g.sCm = bs; g.sCn = 1;
    g.name = "block_grad_generic";
    POETX_TRY(gemm_generic(g, s));
    if (whole * kc == p.N) return POETX_OK;
    g.K = p.N - whole * kc; g.batch = 1;
    g.A = col_off(p, X, whole * kc * ld);
    g.B = col_off(p, Y, whole * kc * ld);
    g.C = parts + whole * bs * bs;
    return gemm_generic(g, s);
  }
  for (int64_t c = 0, t0 = 0; t0 < p.N; ++c, t0 += kc) {
    GemmDesc g;
    g.M = bs; g.N = bs; g.K = p.N - t0 < kc ? p.N - t0 : kc; g.batch = nb;
    g.A = col_off(p, X, t0 * ld); g.a_dt = p.act; g.sAb = bs; g.sAm = 1; g.sAk = ld;
    g.B = col_off(p, Y, t0 * ld); g.b_dt = p.act; g.sBb = bs; g.sBk = ld; g.sBn = 1;
    g.C = parts + c * nb * bs * bs; g.c_dt = POETX_F32; g.sCb = bs * bs; g.sCm = bs; g.sCn = 1;
    g.name = "block_grad_generic";
    POETX_TRY(gemm_generic(g, s));
  }
  return POETX_OK;
}

// Partials of the block gradients of a side: full blocks and the last block apart.
struct GradParts {
  int64_t P = 1, Pl = 1;           // partial counts
  float *full = nullptr, *last = nullptr;
};

// A single partial (P = 1) is the gradient itself: it is written straight into dG and
// takes no workspace.
void carve_grad_parts(Arena &ar, const Plan &p, int64_t d, GradParts &g) {
  const int64_t b = p.b, nb = d / b, bl = d % b;
  g.P = grad_parts(p, d, nb, b);
  g.full = g.P > 1 ? (float *)ar.take((size_t)g.P * nb * b * b * 4) : nullptr;
  g.Pl = bl ? grad_parts(p, d, 1, bl) : 1;
  g.last = bl && g.Pl > 1 ? (float *)ar.take((size_t)g.Pl * bl * bl * 4) : nullptr;
}

// dG of every block of a side into dg ([nb][b][b] then [bl][bl]), via the partials when
// there are several.
int block_grad(const Plan &p, int64_t d, const void *X, const void *Y, const GradParts &gp, float *dg,
               hipStream_t s) {
  const int64_t b = p.b, nb = d / b, bl = d % b;
  if (nb) {
    if (gp.P == 1) {
      POETX_TRY(grad_blocks(p, d, nb, b, X, Y, dg, s));
    } else {
      POETX_TRY(grad_blocks(p, d, nb, b, X, Y, gp.full, s));
      POETX_TRY(reduce_parts(gp.full, dg, nb * b * b, gp.P, nb * b * b, s));
    }
  }
  if (bl) {
    const int64_t c = nb * b;
    float *dgl = dg + nb * b * b;
    if (gp.Pl == 1) {
      POETX_TRY(grad_blocks(p, d, 1, bl, col_off(p, X, c), col_off(p, Y, c), dgl, s));
    } else {
      POETX_TRY(grad_blocks(p, d, 1, bl, col_off(p, X, c), col_off(p, Y, c), gp.last, s));
      POETX_TRY(reduce_parts(gp.last, dgl, bl * bl, gp.Pl, bl * bl, s));
    }
  }
  return POETX_OK;
}

// B = A . W'^T (scaled per output row of W' for int8 weights)
// `tail` (may be null): workspace of gemm_tail_ws_bytes for the product's shape.
int gemm_fwd(const Plan &p, const poetx_layer *L, const void *A, void *B, void *tail, size_t tail_bytes,
             hipStream_t s) {
  if (p.N == 0) return POETX_OK;
  if (p.mfma) {
    MfmaDesc m;
    m.M = p.N; m.N = p.dout; m.K = p.din;
    m.A = A; m.a_km = false; m.lda = p.din;
    m.B = L->w_merged; m.b_km = false; m.b_dt = p.w; m.ldb = p.din;
    m.C = B; m.c_dt = p.act; m.ldc = p.dout;
    m.scaleN = p.w == POETX_I8 ? L->w_scale : nullptr;
    m.name = "gemm_nt";
    m.role = MFMA_GEMM_NT;
    m.tail_ws = tail;
    m.tail_ws_bytes = tail ? tail_bytes : 0;
    return gemm_mfma_best(m, s);
  }
  GemmDesc g;
  g.M = p.N; g.N = p.dout; g.K = p.din;
  g.A = A; g.a_dt = p.act; g.sAm = p.din; g.sAk = 1;
  g.B = L->w_merged; g.b_dt = p.w; g.sBk = 1; g.sBn = p.din;
  g.C = B; g.c_dt = p.act; g.sCm = p.dout; g.sCn = 1;
  g.scaleN = p.w == POETX_I8 ? L->w_scale : nullptr;
  g.name = "gemm_nt_generic";
  return gemm_generic(g, s);
}

// dA = dB' . W'  (dB' already carries the int8 row scales)
// Without a kept W'^T, the backward product still runs on the k-contiguous NT kernel when
// that kernel tiles the shape: W' is transposed into the workspace first (one pass over
// the weight, much less than what reading W' n-major costs the product).
// Widths that the NT kernel tiles only in its tail form (bf16) always take this route: the
// n-major kernels need whole tiles.
bool bwd_transposes_w(const Plan &p, const poetx_layer *L) {
  if (!p.mfma || p.N == 0 || L->w_merged_t) return false;
  const bool tiles = p.din % 256 == 0 && p.dout % 64 == 0;
  return p.w == POETX_BF16 ? tiles || p.din % 128 || p.dout % 128 : p.w == POETX_I8 && tiles;
}

// `wt`: workspace for W'^T when bwd_transposes_w, else null.
int gemm_bwd(const Plan &p, const poetx_layer *L, const void *dB, void *dA, void *tail, size_t tail_bytes,
             void *wt, hipStream_t s) {
  if (p.N == 0) return POETX_OK;
  const void *w_t = p.w == POETX_BF16 ? L->w_merged_t : nullptr;
  if (p.mfma && !w_t && wt) {
    POETX_TRY(transpose(L->w_merged, wt, p.dout, p.din, (int)dtype_size(p.w), s));
    w_t = wt;
  }
  if (p.mfma && w_t) {
    // dA = dB . (W'^T)^T: both operands k-contiguous
    MfmaDesc m;
    m.M = p.N; m.N = p.din; m.K = p.dout;
    m.A = dB; m.a_km = false; m.lda = p.dout;
    m.B = w_t; m.b_km = false; m.b_dt = p.w; m.ldb = p.dout;
    m.C = dA; m.c_dt = p.act; m.ldc = p.din;
    m.name = "gemm_nn";
    m.role = MFMA_GEMM_NT;
    m.tail_ws = tail;
    m.tail_ws_bytes = tail ? tail_bytes : 0;
    return gemm_mfma_best(m, s);
  }
  if (p.mfma) {
    MfmaDesc m;
    m.M = p.N; m.N = p.din; m.K = p.dout;
    m.A = dB; m.a_km = false; m.lda = p.dout;
    m.B = L->w_merged; m.b_km = true; m.b_dt = p.w; m.ldb = p.din;
    m.C = dA; m.c_dt = p.act; m.ldc = p.din;
    m.name = "gemm_nn";
    m.role = MFMA_GEMM_NN;
    m.tail_ws = tail;
    m.tail_ws_bytes = tail ? tail_bytes : 0;
    return gemm_mfma_best(m, s);
  }
  GemmDesc g;
  g.M = p.N; g.N = p.din; g.K = p.dout;
  g.A = dB; g.a_dt = p.act; g.sAm = p.dout; g.sAk = 1;
  g.B = L->w_merged; g.b_dt = p.w; g.sBk = p.din; g.sBn = 1;
  g.C = dA; g.c_dt = p.act; g.sCm = p.din; g.sCn = 1;
  g.name = "gemm_nn_generic";
  return gemm_generic(g, s);
}

struct FwdBufs {
  void *xg = nullptr, *a = nullptr, *bt = nullptr, *zt = nullptr;
  void *gt_r = nullptr, *gt_p = nullptr;  // transposed G blocks for the plain b = 512 products
};

// b = 512 on the MFMA kernels: the plain block products read G^T k-contiguous
// G^T copies serve the plain b = 512 products that the streaming kernel does not take
bool wants_gt(const Plan &p, int64_t d, int64_t nb) {
  return p.mfma && p.b == 512 && p.gdt == POETX_BF16 && !block_stream_supported(p.b, d, nb, p.N);
}

// G^T of a side's nb full blocks into gt; *out = gt, or null where there is no buffer or G
// is not 16-byte aligned (the product then reads G n-major).
int transposed_g(const Plan &p, const void *g, void *gt, int64_t nb, hipStream_t s, const void **out) {
  *out = nullptr;
  if (!gt || nb == 0) return POETX_OK;
  const int st = transpose_batched(g, gt, nb, p.b, p.b, s);
  if (st == POETX_ERR_UNSUPPORTED) return POETX_OK;
  if (st == POETX_OK) *out = gt;
  return st;
}

// Carve forward intermediates.  `want_b` asks for B in the workspace; `saved_x` (the
// caller's buffer for X~, or null) replaces the workspace copy of X~.
// fwd: the forward (both plain products), else the backward (the R side's, recomputed by mem).
void carve_fwd(Arena &ar, const Plan &p, const poetx_layer *L, bool want_b, void *saved_x, FwdBufs &f,
               bool fwd = true) {
  size_t xin = (size_t)p.N * p.din * p.ae, xout = (size_t)p.N * p.dout * p.ae;
  if (p.N > 0) {
    if (p.nr && (fwd || p.mem) && wants_gt(p, p.din, p.nr)) f.gt_r = ar.take((size_t)p.nr * p.b * p.b * 2);
    if (p.np && fwd && wants_gt(p, p.dout, p.np)) f.gt_p = ar.take((size_t)p.np * p.b * p.b * 2);
  }
  if (L->perm_in) f.xg = saved_x ? saved_x : ar.take(xin);
  f.a = ar.take(xin);
  if (want_b) f.bt = ar.take(xout);
  if (L->perm_out) f.zt = ar.take(xout);
}

// workspace for splitting the leftover tiles of the forward W' product
size_t tail_fwd_bytes(const Plan &p) { return p.mfma ? gemm_tail_ws_bytes(p.N, p.dout, p.din) : 0; }
// ... and of the backward one (dA = dB . W', same tiles with or without W'^T)
size_t tail_bwd_bytes(const Plan &p) { return p.mfma ? gemm_tail_ws_bytes(p.N, p.din, p.dout) : 0; }

// Gather(X) -> Xg ; A = Xg . Diag(G_R) ; B = A . W'^T
int run_front(const Plan &p, const poetx_layer *L, const void *x, const FwdBufs &f, void *bt, void *tail,
              size_t tail_bytes, hipStream_t s) {
  const void *xg = x;
  if (L->perm_in) {
    POETX_TRY(permute_cols(x, f.xg, p.N, p.din, (int)p.ae, nullptr, L->perm_in, false, s));
    xg = f.xg;
  }
  const void *gtr;
  POETX_TRY(transposed_g(p, L->g_r, f.gt_r, p.nr, s, &gtr));
  POETX_TRY(block_apply(p, p.din, xg, L->g_r, f.a, false, nullptr, s, gtr));
  return gemm_fwd(p, L, f.a, bt, tail, tail_bytes, s);
}

}  // namespace

extern "C" int poetx_forward(const poetx_layer *L, int64_t n_tokens, const void *x, void *z,
                             void *saved_b, void *saved_x, void *ws, size_t *ws_bytes, void *stream) {
  Plan p;
  POETX_TRY(validate(L, n_tokens, p));
  if (!ws_bytes) return POETX_ERR_INVALID_ARG;
  if (p.mem && (saved_b || saved_x)) return POETX_ERR_INVALID_ARG;
  Arena ar(ws);
  FwdBufs f;
  carve_fwd(ar, p, L, p.mem, L->perm_in ? saved_x : nullptr, f);
  const size_t tb = tail_fwd_bytes(p);
  void *tail = tb ? ar.take(tb) : nullptr;
  if (!ws) {
    *ws_bytes = ar.used;
    return POETX_OK;
  }
  POETX_TRY(check_layer_ptrs(L));
  if (p.N > 0 && (!x || !z || (!p.mem && !saved_b))) return POETX_ERR_INVALID_ARG;
  if (*ws_bytes < ar.used) return POETX_ERR_WORKSPACE;
  if (p.N == 0) return POETX_OK;
  hipStream_t s = (hipStream_t)stream;
  void *bt = p.mem ? f.bt : saved_b;
  POETX_TRY(run_front(p, L, x, f, bt, tail, tb, s));
  void *zt = L->perm_out ? f.zt : z;
  const void *gtp;
  POETX_TRY(transposed_g(p, L->g_p, f.gt_p, p.np, s, &gtp));
  POETX_TRY(block_apply(p, p.dout, bt, L->g_p, zt, false, nullptr, s, gtp));
  if (L->perm_out) POETX_TRY(permute_cols(zt, z, p.N, p.dout, (int)p.ae, nullptr, L->perm_out, true, s));
  return POETX_OK;
}

namespace {

// Bias corrections of Adam step t in double on the host; the kernels take the step size
// and 1 / sqrt(1 - beta2^t).
AdamEpi adam_hyper(float lr, float beta1, float beta2, float eps, int64_t step, float gamma) {
  const double bc1 = 1.0 - std::pow((double)beta1, (double)step), bc2 = 1.0 - std::pow((double)beta2, (double)step);
  AdamEpi h;
  h.step_size = (float)((double)gamma * (double)lr / bc1);
  h.rs2 = (float)(1.0 / std::sqrt(bc2));
  h.b1 = beta1; h.b2 = beta2; h.eps = eps;
  return h;
}

bool adam_args_ok(float beta1, float beta2, float eps, int64_t step) {
  return step >= 1 && beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f && eps > 0.f;
}

// The backward; with `opt`, the Adam update of both sides' theta fused into the pack of
// dtheta (dtheta_r / dtheta_p may then be null).
int backward_impl(const poetx_layer *L, int64_t n_tokens, const void *x, const void *dz, const void *saved_b,
                  const void *saved_x, void *dx, float *dtheta_r, float *dtheta_p, float *dg_r, float *dg_p,
                  const poetx_adam *opt, void *ws, size_t *ws_bytes, void *stream) {
  Plan p;
  POETX_TRY(validate(L, n_tokens, p));
  if (!ws_bytes) return POETX_ERR_INVALID_ARG;
  if (p.mem && (saved_b || saved_x)) return POETX_ERR_INVALID_ARG;
  // X~ kept by the forward (fast variant with an input permutation), else gathered here
  const void *kept_xg = L->perm_in ? saved_x : nullptr;
  const int64_t b = p.b, bb = b * b;
  size_t xin = (size_t)p.N * p.din * p.ae, xout = (size_t)p.N * p.dout * p.ae;
  Arena ar(ws);
  FwdBufs f;
  carve_fwd(ar, p, L, p.mem, const_cast<void *>(kept_xg), f, false);
  void *dzt = L->perm_out ? ar.take(xout) : nullptr;
  void *dbuf = ar.take(xout);
  void *da = ar.take(xin);
  void *dxt = L->perm_in ? ar.take(xin) : nullptr;
  GradParts part_r, part_p;
  carve_grad_parts(ar, p, p.din, part_r);
  carve_grad_parts(ar, p, p.dout, part_p);
  float *gr = dg_r ? dg_r : (float *)ar.take((size_t)(p.nr * bb + p.lr * p.lr) * 4);
  float *gp = dg_p ? dg_p : (float *)ar.take((size_t)(p.np * bb + p.lp * p.lp) * 4);
  // the full blocks of both sides in one CNP backward, then the last blocks; the calls
  // run one after the other and share one workspace region
  const size_t cw_full = cnp_ws_bytes(POETX_CNP_BWD, p.nr, b) + cnp_ws_bytes(POETX_CNP_BWD, p.np, b);
  const size_t cw_last = cnp_ws_bytes(POETX_CNP_BWD, p.lr > 1, p.lr) + cnp_ws_bytes(POETX_CNP_BWD, p.lp > 1, p.lp);
  void *cws = ar.take(cw_full > cw_last ? cw_full : cw_last);
  // one region serves the recomputed forward product (mem) and the dA product in turn
  const size_t tfb = p.mem ? tail_fwd_bytes(p) : 0, tbb = tail_bwd_bytes(p);  // 0: not split
  const size_t tb = tfb > tbb ? tfb : tbb;
  void *tail = tb ? ar.take(tb) : nullptr;
  void *wt = bwd_transposes_w(p, L) ? ar.take((size_t)p.din * p.dout * dtype_size(p.w)) : nullptr;
  if (!ws) {
    *ws_bytes = ar.used;
    return POETX_OK;
  }
  POETX_TRY(check_layer_ptrs(L));
  if (!opt && (!dtheta_r || !dtheta_p)) return POETX_ERR_INVALID_ARG;
  AdamEpi hyper;
  if (opt) {
    if (!adam_args_ok(opt->beta1, opt->beta2, opt->eps, opt->step)) return POETX_ERR_INVALID_ARG;
    if (!opt->theta_r_out || !opt->theta_p_out || !opt->m_r || !opt->v_r || !opt->m_p || !opt->v_p)
      return POETX_ERR_INVALID_ARG;
    hyper = adam_hyper(opt->lr, opt->beta1, opt->beta2, opt->eps, opt->step, opt->gamma);
  }
  const AdamEpi *h = opt ? &hyper : nullptr;
  const int th_bf = L->theta_dtype == POETX_BF16;
  const size_t te = th_bf ? 2 : 4;
  if (p.N > 0 && (!x || !dz || !dx || (!p.mem && !saved_b))) return POETX_ERR_INVALID_ARG;
  if (*ws_bytes < ar.used) return POETX_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;

  // B (kept by the fast variant, recomputed by the mem variant) and X~ = Gather(X)
  const void *bt = saved_b;
  const void *xg = x;
  if (p.N > 0) {
    if (p.mem) {
      POETX_TRY(run_front(p, L, x, f, f.bt, tail, tb, s));
      bt = f.bt;
    } else if (L->perm_in && !kept_xg) {
      POETX_TRY(permute_cols(x, f.xg, p.N, p.din, (int)p.ae, nullptr, L->perm_in, false, s));
    }
    if (L->perm_in) xg = f.xg;
  }
  // P side: dZ~ = Gather_out(dZ); dB = dZ~ Diag(G_P)^T; dG_P = sum_t B^T dZ~
  const void *dzg = dz;
  if (p.N > 0 && L->perm_out) {
    POETX_TRY(permute_cols(dz, dzt, p.N, p.dout, (int)p.ae, nullptr, L->perm_out, false, s));
    dzg = dzt;
  }
  if (p.N > 0) {
    POETX_TRY(block_apply(p, p.dout, dzg, L->g_p, dbuf, true,
                          p.w == POETX_I8 ? L->w_scale : nullptr, s));
    POETX_TRY(block_grad(p, p.dout, bt, dzg, part_p, gp, s));
    // dA = dB W'
    POETX_TRY(gemm_bwd(p, L, dbuf, da, tail, tb, wt, s));
    // R side: dX~ = dA Diag(G_R)^T; dG_R = sum_t X~^T dA; dX = Scatter_in(dX~)
    void *dxw = L->perm_in ? dxt : dx;
    POETX_TRY(block_apply(p, p.din, da, L->g_r, dxw, true, nullptr, s));
    if (L->perm_in) POETX_TRY(permute_cols(dxt, dx, p.N, p.din, (int)p.ae, nullptr, L->perm_in, true, s));
    POETX_TRY(block_grad(p, p.din, xg, da, part_r, gr, s));
  } else {
    POETX_TRY(lincomb(gr, p.nr, b, 0.f, nullptr, 0.f, nullptr, 0.f, nullptr, 0.f, nullptr, 0.f, s));
    POETX_TRY(lincomb(gp, p.np, b, 0.f, nullptr, 0.f, nullptr, 0.f, nullptr, 0.f, nullptr, 0.f, s));
    if (p.lr) POETX_TRY(lincomb(gr + p.nr * bb, 1, p.lr, 0.f, nullptr, 0.f, nullptr, 0.f, nullptr, 0.f, nullptr, 0.f, s));
    if (p.lp) POETX_TRY(lincomb(gp + p.np * bb, 1, p.lp, 0.f, nullptr, 0.f, nullptr, 0.f, nullptr, 0.f, nullptr, 0.f, s));
  }
  // CNP backward (Method §4): the full blocks of both sides together, then each side's
  // last block at its own size (a block of size 1 has no parameters)
  const int64_t pb = b * (b - 1) / 2;
  // a side's blocks from packed offset `off` (elements) on: theta, dtheta, new theta, state
  auto side_at = [&](bool rside, int64_t n, int64_t off, const float *dg) {
    CnpBwdSide sd;
    sd.n = n;
    sd.theta = (const char *)(rside ? L->theta_r : L->theta_p) + off * te;
    sd.dg = dg;
    float *dth = rside ? dtheta_r : dtheta_p;
    sd.dtheta = dth ? dth + off : nullptr;
    if (opt) {
      sd.theta_out = (char *)(rside ? opt->theta_r_out : opt->theta_p_out) + off * te;
      sd.m = (rside ? opt->m_r : opt->m_p) + off;
      sd.v = (rside ? opt->v_r : opt->v_p) + off;
    }
    return sd;
  };
  CnpBwdSide sides[2];
  int ns = 0;
  const bool qok = cnp_bwd5_supported(b);  // saved planes (full blocks only): five-product backward
  if (p.nr) {
    sides[ns] = side_at(true, p.nr, 0, gr);
    sides[ns++].qsave = qok ? L->q_r : nullptr;
  }
  if (p.np) {
    sides[ns] = side_at(false, p.np, 0, gp);
    sides[ns++].qsave = qok ? L->q_p : nullptr;
  }
  if (ns) POETX_TRY(cnp_bwd_impl(b, sides, ns, th_bf, h, cws, s));
  const CnpBwdSide lr = side_at(true, 1, p.nr * pb, gr + p.nr * bb);
  const CnpBwdSide lp = side_at(false, 1, p.np * pb, gp + p.np * bb);
  if (p.lr > 1 && p.lr == p.lp) {
    const CnpBwdSide both[2] = {lr, lp};
    return cnp_bwd_impl(p.lr, both, 2, th_bf, h, cws, s);
  }
  if (p.lr > 1) POETX_TRY(cnp_bwd_impl(p.lr, &lr, 1, th_bf, h, cws, s));
  if (p.lp > 1) POETX_TRY(cnp_bwd_impl(p.lp, &lp, 1, th_bf, h, cws, s));
  return POETX_OK;
}

}  // namespace

extern "C" int poetx_backward(const poetx_layer *L, int64_t n_tokens, const void *x, const void *dz,
                              const void *saved_b, const void *saved_x, void *dx, float *dtheta_r,
                              float *dtheta_p, float *dg_r, float *dg_p, void *ws, size_t *ws_bytes,
                              void *stream) {
  return backward_impl(L, n_tokens, x, dz, saved_b, saved_x, dx, dtheta_r, dtheta_p, dg_r, dg_p, nullptr, ws,
                       ws_bytes, stream);
}

extern "C" int poetx_backward_adam(const poetx_layer *L, int64_t n_tokens, const void *x, const void *dz,
                                   const void *saved_b, const void *saved_x, void *dx, float *dtheta_r,
                                   float *dtheta_p, const poetx_adam *opt, void *ws, size_t *ws_bytes,
                                   void *stream) {
  if (!opt) return POETX_ERR_INVALID_ARG;
  return backward_impl(L, n_tokens, x, dz, saved_b, saved_x, dx, dtheta_r, dtheta_p, nullptr, nullptr, opt, ws,
                       ws_bytes, stream);
}



// ================================================================= fold ====
// Phase-end fold (the consolidation step of merge-then-reinitialize): the layer's
// effective weight in original coordinates,
//   w_out[perm_out[i]][perm_in[k]] = (Diag(G_P)^T . W' . Diag(G_R)^T)[i][k],
// so that x . w_out^T is poetx_forward's z for every token row x.  The block products
// reuse the block-diagonal kernels with the rows of W' (then of the transpose) as the
// token dimension; the final gather uses the inverse permutations.
extern "C" int poetx_fold(const poetx_layer *L, void *w_out, void *ws, size_t *ws_bytes, void *stream) {
  Plan p;
  POETX_TRY(validate(L, 0, p));
  if (!ws_bytes) return POETX_ERR_INVALID_ARG;
  if (L->w_dtype == POETX_I8) return POETX_ERR_UNSUPPORTED;  // a folded int8 weight needs a requantizer
  const size_t es = dtype_size(p.w), wb = (size_t)p.dout * p.din * es;
  Arena ar(ws);
  void *m1 = ar.take(wb), *t1 = ar.take(wb), *t2 = ar.take(wb);
  int32_t *inv_out = L->perm_out ? (int32_t *)ar.take((size_t)p.dout * 4) : nullptr;
  int32_t *inv_in = L->perm_in ? (int32_t *)ar.take((size_t)p.din * 4) : nullptr;
  if (!ws) {
    *ws_bytes = ar.used;
    return POETX_OK;
  }
  if (!L->w_merged || !L->g_r || !L->g_p || !w_out) return POETX_ERR_INVALID_ARG;
  if (w_out == L->w_merged) return POETX_ERR_INVALID_ARG;
  if (*ws_bytes < ar.used) return POETX_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  Plan pr = p;
  pr.N = p.dout;  // rows of W' as tokens over d_in features: M1 = W' . Diag(G_R)^T
  POETX_TRY(block_apply(pr, p.din, L->w_merged, L->g_r, m1, true, nullptr, s));
  POETX_TRY(transpose(m1, t1, p.dout, p.din, (int)es, s));
  Plan pp = p;
  pp.N = p.din;  // M^T = M1^T . Diag(G_P)
  POETX_TRY(block_apply(pp, p.dout, t1, L->g_p, t2, false, nullptr, s));
  const bool perms = L->perm_out || L->perm_in;
  void *m = perms ? m1 : w_out;
  POETX_TRY(transpose(t2, m, p.din, p.dout, (int)es, s));
  if (!perms) return POETX_OK;
  if (inv_out) POETX_TRY(invert_perm(L->perm_out, inv_out, p.dout, s));
  if (inv_in) POETX_TRY(invert_perm(L->perm_in, inv_in, p.din, s));
  return permute_cols(m, w_out, p.dout, p.din, (int)es, inv_out, inv_in, false, s);
}

// ================================================================ optimizer ====
extern "C" int poetx_adam_step(int64_t n_params, void *theta, int32_t theta_dtype, const float *grad, float *m,
                               float *v, float lr, float beta1, float beta2, float eps, int64_t step, float gamma,
                               void *stream) {
  if (n_params < 0 || !adam_args_ok(beta1, beta2, eps, step)) return POETX_ERR_INVALID_ARG;
  if (theta_dtype != POETX_F32 && theta_dtype != POETX_BF16) return POETX_ERR_INVALID_ARG;
  if (n_params == 0) return POETX_OK;
  if (!theta || !grad || !m || !v) return POETX_ERR_INVALID_ARG;
  if (((uintptr_t)theta | (uintptr_t)grad | (uintptr_t)m | (uintptr_t)v) % 16) return POETX_ERR_INVALID_ARG;
  return adam_step(n_params, theta, theta_dtype, grad, m, v, adam_hyper(lr, beta1, beta2, eps, step, gamma),
                   (hipStream_t)stream);
}
