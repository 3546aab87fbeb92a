/*
 * poetx.h -- C ABI of libpoetx, the POET-X linear layer on AMD MI355X (gfx950).
 *
 * The layer (POET-X summary page, Method §1, eq. 3, input-centric form) is
 *
 *     z = G_P^T ( W' ( G_R^T x ) )
 *
 * where W' is the frozen weight with the two weight-side permutations merged
 * in (Method §2), and G_R, G_P are block-diagonal with b x b blocks built by
 * the Cayley-Neumann parameterization (Method §4, eq. 9)
 *
 *     G = I + 2 (Q + Q^2 + Q^2.Q) + Q^2.Q^2,   Q skew,
 *
 * each Q stored as its packed strict upper triangle (b(b-1)/2 floats).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Layouts are row-major and contiguous.  Activations are token-major:
 *    x[N][d_in], z[N][d_out].  The weight is w[d_out][d_in] (torch nn.Linear).
 *    Block j of G_R covers input features [j*b, (j+1)*b) of the permuted
 *    input; G_R is stored g_r[n_R][b][b] with g_r[j][r][c] the (r, c) entry
 *    of block j (n_R = d_in / b, n_P = d_out / b).
 *  - Packed theta: theta[j][k] = Q_j[r][c] for r < c, k running row-major over
 *    the strict upper triangle; Q_j[c][r] = -theta[j][k].
 *  - Token-major form of the layer, with Gather(x)[i] = x[perm_in[i]] and
 *    Scatter(y)[perm_out[i]] = y[i]:
 *        A = Gather(X) . Diag(G_R)        (a = G_R^T x, Method §5)
 *        B = A . W'^T                     (b = W' a)
 *        Z = Scatter(B . Diag(G_P))       (z = G_P^T b)
 *    perm_in / perm_out may be NULL (identity): then the call is exactly the
 *    three-product chain above with no activation permutation.
 *  - All pointers are DEVICE pointers unless marked [host].  Device pointers
 *    must be 16-byte aligned.  The caller owns every buffer; the library never
 *    allocates or frees device memory.  Inputs are read-only, outputs are
 *    overwritten (never accumulated into); inputs and outputs must not alias.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL = the default stream) and never synchronizes.
 *  - Workspace: calls taking (ws, ws_bytes) report the bytes they need when
 *    called with ws == NULL (writing *ws_bytes, launching nothing).  With
 *    ws != NULL, *ws_bytes below the requirement is POETX_ERR_WORKSPACE.  The
 *    requirement can depend on the current device (its compute-unit count sets
 *    how the W' products split their last round of tiles): query on the device
 *    the call will run on.
 *  - Errors: arguments are validated on the host before any launch; on a
 *    validation error nothing is launched and outputs are untouched.  A failed
 *    launch returns POETX_ERR_HIP; faults during execution surface at the
 *    caller's next synchronization.  poetx_status_string() names a code.
 *  - Block sizes: 2 <= b <= 1024.  A side of width d has ceil(d/b) diagonal
 *    blocks (Method §3): d/b full b x b blocks, then, when b does not divide d, one
 *    last block of size d % b.  A side's theta holds the blocks' packed vectors one
 *    after another ([d/b][b(b-1)/2], then (d%b)(d%b-1)/2 values) and its G the
 *    blocks one after another ([d/b][b][b], then [d%b][d%b]).  A block of size 1 has
 *    no parameters and G = [1].  Kernel paths: the W' products of a bf16 layer run
 *    on MFMA when d_in and d_out are multiples of 128, or (bf16 weights) of 8; the
 *    block products on MFMA for b = 64 or a multiple of 128 (a last block of such a
 *    size too); every other shape, and every float32 layer, runs on the float32
 *    vector-ALU product.
 */
#ifndef POETX_H
#define POETX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  POETX_OK = 0,
  POETX_ERR_INVALID_ARG = -1, /* NULL where a buffer is required, bad enum, n < 0 */
  POETX_ERR_SHAPE = -2,       /* block size b out of range                       */
  POETX_ERR_UNSUPPORTED = -3, /* a combination the library does not implement    */
  POETX_ERR_WORKSPACE = -4,   /* *ws_bytes smaller than required                 */
  POETX_ERR_HIP = -5          /* a HIP runtime call or kernel launch failed      */
} poetx_status;

typedef enum { POETX_F32 = 0, POETX_BF16 = 1, POETX_I8 = 2 } poetx_dtype;
typedef enum { POETX_FAST = 0, POETX_MEM = 1 } poetx_variant;
typedef enum { POETX_CNP_FWD = 0, POETX_CNP_BWD = 1 } poetx_cnp_dir;

/* [host] description of one layer.  Pointers inside are device pointers. */
typedef struct {
  int64_t d_in, d_out, b;      /* widths and block size                              */
  int32_t act_dtype;           /* poetx_dtype of x, z, dz, dx, saved_b: F32 or BF16  */
  int32_t w_dtype;             /* F32, BF16 (same as act) or I8 (BF16 act, MEM only) */
  int32_t g_dtype;             /* dtype of g_r / g_p: F32 or BF16 (== act_dtype)     */
  int32_t variant;             /* poetx_variant                                     */
  const void *w_merged;        /* [d_out][d_in] W' from poetx_merge_perm            */
  const void *w_merged_t;      /* optional [d_in][d_out] copy of W'^T (BF16 only: set
                                  with an I8 W' it is POETX_ERR_INVALID_ARG), or NULL;
                                  when given, the backward's dA = dB.W' reads it
                                  k-contiguous (faster, one more weight copy)          */
  const float *w_scale;        /* [d_out] per-row scale of an I8 W', else NULL      */
  const int32_t *perm_in;      /* [d_in]  or NULL (identity)                        */
  const int32_t *perm_out;     /* [d_out] or NULL (identity)                        */
  const void *theta_r;         /* [n_R][b(b-1)/2] packed Q of G_R (n_R = d_in/b; with
                                  a last block of size d_in % b, its packed vector
                                  follows), in theta_dtype                           */
  const void *theta_p;         /* [n_P][b(b-1)/2] packed Q of G_P, likewise         */
  const void *g_r;             /* [n_R][b][b] (then the last block) from poetx_cnp  */
  const void *g_p;             /* [n_P][b][b] (then the last block) from poetx_cnp  */
  int32_t theta_dtype;         /* F32 (0, the default) or BF16: storage of theta; the
                                  CNP widens it exactly and computes in float32, and
                                  dtheta stays float32                               */
  const void *q_r;             /* optional: the qsave buffer that poetx_cnp(FWD) filled
                                  for the n_R full blocks of G_R from this theta_r, or
                                  NULL; the backward's CNP then reads Q from it instead
                                  of unpacking theta_r again (b in {64, 128, 256,
                                  512}; ignored otherwise; results are the same).  16-byte
                                  aligned, n_R * b * b * 4 bytes.                   */
  const void *q_p;             /* the same for the n_P full blocks of G_P           */
} poetx_layer;

/* Size of the static device workspace of poetx_cnp_noalloc, per GPU (64 MiB). */
#define POETX_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * poetx_merge_perm -- Method §2 (permutation merge, once per inner phase):
 *     w_merged[i][k] = w[perm_out[i]][perm_in[k]]
 * and for an I8 weight with per-output-row scales also
 *     w_scale_merged[i] = w_scale[perm_out[i]]   (exact: a row scale moves with its row).
 * When w_merged_t is not NULL it also receives the transpose w_merged_t[k][i] =
 * w_merged[i][k] ([d_in][d_out], same dtype; must not alias w or w_merged).
 * w: [d_out][d_in] of w_dtype (F32, BF16 or I8); w_scale: [d_out] (I8 only, else NULL);
 * perm_out: [d_out], perm_in: [d_in] (each may be NULL = identity; entries must form a
 * permutation -- not checked on the device).  Output w_merged has w's dtype and shape.
 * Bit-exact data movement.  Errors: NULL w/w_merged, I8 without both scale pointers,
 * d_out or d_in < 1 -> POETX_ERR_INVALID_ARG.
 */
int poetx_merge_perm(const void *w, const float *w_scale, int32_t w_dtype, int64_t d_out,
                     int64_t d_in, const int32_t *perm_out, const int32_t *perm_in,
                     void *w_merged, float *w_scale_merged, void *w_merged_t, void *stream);

/*
 * poetx_cnp -- Method §4 (Cayley-Neumann parameterization, eq. 9) on nblocks
 * independent b x b blocks.
 *   theta: packed [n][b(b-1)/2] in theta_dtype (F32, or BF16 storage widened exactly).
 *   dir == POETX_CNP_FWD: g[n][b][b] = I + 2(Q + Q^2 + Q^2.Q) + Q^2.Q^2 from packed
 *     theta; g in g_dtype (F32 or BF16, rounded to nearest even).
 *     dg, dtheta unused (may be NULL).
 *   dir == POETX_CNP_BWD: dtheta[n][b(b-1)/2] = dL/dtheta given dg = dL/dG
 *     ([n][b][b], dg_dtype F32), the exact adjoint of eq. 9 (the page leaves
 *     its eq. 10 unprinted); g unused.
 * Products are evaluated to float32 accuracy (split-bf16 MFMA passes), whatever
 * g_dtype is; a b between 64 and 512 that is not a multiple of 64 runs on blocks padded
 * to 128, 256 or 512 (Q embedded as diag(Q, 0), which leaves G and dtheta exact).  Workspace: query with ws == NULL.  A layer whose b does not divide a
 * width calls this once for the side's full blocks and once for its last block (at
 * that block's size).  theta, dtheta, g and dg need only be aligned to their element
 * size (a last block sits at an offset of whole blocks); g and dg that are not
 * 16-byte aligned take the float32 vector-ALU path.  b == 1: G = [1] per block,
 * no parameters (theta and dtheta may be NULL).
 * qsave (nullable; used for b in {64, 128, 256, 512}, ignored otherwise): the saved
 * operand of the pages' fused kernel, which loads Q and Q^2 on chip.  Here it holds Q
 * itself, as the split-bf16 planes
 * in MFMA fragment order that the CNP kernels read (an internal layout, n * b * b * 4
 * bytes, 16-byte aligned): the forward's chain and the backward's five products are all
 * products by Q (or by the symmetric and skew parts of dG), so no power of Q is kept.  FWD
 * writes it; BWD with qsave reads Q from it instead of unpacking theta again, and theta
 * must then be the theta of the FWD call that wrote it.  Results are the same with or
 * without it.
 * Errors: b < 1 or b > 1024 -> POETX_ERR_SHAPE; NULL theta (b > 1) / output, theta_dtype
 * other than F32 or BF16, qsave not 16-byte aligned -> INVALID_ARG.
 */
int poetx_cnp(int32_t dir, int64_t nblocks, int64_t b, const void *theta, int32_t theta_dtype,
              void *g, int32_t g_dtype, void *qsave, const void *dg, int32_t dg_dtype, float *dtheta,
              void *ws, size_t *ws_bytes, void *stream);

/*
 * poetx_cnp_noalloc -- for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): poetx_cnp, same arguments
 * (no qsave: Q is unpacked from theta in both directions) and results, with its workspace in a static device array of POETX_NOALLOC_SCRATCH_BYTES
 * per GPU, set up on the first call on each device and held until the process ends.  It
 * calls no hipMalloc / hipFree.  Every call on a GPU uses that GPU's one array: calls
 * that overlap on one GPU (two streams, or two threads) race and must not be made; calls
 * in one stream's order are fine.  The CNP writes every workspace byte it reads, so the
 * contents a previous call left behind do not matter.
 * Errors: as poetx_cnp; a call whose workspace (the poetx_cnp query) exceeds
 * POETX_NOALLOC_SCRATCH_BYTES -> POETX_ERR_WORKSPACE, before any launch (for b = 256 that
 * is more than 64 forward or 42 backward blocks).
 */
int poetx_cnp_noalloc(int32_t dir, int64_t nblocks, int64_t b, const void *theta, int32_t theta_dtype,
                      void *g, int32_t g_dtype, const void *dg, int32_t dg_dtype, float *dtheta,
                      void *stream);

/*
 * poetx_forward -- Method §1 eq. 3 with §2 and §3 (batched block-diagonal
 * products), token-major:  z[N][d_out] from x[N][d_in] (see the chain above).
 * L->g_r, L->g_p must hold poetx_cnp(FWD) of L->theta_r, L->theta_p.
 * saved_b: FAST variant -> output B = A.W'^T [N][d_out] in act dtype, kept for
 * the backward (Method §5, POET-X_fast); MEM variant -> must be NULL (B is
 * recomputed in the backward, POET-X_mem).
 * saved_x: FAST variant, optional -> output X~ = Gather_in(x) [N][d_in] in act dtype,
 * kept so that the backward need not gather x again (one more activation copy for one
 * less pass over x; the pages keep only B).  NULL -> not kept.  Not written when
 * perm_in is NULL (then X~ = x).  MEM variant -> must be NULL.  n_tokens == 0 is a
 * no-op.
 * Errors: I8 weight with FAST -> POETX_ERR_UNSUPPORTED (Method §6: POET-XQ
 * builds on the recomputing variant); shape errors -> POETX_ERR_SHAPE.
 */
int poetx_forward(const poetx_layer *L /*[host]*/, int64_t n_tokens, const void *x, void *z,
                  void *saved_b, void *saved_x, void *ws, size_t *ws_bytes, void *stream);

/*
 * poetx_backward -- chain rule through poetx_forward (Method §1: W gets no
 * gradient; only the block-diagonal G_R, G_P do), then the CNP backward:
 *     dZ~ = Gather_out(dz);  dB = dZ~ . Diag(G_P)^T;  dG_P[j] = sum_t B_j^T dZ~_j
 *     dA  = dB . W';          dX~ = dA . Diag(G_R)^T;  dG_R[j] = sum_t X~_j^T dA_j
 *     dx  = Scatter_in(dX~);  dtheta_* = CNP backward of dG_*.
 * saved_b: FAST -> the B written by poetx_forward; MEM -> NULL (recomputed).
 * saved_x: FAST -> the X~ written by poetx_forward into its saved_x, or NULL (X~ is then
 * gathered from x again); MEM -> NULL.  Pass the same saved_x to the workspace query.
 * dx [N][d_in] act dtype; dtheta_r, dtheta_p float32 in theta's layout (overwritten,
 * sums over all N tokens).  dg_r, dg_p float32 in G's layout ([n][b][b], then the last
 * block) are optional outputs of the block gradients (NULL = not written).  Reductions over tokens run
 * in a fixed order: results are bitwise reproducible run to run.
 */
int poetx_backward(const poetx_layer *L /*[host]*/, int64_t n_tokens, const void *x,
                   const void *dz, const void *saved_b, const void *saved_x, void *dx,
                   float *dtheta_r, float *dtheta_p, float *dg_r, float *dg_p, void *ws,
                   size_t *ws_bytes, void *stream);

/*
 * poetx_backward_adam -- poetx_backward with one Adam step of both sides' packed theta
 * fused into the CNP backward's last pass (the pass that forms dtheta from dL/dQ), so the
 * gradient goes straight into the update instead of through a separate optimizer pass
 * over dtheta.  The optimizer state lives on the b(b-1)/2 packed parameters per block
 * (Method §4); gamma scales the learning rate (practical advice 3: 0.5 for POET-XQ).  The
 * update is poetx_adam_step's, element by element (float32 arithmetic; a BF16 theta is
 * rounded to nearest even after it).
 * opt [host]: hyperparameters and the device buffers, in theta's layout: m_r, v_r, m_p,
 * v_p float32 state, updated in place (zero before step 1); theta_r_out, theta_p_out
 * receive the updated theta in L->theta_dtype and may be L->theta_r / L->theta_p
 * themselves (an in-place update: every element is read and written by one thread).
 * dtheta_r, dtheta_p: also written when not NULL.  Other arguments and the workspace as
 * poetx_backward (the block gradients dg_* are not offered).
 * Errors: as poetx_backward; NULL opt or state/theta buffers, step < 1, beta outside
 * [0, 1), eps <= 0 -> POETX_ERR_INVALID_ARG.
 */
typedef struct {
  float lr, beta1, beta2, eps, gamma;
  int64_t step;                  /* t >= 1 (bias corrections 1 - beta^t)             */
  float *m_r, *v_r, *m_p, *v_p;  /* Adam state of theta_r, theta_p                    */
  void *theta_r_out, *theta_p_out;
} poetx_adam;

int poetx_backward_adam(const poetx_layer *L /*[host]*/, int64_t n_tokens, const void *x,
                        const void *dz, const void *saved_b, const void *saved_x, void *dx,
                        float *dtheta_r, float *dtheta_p, const poetx_adam *opt /*[host]*/,
                        void *ws, size_t *ws_bytes, void *stream);

/*
 * poetx_fold -- the consolidation step of merge-then-reinitialize (the POET training
 * recipe's periodic merge, on the "Poet Orthogonal LLM Training" skill page under its
 * memory optimization; with POET-X's merged permutations, Method §2): the layer's
 * effective weight in original coordinates,
 *     w_out[perm_out[i]][perm_in[k]] = (Diag(G_P)^T . W' . Diag(G_R)^T)[i][k],
 * so that x . w_out^T equals poetx_forward's z for every token row x.  A caller starts
 * the next phase by zeroing theta (then G = I), drawing new permutations and calling
 * poetx_merge_perm(w_out, ...).
 * w_out: [d_out][d_in] of L->w_dtype (F32 or BF16; must not alias L->w_merged).
 * Uses L->w_merged, g_r, g_p, perm_in, perm_out (theta and variant unused).  With BF16
 * the two block products round their outputs to bf16 (fp32 accumulation).  Workspace:
 * query with ws == NULL.  Errors: I8 weight -> POETX_ERR_UNSUPPORTED (a folded weight
 * would need a requantizer the pages do not give); shapes as poetx_forward.
 */
int poetx_fold(const poetx_layer *L /*[host]*/, void *w_out, void *ws, size_t *ws_bytes, void *stream);

/*
 * poetx_adam_step -- one Adam update of packed theta, fused in a single pass.  The
 * optimizer state lives on the b(b-1)/2 packed parameters per block, half of a dense
 * b x b (Method §4); gamma scales the learning rate (the pages set it below 1, to 0.5,
 * for POET-XQ: practical advice 3).  With g = dtheta from poetx_backward:
 *     m = beta1 m + (1 - beta1) g,   v = beta2 v + (1 - beta2) g^2,
 *     theta -= gamma lr (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 * theta: [n_params] in theta_dtype (F32, or BF16: widened, updated in float32, rounded to
 * nearest even), updated in place; m, v: [n_params] float32, updated in place (m, v start
 * at zero); grad: [n_params] float32, read-only; all 16-byte aligned.  t = step >= 1.  The
 * pages do not fix the other hyperparameters: the caller passes them.
 * Errors: step < 1, beta outside [0, 1), eps <= 0, theta_dtype other than F32 or BF16,
 * NULL or misaligned pointers -> POETX_ERR_INVALID_ARG.
 */
int poetx_adam_step(int64_t n_params, void *theta, int32_t theta_dtype, const float *grad, float *m,
                    float *v, float lr, float beta1, float beta2, float eps, int64_t step, float gamma,
                    void *stream);

/* Human-readable name of a poetx_status code (static string). */
const char *poetx_status_string(int status);

/* Library version, e.g. "0.1.0" (static string). */
const char *poetx_version(void);

/*
 * Measurement hooks (not part of the layer's math).  poetx_prof_enable(1) turns on the
 * CALLING THREAD's recorder: every later kernel launch that this thread makes through
 * the library carries a start and a stop event bound to the dispatch itself
 * (hipExtLaunchKernel), so a recorded duration is that kernel's own execution time and
 * no marker packet is placed between kernels (the events carry no system-scope fence, so
 * recording leaves the caches alone).  poetx_prof_read() synchronizes this
 * thread's recorded events and writes one line per kernel label,
 * "label launches total_ms min_ms max_ms\n", into buf (truncated to len bytes,
 * NUL-terminated), then clears this thread's record.  poetx_prof_enable(0) stops
 * recording.  poetx_prof_only(label) limits this thread's recording to the launches with
 * that label (NULL or "" = every launch): each recorded dispatch still waits on its
 * events' bookkeeping (a few us of idle GPU before it), so a timing of one kernel inside
 * a longer sequence records that kernel alone.  The recorder is thread-local: calls from
 * different threads neither see nor disturb each other's records.  Returns POETX_OK or
 * POETX_ERR_HIP.
 */
int poetx_prof_enable(int32_t on);
int poetx_prof_only(const char *label);
int poetx_prof_read(char *buf, size_t len);

#ifdef __cplusplus
}
#endif
#endif /* POETX_H */
