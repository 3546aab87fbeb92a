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
// int8 weights (BI8) travel to LDS as int8 (half the bytes of a bf16 tile) and are
// widened to bf16 in registers, exactly, right before the MFMAs; their per-row scale is
// applied in the epilogue.
#include <atomic>

#include "lds_tiles.h"

// fragment read distance (substeps) of the four-wave W' kernel: 1, 2 and 3 measured alike
// (237-238 us per W' product at workload 3), so LDS latency is not what holds it back
#ifndef POETX_G4_RD
#define POETX_G4_RD 1
#endif

// bf16 256 x 256 tiles leave through LDS (off: straight from the accumulators)
#ifndef POETX_EPI_LDS
#define POETX_EPI_LDS 1
#endif

#ifndef POETX_NT_LATE
#define POETX_NT_LATE 0
#endif
// The k-contiguous products' fragment reads interleaved with their MFMAs (below; off: all
// reads before the first MFMA).  W' product at workload 3: 206.5 -> 201.4 us.
#ifndef POETX_NT_ILV
#define POETX_NT_ILV 1
#endif

// Two-stage NT loop that frees a stage with a second barrier once it has been read and
// issues the loads two k steps ahead there (off: 236 against 218 us per W' product at
// workload 3 on one box).
#ifndef POETX_NT_EARLY
#define POETX_NT_EARLY 0
#endif

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
  // Tiles at or past full_tiles (in the order of the m-group map) are each shared by
  // tail_splits blocks, block p taking k in [p*tail_kc, (p+1)*tail_kc); their fp32
  // partials go to part[tail tile][p][BM*BN] and are summed by k_tail_reduce.
  // full_tiles = tiles_m * tiles_n when no tile is split.
  int full_tiles, tail_splits;
  int64_t tail_kc;
  float *part;
};

namespace {

// The tile a block computes and its k range.  Whole tiles keep the XCD-aware order
// (consecutive ids land on one XCD); split tiles follow them, their parts adjacent.
struct TileSel {
  int L, tail, part;
  int64_t kbeg, kend;
};
__device__ inline TileSel select_tile(const G2Args &a, int64_t kz, int L) {
  TileSel t;
  if (L >= a.full_tiles) {
    const int u = L - a.full_tiles;
    t.tail = u / a.tail_splits;
    t.part = u % a.tail_splits;
    t.L = a.full_tiles + t.tail;
    t.kbeg = (int64_t)t.part * a.tail_kc;
    t.kend = t.kbeg + a.tail_kc < a.K ? t.kbeg + a.tail_kc : a.K;
  } else {
    if (a.full_tiles % 8 == 0) L = (L % 8) * (a.full_tiles / 8) + L / 8;
    t.L = L;
    t.tail = -1;
    t.part = 0;
    t.kbeg = kz * a.Kc;
    t.kend = t.kbeg + a.Kc < a.K ? t.kbeg + a.Kc : a.K;
  }
  return t;
}

// (tile, batch/split entry) of this workgroup.  Workgroups go to the XCDs round-robin in
// linear order (x fastest).  A batched launch with fewer than 8 whole tiles per entry (the
// b = 512 block gradients: 2 x 2 tiles of 256 per block and token part) would put the tiles
// of one entry, which share their operand panels, on different XCDs; they are instead
// placed on one XCD, so a panel's second read is an L2 hit.
__device__ inline void batch_coords(const G2Args &a, int &bx, int64_t &bz) {
  bx = blockIdx.x;
  bz = blockIdx.z;
  const int ft = (int)gridDim.x;
  if (a.full_tiles == ft && ft < 8 && gridDim.y == 1 && gridDim.z % 8 == 0) {
    const int lin = (int)blockIdx.x + ft * (int)blockIdx.z, slot = lin >> 3;
    bz = __builtin_amdgcn_readfirstlane((lin & 7) + 8 * (slot / ft));
    bx = __builtin_amdgcn_readfirstlane(slot % ft);
  }
}

// (m, n) tile of tile-order index L: groups of 4 m-tiles sweep over n, so the
// blocks running together share their A and B panels.
__device__ inline void tile_coords(const G2Args &a, int L, int &tm, int &tn) {
  const int GM = a.tiles_m < 4 ? a.tiles_m : 4;
  const int grp_size = GM * a.tiles_n;
  const int grp = L / grp_size, first_m = grp * GM;
  const int gm = (a.tiles_m - first_m) < GM ? (a.tiles_m - first_m) : GM;
  const int local = L % grp_size;
  tm = first_m + local % gm;
  tn = local / gm;
}

// A part of a split tile stores its fp32 accumulators thread-major (whole lines per
// wave store); k_tail_reduce sums the parts after the product kernel has ended.
template <int FM, int FN, int NTH>
__device__ inline void tail_store(const f32x4 (&acc)[FM][FN], const G2Args &a, int tail, int part) {
  f32x4 *dst = (f32x4 *)a.part + ((int64_t)tail * a.tail_splits + part) * (FM * FN * NTH);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) dst[(i * FN + j) * NTH + threadIdx.x] = acc[i][j];
}

}  // namespace


// ROLE separates instantiations per use.  WGM x WGN waves, each computing a
// (BM/WGM) x (BN/WGN) patch; k advances BKT per step through NST LDS stages with
// NST-1 steps of prefetch in flight.
//
// With an int8 k-contiguous B (BI8) the 64 k of a step are dealt out in a different
// order, identically on both operands: lane group g (lanes 16g .. 16g+15) of the h-th
// MFMA covers k = 16g + 8h + 0..7, so one 16-byte LDS read of a B row (k = 16g .. +15)
// feeds both MFMAs of the step, and the A reads take bf16 chunk 2g + h.
//
// TAIL (bf16 operands, batch 1): M, N and K need only be multiples of 8.  Rows past M and
// columns past N are not stored; a k-contiguous operand's last k step has its chunks past K,
// which the loads fill from the next rows, zeroed in LDS before they are read, while a
// k-major operand's rows past K read as zero through the buffer range.  Operand rows or
// columns past M or N only reach outputs that are not stored.
template <int ROLE, int BM, int BN, int WGM, int WGN, int BKT, int NST, bool AKM, bool BKM, bool OUTF32,
          bool BI8 = false, bool TAIL = false>
__global__ __launch_bounds__(64 * WGM * WGN) void k_gemm2(G2Args a) {
  static_assert(!BI8 || (!AKM && !BKM && BKT == 64), "int8 B: k-contiguous operands, 64-deep steps");
  static_assert(!TAIL || !BI8, "tails: bf16 operands");
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN, FM = WTM / 16, FN = WTN / 16;
  constexpr int EB = BI8 ? 1 : 2;  // bytes per B element
  constexpr int A_ELEMS = BM * BKT, B_ELEMS = BN * BKT * EB / 2;  // in bf16 slots
  constexpr int PF = NST - 1;
  extern __shared__ __align__(16) bf16_t smem[];
  // stage s: A tile at smem + s*A_ELEMS, B tile at smem + NST*A_ELEMS + s*B_ELEMS

  // ---- tile mapping: batch/split in z; (m, n) from an XCD-aware order of blockIdx.x
  int bx;
  int64_t z;
  batch_coords(a, bx, z);
  // batch entry and k split as wave-uniform 32-bit values (a 64-bit division is expanded
  // into vector code, and operand bases derived from it would count as divergent)
  const int64_t bidx = __builtin_amdgcn_readfirstlane((int)z / a.splits),
                kz = __builtin_amdgcn_readfirstlane((int)z % a.splits);
  const TileSel sel = select_tile(a, kz, bx);
  int tm, tn;
  tile_coords(a, sel.L, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int64_t kbeg = sel.kbeg, kend = sel.kend;
  const bf16_t *A = a.A + bidx * a.sAb;
  const bf16_t *B = (const bf16_t *)((const char *)a.B + bidx * a.sBb * EB);
  // valid extents: k-contiguous operands end at their last row, k-major at kend
  const __amdgpu_buffer_rsrc_t ra = AKM ? make_rsrc(A, kend * a.lda * 2) : make_rsrc(A, a.M * a.lda * 2);
  const __amdgpu_buffer_rsrc_t rb = BKM ? make_rsrc(B, kend * a.ldb * EB) : make_rsrc(B, a.N * a.ldb * EB);

  const int wave = threadIdx.x >> 6;
  const int wm = (wave / WGN) * WTM, wn = (wave % WGN) * WTN;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // an int8 row of BKT bytes loads as a bf16 row of BKT/2 (k and ld halve with it)
  constexpr int BKB = BI8 ? BKT / 2 : BKT;
  const int64_t ldb_s = BI8 ? a.ldb / 2 : a.ldb;
  using LA = typename std::conditional<AKM, LoaderKM<BM, NW, BKT>, LoaderKC<BM, NW, BKT>>::type;
  using LB = typename std::conditional<BKM, LoaderKM<BN, NW, BKT>, LoaderKC<BN, NW, BKB>>::type;
  constexpr int LPS = LA::INSTR + LB::INSTR;  // loads per wave per stage
  LA la;
  LB lb;
  la.init(a.lda, m0);
  lb.init(ldb_s, n0);
  auto issue = [&](int buf, int64_t k0) {
    la.issue(ra, k0, a.lda, smem + buf * A_ELEMS);
    lb.issue(rb, BI8 ? k0 / 2 : k0, ldb_s, smem + NST * A_ELEMS + buf * B_ELEMS);
  };

  const int nk = (int)((kend - kbeg + BKT - 1) / BKT);
  // EARLY (two stages): a step reads all its fragments first, so its stage is free once every
  // wave has read it: a second barrier there lets the loads two steps ahead go out a step
  // sooner than the load of the next stage at the top of the step would
  constexpr bool EARLY = POETX_NT_EARLY && !BI8 && NST == 2 && ROLE == MFMA_GEMM_NT;
  // LATE: the next stage's loads go out after this step's fragment reads instead of right
  // after the barrier, so the reads do not queue behind them.  On for the block gradients
  // (b = 512 at workload 4: 118 -> 106 us); measured flat for the W' products and 2.5 us
  // slower for the batched block products, so off there.
  constexpr bool LATE = !EARLY && !BI8 && (POETX_NT_LATE || ROLE == MFMA_BLOCK_GRAD);
  if constexpr (EARLY) {
    if (nk > 0) issue(0, kbeg);
    if (nk > 1) issue(1, kbeg + BKT);
  } else {
#pragma unroll
    for (int s = 0; s < PF; ++s)
      if (s < nk) issue(s, kbeg + (int64_t)s * BKT);
  }
  for (int t = 0; t < nk; ++t) {
    if constexpr (EARLY) {
      // stage t landed; stage t+1 (issued a step ago) may still be in flight
      if (t + 1 < nk) wait_vmcnt<LPS>();
      else __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    } else {
      // stage t has landed for this wave once at most (PF-1) newer stages are outstanding
      if (t + PF <= nk) wait_vmcnt<(PF - 1) * LPS>();
      else __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // everyone's stage t is in LDS; stage t-1 is no longer read
      if (!LATE && t + PF < nk) issue((t + PF) % NST, kbeg + (int64_t)(t + PF) * BKT);
      if constexpr (TAIL && (!AKM || !BKM)) {
        const int kr = (int)(kend - kbeg - (int64_t)t * BKT);  // valid k of this step
        if (kr < BKT) {
          // the k-contiguous tiles' chunks past K (k-major tiles are zero there already)
          bf16_t *za = smem + (t % NST) * A_ELEMS, *zb = smem + NST * A_ELEMS + (t % NST) * B_ELEMS;
          constexpr int CR = BKT / 8, RA = AKM ? 0 : BM, RB = BKM ? 0 : BN;
          const int c0 = kr / 8;
          for (int q = threadIdx.x; q < (RA + RB) * CR; q += 64 * NW) {
            const int r = q / CR, c = q % CR;
            if (c < c0) continue;
            bf16_t *row = r < RA ? za + r * BKT : zb + (r - RA) * BKT;
            const int rr = r < RA ? r : r - RA;
            *(uint4 *)(row + (c ^ kc_key<BKT>(rr)) * 8) = make_uint4(0u, 0u, 0u, 0u);
          }
          __syncthreads();
        }
      }
    }
    const int cur = t % NST;
    const bf16_t *ta = smem + cur * A_ELEMS, *tb = smem + NST * A_ELEMS + cur * B_ELEMS;
    if constexpr (BI8) {
      const int l = threadIdx.x & 63, g = l >> 4;
      bf16x8 fa[2][FM];
      u32x4v rq[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm + 16 * i + (l & 15);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          fa[h][i] = __builtin_bit_cast(bf16x8, *(const s16x8 *)(ta + row * BKT + ((2 * g + h) ^ kc_key<BKT>(row)) * 8));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn + 16 * j + (l & 15);
        rq[j] = *(const u32x4v *)((const char *)tb + row * BKT + ((g ^ kc_key<BKB>(row)) << 4));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const bf16x8 fb = widen_i8x8(rq[j][2 * h], rq[j][2 * h + 1]);
#pragma unroll
          for (int i = 0; i < FM; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, fa[h][i], acc[i][j], 0, 0, 0);
        }
      continue;
    }
    // Fragment reads.  ILV (k-contiguous tiles, two 32-deep halves): the B fragments and the
    // first A fragment go out first, since the first MFMAs need them, then one read per MFMA
    // until the whole step's fragments are in flight (scheduling groups below); otherwise all
    // reads go out before the first MFMA, a scheduling barrier keeping the compiler from
    // sinking them into the MFMA chain.
    constexpr int KH = BKT / 32;
    constexpr bool ILV = POETX_NT_ILV && KH == 2 && !AKM && !BKM;
    bf16x8 fa[KH][FM], fb[KH][FN];
#pragma unroll
    for (int h = 0; h < KH; ++h) {
      if constexpr (ILV) {
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[h][j] = frag_kc<BKT>(tb, wn + 16 * j, 32 * h);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[h][i] = AKM ? frag_km<BM>(ta, wm + 16 * i, 32 * h) : frag_kc<BKT>(ta, wm + 16 * i, 32 * h);
      if constexpr (!ILV) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          fb[h][j] = BKM ? frag_km<BN>(tb, wn + 16 * j, 32 * h) : frag_kc<BKT>(tb, wn + 16 * j, 32 * h);
      }
    }
    if constexpr (!ILV) __builtin_amdgcn_sched_barrier(0);
    if constexpr (EARLY) {
      __syncthreads();  // every wave's reads of stage t have returned: its buffer takes stage t+2
      if (t + 2 < nk) issue(cur, kbeg + (int64_t)(t + 2) * BKT);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (LATE) {
      if (t + PF < nk) issue((t + PF) % NST, kbeg + (int64_t)(t + PF) * BKT);
    }
#pragma unroll
    for (int h = 0; h < KH; ++h)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          // operands swapped: lane l then holds C[m = l%16][n = 4*(l/16) + 0..3]
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[h][j], fa[h][i], acc[i][j], 0, 0, 0);
    if constexpr (ILV) {
      // DS reads: FN + 1 first, then one after each MFMA; then the remaining MFMAs
      constexpr int NR = KH * (FM + FN), NM = KH * FM * FN, FIRST = FN + 1;
      __builtin_amdgcn_sched_group_barrier(0x100, FIRST, 0);
#pragma unroll
      for (int q = 0; q < NR - FIRST; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NM - (NR - FIRST), 0);
    }
  }

  if constexpr (BM == 256 && BN == 256) {  // only the W' products split tiles
    if (sel.tail >= 0) {
      tail_store<FM, FN, 64 * NW>(acc, a, sel.tail, sel.part);
      return;
    }
  }
  const int l = threadIdx.x & 63;
  char *Cb = (char *)a.C + (bidx * a.sCb + kz * a.sCsplit) * (OUTF32 ? 4 : 2);
  if constexpr (!OUTF32 && BM == 256 && BN == 256 && POETX_EPI_LDS) {
    // bf16 tile through LDS: an accumulator's lanes hold 16 rows x 32 bytes, which as
    // global stores are 16 partial cache lines per instruction; staged, every store
    // instruction writes two whole 512-byte rows.  Rows are EPI_LD bytes apart (16 over a
    // row) so the 16 rows of one accumulator write fall on different banks.
    constexpr int EPI_LD = BN * 2 + 16;
    if ((((uintptr_t)Cb | (uintptr_t)(n0 * 2)) & 15) == 0 && (a.ldc & 7) == 0) {
      char *st = (char *)smem;
      __syncthreads();  // every wave is done with the last stage
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = wm + 16 * i + (l & 15);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int n = wn + 16 * j + 4 * (l >> 4);
          f32x4 v = acc[i][j];
          if (a.scaleN) {
            float4 sc = *(const float4 *)(a.scaleN + bidx * a.sSNb + n0 + n);
            v[0] *= sc.x; v[1] *= sc.y; v[2] *= sc.z; v[3] *= sc.w;
          }
          uint2 p;
          p.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
          p.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
          *(uint2 *)(st + m * EPI_LD + n * 2) = p;
        }
      }
      __syncthreads();
      constexpr int NTH = 64 * NW, RPP = NTH / 32;  // rows per pass: 32 lanes x 16 bytes a row
      const int ch = threadIdx.x & 31;
#pragma unroll
      for (int r = threadIdx.x >> 5; r < BM; r += RPP) {
        const int64_t m = m0 + r;
        if (m < a.M && (!TAIL || n0 + ch * 8 < a.N))
          *(uint4 *)(Cb + (m * a.ldc + n0 + ch * 8) * 2) = *(const uint4 *)(st + r * EPI_LD + ch * 16);
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wm + 16 * i + (l & 15);
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn + 16 * j + 4 * (l >> 4);
      if (TAIL && n >= a.N) continue;
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
// An int8 B (BI8, k-major only) stays int8 in LDS, 256-byte rows, and is read with the
// 8-bit transposing LDS read, one per fragment.
template <int ROLE, bool AKM, bool BKM, bool OUTF32, bool BI8 = false>
__global__ __launch_bounds__(512) void k_gemm_pp(G2Args a) {
  static_assert(!BI8 || (!AKM && BKM), "int8 B: k-major B, k-contiguous A");
  constexpr int BM = 256, BN = 256, BKT = 64, WGN = 4, NW = 8;
  constexpr int WTM = 128, WTN = 64, FM = WTM / 16, FN = WTN / 16;
  constexpr int EB = BI8 ? 1 : 2;
  constexpr int A_ELEMS = BM * BKT, B_ELEMS = BN * BKT * EB / 2;
  extern __shared__ __align__(16) bf16_t smem[];

  const int64_t z = blockIdx.z, bidx = z / a.splits, kz = z % a.splits;
  const TileSel sel = select_tile(a, kz, (int)blockIdx.x);
  int tm, tn;
  tile_coords(a, sel.L, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int64_t kbeg = sel.kbeg, kend = sel.kend;
  const bf16_t *A = a.A + bidx * a.sAb;
  const bf16_t *B = (const bf16_t *)((const char *)a.B + bidx * a.sBb * EB);
  const __amdgpu_buffer_rsrc_t ra = AKM ? make_rsrc(A, kend * a.lda * 2) : make_rsrc(A, a.M * a.lda * 2);
  const __amdgpu_buffer_rsrc_t rb = BKM ? make_rsrc(B, kend * a.ldb * EB) : make_rsrc(B, a.N * a.ldb * EB);

  const int wave = threadIdx.x >> 6, group = wave >> 2;
  const int wm = (wave / WGN) * WTM, wn = (wave % WGN) * WTN;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // an int8 row of 256 bytes loads as a bf16 row of 128 (ld and column offsets halve)
  constexpr int BNS = BI8 ? BN / 2 : BN;
  const int64_t ldb_s = BI8 ? a.ldb / 2 : a.ldb;
  using LA = typename std::conditional<AKM, LoaderKM<BM, 4, BKT>, LoaderKC<BM, 4, BKT>>::type;
  using LB = typename std::conditional<BKM, LoaderKM<BNS, 4, BKT, 0, BI8>, LoaderKC<BN, 4, BKT>>::type;
  LA la;
  LB lb;
  if (group == 0) {
    la.init(a.lda, m0);
    lb.init(ldb_s, BI8 ? n0 / 2 : n0);
  }
  auto issue = [&](int buf, int64_t k0) {
    la.issue(ra, k0, a.lda, smem + buf * A_ELEMS);
    lb.issue(rb, k0, ldb_s, smem + 2 * A_ELEMS + buf * B_ELEMS);
  };
  bf16x8 fa[FM], fb[FN];  // fragments of one 32-deep half step
  auto read_frags = [&](int buf, int h) {
    const bf16_t *ta = smem + buf * A_ELEMS, *tb = smem + 2 * A_ELEMS + buf * B_ELEMS;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[i] = AKM ? frag_km<BM>(ta, wm + 16 * i, 32 * h) : frag_kc<BKT>(ta, wm + 16 * i, 32 * h);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (BI8) fb[j] = frag_km8<BN>(tb, wn + 16 * j, 32 * h);
      else fb[j] = BKM ? frag_km<BN>(tb, wn + 16 * j, 32 * h) : frag_kc<BKT>(tb, wn + 16 * j, 32 * h);
    }
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

  if (sel.tail >= 0) {
    tail_store<FM, FN, 512>(acc, a, sel.tail, sel.part);
    return;
  }
  const int l = threadIdx.x & 63;
  char *Cb = (char *)a.C + (bidx * a.sCb + kz * a.sCsplit) * (OUTF32 ? 4 : 2);
  if constexpr (!OUTF32 && BM == 256 && BN == 256 && POETX_EPI_LDS) {
    // bf16 tile through LDS: an accumulator's lanes hold 16 rows x 32 bytes, which as
    // global stores are 16 partial cache lines per instruction; staged, every store
    // instruction writes two whole 512-byte rows.  Rows are EPI_LD bytes apart (16 over a
    // row) so the 16 rows of one accumulator write fall on different banks.
    constexpr int EPI_LD = BN * 2 + 16;
    if ((((uintptr_t)Cb | (uintptr_t)(n0 * 2)) & 15) == 0 && (a.ldc & 7) == 0) {
      char *st = (char *)smem;
      __syncthreads();  // every wave is done with the last stage
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = wm + 16 * i + (l & 15);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int n = wn + 16 * j + 4 * (l >> 4);
          f32x4 v = acc[i][j];
          if (a.scaleN) {
            float4 sc = *(const float4 *)(a.scaleN + bidx * a.sSNb + n0 + n);
            v[0] *= sc.x; v[1] *= sc.y; v[2] *= sc.z; v[3] *= sc.w;
          }
          uint2 p;
          p.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
          p.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
          *(uint2 *)(st + m * EPI_LD + n * 2) = p;
        }
      }
      __syncthreads();
      constexpr int NTH = 64 * NW, RPP = NTH / 32;  // rows per pass: 32 lanes x 16 bytes a row
      const int ch = threadIdx.x & 31;
#pragma unroll
      for (int r = threadIdx.x >> 5; r < BM; r += RPP) {
        const int64_t m = m0 + r;
        if (m < a.M)
          *(uint4 *)(Cb + (m * a.ldc + n0 + ch * 8) * 2) = *(const uint4 *)(st + r * EPI_LD + ch * 16);
      }
      return;
    }
  }
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


// The W' product B = A . W'^T (both operands k-contiguous, bf16) on v_mfma_f32_32x32x16_bf16,
// 256 x 256 tiles over WGM x WGN waves (2 x 2: one wave per SIMD, 128 x 128 each, the
// accumulators in AGPRs).  A 128 x 128 wave patch reads (128 + 128) x 16 x 2 bytes of LDS
// per 16 MFMAs: a third less LDS traffic per flop than eight 128 x 64 patches, which keeps
// the LDS below the MFMA rate.  With one wave per SIMD nothing else hides a wave's global
// loads, so the k range goes through NST stages of BKT (32: four or five 32 KB stages), the
// loads of a stage issued NST - 1 stages before its first read.
// The schedule is fixed by hand (a scheduling fence after every group): each 16-deep
// substep's MFMAs are dealt out one by one, and after each comes one fragment read of the
// next substep (in the order its MFMAs consume them) and, in a stage's last substep, one of
// the loads NST stages ahead.  The stage's barrier sits after the reads of its last substep
// have returned and before that substep's MFMAs: they then cover both the barrier and the
// LDS latency of the next stage's first fragments, and the stage just read is free for the
// loads.
template <int WGM, int WGN, int BKT, int NST>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void k_gemm4(G2Args a) {
  constexpr int BM = 256, BN = 256, NSUB = BKT / 16, NW = WGM * WGN;
  static_assert(NSUB % 2 == 0 && NST >= 2, "fragment buffers alternate by substep");
  constexpr int A_ELEMS = BM * BKT, B_ELEMS = BN * BKT;
  constexpr int WTM = BM / WGM, WTN = BN / WGN, FM = WTM / 32, FN = WTN / 32;  // 32 x 32 tiles per wave
  extern __shared__ __align__(16) bf16_t smem[];

  const TileSel sel = select_tile(a, 0, (int)blockIdx.x);
  int tm, tn;
  tile_coords(a, sel.L, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t kbeg = sel.kbeg, kend = sel.kend;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, a.M * a.lda * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.B, a.N * a.ldb * 2);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const int wm = (wave / WGN) * WTM, wn = (wave % WGN) * WTN;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  using LA = LoaderKC<BM, NW, BKT>;
  using LB = LoaderKC<BN, NW, BKT>;
  constexpr int LPS = LA::INSTR + LB::INSTR;
  LA la;
  LB lb;
  la.init(a.lda, m0);
  lb.init(a.ldb, n0);
  auto issue = [&](int buf, int64_t k0) {
    la.issue(ra, k0, a.lda, smem + buf * A_ELEMS);
    lb.issue(rb, k0, a.ldb, smem + NST * A_ELEMS + buf * B_ELEMS);
  };
  // fragment of a 32 x 16 operand slice: lane l holds row r0 + l % 32, k = ks + 8 (l / 32) .. +7
  auto frag = [&](const bf16_t *t, int r0, int ks) {
    const int row = r0 + (l & 31);
    const int pchunk = ((ks >> 3) + (l >> 5)) ^ kc_key<BKT>(row);
    return __builtin_bit_cast(bf16x8, *(const s16x8 *)(t + row * BKT + pchunk * 8));
  };
  // fragments are read RDI substeps ahead of their MFMAs, into NSL register slots
  constexpr int RDI = POETX_G4_RD, NSL = RDI == 1 ? 2 : NSUB;
  static_assert(RDI >= 1 && RDI < NSUB, "read distance within a stage");
  bf16x8 fa[NSL][FM], fb[NSL][FN];
  auto read = [&](int q, int buf, int s) {
    const bf16_t *ta = smem + buf * A_ELEMS, *tb = smem + NST * A_ELEMS + buf * B_ELEMS;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[q][i] = frag(ta, wm + 32 * i, 16 * s);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[q][j] = frag(tb, wn + 32 * j, 16 * s);
  };
  // the g-th fragment read of a substep, in the order the MFMAs (row tile i major) use
  // them: A0, B0 .. B(FN-1), A1 .. A(FM-1)
  auto read1 = [&](int q, int buf, int s, int g) {
    const bf16_t *ta = smem + buf * A_ELEMS, *tb = smem + NST * A_ELEMS + buf * B_ELEMS;
    if (g == 0) fa[q][0] = frag(ta, wm, 16 * s);
    else if (g <= FN) fb[q][g - 1] = frag(tb, wn + 32 * (g - 1), 16 * s);
    else fa[q][g - FN] = frag(ta, wm + 32 * (g - FN), 16 * s);
  };
  auto mma1 = [&](int q, int i, int j) {
    // operands swapped: lane l holds C[m = l % 32][n = 8 (e / 4) + 4 (l / 32) + e % 4]
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[q][j], fa[q][i], acc[i][j], 0, 0, 0);
  };
  constexpr int NM = FM * FN, NR = FM + FN, NL = LA::INSTR;  // LB::INSTR == LA::INSTR
  static_assert(NR <= NM && NL <= NM && LB::INSTR == NL, "one read and one load pair per MFMA at most");

  const int nk = (int)((kend - kbeg + BKT - 1) / BKT);
  // every buffer takes a stage up front; stage t+NST goes into stage t's buffer once it is read
#pragma unroll
  for (int t = 0; t < NST; ++t)
    if (t < nk) issue(t, kbeg + (int64_t)t * BKT);
  // stage 0 in LDS for every wave: the stages after it (at most NST - 1) may still be in flight
  wait_tiles<LPS, NST - 1>(nk - 1);
  __syncthreads();
  if (nk > 0) {
#pragma unroll
    for (int r = 0; r < RDI; ++r) read(r % NSL, 0, r);
  }
  // One stage: RD (a next stage exists: read its first fragments, after the stage barrier)
  // and LD (the stage NST ahead exists: load it) are compile-time flags, so the steady
  // state runs without a branch between its MFMAs; the last NST stages run the other forms.
  int cur = 0;  // t % NST
  auto stage = [&](int t, auto rd_c, auto ld_c) {
    constexpr bool RD = decltype(rd_c)::value, LD = decltype(ld_c)::value;
    const int nxt = cur + 1 == NST ? 0 : cur + 1;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int q = s % NSL, rs = s + RDI;  // rs: the substep whose fragments are read now
      const bool nx = rs >= NSUB;           // ... from stage t+1
      if (rs == NSUB && RD) {
        // every fragment of stage t is in registers or on its way (the barrier waits for
        // them): stage t is no longer read by this wave, and stage t+1 has landed for it once
        // the stages issued after it (up to t+NST-1, those that exist) are all in flight
        if (LD) wait_vmcnt<(NST - 2) * LPS>();
        else wait_tiles<LPS, NST - 2>(nk - 2 - t);
        __syncthreads();
      }
      const bool rd = !nx || RD, ld = rs == NSUB && LD;
      const int64_t kl = kbeg + (int64_t)(t + NST) * BKT;
#pragma unroll
      for (int g = 0; g < NM; ++g) {
        mma1(q, g / FN, g % FN);
        if (rd && g < NR) read1(rs % NSL, nx ? nxt : cur, rs % NSUB, g);
        if (ld && g < NL) {
          la.issue_one(ra, kl, smem + cur * A_ELEMS, g);
          lb.issue_one(rb, kl, smem + NST * A_ELEMS + cur * B_ELEMS, g);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    cur = nxt;
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  int t = 0;
  for (; t < nk - NST; ++t) stage(t, T_{}, T_{});
  for (; t < nk - 1; ++t) stage(t, T_{}, F_{});
  if (t < nk) stage(t, F_{}, F_{});
  char *Cb = (char *)a.C;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wm + 32 * i + (l & 31);
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + wn + 32 * j + 8 * g + 4 * (l >> 5);
        f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        if (a.scaleN) {
          float4 sc = *(const float4 *)(a.scaleN + n);
          v[0] *= sc.x; v[1] *= sc.y; v[2] *= sc.z; v[3] *= sc.w;
        }
        uint2 p;
        p.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        p.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *(uint2 *)(Cb + (m * a.ldc + n) * 2) = p;
      }
  }
}


// Sum of the parts of each split tile, in part order 0, 1, ... (so the result does not
// depend on which part finished first), times scaleN, to bf16 C.  The 256 x 256 tiles
// of both W' kernels share one fragment layout: 8 waves as 2 (m) x 4 (n), 128 x 64 per
// wave, lane l of fragment (i, j) holding C[16i + l%16][16j + 4(l/16) + 0..3].  Eight
// blocks per tile, each over an eighth of the fragments.
__global__ __launch_bounds__(256) void k_tail_reduce(G2Args a) {
  constexpr int FM = 8, FN = 4, NTH = 512, QP = FM * FN * NTH;  // f32x4 per part
  constexpr int SL = 8, PER = QP / SL / 256;
  const int tail = blockIdx.x / SL, sl = blockIdx.x % SL;
  int tm, tn;
  tile_coords(a, a.full_tiles + tail, tm, tn);
  const f32x4 *P = (const f32x4 *)a.part + (int64_t)tail * a.tail_splits * QP;
  f32x4 v[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) v[e] = P[(sl * PER + e) * 256 + threadIdx.x];
  for (int p = 1; p < a.tail_splits; ++p)
#pragma unroll
    for (int e = 0; e < PER; ++e) v[e] += P[(int64_t)p * QP + (sl * PER + e) * 256 + threadIdx.x];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int q = (sl * PER + e) * 256 + threadIdx.x;
    const int fr = q / NTH, src = q % NTH, i = fr / FN, j = fr % FN, wave = src >> 6, l = src & 63;
    const int64_t m = (int64_t)tm * 256 + (wave / 4) * 128 + 16 * i + (l & 15);
    const int64_t n = (int64_t)tn * 256 + (wave % 4) * 64 + 16 * j + 4 * (l >> 4);
    if (m >= a.M) continue;
    f32x4 w = v[e];
    if (a.scaleN) {
      const float4 sc = *(const float4 *)(a.scaleN + n);
      w[0] *= sc.x; w[1] *= sc.y; w[2] *= sc.z; w[3] *= sc.w;
    }
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(w[0]) | ((uint32_t)f32_to_bf16(w[1]) << 16);
    pk.y = (uint32_t)f32_to_bf16(w[2]) | ((uint32_t)f32_to_bf16(w[3]) << 16);
    *(uint2 *)((char *)a.C + (m * a.ldc + n) * 2) = pk;
  }
}

// The four-wave form passes the parity tests but measured slower than the eight-wave
// kernel at workload 3, per W' product on one box each: 248-254 against 215 us (two 64-deep
// stages, a branch around every guarded read and load); 260 (four 32-deep stages) and 262
// (five) against 214 us; with the branch-free steady state, 238 (two 64-deep stages), 250
// (four 32-deep) and 253 us (three) against 214 us.  It stays off.
#ifndef POETX_GEMM4
#define POETX_GEMM4 0
#endif
constexpr bool kUseGemm4 = POETX_GEMM4 != 0;
#ifndef POETX_G4_WGM
#define POETX_G4_WGM 2
#define POETX_G4_WGN 2
#endif
#ifndef POETX_G4_BK
#define POETX_G4_BK 64
#define POETX_G4_NST 2
#endif
#ifndef POETX_NT_BK
#define POETX_NT_BK 64
#define POETX_NT_NST 2
#endif
// batched NT products (the b = 512 block products: K = 512, eight 64-deep steps per tile)
#ifndef POETX_BNT_BK
#define POETX_BNT_BK 64
#define POETX_BNT_NST 2
#endif

// explicit instantiations (every configuration the dispatcher below launches)
#define POETX_G2_INST(R, BMv, BNv, WM, WN, BKv, NS, AK, BKm)                                     \
  template __global__ void k_gemm2<R, BMv, BNv, WM, WN, BKv, NS, AK, BKm, true>(G2Args);       \
  template __global__ void k_gemm2<R, BMv, BNv, WM, WN, BKv, NS, AK, BKm, false>(G2Args);
POETX_G2_INST(MFMA_GEMM_NT, 256, 256, 2, 4, POETX_NT_BK, POETX_NT_NST, false, false)
#if POETX_BNT_BK != POETX_NT_BK || POETX_BNT_NST != POETX_NT_NST
POETX_G2_INST(MFMA_GEMM_NT, 256, 256, 2, 4, POETX_BNT_BK, POETX_BNT_NST, false, false)
#endif
POETX_G2_INST(MFMA_BLOCK_APPLY, 128, 128, 2, 2, 64, 2, false, true)
POETX_G2_INST(MFMA_BLOCK_APPLY_T, 128, 128, 2, 2, 64, 2, false, false)
POETX_G2_INST(MFMA_BLOCK_GRAD, 128, 128, 2, 2, 64, 2, true, true)
POETX_G2_INST(MFMA_BLOCK_GRAD, 256, 256, 2, 4, 64, 2, true, true)
#undef POETX_G2_INST
template __global__ void k_gemm2<MFMA_GEMM_NT, 256, 256, 2, 4, 64, 2, false, false, false, true>(G2Args);
template __global__ void k_gemm2<MFMA_GEMM_NT, 256, 256, 2, 4, 64, 2, false, false, false, false, true>(G2Args);
template __global__ void k_gemm2<MFMA_BLOCK_APPLY, 128, 128, 2, 2, 64, 2, false, true, false, false, true>(G2Args);
template __global__ void k_gemm2<MFMA_BLOCK_APPLY_T, 128, 128, 2, 2, 64, 2, false, false, false, false, true>(G2Args);
template __global__ void k_gemm2<MFMA_BLOCK_GRAD, 128, 128, 2, 2, 64, 2, true, true, true, false, true>(G2Args);
template __global__ void k_gemm4<POETX_G4_WGM, POETX_G4_WGN, POETX_G4_BK, POETX_G4_NST>(G2Args);
template __global__ void k_gemm_pp<MFMA_GEMM_NN, false, true, false>(G2Args);
template __global__ void k_gemm_pp<MFMA_GEMM_NN, false, true, true>(G2Args);
template __global__ void k_gemm_pp<MFMA_GEMM_NN, false, true, false, true>(G2Args);

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

namespace {

// Leftover tiles of a W' product (256 x 256 tiles, one block per CU): when the last
// round would leave at least half the CUs idle, its tiles are split along k so that
// about one block per CU runs in that round.  Every part keeps at least 4 k steps.
struct TailPlan {
  int64_t full, r, s, kc;
};
TailPlan tail_plan(int64_t tiles, int64_t K, int cus) {
  TailPlan t{tiles, 0, 1, K};
  if (cus <= 0 || K % 64) return t;
  const int64_t r = tiles % cus, nk = K / 64;
  if (r == 0 || 2 * r > cus) return t;
  int64_t sp = cus / r;
  if (sp > 8) sp = 8;
  if (sp > nk / 4) sp = nk / 4;
  if (sp < 2) return t;
  const int64_t kc = cdiv(nk, sp) * 64;
  sp = cdiv(K, kc);
  if (sp < 2) return t;
  t.full = tiles - r; t.r = r; t.s = sp; t.kc = kc;
  return t;
}

// Fill in the split of the leftover tiles: none without a large enough workspace, for
// other tile shapes, batches, k splits or fp32 results.
void plan_tail(G2Args &a, const MfmaDesc &d, int bm, int bn) {
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  a.full_tiles = (int)tiles; a.tail_splits = 1; a.tail_kc = a.K; a.part = nullptr;
  if (!d.tail_ws || d.batch != 1 || d.splits != 1 || bm != 256 || bn != 256 || d.c_dt != POETX_BF16) return;
  const TailPlan t = tail_plan(tiles, d.K, device_cus());
  if (t.r == 0 || (size_t)t.r * t.s * bm * bn * 4 > d.tail_ws_bytes) return;
  a.full_tiles = (int)t.full; a.tail_splits = (int)t.s; a.tail_kc = t.kc;
  a.part = (float *)d.tail_ws;
}

int tail_reduce(const G2Args &a, const MfmaDesc &d, hipStream_t s) {
  const int r = a.tiles_m * a.tiles_n - a.full_tiles;
  if (r == 0) return POETX_OK;
  return launch_k("gemm_tail_reduce", s, k_tail_reduce, r * 8, 256, 0, a);
}

}  // namespace

size_t gemm_tail_ws_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N % 256 || K % 64) return 0;
  const TailPlan t = tail_plan(cdiv(M, 256) * (N / 256), K, device_cus());
  return (size_t)t.r * t.s * 256 * 256 * 4;
}

template <int ROLE, bool AKM, bool BKM, bool BI8 = false>
static int run_pp(const G2Args &k, const MfmaDesc &d, hipStream_t s) {
  size_t lds = (size_t)2 * 64 * (256 * 2 + 256 * (BI8 ? 1 : 2));
  if (POETX_EPI_LDS && lds < (size_t)256 * (256 * 2 + 16)) lds = (size_t)256 * (256 * 2 + 16);  // staged epilogue
  if (d.M <= 0 || d.N % 256 || d.K % 64) return POETX_ERR_UNSUPPORTED;
  G2Args a = k;
  a.tiles_m = (int)cdiv(d.M, 256);
  a.tiles_n = (int)(d.N / 256);
  plan_tail(a, d, 256, 256);
  dim3 grid((unsigned)(a.full_tiles + (a.tiles_m * a.tiles_n - a.full_tiles) * a.tail_splits), 1,
            (unsigned)(d.batch * d.splits));
  if constexpr (BI8) {  // int8 W' products write bf16 gradients only
    if (d.c_dt != POETX_BF16) return POETX_ERR_UNSUPPORTED;
    static std::atomic<uint64_t> attr{0};  // dynamic-LDS limit, per device
    POETX_TRY(lds_limit(reinterpret_cast<const void *>(&k_gemm_pp<ROLE, AKM, BKM, false, true>), lds, attr));
    POETX_TRY(launch_k(d.name, s, k_gemm_pp<ROLE, AKM, BKM, false, true>, grid, 512, lds, a));
    return tail_reduce(a, d, s);
  }
  if (d.c_dt == POETX_F32) {
    static std::atomic<uint64_t> attr{0};  // dynamic-LDS limit, per device
    POETX_TRY(lds_limit(reinterpret_cast<const void *>(&k_gemm_pp<ROLE, AKM, BKM, true>), lds, attr));
    return launch_k(d.name, s, k_gemm_pp<ROLE, AKM, BKM, true>, grid, 512, lds, a);
  }
  static std::atomic<uint64_t> attr{0};  // dynamic-LDS limit, per device
  POETX_TRY(lds_limit(reinterpret_cast<const void *>(&k_gemm_pp<ROLE, AKM, BKM, false>), lds, attr));
  POETX_TRY(launch_k(d.name, s, k_gemm_pp<ROLE, AKM, BKM, false>, grid, 512, lds, a));
  return tail_reduce(a, d, s);
}

template <int ROLE, int BM, int BN, int WGM, int WGN, int BKT, int NST, bool AKM, bool BKM, bool OUTF32,
          bool BI8 = false, bool TAIL = false>
static int run2o(const G2Args &a, const char *name, dim3 grid, size_t lds, hipStream_t s) {
  constexpr int NT = 64 * WGM * WGN;
  auto kern = &k_gemm2<ROLE, BM, BN, WGM, WGN, BKT, NST, AKM, BKM, OUTF32, BI8, TAIL>;
  static std::atomic<uint64_t> attr{0};  // dynamic-LDS limit, per device
  POETX_TRY(lds_limit(reinterpret_cast<const void *>(kern), lds, attr));
  return launch_k(name, s, kern, grid, NT, lds, a);
}

template <int ROLE, int BM, int BN, int WGM, int WGN, int BKT, int NST, bool AKM, bool BKM, bool BI8 = false,
          bool TAIL = false>
static int run2(const G2Args &k, const MfmaDesc &d, hipStream_t s) {
  size_t lds = (size_t)NST * (BM * 2 + BN * (BI8 ? 1 : 2)) * BKT;
  if (BM == 256 && BN == 256 && POETX_EPI_LDS && lds < (size_t)BM * (BN * 2 + 16))
    lds = (size_t)BM * (BN * 2 + 16);  // the staged bf16 epilogue tile
  if (TAIL ? (d.M <= 0 || d.N % 8 || d.K % 8 || d.batch != 1 || (ROLE == MFMA_BLOCK_GRAD && d.M % 8))
           : (d.M <= 0 || d.N % BN || (d.K % BKT && (!AKM || !BKM))))
    return POETX_ERR_UNSUPPORTED;
  G2Args a = k;
  a.tiles_m = (int)cdiv(d.M, BM);
  a.tiles_n = (int)(TAIL ? cdiv(d.N, BN) : d.N / BN);
  plan_tail(a, d, BM, BN);
  dim3 grid((unsigned)(a.full_tiles + (a.tiles_m * a.tiles_n - a.full_tiles) * a.tail_splits), 1,
            (unsigned)(d.batch * d.splits));
  if constexpr (BI8) {  // int8 W' products write bf16 activations only
    if (d.c_dt != POETX_BF16) return POETX_ERR_UNSUPPORTED;
    POETX_TRY((run2o<ROLE, BM, BN, WGM, WGN, BKT, NST, AKM, BKM, false, true>(a, d.name, grid, lds, s)));
    return tail_reduce(a, d, s);
  }
  if constexpr (TAIL) {  // whole-k tiles only (plan_tail splits none of these shapes)
    if (a.full_tiles != a.tiles_m * a.tiles_n) return POETX_ERR_UNSUPPORTED;
    if constexpr (ROLE == MFMA_BLOCK_GRAD) {  // fp32 partials
      if (d.c_dt != POETX_F32) return POETX_ERR_UNSUPPORTED;
      return run2o<ROLE, BM, BN, WGM, WGN, BKT, NST, AKM, BKM, true, false, true>(a, d.name, grid, lds, s);
    } else {  // bf16 products
      if (d.c_dt != POETX_BF16) return POETX_ERR_UNSUPPORTED;
      return run2o<ROLE, BM, BN, WGM, WGN, BKT, NST, AKM, BKM, false, false, true>(a, d.name, grid, lds, s);
    }
  } else {
    if (d.c_dt == POETX_F32) return run2o<ROLE, BM, BN, WGM, WGN, BKT, NST, AKM, BKM, true>(a, d.name, grid, lds, s);
    POETX_TRY((run2o<ROLE, BM, BN, WGM, WGN, BKT, NST, AKM, BKM, false>(a, d.name, grid, lds, s)));
    return tail_reduce(a, d, s);
  }
}

// The four-wave W' product: whole tiles only (a plan that splits leftover tiles along k
// takes the eight-wave kernel, whose partial layout the reduce kernel reads).
static int run4(const G2Args &k, const MfmaDesc &d, hipStream_t s, bool *done) {
  constexpr int WGM = POETX_G4_WGM, WGN = POETX_G4_WGN, BKT = POETX_G4_BK, NST = POETX_G4_NST;
  *done = false;
  if (d.K % BKT || d.c_dt != POETX_BF16) return POETX_OK;
  const size_t lds = (size_t)NST * (256 + 256) * BKT * 2;
  G2Args a = k;
  a.tiles_m = (int)cdiv(d.M, 256);
  a.tiles_n = (int)(d.N / 256);
  plan_tail(a, d, 256, 256);
  if (a.full_tiles != a.tiles_m * a.tiles_n) return POETX_OK;
  *done = true;
  const dim3 grid((unsigned)a.full_tiles);
  static std::atomic<uint64_t> attr{0};
  POETX_TRY(lds_limit(reinterpret_cast<const void *>(&k_gemm4<WGM, WGN, BKT, NST>), lds, attr));
  return launch_k(d.name, s, k_gemm4<WGM, WGN, BKT, NST>, grid, 64 * WGM * WGN, lds, a);
}

bool mfma2_supported(const MfmaDesc &d) {
  if (d.b_dt == POETX_I8) {
    // int8 W' in the two W' products only (16-byte aligned rows), bf16 results
    if (d.role != MFMA_GEMM_NT && d.role != MFMA_GEMM_NN) return false;
    if (d.c_dt != POETX_BF16 || d.ldb % 16 || d.batch != 1 || d.splits != 1) return false;
  } else if (d.b_dt != POETX_BF16) {
    return false;
  }
  if (d.c_dt != POETX_BF16 && d.c_dt != POETX_F32) return false;
  if (d.splits < 1 || d.batch * d.splits > 65535) return false;
  if (d.splits > 1 && (d.kchunk <= 0 || d.kchunk % 64 || cdiv(d.K, d.kchunk) != d.splits)) return false;
  // shapes that do not tile (multiples of 8), batch 1: the TAIL forms of the NT kernel (W'
  // products, bf16 results) and of the 128 x 128 block kernels (a last block of a size with
  // no block kernel: its products, bf16, and its gradient, fp32 parts)
  const bool tail = d.batch == 1 &&
                    ((d.role == MFMA_GEMM_NT && !d.a_km && !d.b_km && (d.N % 256 || d.K % 64)) ||
                     (d.role == MFMA_BLOCK_APPLY && !d.a_km && d.b_km && (d.N % 128 || d.K % 64)) ||
                     (d.role == MFMA_BLOCK_APPLY_T && !d.a_km && !d.b_km && (d.N % 128 || d.K % 64)) ||
                     (d.role == MFMA_BLOCK_GRAD && d.a_km && d.b_km && (d.M % 128 || d.N % 128)));
  if (tail) {
    if (d.b_dt != POETX_BF16) return false;
    if (d.role == MFMA_BLOCK_GRAD ? d.c_dt != POETX_F32 : (d.c_dt != POETX_BF16 || d.splits != 1)) return false;
    if (d.N % 8 || d.K % 8 || d.lda % 8 || d.ldb % 8 || d.ldc % 8) return false;
    if (d.role == MFMA_BLOCK_GRAD && d.M % 8) return false;
    if ((((uintptr_t)d.A | (uintptr_t)d.B | (uintptr_t)d.C) & 15) != 0) return false;
  } else if ((!d.a_km || !d.b_km) && d.K % 64) {
    return false;
  }
  // 32-bit buffer offsets, with room for the rows a last partial tile addresses
  const int64_t a_ext = ((d.a_km ? d.K : d.M) + 256) * d.lda * 2, b_ext = ((d.b_km ? d.K : d.N) + 256) * d.ldb * 2;
  if (a_ext > 0x7fffffff || b_ext > 0x7fffffff) return false;
  switch (d.role) {
    case MFMA_GEMM_NT: return (tail || d.N % 256 == 0) && cdiv(d.M, 256) * cdiv(d.N, 256) < (1 << 30);
    case MFMA_GEMM_NN: return d.N % 256 == 0 && cdiv(d.M, 256) * (d.N / 256) < (1 << 30);
    default: return tail || (d.N % 128 == 0 && (!d.a_km || d.M % 128 == 0));
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
  const bool i8 = d.b_dt == POETX_I8;
  switch (d.role) {
    case MFMA_GEMM_NT:
      if (d.a_km || d.b_km) return POETX_ERR_UNSUPPORTED;
      if (i8) return run2<MFMA_GEMM_NT, 256, 256, 2, 4, 64, 2, false, false, true>(k, d, s);
      if (d.N % 256 || d.K % 64) return run2<MFMA_GEMM_NT, 256, 256, 2, 4, 64, 2, false, false, false, true>(k, d, s);
      if (d.batch == 1 && d.splits == 1 && kUseGemm4) {
        bool done = false;
        POETX_TRY(run4(k, d, s, &done));
        if (done) return POETX_OK;
      }
      if (d.batch > 1) return run2<MFMA_GEMM_NT, 256, 256, 2, 4, POETX_BNT_BK, POETX_BNT_NST, false, false>(k, d, s);
      return run2<MFMA_GEMM_NT, 256, 256, 2, 4, POETX_NT_BK, POETX_NT_NST, false, false>(k, d, s);
    case MFMA_GEMM_NN:
      if (d.a_km || !d.b_km) return POETX_ERR_UNSUPPORTED;
      // the k-major W' operand goes through the transposing LDS reads; the ping-pong
      // schedule hides their extra latency best (measured against the plain schedule)
      if (i8) return run_pp<MFMA_GEMM_NN, false, true, true>(k, d, s);
      return run_pp<MFMA_GEMM_NN, false, true>(k, d, s);
    case MFMA_BLOCK_APPLY:
      if (d.a_km || !d.b_km) return POETX_ERR_UNSUPPORTED;
      if (d.N % 128 || d.K % 64) return run2<MFMA_BLOCK_APPLY, 128, 128, 2, 2, 64, 2, false, true, false, true>(k, d, s);
      return run2<MFMA_BLOCK_APPLY, 128, 128, 2, 2, 64, 2, false, true>(k, d, s);
    case MFMA_BLOCK_APPLY_T:
      if (d.a_km || d.b_km) return POETX_ERR_UNSUPPORTED;
      if (d.N % 128 || d.K % 64) return run2<MFMA_BLOCK_APPLY_T, 128, 128, 2, 2, 64, 2, false, false, false, true>(k, d, s);
      return run2<MFMA_BLOCK_APPLY_T, 128, 128, 2, 2, 64, 2, false, false>(k, d, s);
    case MFMA_BLOCK_GRAD:
      if (!d.a_km || !d.b_km) return POETX_ERR_UNSUPPORTED;
      if (d.M % 128 || d.N % 128) return run2<MFMA_BLOCK_GRAD, 128, 128, 2, 2, 64, 2, true, true, false, true>(k, d, s);
      // blocks of a multiple of 256: 256 x 256 tiles, each operand slice read by two of them
      if (d.M % 256 == 0 && d.N % 256 == 0) return run2<MFMA_BLOCK_GRAD, 256, 256, 2, 4, 64, 2, true, true>(k, d, s);
      return run2<MFMA_BLOCK_GRAD, 128, 128, 2, 2, 64, 2, true, true>(k, d, s);
    default:
      return POETX_ERR_UNSUPPORTED;
  }
}

}  // namespace poetx
