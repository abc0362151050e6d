// gemm_prefill.hip -- output-tiled hybrid GEMM for many tokens (M > 16).
//
// PATCH (arXiv 2509.23410), gist.science explainer, section 2 "Inference &
// Deployment": each tile runs on the dense matrix units or, when it is 2:4,
// on the sparse ones.  With M >= 512 the product is bound by the matrix
// cores, so the kernel is built around feeding them:
//
//   * A workgroup (8 waves, one per CU) owns TWO row-blocks of W -- row-block
//     p and row-block NT-1-p -- and BM columns of M (BM = 128, 192 or 256,
//     chosen per shape so the grid fills the GPU): a 256 x BM block of Y^T.
//     Both row-blocks read the same X[m0 .. m0+BM-1][k] slices, so every X
//     byte brought into the CU feeds 256 rows of W.
//   * Wave w: row-block r = w/4, bands 4*((w/2)&1) .. +3 of it (64 rows of W)
//     and BM/2 columns of M (w&1): 4 x BM/32 fp32 accumulators of 16 x 16.
//     Waves w and w+4 -- one per row-block -- share a SIMD, so when one
//     row-block's tile is dense and the other's is 2:4 the SIMD's matrix
//     core is busy for the sum of the two, with no wave idling on the other's
//     kind.  Pairing row-block p with NT-1-p also evens out maps whose dense
//     tiles cluster in a band of rows.
//   * The K loop walks the tile columns in order, 64 columns a step, and
//     runs both kinds on v_smfmac_f32_16x16x64: a 2:4 slice once with its
//     own index codes, a dense slice twice (its halves holding positions
//     (0,1) and (2,3) of every group, fixed codes) -- so both kinds share one
//     instruction, one B fragment set and one accumulator layout, and the
//     per-wave choice of kind is just a trip count.
//   * X[m0 .. m0+BM-1][64 columns] of the next step is loaded into registers
//     while the current step computes, then written to the other of two LDS
//     buffers; 16-byte chunks are XOR-swizzled by row so the B-operand reads
//     hit distinct banks.  Every memory operation in the loop is an ordinary
//     vector load, so the compiler's wait counts stay exact (mixing in
//     global -> LDS copies makes it wait for everything before each LDS
//     read).  Where registers allow, B fragments for the next 32 columns of
//     M are read from LDS while the current ones feed the matrix cores.
//   * W comes straight from the packed blob into A-operand registers (a 1 KB
//     fragment is one 16-byte load a lane), one step ahead; eight loads a
//     lane per step for either kind.  A wave's four bands of a tile are four
//     pieces one band stride apart, so one descriptor and four scalar
//     offsets address them.
//   * All loads are buffer loads: a scalar descriptor (tile or X block base)
//     plus a 32-bit lane offset, so addresses cost no 64-bit vector
//     arithmetic; X rows past M fall outside the X descriptor's range and
//     read as zero.
//   * Workgroups are numbered so that each of the 8 XCDs gets a contiguous
//     run of output blocks that is close to a rectangle -- a range of
//     row-block pairs times one group of M-blocks -- so that neither all of
//     W nor all of X passes through every XCD's L2 (the M-blocks of a pair
//     share its W tiles in that L2; the pairs share the X slices).
//
// With SRC_ROWMAJOR the same kernel reads plain row-major W with every tile
// dense, on v_mfma_f32_16x16x32: the same-shape dense baseline.
#include "prefill_common.h"

#include <algorithm>
#include <atomic>
#include <random>

namespace patch {

constexpr int kPfWaves = 8;
constexpr int kPfMGroup = 2;      // 16-column blocks of M whose B fragments are read together

// A operands of one step, [.][band]: packed dense tile: a[e] = half e
// (positions 2e, 2e+1 of every group of four); 2:4 tile: a[0] = values,
// a[1] = the 16 bytes of the band's codes that hold this lane's word (word
// l & 3); row-major W (dense baseline): a[qq] = 32-column slice qq in the
// v_mfma_f32_16x16x32 layout.
struct StepA {
  u32x4 a[2][4];
};

// Fused gate/up epilogue: the pair is (gate row-block 2p, up row-block 2p+1),
// waves r = 0 hold gate sums and waves r = 1 the up sums of the same output
// positions; the up sums go through LDS (scratch, at least 2 KB per wave
// pair), and the gate waves write H[m][128 p + ...] = SiLU(gate) * up.
template <bool BF16, bool OUT_F32, int kNMB, int NBR>
__device__ __forceinline__ void fused_epilogue(const f32x4 (&acc)[4][kNMB], uint8_t* scratch, void* H, int M, int F,
                                               int p, int m0, int r, int wn, int wm, int l, int half_cols) {
  constexpr int nbr = NBR;  // bands exchanged per round: scratch holds 4 * NBR KB
  const int hl = l >> 4;
  f32x4* sc = reinterpret_cast<f32x4*>(scratch);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of the last stage are done
  wg_barrier();
#pragma unroll
  for (int mblk = 0; mblk < kNMB; mblk++) {
#pragma unroll
    for (int b0 = 0; b0 < 4; b0 += nbr) {
      if (r == 1)
#pragma unroll
        for (int bb = 0; bb < nbr; bb++) sc[(((wn * 2 + wm) * nbr) + bb) * 64 + l] = acc[b0 + bb][mblk];
      __builtin_amdgcn_s_waitcnt(0xC07F);
      wg_barrier();
      if (r == 0) {
        const int m = m0 + wm * half_cols + mblk * 16 + (l & 15);
#pragma unroll
        for (int bb = 0; bb < nbr; bb++) {
          const f32x4 u = sc[(((wn * 2 + wm) * nbr) + bb) * 64 + l];
          const int64_t n = (int64_t)p * kTile + 16 * (4 * wn + b0 + bb) + 4 * hl;
          if (m < M) store4<BF16, OUT_F32>(H, (int64_t)m * F + n, silu_mul(acc[b0 + bb][mblk], u));
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      wg_barrier();
    }
  }
}

template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32, int BM, int DIST, bool FUSE>
__global__ __launch_bounds__(kPfWaves * 64, 1) void k_prefill(PfArgs P) {
  constexpr int kNMB = BM / 32;                       // 16-column M blocks per wave
  constexpr int kStageBytes = BM * kPfRowBytes;       // one X stage
  constexpr int kXChunks = kStageBytes / 16 / (kPfWaves * 64);  // 16-byte chunks a lane stages per step
  static_assert(kNMB % kPfMGroup == 0 && kXChunks * 16 * kPfWaves * 64 == kStageBytes, "tile shape");

  static_assert(DIST == 1 || DIST == 2, "prefetch distance");
  __shared__ __attribute__((aligned(16))) uint8_t s_x0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_x1[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_x2[DIST == 2 ? kStageBytes : 16];
  // per row-block of the pair and tile column: (byte offset >> 8) | kind << 30
  // (kind 0 dense, 1 2:4, 2 4:8; blobs stay below 2^38 bytes)
  __shared__ uint32_t s_ent[2][kPfMaxKT];
  __shared__ uint32_t s_stride[2];  // band stride of each row-block of the pair

  // Output blocks in order: K range, M-group (mg M-blocks each), row-block
  // pair, M-block; XCD x (workgroups are dealt to the 8 XCDs in turn) takes
  // the x-th eighth of that order, so its blocks are a few pairs times one
  // group's M-blocks, mostly in one K range.
  const int t = (blockIdx.x & 7) * P.per_xcd + (blockIdx.x >> 3);
  if (t >= P.n_blocks) return;  // whole workgroup
  const int per_split = P.n_pairs * P.n_mblk;
  const int ks = t / per_split, tk = t - (t / per_split) * per_split;
  const int grp = P.n_pairs * P.mg;
  const int gi = tk / grp, rem = tk - (tk / grp) * grp;
  const int m_cnt = min(P.mg, P.n_mblk - gi * P.mg);
  const int p = rem / m_cnt, mb = gi * P.mg + rem % m_cnt;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l = threadIdx.x & 63;
  const int r = w >> 2, wn = (w >> 1) & 1, wm = w & 1;
  const int hl = l >> 4;
  const int KT = P.KT, K = P.K;
  const int m0 = mb * BM;
  // pair: row-blocks p and NT-1-p; fused gate/up: 2p (gate) and 2p+1 (up)
  const int i0 = FUSE ? 2 * p : p, i1 = FUSE ? 2 * p + 1 : P.NT - 1 - p;
  const int i_mine = r == 0 ? i0 : i1;
  const bool active = r == 0 || i1 != i0;  // a lone middle row-block has no second half (never when fused)
  // this workgroup's tile columns j0 .. j0 + nt - 1 (all of them unless split)
  const int j0 = ks * P.kt_split;
  const int nt = min(P.kt_split, KT - j0);
  const int n_steps = 2 * nt;

  if constexpr (!SRC_ROWMAJOR) {
    const TileEntry* table = reinterpret_cast<const TileEntry*>(P.src + kHeaderBytes);
    for (int e = threadIdx.x; e < 2 * nt; e += kPfWaves * 64) {
      const int rr = e >= nt ? 1 : 0;
      const int j = e - rr * nt;
      const TileEntry te = table[(int64_t)(rr ? i1 : i0) * KT + j0 + j];
      s_ent[rr][j] = (uint32_t)(te.offset >> 8) | (te.kind << 30);
      if (j == 0) s_stride[rr] = te.band_stride;
    }
    __syncthreads();
  }
  const uint32_t stride = SRC_ROWMAJOR ? 0u : (uint32_t)__builtin_amdgcn_readfirstlane((int)s_stride[r]);

  const uint32_t lane16 = 16u * (uint32_t)l;

  // A operands of step s (tile column s/2, half s&1) for this wave; returns
  // the tile kind (0 dense, 1 2:4), wave-uniform.  Both kinds issue the same
  // eight 16-byte loads (only offsets differ), so registers and wait counts
  // are identical on both paths.
  auto load_a = [&](int s, StepA& A) -> uint32_t {
    const int jl = s >> 1, h = s & 1, j = j0 + jl;
    if constexpr (SRC_ROWMAJOR) {
      // rows 64wn + 16b + (l & 15) of row-block i_mine, columns 128j + 64h + 32qq + 8hl
      // (fused: row-block i_mine/2 of the gate or the up matrix)
      const uint8_t* Wsrc = (FUSE && (i_mine & 1)) ? P.src2 : P.src;
      const int ib = FUSE ? (i_mine >> 1) : i_mine;
      const uint8_t* W = Wsrc + (((int64_t)ib * kTile + 64 * wn) * K + (int64_t)j * kTile + 64 * h) * 2;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(W, 0xffffffffu);
      const uint32_t lane_rm = ((uint32_t)(l & 15) * (uint32_t)K + 8u * (uint32_t)hl) * 2u;
#pragma unroll
      for (int qq = 0; qq < 2; qq++)
#pragma unroll
        for (int b = 0; b < 4; b++) A.a[qq][b] = bload16(rs, lane_rm, (uint32_t)(16 * b * K + 32 * qq) * 2u);
      return 0u;
    } else {
      const uint32_t e = __builtin_amdgcn_readfirstlane(s_ent[r][jl]);
      const uint32_t kind = e >> 30;
      // the wave's first band piece; band 4wn+b is b * stride further on
      const uint8_t* piece = P.src + ((uint64_t)(e & 0x3fffffffu) << 8) + (uint64_t)(4 * wn) * stride;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(piece, 3u * stride + (uint32_t)kDensePieceBytes);
      // dense: a[e][b] = half e of band 4wn+b in 64-column slice h, at
      //        2048h + 1024e in its piece;
      // 2:4  : a[0][b] = values of band 4wn+b in slice h, at 1024h;
      //        a[1][b] = its codes chunk 16 * (l/4) past the values.
      // (This kernel runs dense and 2:4 tiles only; the host routes blobs
      // with 4:8 tiles to k_prefill_lds.)
      const uint32_t v1 = kind ? 16u * (uint32_t)(l >> 2) : lane16;
      const uint32_t o0 = kind ? 1024u * (uint32_t)h : 2048u * (uint32_t)h;
      const uint32_t o1 = kind ? (uint32_t)kSparseMetaOffset : 2048u * (uint32_t)h + 1024u;
#pragma unroll
      for (int b = 0; b < 4; b++) A.a[0][b] = bload16(rs, lane16, o0 + stride * b);
#pragma unroll
      for (int b = 0; b < 4; b++) A.a[1][b] = bload16(rs, v1, o1 + stride * b);
      return kind;
    }
  };

  // X of step s, BM rows x 64 columns = BM*8 chunks of 16 bytes: lane chunk
  // c = u * 512 + threadIdx.x is row c / 8, stored at chunk position c % 8 of
  // that row, so it holds the source chunk whose swizzled position is c % 8.
  // Rows past M are outside the descriptor's range and load as zero (never
  // stored).  Lane offsets stay below BM * K * 2 bytes (< 2^31).
  uint32_t lane_x[kXChunks];
#pragma unroll
  for (int u = 0; u < kXChunks; u++) {
    const int c = u * kPfWaves * 64 + (int)threadIdx.x;
    const int row = c >> 3;
    lane_x[u] = ((uint32_t)row * (uint32_t)K + 8u * (uint32_t)((c & 7) ^ swz_f(row))) * 2u;
  }
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(P.X + (int64_t)m0 * K, (uint32_t)min(BM, P.M - m0) * (uint32_t)K * 2u);
  auto load_x = [&](int s, u32x4 (&xr)[kXChunks]) {
    const uint32_t col = (uint32_t)((j0 + (s >> 1)) * kTile + 64 * (s & 1)) * 2u;
#pragma unroll
    for (int u = 0; u < kXChunks; u++) xr[u] = bload16(rx, lane_x[u], col);
  };
  auto store_x = [&](const u32x4 (&xr)[kXChunks], uint8_t* dst) {
#pragma unroll
    for (int u = 0; u < kXChunks; u++)
      *reinterpret_cast<u32x4*>(dst + 16 * (u * kPfWaves * 64 + (int)threadIdx.x)) = xr[u];
  };

  f32x4 acc[4][kNMB];
#pragma unroll
  for (int a = 0; a < 4; a++)
#pragma unroll
    for (int c = 0; c < kNMB; c++) acc[a][c] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // B fragments of M blocks kPfMGroup*g .. +kPfMGroup-1: chunks hl (K 8hl..)
  // and 4+hl (K 32+8hl..) of their rows.
  auto read_b = [&](const uint8_t* xs, int g, u32x4 (&blo)[kPfMGroup], u32x4 (&bhi)[kPfMGroup]) {
#pragma unroll
    for (int mm = 0; mm < kPfMGroup; mm++) {
      const int row = wm * (BM / 2) + (kPfMGroup * g + mm) * 16 + (l & 15);
      blo[mm] = *reinterpret_cast<const u32x4*>(xs + swz(row, hl));
      bhi[mm] = *reinterpret_cast<const u32x4*>(xs + swz(row, 4 + hl));
    }
  };

  // One step from stage buffer xs.
  auto compute = [&](const StepA& A, uint32_t kind, int h, const uint8_t* xs) {
    if (!active) return;
    if constexpr (SRC_ROWMAJOR) {
#pragma unroll
      for (int qq = 0; qq < 2; qq++) {
        u32x4 bf[kNMB];
#pragma unroll
        for (int mblk = 0; mblk < kNMB; mblk++)
          bf[mblk] = *reinterpret_cast<const u32x4*>(xs + swz(wm * (BM / 2) + mblk * 16 + (l & 15), 4 * qq + hl));
#pragma unroll
        for (int mblk = 0; mblk < kNMB; mblk++)
#pragma unroll
          for (int b = 0; b < 4; b++) acc[b][mblk] = mma_dense<BF16>(A.a[qq][b], bf[mblk], acc[b][mblk]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // Both kinds on v_smfmac_f32_16x16x64 with the same B fragments: a 2:4
      // slice once with its own codes, a dense slice twice -- half (0,1) with
      // code 4 in every group, half (2,3) with code 14.
      const int nsub = kind == 0 ? 2 : 1;
      // 2:4: word l & 3 of the chunk by two bit tests (plain selects; a
      // dynamic vector index would put the fragments in scratch memory)
      uint32_t idx0[4];
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const u32x4 mc = A.a[1][b];
        const uint32_t lo = (l & 1) ? mc[1] : mc[0], hi = (l & 1) ? mc[3] : mc[2];
        idx0[b] = kind == 0 ? 0x4444u : (((l & 2) ? hi : lo) >> (16 * h));
      }
      // B fragments double-buffered across groups where registers allow
      // (the 256-wide tile has no room for the second set).
      constexpr int kGroups = kNMB / kPfMGroup;
      constexpr bool kPipeB = BM < 256;
      u32x4 blo[2][kPfMGroup], bhi[2][kPfMGroup];
      if (kPipeB) read_b(xs, 0, blo[0], bhi[0]);
#pragma unroll
      for (int g = 0; g < kGroups; g++) {
        if (!kPipeB) read_b(xs, g, blo[g & 1], bhi[g & 1]);
        if (kPipeB && g + 1 < kGroups) read_b(xs, g + 1, blo[(g + 1) & 1], bhi[(g + 1) & 1]);
        for (int sub = 0; sub < nsub; sub++) {
#pragma unroll
          for (int mm = 0; mm < kPfMGroup; mm++)
#pragma unroll
            for (int b = 0; b < 4; b++)
              acc[b][kPfMGroup * g + mm] =
                  mma_sparse<BF16, 0>(sub ? A.a[1][b] : A.a[0][b], blo[g & 1][mm], bhi[g & 1][mm],
                                      acc[b][kPfMGroup * g + mm], sub ? 0xEEEEu : idx0[b]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  const int last = n_steps - 1;
  if constexpr (DIST == 1) {
    // ---- prologue: X of step 0 into buffer 0, A of step 0.  Every step
    // issues the same loads (X of the next step, then its A); past the last
    // step they repeat the last step's offsets and land in registers and a
    // buffer nobody reads again, so the wait counts hold on every path.
    u32x4 xr[kXChunks];
    StepA A0, A1;
    load_x(0, xr);
    uint32_t k0 = load_a(0, A0), k1 = 0;
    store_x(xr, s_x0);
    __syncthreads();

    // Step s (X buffer s % 2, A buffer s % 2): load X and A of step s+1 into
    // registers, compute step s, write X of s+1 into the other buffer (read
    // at step s-1; every wave has passed the barrier after it), and meet at
    // the barrier once the LDS writes are done.
    auto step = [&](int s, StepA& cur, uint32_t kc, StepA& nxt, uint32_t& kn, const uint8_t* xs, uint8_t* xo) {
      load_x(min(s + 1, last), xr);
      kn = load_a(min(s + 1, last), nxt);
      compute(cur, kc, s & 1, xs);
      store_x(xr, xo);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
      wg_barrier();
    };
    for (int s = 0; s < n_steps; s += 2) {  // n_steps is even
      step(s, A0, k0, A1, k1, s_x0, s_x1);
      step(s + 1, A1, k1, A0, k0, s_x1, s_x0);
    }
  } else {
    // ---- two steps ahead: A of step s+2 and X of step s+2 are loaded at
    // step s; X of s+1 (loaded at step s-1) is written to LDS at the end of
    // step s.  Three A register sets, three X buffers, two X register sets:
    // the pattern repeats every 6 steps.
    u32x4 xr0[kXChunks], xr1[kXChunks];
    StepA A0, A1, A2;
    uint32_t k0, k1, k2 = 0;
    load_x(0, xr0);
    k0 = load_a(0, A0);
    load_x(min(1, last), xr1);
    k1 = load_a(min(1, last), A1);
    store_x(xr0, s_x0);
    __syncthreads();

    // xl: registers receiving X of s+2; xw: registers holding X of s+1.
    auto step = [&](int s, StepA& cur, uint32_t kc, StepA& ahead, uint32_t& ka, u32x4 (&xl)[kXChunks],
                    const u32x4 (&xw)[kXChunks], const uint8_t* xs, uint8_t* xo) {
      load_x(min(s + 2, last), xl);
      ka = load_a(min(s + 2, last), ahead);
      compute(cur, kc, s & 1, xs);
      store_x(xw, xo);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
      wg_barrier();
    };
    int s = 0;
    for (; s + 6 <= n_steps; s += 6) {
      step(s + 0, A0, k0, A2, k2, xr0, xr1, s_x0, s_x1);
      step(s + 1, A1, k1, A0, k0, xr1, xr0, s_x1, s_x2);
      step(s + 2, A2, k2, A1, k1, xr0, xr1, s_x2, s_x0);
      step(s + 3, A0, k0, A2, k2, xr1, xr0, s_x0, s_x1);
      step(s + 4, A1, k1, A0, k0, xr0, xr1, s_x1, s_x2);
      step(s + 5, A2, k2, A1, k1, xr1, xr0, s_x2, s_x0);
    }
    if (s < n_steps) {  // n_steps = 2 or 4 (mod 6): the first steps of the pattern
      step(s + 0, A0, k0, A2, k2, xr0, xr1, s_x0, s_x1);
      step(s + 1, A1, k1, A0, k0, xr1, xr0, s_x1, s_x2);
      if (s + 2 < n_steps) {
        step(s + 2, A2, k2, A1, k1, xr0, xr1, s_x2, s_x0);
        step(s + 3, A0, k0, A2, k2, xr1, xr0, s_x0, s_x1);
      }
    }
  }

  // ---- epilogue: round and store Y[m][n .. n+3] (split: the fp32 partial
  // of K range ks, at plane ks of the partial buffer; fused and unsplit:
  // H = SiLU(gate) * up)
  if constexpr (FUSE) {
    if (P.splits == 1) {
      fused_epilogue<BF16, OUT_F32, kNMB, (kStageBytes >= 4 * 4096 ? 4 : 2)>(acc, s_x0, P.Y, P.M, P.N / 2, p, m0, r,
                                                                              wn, wm, l, BM / 2);
      return;
    }
  }
  void* Yp = P.Y;
  if (P.splits > 1) Yp = reinterpret_cast<float*>(P.Y) + (int64_t)ks * P.M * P.N;
  if (active) {
#pragma unroll
    for (int mblk = 0; mblk < kNMB; mblk++) {
      const int m = m0 + wm * (BM / 2) + mblk * 16 + (l & 15);
      if (m < P.M) {
#pragma unroll
        for (int b = 0; b < 4; b++) {
          const int64_t n = (int64_t)i_mine * kTile + 16 * (4 * wn + b) + 4 * hl;
          store4<BF16, OUT_F32>(Yp, (int64_t)m * P.N + n, acc[b][mblk]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------------------
// k_prefill_lds: the same output tiling with W and X staged through LDS by
// global -> LDS copies, two or three steps deep.
//
//   * Per step every wave issues exactly 4 + BM/64 copies of 1 KB (16 bytes
//     a lane, straight into LDS, no registers): BM/64 8-row chunks of the X
//     stage and four W fragments -- wave (r, wn, wm) copies half wm of bands
//     4wn..4wn+3 of row-block r (a 2:4 tile: the values if wm = 0, the
//     band's codes, 4 bytes a lane, if wm = 1), so each W byte enters the CU
//     once, where the register-staged kernel loads every W fragment into
//     both M-halves' waves.  A step's copies go out as a few blocks of
//     back-to-back copies whose addresses are scalar (one scalar add a copy).
//   * Copies for the later steps go out while step s computes; a wave waits
//     for its own copies of step s with vmcnt (the copies of the next step
//     may stay in flight) and the barrier after it publishes everyone's.  The
//     copies are inline asm, so the compiler neither waits for them nor for
//     anything else before LDS reads; the wait counts are exact because every
//     wave issues the same copies every step.
//   * Fragments are then read from LDS with one 16-byte read a lane (a 2:4
//     or 4:8 tile's codes: one 16-bit read a lane, its half of its word) and
//     fed to the same v_smfmac_f32_16x16x64 sequence as the register-staged
//     kernel.  The barrier of step s + 1 sits before the last group of step
//     s's matrix instructions; right after it each wave reads step s + 1's
//     A fragments and first B fragments, then issues its copies, then runs
//     that group, so the reads the next step waits for go out first and run
//     under the group (two sets of A fragments; B fragments alternate
//     between two buffers by group).  Within the other groups the next
//     group's reads are spread between the matrix instructions (one or two
//     after each), so the waves sharing a SIMD do not all queue at the LDS
//     and then all at the matrix core.
// LDS per stage: 32 KB of W + BM * 128 bytes of X; three stages up to width
// 128 (120 KB at 64, 144 KB at 128), two at 192 and 256 (112 and 128 KB),
// plus the tile entries and, for packed W, the 4 KB table that rebuilds 4:8
// tiles: one workgroup per CU.
//   * Tile kinds: dense and 2:4 as above; a 4:8 tile's band is copied like a
//     2:4 one (values, then the chunk holding the lane's position masks) and
//     rebuilt in registers into a dense piece's two halves (one table read
//     and four byte permutes per group of eight), then runs as a dense tile.
// ---------------------------------------------------------------------------
constexpr int kLdsWStage = 32768;  // 2 row-blocks x 8 bands x 2 fragments of 1 KB
// stages of the LDS ring for an M-block width: three up to 128, two at 192
// and 256 (a third would not fit the 160 KB of LDS; at 192 three X stages
// beside two W stages measured 2-4% slower than two beside three)
constexpr int lds_stages(int bm) { return bm <= 128 ? 3 : 2; }
// W stages: three also at width 192 (two X stages of 24 KB beside three W
// stages of 32 KB and 8 KB of tile entries fill the 160 KB exactly; not with
// the 16 KB of entries of 64 x 64 tiles), so W copies run two steps ahead
// there while X copies run one
constexpr int lds_w_stages(int bm, bool q64) { return bm <= 128 || (bm == 192 && !q64) ? 3 : 2; }
// Polls of a tail range's flag (each a round trip to the L2 plus 256
// cycles of sleep) before range 0 gives up on it: a second or more, far
// beyond any range's run time.
constexpr int kTailSpinLimit = 1 << 20;
// Cache-policy operand of the buffer loads and stores: sc1, agent scope.
constexpr int kCoherent = 16;

// Q64: a blob of 64 x 64 execution tiles (format 4).  Its table has one
// entry per 64-row half of a row-block and 128-column tile column, whose
// kind bits give each 64-column slice's kind (bit q set: slice q is 2:4) and
// whose pieces hold the slices back to back (a dense slice 2048 bytes, a 2:4
// one 1024) and then, if either is 2:4, the 256-byte codes block.  A wave
// (r, wn, wm) works on half wn of row-block r, so it reads that half's
// entries and, per step (one slice), that slice's kind: the waves of one
// workgroup may run different kinds in the same step.
template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32, bool FUSE, int BM, bool Q64 = false>
__global__ __launch_bounds__(kPfWaves * 64, 1) void k_prefill_lds(PfArgs P) {
  static_assert(!Q64 || (!SRC_ROWMAJOR && !FUSE), "64 x 64 execution tiles: packed W, not fused");
  constexpr int kNMB = BM / 32;                     // 16-column M blocks per wave
  constexpr int kXStages = lds_stages(BM);
  constexpr int kWStages = lds_w_stages(BM, Q64);
  constexpr int kLdsXStage = BM * kPfRowBytes;       // X rows of one step
  constexpr int kXC = BM / 64;                       // 1 KB X chunks a wave copies per step
  constexpr int kLdsCopies = 4 + kXC;                // copies a wave issues per step
  // 16-column M blocks whose B fragments are read together (one at width
  // 256, where two steps' A fragments and the accumulators leave no room)
  constexpr int kMG = BM == 256 ? 1 : kPfMGroup;
  static_assert(kXC * 1024 * kPfWaves == kLdsXStage, "X stage split");
  __shared__ __attribute__((aligned(1024))) uint8_t s_w[kWStages * kLdsWStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s_x[kXStages * kLdsXStage];
  constexpr int kEntRows = Q64 ? 4 : 2;  // row-blocks (Q64: their 64-row halves) of a workgroup
  __shared__ uint32_t s_ent[kEntRows][kPfMaxKT];
  __shared__ u32x4 s_sel[SRC_ROWMAJOR || Q64 ? 1 : 256];  // 4:8 rebuild selectors

  // block tk, K range ks; tb: the tail block (tail split), else -1
  int ks, tk, tb = -1;
  if (!FUSE && P.tail_s > 1 && P.n_full == 0) {
    // no whole blocks: range-major, as the K split (an XCD streams one K
    // range of its blocks), the waiting range 0 last -- on the XCDs after
    // the writers', so the waiting workgroups never hold the CUs that the
    // ranges they wait for need
    const int t = (blockIdx.x & 7) * P.per_xcd + (blockIdx.x >> 3);
    if (t >= P.tail_s * P.n_tail) return;  // whole workgroup
    const int r = t / P.n_tail;
    tb = t - r * P.n_tail;
    ks = P.tail_s - 1 - r;
    tk = tb;
  } else if (!FUSE && P.tail_s > 1) {
    // an XCD runs its share of the whole blocks first, then its tail blocks,
    // each block's ranges back to back with range 0 -- the one that waits --
    // last, so it is dispatched after the ranges it waits for
    const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
    const int full_per = P.n_full >> 3;
    if (i < full_per) {
      tk = x * full_per + i;
      ks = 0;
    } else {
      const int j = i - full_per;
      const int tl = j / P.tail_s;
      tb = x * P.tail_per + tl;
      if (tl >= P.tail_per || tb >= P.n_tail) return;  // whole workgroup
      ks = P.tail_s - 1 - (j - tl * P.tail_s);
      tk = P.n_full + tb;
    }
  } else {
    const int t = (blockIdx.x & 7) * P.per_xcd + (blockIdx.x >> 3);
    if (t >= P.n_blocks) return;  // whole workgroup
    const int per_split = P.n_pairs * P.n_mblk;
    ks = t / per_split;
    tk = t - ks * per_split;
  }
  const int grp = P.n_pairs * P.mg;
  const int gi = tk / grp, rem = tk - (tk / grp) * grp;
  const int m_cnt = min(P.mg, P.n_mblk - gi * P.mg);
  const int p = rem / m_cnt, mb = gi * P.mg + rem % m_cnt;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l = threadIdx.x & 63;
  const int r = w >> 2, wn = (w >> 1) & 1, wm = w & 1;
  const int hl = l >> 4;
  const int KT = P.KT, K = P.K, M = P.M;
  const int m0 = mb * BM;
  // pair: row-blocks p and NT-1-p; fused gate/up: 2p (gate) and 2p+1 (up)
  const int i0 = FUSE ? 2 * p : p, i1 = FUSE ? 2 * p + 1 : P.NT - 1 - p;
  const bool active = r == 0 || i1 != i0;  // a lone middle row-block has no second half (never when fused)
  const int i_mine = r == 0 ? i0 : i1;
  // a wave with no row-block of its own copies row-block i0's fragments into
  // its own (never read) LDS slots, so every wave issues the same copies
  const int r_src = active ? r : 0;
  const int i_src = active ? i_mine : i0;
  const int j0 = ks * P.kt_split;
  // (a whole block of a tail split: all of K)
  const int nt = !FUSE && P.tail_s > 1 && tb < 0 ? KT : min(P.kt_split, KT - j0);
  const int n_steps = 2 * nt;

  if constexpr (Q64) {
    // entry rows 2 rr + hh: half hh of row-block i0 (rr = 0) or i1 (rr = 1)
    const TileEntry* table = reinterpret_cast<const TileEntry*>(P.src + kHeaderBytes);
    for (int e = threadIdx.x; e < 4 * nt; e += kPfWaves * 64) {
      const int rh = e / nt;
      const int j = e - rh * nt;
      const TileEntry te = table[(int64_t)(2 * ((rh >> 1) ? i1 : i0) + (rh & 1)) * KT + j0 + j];
      s_ent[rh][j] = (uint32_t)(te.offset >> 8) | (te.kind << 30);
    }
    __syncthreads();
  } else if constexpr (!SRC_ROWMAJOR) {
    const TileEntry* table = reinterpret_cast<const TileEntry*>(P.src + kHeaderBytes);
    for (int e = threadIdx.x; e < 2 * nt; e += kPfWaves * 64) {
      const int rr = e >= nt ? 1 : 0;
      const int j = e - rr * nt;
      const TileEntry te = table[(int64_t)(rr ? i1 : i0) * KT + j0 + j];
      s_ent[rr][j] = (uint32_t)(te.offset >> 8) | (te.kind << 30);
    }
    fill_sel48(s_sel, (int)threadIdx.x, kPfWaves * 64);
    __syncthreads();
  }
  const int er = Q64 ? 2 * r_src + wn : r_src;  // this wave's entry row
  // the band stride of this wave's row-block (Q64: of its half), read by
  // each wave from its first table entry
  uint32_t stride = 0u;
  if constexpr (!SRC_ROWMAJOR)
    stride = (uint32_t)__builtin_amdgcn_readfirstlane((int)reinterpret_cast<const TileEntry*>(
        P.src + kHeaderBytes)[(int64_t)(Q64 ? 2 * (r_src ? i1 : i0) + wn : i_src) * KT + j0].band_stride);

  // this wave's kXC 8-row chunks of each X stage: rows 8 (kXC w + u) + l/8,
  // the lane fetching the source chunk whose swizzled position is l % 8;
  // rows past M read row M - 1 (their outputs are never stored).  Lane byte
  // offsets from row m0 of X (at most 256 K elements: 32 bits suffice).
  const uint8_t* const xrow0 = reinterpret_cast<const uint8_t*>(P.X + (int64_t)m0 * K);
  uint32_t xoff[kXC];
#pragma unroll
  for (int u = 0; u < kXC; u++) {
    const int row = 8 * (kXC * w + u) + (l >> 3);
    const int gm = min(m0 + row, M - 1);
    xoff[u] = 2u * (uint32_t)((gm - m0) * K + 8 * ((l & 7) ^ swz_f(row)));
  }
  const uint32_t w_lds = lds_addr(s_w), x_lds = lds_addr(s_x);
  // lane byte offsets of the W copies: a dense fragment half wm (or a 2:4
  // band's values, wm = 0) 16 bytes a lane, a 2:4 band's codes 4 bytes a lane;
  // row-major W: rows 64 wn + l % 16 (+ 16 b), columns 32 wm + 8 (l / 16) of
  // the step's 64 from the row-block's first row (at most 128 K elements)
  const uint32_t vw16 = 1024u * (uint32_t)wm + 16u * (uint32_t)l, vw4 = 4u * (uint32_t)l;
  const uint32_t vrm = 2u * (uint32_t)((64 * wn + (l & 15)) * K + 32 * wm + 8 * hl);
  const uint32_t vw16s[4] = {vw16, vw16, vw16, vw16}, vw4s[4] = {vw4, vw4, vw4, vw4};
  const uint32_t vrms[4] = {vrm, vrm, vrm, vrm};

  // the X copies of step s into X stage xst (= s % kXStages)
  auto issue_x = [&](int s, int xst) {
    const int col = (j0 + (s >> 1)) * kTile + 64 * (s & 1);
    const uint8_t* const base = xrow0 + 2 * (int64_t)col;
    const uint8_t* srcs[kXC];
#pragma unroll
    for (int u = 0; u < kXC; u++) srcs[u] = base;
    dma_n<kXC, 1024, true>(srcs, xoff, x_lds + (uint32_t)(xst * kLdsXStage) + 1024u * (uint32_t)(kXC * w));
  };
  // the W copies of step s into W stage wst (= s % kWStages); e_v: the tile
  // entry of step s for this wave's row-block (a VGPR loaded from LDS
  // earlier, so no LDS round trip sits between the step's barrier and its
  // copies)
  auto issue_w = [&](int s, int wst, uint32_t e_v) {
    const int jl = s >> 1, h = s & 1, j = j0 + jl;
    const uint32_t wb = w_lds + (uint32_t)(wst * kLdsWStage);
    const int col = j * kTile + 64 * h;
    // fragment slot of band 4wn + b, half e of row-block r: ((r*8 + 4wn + b)*2 + e) KB
    const uint32_t slot0 = wb + 1024u * (uint32_t)((r * 8 + 4 * wn) * 2);
    const uint8_t* srcs[4];
    if constexpr (SRC_ROWMAJOR) {
      // rows 16 (4wn + b) + l % 16 of row-block i_src, columns 64h + 32wm + 8(l/16) of tile j
      // (fused: row-block i_src/2 of the gate or the up matrix)
      const uint8_t* Wsrc = (FUSE && (i_src & 1)) ? P.src2 : P.src;
      const int ib = FUSE ? (i_src >> 1) : i_src;
      const uint8_t* const base = Wsrc + 2 * ((int64_t)ib * kTile * K + col);
#pragma unroll
      for (int b = 0; b < 4; b++) srcs[b] = base + (int64_t)32 * b * K;
      dma_n<4, 2048, true>(srcs, vrms, slot0 + 1024u * (uint32_t)wm);
    } else {
      const uint32_t e = (uint32_t)__builtin_amdgcn_readfirstlane((int)e_v);
      // the slice's kind, where its part starts in the band piece, where the codes are
      uint32_t sparse, part, codes;
      if constexpr (Q64) {
        const uint32_t kb = e >> 30, a1 = (kb & 1u) ? 1024u : 2048u;
        sparse = (kb >> h) & 1u;
        part = h ? a1 : 0u;
        codes = a1 + ((kb & 2u) ? 1024u : 2048u);
      } else {
        sparse = (e >> 30) != 0u;
        part = sparse ? 1024u * h : 2048u * h;
        codes = kSparseMetaOffset;
      }
      const uint8_t* const piece = P.src + ((uint64_t)(e & 0x3fffffffu) << 8) + (Q64 ? 0 : (uint64_t)(4 * wn) * stride);
      if (!sparse || wm == 0) {
        // a dense fragment half wm, or a 2:4 band's values
#pragma unroll
        for (int b = 0; b < 4; b++) srcs[b] = piece + (uint64_t)b * stride + part;
        dma_n<4, 2048, true>(srcs, vw16s, slot0 + 1024u * (uint32_t)wm);
      } else {
#pragma unroll
        for (int b = 0; b < 4; b++) srcs[b] = piece + (uint64_t)b * stride + codes;
        dma_n<4, 2048, false>(srcs, vw4s, slot0 + 1024u);
      }
    }
  };

  f32x4 acc[4][kNMB];
#pragma unroll
  for (int a = 0; a < 4; a++)
#pragma unroll
    for (int c = 0; c < kNMB; c++) acc[a][c] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto read_b = [&](const uint8_t* xs, int g, u32x4 (&blo)[kMG], u32x4 (&bhi)[kMG]) {
#pragma unroll
    for (int mm = 0; mm < kMG; mm++) {
      const int row = wm * (BM / 2) + (kMG * g + mm) * 16 + (l & 15);
      blo[mm] = *reinterpret_cast<const u32x4*>(xs + swz(row, hl));
      bhi[mm] = *reinterpret_cast<const u32x4*>(xs + swz(row, 4 + hl));
    }
  };
  // row-major W: B fragments of K half qq (32 columns), M blocks kRG p .. kRG p + kRG - 1
  // (parts at the larger widths: registers)
  constexpr int kRG = BM == 256 ? kNMB / 4 : (BM == 192 ? kNMB / 2 : kNMB);
  constexpr int kRParts = kNMB / kRG;
  auto read_bq = [&](const uint8_t* xs, int qq, int part, u32x4 (&bf)[kRG]) {
#pragma unroll
    for (int mm = 0; mm < kRG; mm++)
      bf[mm] = *reinterpret_cast<const u32x4*>(xs + swz(wm * (BM / 2) + (kRG * part + mm) * 16 + (l & 15), 4 * qq + hl));
  };
  auto x_stage = [&](int xi) { return s_x + xi * kLdsXStage; };
  // stage indices of the next step
  auto next_x = [](int xi) { return xi + 1 == kXStages ? 0 : xi + 1; };
  auto next_w = [](int wi) { return wi + 1 == kWStages ? 0 : wi + 1; };
  // the tile kind of step s (0 for row-major W)
  // (Q64: the kind of slice s & 1 of the entry's two)
  auto kind_of = [&](uint32_t ent, int s) -> uint32_t {
    if constexpr (Q64) return ((ent >> 30) >> (s & 1)) & 1u;
    return ent >> 30;
  };
  auto step_kind = [&](int s) -> uint32_t {
    if constexpr (SRC_ROWMAJOR) return 0u;
    return kind_of((uint32_t)__builtin_amdgcn_readfirstlane((int)s_ent[er][s >> 1]), s);
  };
  // this wave's tile entry of step s as a VGPR (an LDS load nobody waits
  // for until the value is used)
  auto ent_v = [&](int s) -> uint32_t {
    if constexpr (SRC_ROWMAJOR) return 0u;
    return s_ent[er][min(s, n_steps - 1) >> 1];
  };
  // this wave's A fragments of a step in W stage wi, 64-column half h, tile
  // kind `kind`: the first fragment a0 (a dense tile's first half, a 2:4 or
  // 4:8 tile's values); cw = the lane's 16-bit half h of word l of the band's
  // codes (mask) chunk, read whatever the kind (128 bytes a wave); a dense
  // tile's second half a1 only for a dense tile (a1 is written on that path
  // alone, so no wait for a read that did not happen lands on it)
  auto read_a = [&](int wi, int h, uint32_t kind, u32x4 (&a0)[4], u32x4 (&a1)[4], uint32_t (&cw)[4]) {
    const uint8_t* ws = s_w + wi * kLdsWStage + 1024 * ((r * 8 + 4 * wn) * 2);
#pragma unroll
    for (int b = 0; b < 4; b++) a0[b] = *reinterpret_cast<const u32x4*>(ws + 2048 * b + 16 * l);
    if constexpr (!SRC_ROWMAJOR) {
#pragma unroll
      for (int b = 0; b < 4; b++) cw[b] = *reinterpret_cast<const uint16_t*>(ws + 2048 * b + 1024 + 4 * l + 2 * h);
    }
    if (kind == 0) {
#pragma unroll
      for (int b = 0; b < 4; b++) a1[b] = *reinterpret_cast<const u32x4*>(ws + 2048 * b + 1024 + 16 * l);
    }
  };

  // ---- pipeline: X copies kXStages - 1 steps ahead, W copies kWStages - 1;
  // the fragments of step s + 1 are read from LDS while the last group of
  // step s's matrix instructions runs, so a step starts with its first
  // operands in registers
  constexpr int kXAhead = kXStages - 1, kWAhead = kWStages - 1;
  constexpr int kAhead = kXAhead > kWAhead ? kXAhead : kWAhead;
  // Every advance issues the copies of the ring that runs fewer steps ahead
  // first (X, also when both run as far), then the other's; kLater = the
  // copies issued after step s + 1's last one (step s + 2's), which may stay
  // in flight at step s's barrier
  constexpr bool kXFirst = kXAhead <= kWAhead;
  constexpr int kLater = (kXAhead == 2 ? kXC : 0) + (kWAhead == 2 ? 4 : 0);
  static_assert(kXAhead >= 1 && kWAhead >= 1 && kAhead <= 2 && kLater <= kLdsCopies, "copy pipeline");
  // called in step s (s + 1 < n_steps) once this wave's reads of stage s
  // are issued: step s + 1's copies have landed everywhere and nobody reads
  // stage s any more, which the copies of step s + 1 + kXAhead (X) and
  // s + 1 + kWAhead (W) then refill
  // (xi, wi: the X and W stages of step s, which the copies refill)
  // advance_wait: the wait and the barrier; advance_issue: the copies
  auto advance_wait = [&](int s) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage s are done
    if (kLater > 0 && s + 2 < n_steps)
      wait_copies<kLater>();  // step s + 2's copies may stay in flight
    else
      wait_copies<0>();
    wg_barrier();
  };
  auto advance_issue = [&](int s, int xi, int wi, uint32_t e_copy) {
    if (kXFirst && s + 1 + kXAhead < n_steps) issue_x(s + 1 + kXAhead, xi);
    if (s + 1 + kWAhead < n_steps) issue_w(s + 1 + kWAhead, wi, e_copy);
    if (!kXFirst && s + 1 + kXAhead < n_steps) issue_x(s + 1 + kXAhead, xi);
  };

  // packed W, step s: A fragments a0/a1 (kind), B group 0 in buffer par * G & 1
  // (the buffers alternate by group across steps; par = s & 1); reads step
  // s + 1's A fragments into na0/na1 and its B group 0 into the next buffer
  constexpr int kGroups = kNMB / kMG;
  auto step_packed = [&](int s, int par, int xi, int wi, u32x4 (&a0)[4], u32x4 (&a1)[4], uint32_t (&cw)[4],
                         uint32_t kind, u32x4 (&na0)[4], u32x4 (&na1)[4], uint32_t (&ncw)[4], uint32_t& nkind,
                         u32x4 (&blo)[2][kMG], u32x4 (&bhi)[2][kMG]) {
    const int h = s & 1;
    // step s + 1's entry (its kind: its fragments' addresses depend on it)
    // and that of the step whose copies this step issues, loaded now and
    // read after the step's barrier
    const uint32_t nk_v = ent_v(s + 1), ecopy_v = ent_v(s + 1 + kWAhead);
    if (!Q64 && kind == 2) {
      // 4:8: each band's sixteen columns rebuilt into a dense piece's two
      // halves (values in a0, the lane's masks in the codes chunk a1),
      // then run as a dense tile
#pragma unroll
      for (int b = 0; b < 4; b++) dense_halves48(a0[b], cw[b], s_sel, a0[b], a1[b]);
      kind = 0;
    }
    uint32_t idx0[4];
#pragma unroll
    for (int b = 0; b < 4; b++) idx0[b] = kind == 0 ? 0x4444u : cw[b];
    const uint8_t* xs = x_stage(xi);
    const int xn = next_x(xi), wn1 = next_w(wi);
#pragma unroll
    for (int g = 0; g < kGroups; g++) {
      const int cb = (g + par * kGroups) & 1, nb = (g + 1 + par * kGroups) & 1;
      const bool last = g + 1 == kGroups;
      if (last && s + 1 < n_steps) advance_wait(s);
      if (last) {
        // step s + 1's A fragments and first B fragments right after the
        // barrier, before this step's copies go out: the next step waits
        // for them (after the last step: a stage never used again)
        nkind = kind_of((uint32_t)__builtin_amdgcn_readfirstlane((int)nk_v), s + 1);
        read_a(wn1, h ^ 1, nkind, na0, na1, ncw);
        read_b(x_stage(xn), 0, blo[nb], bhi[nb]);
      }
      if (last && s + 1 < n_steps) advance_issue(s, xi, wi, ecopy_v);
      __builtin_amdgcn_sched_barrier(0);
      // the first half (a 2:4 tile's only one) with the next group's reads
      // -- or, in the last group, step s + 1's first fragments -- spread
      // between its matrix instructions.  (Waves without a row-block of
      // their own compute on row-block i0's copy and store nothing.)
#pragma unroll
      for (int mm = 0; mm < kMG; mm++)
#pragma unroll
        for (int b = 0; b < 4; b++)
          acc[b][kMG * g + mm] = mma_sparse<BF16, 0>(a0[b], blo[cb][mm], bhi[cb][mm], acc[b][kMG * g + mm], idx0[b]);
      if (!last) read_b(xs, g + 1, blo[nb], bhi[nb]);
      constexpr int kMma = 4 * kMG;
      constexpr int kPerMid = (2 * kMG + kMma - 1) / kMma, kPerLast = (2 * kMG + kMma - 1) / kMma;
      if (last) {
#pragma unroll
        for (int i = 0; i < kMma; i++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // one matrix instruction
          __builtin_amdgcn_sched_group_barrier(0x100, kPerLast, 0);  // then LDS reads
        }
      } else {
#pragma unroll
        for (int i = 0; i < kMma; i++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, kPerMid, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kind == 0) {
        // dense tile: the second half (positions 2, 3 of each group of four)
#pragma unroll
        for (int mm = 0; mm < kMG; mm++)
#pragma unroll
          for (int b = 0; b < 4; b++)
            acc[b][kMG * g + mm] = mma_sparse<BF16, 0>(a1[b], blo[cb][mm], bhi[cb][mm], acc[b][kMG * g + mm], 0xEEEEu);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // row-major W (the dense baseline), step s: K halves qq = 0, 1 on
  // v_mfma_f32_16x16x32, in groups g = (qq, part) whose B fragments
  // alternate between bq[0] and bq[1] (an even number of groups a step)
  auto step_rowmajor = [&](int s, int xi, int wi, u32x4 (&a0)[4], u32x4 (&a1)[4], u32x4 (&na0)[4],
                           u32x4 (&na1)[4], u32x4 (&bq)[2][kRG]) {
    const uint8_t* xs = x_stage(xi);
    uint32_t cw_unused[4];
#pragma unroll
    for (int g = 0; g < 2 * kRParts; g++) {
      const int qq = g / kRParts, part = g % kRParts;
      const bool last = g + 1 == 2 * kRParts;
      if (last && s + 1 < n_steps) {
        advance_wait(s);
        advance_issue(s, xi, wi, 0u);
      }
      if (last) read_a(next_w(wi), 0, 0u, na0, na1, cw_unused);  // step s + 1's A fragments first
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mm = 0; mm < kRG; mm++)
#pragma unroll
        for (int b = 0; b < 4; b++)
          acc[b][kRG * part + mm] = mma_dense<BF16>(qq ? a1[b] : a0[b], bq[g & 1][mm], acc[b][kRG * part + mm]);
      if (!last) {
        read_bq(xs, (g + 1) / kRParts, (g + 1) % kRParts, bq[(g + 1) & 1]);
      } else {
        read_bq(x_stage(next_x(xi)), 0, 0, bq[0]);
      }
      // the reads spread between the matrix instructions
      constexpr int kMma = 4 * kRG;
      constexpr int kPerMid = (kRG + kMma - 1) / kMma, kPerLast = (kRG + kMma - 1) / kMma;
      if (last) {
#pragma unroll
        for (int i = 0; i < kMma; i++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, kPerLast, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kMma; i++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, kPerMid, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // before step 0: the copies the advances of steps -kAhead - 1 .. -2 would
  // have issued (all exist: n_steps >= 2 >= kAhead), then step 0's wait and
  // barrier and what the advance of step -1 issues
#pragma unroll
  for (int t = -(kAhead + 1); t <= -2; t++) {
    if (kXFirst && t + 1 + kXAhead >= 0) issue_x(t + 1 + kXAhead, (t + 1 + kXAhead) % kXStages);
    if (t + 1 + kWAhead >= 0) issue_w(t + 1 + kWAhead, (t + 1 + kWAhead) % kWStages, ent_v(t + 1 + kWAhead));
    if (!kXFirst && t + 1 + kXAhead >= 0) issue_x(t + 1 + kXAhead, (t + 1 + kXAhead) % kXStages);
  }
  wait_copies<kLater>();
  wg_barrier();
  if (kXFirst && kXAhead < n_steps) issue_x(kXAhead, kXAhead);
  if (kWAhead < n_steps) issue_w(kWAhead, kWAhead, ent_v(kWAhead));
  if (!kXFirst && kXAhead < n_steps) issue_x(kXAhead, kXAhead);
  u32x4 fa0[4], fa1[4], fb0[4], fb1[4];
  uint32_t fac[4], fbc[4];
  uint32_t ka = step_kind(0), kb;
  read_a(0, 0, ka, fa0, fa1, fac);
  // stage indices of step s (X and W rings)
  int xi = 0, wi = 0;
  if constexpr (SRC_ROWMAJOR) {
    u32x4 bq[2][kRG];
    read_bq(x_stage(0), 0, 0, bq[0]);
    for (int s = 0; s < n_steps; s += 2) {  // n_steps is even
      step_rowmajor(s, xi, wi, fa0, fa1, fb0, fb1, bq);
      xi = next_x(xi), wi = next_w(wi);
      step_rowmajor(s + 1, xi, wi, fb0, fb1, fa0, fa1, bq);
      xi = next_x(xi), wi = next_w(wi);
    }
  } else {
    u32x4 blo[2][kMG], bhi[2][kMG];
    read_b(x_stage(0), 0, blo[0], bhi[0]);
    for (int s = 0; s < n_steps; s += 2) {  // n_steps is even
      step_packed(s, 0, xi, wi, fa0, fa1, fac, ka, fb0, fb1, fbc, kb, blo, bhi);
      xi = next_x(xi), wi = next_w(wi);
      step_packed(s + 1, 1, xi, wi, fb0, fb1, fbc, kb, fa0, fa1, fac, ka, blo, bhi);
      xi = next_x(xi), wi = next_w(wi);
    }
  }

  if constexpr (FUSE) {
    if (P.splits == 1) {
      fused_epilogue<BF16, OUT_F32, kNMB, 4>(acc, s_x, P.Y, M, P.N / 2, p, m0, r, wn, wm, l, BM / 2);
      return;
    }
  }
  if (!FUSE && tb >= 0) {
    // A tail block's ranges: lane l of wave w keeps its sums at f32x4 index
    // ((w * 4 + b) * kNMB + mblk) * 64 + l of a slot.  The slots are written
    // and read with the agent-coherent cache policy (sc1: the value every
    // XCD's L2 sees), so the hand-over needs no cache-wide write-back or
    // invalidation -- which would also evict what the other workgroups of
    // the XCD are streaming.  Order: a range's stores complete (vmcnt 0)
    // before its barrier and flag; range 0 loads after it has seen the
    // flags.
    const int slot0 = tb * (P.tail_s - 1);
    constexpr uint32_t kSlotBytes = 256u * BM * 4u;
    if (ks > 0) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(P.part + (int64_t)(slot0 + ks - 1) * (256 * BM), kSlotBytes);
#pragma unroll
      for (int b = 0; b < 4; b++)
#pragma unroll
        for (int mblk = 0; mblk < kNMB; mblk++)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[b][mblk]), rs,
                                                 16 * (((w * 4 + b) * kNMB + mblk) * 64 + l), 0, kCoherent);
      wait_copies<0>();
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_store(P.flags + slot0 + ks - 1, P.token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    // range 0: a bounded wait (one thread) that marks the block when it runs
    // out, so a missing range shows as NaN outputs rather than a hang; the
    // first barrier: every wave is done with the tile entries, whose first
    // word then carries the mark
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t late = 0;
      for (int q = 1; q < P.tail_s; q++) {
        uint64_t* f = P.flags + slot0 + q - 1;
        int spins = 0;
        while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != P.wait_token) {
          if (++spins > P.wait_polls) {
            late = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
        // back to 0 for the next launch (the sums are read below; the flag
        // is no longer needed)
        __hip_atomic_store(f, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      s_ent[0][0] = late;
    }
    __syncthreads();
    const bool late = s_ent[0][0] != 0;
    // the ranges' sums in range order, one band at a time (the loads of all
    // four at once would need as many registers again as the sums)
    for (int q = 1; q < P.tail_s; q++) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(P.part + (int64_t)(slot0 + q - 1) * (256 * BM), kSlotBytes);
#pragma unroll
      for (int b = 0; b < 4; b++) {
#pragma unroll
        for (int mblk = 0; mblk < kNMB; mblk++)
          acc[b][mblk] += __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (((w * 4 + b) * kNMB + mblk) * 64 + l), 0,
                                                           kCoherent));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (late) {
#pragma unroll
      for (int b = 0; b < 4; b++)
#pragma unroll
        for (int mblk = 0; mblk < kNMB; mblk++)
          acc[b][mblk] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }
  }
  void* Yp = P.Y;
  if (P.splits > 1) Yp = reinterpret_cast<float*>(P.Y) + (int64_t)ks * P.M * P.N;
  if (active) {
#pragma unroll
    for (int mblk = 0; mblk < kNMB; mblk++) {
      const int m = m0 + wm * (BM / 2) + mblk * 16 + (l & 15);
      if (m < M) {
#pragma unroll
        for (int b = 0; b < 4; b++) {
          const int64_t n = (int64_t)i_mine * kTile + 16 * (4 * wn + b) + 4 * hl;
          store4<BF16, OUT_F32>(Yp, (int64_t)m * P.N + n, acc[b][mblk]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Launch shape: the M-block width BM and the number of K ranges, chosen
// by a cost model of the LDS-staged kernel fitted to its measured times on
// the LLaMA-2 7B q_proj, gate_proj and down_proj shapes (32 <= M <= 2048,
// every width, 1 to 12 ranges; 5% rms error; its pick is the fastest
// measured choice on 25 of the 30 shapes and 1% slower on average):
//   t = rounds * (2.33 + tiles * (0.79 * (1 + 0.086 * fill) + 0.0072 * BM)) us
//       + with a split: 6.4 us + partial bytes / 3.24 TB/s (second kernel),
// rounds = ceil(workgroups / CUs), fill = the busy fraction of the CUs in a
// full round (a tile's W copy costs more when every CU streams at once),
// tiles = tile columns per K range.  A K
// range holds at least two tile columns, and the partial sums (ranges * M *
// N * 4 bytes) stay within 2 * N * K bytes.  Then the number of M-groups:
// each XCD (one L2) works on about 1/8 of the output blocks in the
// group-major order, i.e. on about (its share / M-blocks a group) row-block
// pairs times the M-blocks of one group, and its L2 fetches that many pairs'
// W and that many M-blocks' X.  Two groups come closest to the fewest bytes
// for such a split on the LLaMA-2 7B prefill shapes (gate/up: ~10 pairs x 6
// M-blocks an XCD; down: 8 pairs x 4 M-blocks), and measured as fast as four
// (within 1% on the 7B and 13B prefill shapes) with 30-40% fewer bytes
// fetched past the L2s; one group (every XCD reading all of X) was 3-10%
// slower.  With fewer than 4 M-blocks, one group.
struct PfShape {
  int bm, groups, splits, kt_split;
  bool lds;  // W and X staged through LDS (k_prefill_lds), else through registers (k_prefill)
  bool big;  // the kernel whose waves hold 128-row register tiles (k_prefill_big)
  int waves; // its waves a workgroup: 4 or 8
  // tail split (k_prefill_lds, splits = 1): n_full blocks whole, the rest
  // in tail_s K ranges (0: none)
  int tail_s = 0, n_full = 0;
};
static double shape_cost_us(int64_t M, int64_t N, int64_t K, int bm, int64_t splits, int64_t kt_split, int cus) {
  const int64_t pairs = (N / kTile + 1) / 2;
  const int64_t blocks = pairs * ((M + bm - 1) / bm) * splits;
  const int64_t rounds = (blocks + cus - 1) / cus;
  const double fill = (double)std::min<int64_t>(blocks, cus) / (double)cus;
  double t = (double)rounds * (2.33 + (double)kt_split * (0.79 * (1.0 + 0.086 * fill) + 0.0072 * bm));
  if (splits > 1) t += 6.4 + (double)splits * (double)M * (double)N * 4.0 / 3.24e6;
  return t;
}
// only_bm: consider that width alone (0: every width).
// The tail split at width bm: whole rounds of blocks as usual (R = the CUs
// rounded down to a multiple of 8 blocks a round), the blocks left over (too
// few to fill a round, or all of them when there are too few for one) each
// cut into S K ranges so that they fill one short round; a range hands its
// fp32 sums to the block's range 0 (the cost: the slots written and range 0
// reading them).  Returns -1 where it does not apply (no
// left-over blocks, too many to cut in two, or short ranges without a
// whole round).
static double tail_cost_us(int64_t M, int64_t N, int64_t K, int bm, int cus, int* n_full, int* tail_s,
                           int* kt_split) {
  const int64_t KT = K / kTile;
  const int64_t R = cus - cus % 8;
  const int64_t blocks = ((N / kTile + 1) / 2) * ((M + bm - 1) / bm);
  if (R < 8 || blocks % R == 0) return -1.0;
  const int64_t full = blocks / R * R, tail = blocks - full;
  int64_t S = std::min<int64_t>(R / tail, KT / 2);
  if (full == 0) {
    // no whole round: two ranges, and only long ones (measured: down_proj,
    // 43 tile columns a range, 3.7% faster than the split with its
    // reduction kernel; 16-column ranges of q_proj 4-40% slower)
    S = std::min<int64_t>(S, 2);
    if ((KT + 1) / 2 < 32) return -1.0;
  }
  if (S < 2) return -1.0;
  const int64_t kt = (KT + S - 1) / S;
  S = (KT + kt - 1) / kt;
  const double fill = (double)(tail * S) / (double)cus;
  // range 0 reads the other ranges' slots (256 x bm fp32 each) at about
  // 150 GB/s a CU
  const double t = (double)(full / R) * (2.33 + (double)KT * (0.79 * 1.086 + 0.0072 * bm)) + 2.33 +
                   (double)kt * (0.79 * (1.0 + 0.086 * fill) + 0.0072 * bm) + 1.0 +
                   (double)(S - 1) * 256.0 * bm * 4.0 / 1.5e5;
  *n_full = (int)full;
  *tail_s = (int)S;
  *kt_split = (int)kt;
  return t;
}

// Tests of the tail split's bounded wait (tail_wait_test): above 0, range 0
// of the launches that follow waits for a value no range stores, this many
// polls, and marks its block's outputs NaN.
static std::atomic<int> g_tail_test_polls{0};

void tail_wait_test(int polls) { g_tail_test_polls.store(polls > 0 ? polls : 0, std::memory_order_relaxed); }

// This launch's tail-split token: a counter mixed with a random salt
// drawn once per process (splitmix64's finaliser), never 0.  Stale or
// uninitialised flag words would have to equal a fresh 64-bit value to pass
// for it.
static uint64_t tail_token() {
  static const uint64_t salt = [] {
    std::random_device rd;
    return ((uint64_t)rd() << 32) ^ (uint64_t)rd();
  }();
  static std::atomic<uint64_t> counter{1};
  uint64_t z = salt + 0x9e3779b97f4a7c15ull * counter.fetch_add(1, std::memory_order_relaxed);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return z == 0 || z == ~0ull ? 1 : z;  // neither 0 (a cleared flag) nor ~0 (~token: the tests' value)
}

// Workspace bytes of a tail split: a slot of 256 x bm fp32 sums for every
// range but the first of every tail block, then their 8-byte flags
// (rounded to 256 bytes).
static uint64_t tail_ws_bytes(int64_t M, int64_t N, int bm, int n_full, int tail_s) {
  const int64_t blocks = ((N / kTile + 1) / 2) * ((M + bm - 1) / bm);
  const uint64_t slots = (uint64_t)(blocks - n_full) * (uint64_t)(tail_s - 1);
  return slots * 256u * (uint64_t)bm * 4u + (slots * 8u + 255u) / 256u * 256u;
}

// tail_ok: the tail split may be chosen (the LDS-staged kernel, not fused).
static PfShape choose_shape_uncached(int64_t M, int64_t N, int64_t K, int cus, int only_bm = 0,
                                     bool tail_ok = false) {
  const int64_t KT = K / kTile;
  const int widths[4] = {256, 192, 128, 64};
  const int wants[10] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32};
  const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(KT / 2, K / (2 * M)));
  PfShape best = {256, 1, 1, (int)KT, false, false, 4};
  double best_t = -1.0;
  for (int c = 0; c < 4; c++) {
    if (only_bm && widths[c] != only_bm) continue;
    for (int w = 0; w < 10 && wants[w] <= smax; w++) {
      const int64_t kt_split = (KT + wants[w] - 1) / wants[w];
      const int64_t splits = (KT + kt_split - 1) / kt_split;
      const double t = shape_cost_us(M, N, K, widths[c], splits, kt_split, cus);
      if (best_t < 0 || t < best_t) {
        best_t = t;
        best = {widths[c], 1, (int)splits, (int)kt_split, false, false, 4};
      }
    }
    if (tail_ok) {
      int n_full = 0, tail_s = 0, kt = 0;
      const double t = tail_cost_us(M, N, K, widths[c], cus, &n_full, &tail_s, &kt);
      if (t >= 0 && t < best_t) {
        best_t = t;
        best = {widths[c], 1, 1, kt, false, false, 4, tail_s, n_full};
      }
    }
  }
  const int64_t mblk = (M + best.bm - 1) / best.bm;
  while (best.groups < 2 && 2 * best.groups * 2 <= mblk) best.groups *= 2;
  return best;
}

// The same, remembered for the last few shapes of this thread (a GEMM call
// asks for it twice: the workspace query and the launch).  The LDS-staged
// kernel (k_prefill_lds) runs at every width: on the LLaMA-2 7B/13B prefill
// shapes it measured as fast as or faster than the register-staged kernel
// at each width -- 5-10% at width 64, 2-12% from 128 up for packed W, 20-45%
// for row-major W (the dense baseline).
static PfShape choose_shape(int64_t M, int64_t N, int64_t K, bool rowmajor, bool tail_ok = true) {
  struct Entry {
    int64_t M, N, K;
    int cus;
    bool rowmajor, tail_ok;
    PfShape sh;
  };
  constexpr int kSlots = 8;
  thread_local Entry cache[kSlots];
  thread_local int filled = 0, next = 0;
  const int cus = cu_count();
  for (int i = 0; i < filled; i++)
    if (cache[i].M == M && cache[i].N == N && cache[i].K == K && cache[i].cus == cus &&
        cache[i].rowmajor == rowmajor && cache[i].tail_ok == tail_ok)
      return cache[i].sh;
  PfShape sh = choose_shape_uncached(M, N, K, cus, 0, tail_ok);
  sh.lds = true;
  cache[next] = {M, N, K, cus, rowmajor, tail_ok, sh};
  next = (next + 1) % kSlots;
  if (filled < kSlots) filled++;
  return sh;
}

// Adds the fp32 partial sums of the K ranges in range order (so the result
// does not depend on which workgroup finished first) and rounds to Y.
template <bool BF16, bool OUT_F32>
__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ part, int splits, int64_t mn,
                                                      void* __restrict__ Y) {
  const int64_t q = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (q >= mn) return;
  f32x4 sum = *reinterpret_cast<const f32x4*>(part + q);
  for (int k = 1; k < splits; k++) sum += *reinterpret_cast<const f32x4*>(part + (int64_t)k * mn + q);
  store4<BF16, OUT_F32>(Y, q, sum);
}

// Fused gate/up: H[m][f .. f+3] = SiLU(gate) * up from the partial planes of
// the interleaved matrix (N = 2F columns: H column f of row-block f/128 is
// column 256 (f/128) + f%128 for gate and 128 further on for up).
template <bool BF16, bool OUT_F32>
__global__ __launch_bounds__(256) void k_split_reduce_fused(const float* __restrict__ part, int splits, int64_t M,
                                                            int64_t F, void* __restrict__ H) {
  const int64_t q = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (q >= M * F) return;
  const int64_t m = q / F, f = q - (q / F) * F;
  const int64_t N = 2 * F, mn = M * N;
  const int64_t gcol = m * N + 2 * kTile * (f / kTile) + f % kTile;
  f32x4 g = *reinterpret_cast<const f32x4*>(part + gcol);
  f32x4 u = *reinterpret_cast<const f32x4*>(part + gcol + kTile);
  for (int k = 1; k < splits; k++) {
    g += *reinterpret_cast<const f32x4*>(part + (int64_t)k * mn + gcol);
    u += *reinterpret_cast<const f32x4*>(part + (int64_t)k * mn + gcol + kTile);
  }
  store4<BF16, OUT_F32>(H, q, silu_mul(g, u));
}

hipError_t launch_prefill_big(bool bf16, bool rowmajor, bool out_f32, bool fuse, int bm, int waves, const PfArgs& a,
                              hipStream_t s);

// The fp32 partials of sh.splits K ranges in part -> Y (fused: H).
template <bool BF16, bool OUT_F32, bool FUSE>
static hipError_t launch_split_reduce(const float* part, int splits, int64_t M, int64_t N, void* Y, hipStream_t s) {
  if constexpr (FUSE) {
    const int64_t mf = M * (N / 2);
    hipLaunchKernelGGL((k_split_reduce_fused<BF16, OUT_F32>), dim3((unsigned)((mf / 4 + 255) / 256)), dim3(256), 0, s,
                       part, splits, M, N / 2, Y);
  } else {
    const int64_t mn = M * N;
    hipLaunchKernelGGL((k_split_reduce<BF16, OUT_F32>), dim3((unsigned)((mn / 4 + 255) / 256)), dim3(256), 0, s, part,
                       splits, mn, Y);
  }
  return hipGetLastError();
}

static PfArgs prefill_args(const void* src, const void* src2, const void* X, int64_t M, int64_t N, int64_t K, void* Y,
                           const PfShape& sh, float* part, int bm) {
  PfArgs a;
  a.src = reinterpret_cast<const uint8_t*>(src);
  a.src2 = reinterpret_cast<const uint8_t*>(src2);
  a.X = reinterpret_cast<const uint16_t*>(X);
  a.Y = sh.splits > 1 ? static_cast<void*>(part) : Y;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.NT = (int)(N / kTile);
  a.KT = (int)(K / kTile);
  a.n_mblk = (int)((M + bm - 1) / bm);
  a.n_pairs = (a.NT + 1) / 2;
  a.mg = (a.n_mblk + sh.groups - 1) / sh.groups;
  a.splits = sh.splits;
  a.kt_split = sh.kt_split;
  a.n_blocks = a.n_pairs * a.n_mblk * sh.splits;
  a.per_xcd = (a.n_blocks + 7) / 8;
  a.n_full = a.n_tail = a.tail_s = a.tail_per = 0;
  a.part = nullptr;
  a.flags = nullptr;
  a.token = a.wait_token = 0;
  a.wait_polls = 0;
  return a;
}

template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32, bool FUSE>
static hipError_t launch_big_t(const void* src, const void* src2, const void* X, int64_t M, int64_t N, int64_t K,
                               void* Y, const PfShape& sh, float* part, hipStream_t s) {
  const PfArgs a = prefill_args(src, src2, X, M, N, K, Y, sh, part, sh.bm);
  hipError_t e = launch_prefill_big(BF16, SRC_ROWMAJOR, OUT_F32, FUSE, sh.bm, sh.waves, a, s);
  if (e != hipSuccess || sh.splits == 1) return e;
  return launch_split_reduce<BF16, OUT_F32, FUSE>(part, sh.splits, M, N, Y, s);
}

template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32, bool FUSE, int BM, int DIST, bool LDS = false, bool Q64 = false>
static hipError_t launch_prefill_bm(const void* src, const void* src2, const void* X, int64_t M, int64_t N, int64_t K,
                                    void* Y, const PfShape& sh, float* part, hipStream_t s) {
  static_assert(!Q64 || LDS, "64 x 64 execution tiles run on the LDS-staged kernel");
  PfArgs a;
  a.src = reinterpret_cast<const uint8_t*>(src);
  a.src2 = reinterpret_cast<const uint8_t*>(src2);
  a.X = reinterpret_cast<const uint16_t*>(X);
  a.Y = sh.splits > 1 ? static_cast<void*>(part) : Y;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.NT = (int)(N / kTile);
  a.KT = (int)(K / kTile);
  a.n_mblk = (int)((M + BM - 1) / BM);
  a.n_pairs = (a.NT + 1) / 2;
  a.mg = (a.n_mblk + sh.groups - 1) / sh.groups;
  a.splits = sh.splits;
  a.kt_split = sh.kt_split;
  a.n_blocks = a.n_pairs * a.n_mblk * sh.splits;
  a.per_xcd = (a.n_blocks + 7) / 8;
  a.n_full = a.n_tail = a.tail_s = a.tail_per = 0;
  a.part = nullptr;
  a.flags = nullptr;
  a.token = a.wait_token = 0;
  a.wait_polls = 0;
  if constexpr (LDS && !FUSE) {
    if (sh.tail_s > 1) {
      // tail split: the slots, then the flags, in the workspace
      a.n_full = sh.n_full;
      a.n_tail = a.n_pairs * a.n_mblk - sh.n_full;
      a.tail_s = sh.tail_s;
      a.tail_per = (a.n_tail + 7) / 8;
      a.part = part;
      const int nf = a.n_tail * (sh.tail_s - 1);
      a.flags = reinterpret_cast<uint64_t*>(part + (int64_t)nf * 256 * BM);
      a.token = tail_token();
      // a test of the bounded wait makes range 0 wait for a value no range
      // stores, with a short limit (tail_wait_test)
      const int test_polls = g_tail_test_polls.load(std::memory_order_relaxed);
      a.wait_token = test_polls > 0 ? ~a.token : a.token;
      a.wait_polls = test_polls > 0 ? test_polls : kTailSpinLimit;
      // no whole blocks: range-major over per_xcd workgroups an XCD
      a.per_xcd = (sh.tail_s * a.n_tail + 7) / 8;
      const unsigned grid =
          (unsigned)(sh.n_full > 0 ? 8 * (sh.n_full / 8 + a.tail_per * sh.tail_s) : 8 * a.per_xcd);
      hipLaunchKernelGGL((k_prefill_lds<BF16, SRC_ROWMAJOR, OUT_F32, false, BM, Q64>), dim3(grid),
                         dim3(kPfWaves * 64), 0, s, a);
      return hipGetLastError();
    }
  }
  const dim3 grid((unsigned)(8 * a.per_xcd)), block(kPfWaves * 64);
  if (sh.splits > 1) {
    // fp32 partials of the K ranges, then the ordered reduction (fused:
    // SiLU(gate) * up) into Y
    if constexpr (LDS)
      hipLaunchKernelGGL((k_prefill_lds<BF16, SRC_ROWMAJOR, true, FUSE, BM, Q64>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((k_prefill<BF16, SRC_ROWMAJOR, true, BM, DIST, FUSE>), grid, block, 0, s, a);
    if constexpr (FUSE) {
      const int64_t mf = M * (N / 2);
      hipLaunchKernelGGL((k_split_reduce_fused<BF16, OUT_F32>), dim3((unsigned)((mf / 4 + 255) / 256)), dim3(256), 0,
                         s, part, sh.splits, M, N / 2, Y);
    } else {
      const int64_t mn = M * N;
      hipLaunchKernelGGL((k_split_reduce<BF16, OUT_F32>), dim3((unsigned)((mn / 4 + 255) / 256)), dim3(256), 0, s,
                         part, sh.splits, mn, Y);
    }
  } else if constexpr (LDS) {
    hipLaunchKernelGGL((k_prefill_lds<BF16, SRC_ROWMAJOR, OUT_F32, FUSE, BM, Q64>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((k_prefill<BF16, SRC_ROWMAJOR, OUT_F32, BM, DIST, FUSE>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// Launch shape of the big-tile kernel (k_prefill_big): the token-block
// width BM in {128, 192, 256} and the K split, from its time model
//   t = rounds * (c0 + tiles * c1 * BM / 256) + split cost (as above),
// rounds = ceil(workgroups / CUs): a 256 x BM block of output per
// workgroup, one workgroup per CU.  only_bm: that width alone.
static double big_cost_us(int64_t M, int64_t N, int64_t K, int bm, int64_t splits, int64_t kt_split, int cus) {
  const int64_t pairs = (N / kTile + 1) / 2;
  const int64_t blocks = pairs * ((M + bm - 1) / bm) * splits;
  const int64_t rounds = (blocks + cus - 1) / cus;
  double t = (double)rounds * (3.0 + (double)kt_split * 1.6 * (double)bm / 256.0);
  if (splits > 1) t += 6.4 + (double)splits * (double)M * (double)N * 4.0 / 3.24e6;
  return t;
}
constexpr int64_t kBigMaxKT = 256;  // tile columns a workgroup of the big-tile kernel keeps entries of
static PfShape choose_shape_big(int64_t M, int64_t N, int64_t K, int cus, int only_bm = 0, int waves = 4) {
  const int64_t KT = K / kTile;
  const int widths[3] = {256, 192, 128};
  const int wants[10] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32};
  const int64_t smin = (KT + kBigMaxKT - 1) / kBigMaxKT;
  const int64_t smax = std::max<int64_t>(smin, std::min<int64_t>(KT / 2, K / (2 * M)));
  PfShape best = {256, 1, (int)smin, (int)((KT + smin - 1) / smin), true, true, waves};
  double best_t = -1.0;
  for (int c = 0; c < 3; c++) {
    if (only_bm && widths[c] != only_bm) continue;
    if (waves == 8 && widths[c] == 192) continue;
    for (int w = 0; w < 10 && wants[w] <= smax; w++) {
      const int64_t kt_split = (KT + wants[w] - 1) / wants[w];
      const int64_t splits = (KT + kt_split - 1) / kt_split;
      if (kt_split > kBigMaxKT) continue;
      const double t = big_cost_us(M, N, K, widths[c], splits, kt_split, cus);
      if (best_t < 0 || t < best_t) {
        best_t = t;
        best = {widths[c], 1, (int)splits, (int)kt_split, true, true, waves};
      }
    }
  }
  const int64_t mblk = (M + best.bm - 1) / best.bm;
  while (best.groups < 4 && 2 * best.groups * 2 <= mblk) best.groups *= 2;
  return best;
}

// The shape for these sizes with the split limited to what the workspace
// holds (no workspace: no split).
static PfShape shape_for(int64_t M, int64_t N, int64_t K, bool rowmajor, uint64_t ws_bytes, int force_bm = 0,
                         bool force_lds = false, int force_big = 0, bool fuse = false) {
  PfShape sh;
  if (force_big) {
    sh = choose_shape_big(M, N, K, cu_count(), force_bm, force_big);
  } else if (force_bm) {
    sh = choose_shape_uncached(M, N, K, cu_count(), force_bm, force_lds && !fuse);
    sh.lds = force_lds;
  } else {
    sh = choose_shape(M, N, K, rowmajor, !fuse);
  }
  if (sh.tail_s > 1 && tail_ws_bytes(M, N, sh.bm, sh.n_full, sh.tail_s) > ws_bytes) {
    // no room for the tail split's slots: the best shape without it
    const bool lds = sh.lds;
    sh = force_bm ? choose_shape_uncached(M, N, K, cu_count(), force_bm, false) : choose_shape(M, N, K, rowmajor, false);
    sh.lds = lds;
  }
  const uint64_t plane = (uint64_t)M * (uint64_t)N * 4u;
  const int64_t KT = K / kTile;
  if (sh.splits > 1 && (uint64_t)sh.splits * plane > ws_bytes) {
    int64_t fit = (int64_t)(ws_bytes / plane);
    if (fit < 2) {
      sh.splits = 1;
      sh.kt_split = (int)KT;
    } else {
      sh.kt_split = (int)((KT + fit - 1) / fit);
      sh.splits = (int)((KT + sh.kt_split - 1) / sh.kt_split);
    }
  }
  if (sh.big && sh.kt_split > kBigMaxKT) {
    // the big-tile kernel keeps at most kBigMaxKT tile columns a range and
    // the workspace allows no split that short: the 8-wave kernel
    PfShape lds = choose_shape(M, N, K, rowmajor, false);
    lds.lds = true;
    lds.splits = 1;
    lds.kt_split = (int)KT;
    return lds;
  }
  return sh;
}

// Room for the shape with the tail split and for the one without (the
// fused product runs without it).
uint64_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K, bool rowmajor) {
  uint64_t b = 0;
  for (int tail_ok = 0; tail_ok < 2; tail_ok++) {
    const PfShape sh = choose_shape(M, N, K, rowmajor, tail_ok != 0);
    if (sh.splits > 1) b = std::max<uint64_t>(b, (uint64_t)sh.splits * (uint64_t)M * (uint64_t)N * 4u);
    if (sh.tail_s > 1) b = std::max<uint64_t>(b, tail_ws_bytes(M, N, sh.bm, sh.n_full, sh.tail_s));
  }
  return b;
}

// The cost model's time for the shape this workspace allows.
double prefill_estimate_us(int64_t M, int64_t N, int64_t K, bool rowmajor, uint64_t ws_bytes) {
  const PfShape sh = shape_for(M, N, K, rowmajor, ws_bytes);
  if (sh.tail_s > 1) {
    int n_full = 0, tail_s = 0, kt = 0;
    return tail_cost_us(M, N, K, sh.bm, cu_count(), &n_full, &tail_s, &kt);
  }
  return shape_cost_us(M, N, K, sh.bm, sh.splits, sh.kt_split, cu_count());
}

template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32, bool FUSE>
static hipError_t launch_prefill_t(const void* src, const void* src2, const void* X, int64_t M, int64_t N, int64_t K,
                                   void* Y, void* ws, uint64_t ws_bytes, int force_bm, bool force_lds, int force_big,
                                   hipStream_t s) {
  const PfShape sh = shape_for(M, N, K, SRC_ROWMAJOR, ws ? ws_bytes : 0u, force_bm, force_lds, force_big, FUSE);
  float* part = reinterpret_cast<float*>(ws);
  if (sh.big) return launch_big_t<BF16, SRC_ROWMAJOR, OUT_F32, FUSE>(src, src2, X, M, N, K, Y, sh, part, s);
#define PATCH_BM(W, D, L) \
  launch_prefill_bm<BF16, SRC_ROWMAJOR, OUT_F32, FUSE, W, D, L>(src, src2, X, M, N, K, Y, sh, part, s)
  if (sh.lds) {
    switch (sh.bm) {
      case 64: return PATCH_BM(64, 1, true);
      case 128: return PATCH_BM(128, 1, true);
      case 192: return PATCH_BM(192, 1, true);
      case 256: return PATCH_BM(256, 1, true);
      default: return hipErrorInvalidValue;
    }
  }
  switch (sh.bm) {
    case 64: return PATCH_BM(64, 2, false);
    case 128: return PATCH_BM(128, 2, false);
    case 192: return PATCH_BM(192, 1, false);
    default: return PATCH_BM(256, 1, false);
  }
#undef PATCH_BM
}

// A blob of 64 x 64 execution tiles: the LDS-staged kernel at the width the
// cost model picks (or force_bm), its per-half entries and per-slice kinds.
template <bool BF16, bool OUT_F32>
static hipError_t launch_prefill_q64_t(const void* src, const void* X, int64_t M, int64_t N, int64_t K, void* Y,
                                       void* ws, uint64_t ws_bytes, int force_bm, hipStream_t s) {
  const PfShape sh = shape_for(M, N, K, false, ws ? ws_bytes : 0u, force_bm, true, 0);
  float* part = reinterpret_cast<float*>(ws);
#define PATCH_BQ(W) launch_prefill_bm<BF16, false, OUT_F32, false, W, 1, true, true>(src, nullptr, X, M, N, K, Y, sh, part, s)
  switch (sh.bm) {
    case 64: return PATCH_BQ(64);
    case 128: return PATCH_BQ(128);
    case 192: return PATCH_BQ(192);
    case 256: return PATCH_BQ(256);
    default: return hipErrorInvalidValue;
  }
#undef PATCH_BQ
}

// force_bm: 0 (the shape the cost model picks) or a width in {64, 128, 192,
// 256}; force_lds: LDS staging (any of those widths).  src2 non-null: fused
// gate/up (src2 = the up matrix when rowmajor; for a packed blob the two are
// interleaved in src and src2 is src); Y is then H, M x N/2.  q64: a blob of
// 64 x 64 execution tiles (packed, not fused; LDS-staged kernel only).
hipError_t launch_prefill(bool bf16, bool rowmajor, bool out_f32, const void* src, const void* src2, const void* X,
                          int64_t M, int64_t N, int64_t K, void* Y, void* ws, uint64_t ws_bytes, int force_bm,
                          bool force_lds, int force_big, bool q64, hipStream_t s) {
  if (K / kTile > kPfMaxKT) return hipErrorInvalidValue;
  if (q64) {
    if (rowmajor || src2 || force_big) return hipErrorInvalidValue;
    if (force_bm && force_bm != 64 && force_bm != 128 && force_bm != 192 && force_bm != 256)
      return hipErrorInvalidValue;
    if (bf16)
      return out_f32 ? launch_prefill_q64_t<true, true>(src, X, M, N, K, Y, ws, ws_bytes, force_bm, s)
                     : launch_prefill_q64_t<true, false>(src, X, M, N, K, Y, ws, ws_bytes, force_bm, s);
    return out_f32 ? launch_prefill_q64_t<false, true>(src, X, M, N, K, Y, ws, ws_bytes, force_bm, s)
                   : launch_prefill_q64_t<false, false>(src, X, M, N, K, Y, ws, ws_bytes, force_bm, s);
  }
  if (force_bm && force_bm != 64 && force_bm != 128 && force_bm != 192 && force_bm != 256) return hipErrorInvalidValue;
  if (force_lds && force_bm < 64) return hipErrorInvalidValue;
  if (force_big && force_bm != 0 && force_bm < 128) return hipErrorInvalidValue;
  if (force_big == 8 && force_bm == 192) return hipErrorInvalidValue;
  const bool fuse = src2 != nullptr;
  if (fuse && (N % (2 * kTile))) return hipErrorInvalidValue;
#define PATCH_PF(B, R, F, U) \
  launch_prefill_t<B, R, F, U>(src, src2, X, M, N, K, Y, ws, ws_bytes, force_bm, force_lds, force_big, s)
#define PATCH_PF2(B, R, F) (fuse ? PATCH_PF(B, R, F, true) : PATCH_PF(B, R, F, false))
  if (bf16) {
    if (rowmajor) return out_f32 ? PATCH_PF2(true, true, true) : PATCH_PF2(true, true, false);
    return out_f32 ? PATCH_PF2(true, false, true) : PATCH_PF2(true, false, false);
  }
  if (rowmajor) return out_f32 ? PATCH_PF2(false, true, true) : PATCH_PF2(false, true, false);
  return out_f32 ? PATCH_PF2(false, false, true) : PATCH_PF2(false, false, false);
#undef PATCH_PF2
#undef PATCH_PF
}

}  // namespace patch
