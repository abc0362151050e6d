// gemm_prefill_big.hip -- hybrid GEMM for many tokens on large per-wave
// register tiles (the matrix-core-bound case, M in the hundreds and up).
//
// PATCH (arXiv 2509.23410), gist.science explainer, section 2 "Inference &
// Deployment": dense tiles run on the dense matrix path and 2:4 tiles on the
// sparse one.  A 2:4 tile runs at twice the dense rate on the sparse matrix
// instruction, so its operands must reach the matrix cores twice as fast per
// flop; what limits the kernel is then the bytes read from LDS per flop,
// which only the size of each wave's register tile lowers:
//
//   * A workgroup is 4 waves (one per SIMD, 512 registers a lane: the fp32
//     accumulators take up to 256 of them) and owns TWO row-blocks of W --
//     p and NT-1-p, or gate row-block 2p and up row-block 2p+1 when fused --
//     times BM tokens (BM = 128, 192 or 256): a 256 x BM block of Y^T.
//   * Wave w holds bands 4*(w>>1) .. +3 of BOTH row-blocks (128 rows of W)
//     times BM/2 tokens (w & 1): 2 x 4 x BM/32 accumulators of 16 x 16.
//     Per 64-column step it reads 128 rows of A and BM/2 rows of B from LDS
//     (twice the rows of either operand of an 8-wave layout for the same
//     flops), and because every wave covers both row-blocks, a step whose
//     two tiles differ in kind costs every wave the same: no wave waits for
//     another's dense tile at the barrier.
//   * Both tile kinds run on v_smfmac_f32_16x16x64: a 2:4 slice once with its
//     index codes, a dense slice as its two fixed-pattern halves (positions
//     (0,1) and (2,3) of every group of four, codes 0x4444 and 0xEEEE).  The
//     step body is instantiated for the four (dense?, dense?) kind pairs, so
//     the choice of kind costs no branch inside the matrix-instruction
//     stream.  4:8 tiles are rebuilt into dense halves in registers at the
//     start of their step and run as dense.
//   * W pieces and X rows come into LDS by global -> LDS copies
//     (global_load_lds_dwordx4, 16 bytes a lane), kStages-1 steps ahead of
//     use in a ring of 2 or 3 stages; every wave issues the same number of
//     copies a step whatever the kinds (2:4 and 4:8 bands copy their values
//     and their codes, dense bands their two halves), so each wave waits for
//     its own copies with an exact vmcnt and one barrier a step publishes
//     everyone's.  X rows (and the rows of row-major W) are XOR-swizzled by
//     16-byte chunk, so fragment reads hit distinct banks.
//   * The next step's A fragments and first B fragments are read from LDS
//     under the last group of matrix instructions of the current step (the
//     step's barrier sits just before that group); within a group the next
//     group's B reads are spread between the matrix instructions.
//
// With SRC_ROWMAJOR the same kernel reads plain row-major W, staged like X,
// with every tile dense on v_mfma_f32_16x16x32: the same-shape dense
// baseline.
#include "prefill_common.h"

namespace patch {

constexpr int kBgWStage = 32768;  // 2 row-blocks x 8 bands x 2 slots of 1 KB (row-major W: 256 rows x 128 B)
constexpr int kBgEntRegs = 4;                 // tile-entry registers a row-block (64 tile columns each)
constexpr int kBgMaxKT = 64 * kBgEntRegs;     // tile columns a workgroup can hold entries of
static_assert(kBgMaxKT == 256, "the launcher gives this kernel K ranges of at most 256 tile columns");

// WAVES = 4 (one a SIMD: waves = 2 band halves x 2 token halves) or 8 (two
// a SIMD: 2 band halves x 4 token quarters).  Every wave holds its band
// half of BOTH row-blocks.
template <int BM, int WAVES>
struct BigCfg {
  static constexpr int kTQ = WAVES / 2;                 // token parts
  static constexpr int kTok = BM / kTQ;                 // tokens a wave
  static constexpr int kNMB = kTok / 16;                // 16-token blocks a wave
  static constexpr int kXStage = BM * kPfRowBytes;      // X rows of one step
  static constexpr int kStages = BM <= 128 ? 3 : 2;     // LDS ring (a third stage does not fit above 128)
  static constexpr int kXC = BM / (8 * WAVES);          // 1 KB X chunks a wave copies a step
  static constexpr int kWB = 16 / WAVES;                // bands of its row-block a wave copies a step
  static constexpr int kWC = 32 / WAVES;                // 1 KB row-major W chunks a wave copies a step
  static constexpr int kCopies = 2 * kWB + kXC;         // copies a wave issues a step
  static_assert(kXC * 8 * WAVES == BM && kNMB * 16 == kTok, "tile shape");
};

// A fragments of one step: a[rb][b][0] = values (2:4) or half 0 (dense),
// a[rb][b][1] = the 16 bytes holding the lane's code word (2:4, 4:8) or
// half 1 (dense); row-major W: the two 32-column K halves.
struct BigA {
  u32x4 a[2][4][2];
};

// The matrix instructions with their accumulator in AGPRs.  They are
// written out because the compiler, given 2 x 4 x BM/32 accumulators and a
// branch around the dense tiles' second halves, keeps choosing the
// instructions' VGPR form and copies every accumulator between the register
// files around each one.  Hazards the compiler cannot see inside asm are
// covered here: "s_nop 1" before each instruction gives its operands two
// wait states after any vector-ALU write (operands loaded from LDS are
// covered by the compiler's lgkmcnt waits, which it inserts for asm inputs
// too); the accumulators are only read by vector instructions after
// acc_drain(); uses of one accumulator are always at least four matrix
// instructions apart.
template <bool BF16>
__device__ __forceinline__ void smfmac_acc(f32x4& acc, u32x4 a, u32x4 blo, u32x4 bhi, uint32_t idx) {
  const u32x8 b = {blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
  if constexpr (BF16)
    asm volatile("s_nop 1\n\tv_smfmac_f32_16x16x64_bf16 %0, %1, %2, %3" : "+a"(acc) : "v"(a), "v"(b), "v"(idx));
  else
    asm volatile("s_nop 1\n\tv_smfmac_f32_16x16x64_f16 %0, %1, %2, %3" : "+a"(acc) : "v"(a), "v"(b), "v"(idx));
}
template <bool BF16>
__device__ __forceinline__ void mfma_acc(f32x4& acc, u32x4 a, u32x4 b) {
  if constexpr (BF16)
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last matrix instruction and vector reads of its
// result (more than the longest instruction here needs).
__device__ __forceinline__ void acc_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32, bool FUSE, int BM, int WAVES>
__global__ __launch_bounds__(WAVES * 64, 1) void k_prefill_big(PfArgs P) {
  using C = BigCfg<BM, WAVES>;
  constexpr int kBgWaves = WAVES, kTQ = C::kTQ, kTok = C::kTok, kWB = C::kWB, kWC = C::kWC;
  constexpr int kNMB = C::kNMB, kStages = C::kStages, kXC = C::kXC, kXStage = C::kXStage;
  constexpr int kAhead = kStages - 1;
  static_assert(kNMB % 2 == 0, "an even number of token blocks a wave (B buffers alternate by group)");
  __shared__ __attribute__((aligned(1024))) uint8_t s_w[kStages * kBgWStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s_x[kStages * kXStage];
  // per row-block of the pair and tile column: (byte offset >> 8) | kind << 30
  __shared__ u32x4 s_sel[SRC_ROWMAJOR ? 1 : 256];  // 4:8 rebuild selectors

  // output blocks in order: K range, M-group, row-block pair, M-block; XCD x
  // (workgroups are dealt to the 8 XCDs in turn) takes the x-th eighth
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
  const int wm = w % kTQ, wn = w / kTQ;  // token part, band half (of both row-blocks)
  const int hl = l >> 4;
  const int KT = P.KT, K = P.K, M = P.M;
  const int m0 = mb * BM;
  const int i0 = FUSE ? 2 * p : p, i1 = FUSE ? 2 * p + 1 : P.NT - 1 - p;
  const bool second = FUSE || i1 != i0;  // a lone middle row-block: the second half repeats it, unstored
  const int j0 = ks * P.kt_split;
  const int nt = min(P.kt_split, KT - j0);
  const int n_steps = 2 * nt;

  // Tile entries of the two row-blocks, (byte offset >> 8) | kind << 30, in
  // registers: lane t of ev[rb][q] holds tile column j0 + 64 q + t of
  // row-block rb, so a step reads its entries with v_readlane (scalar
  // latency) instead of an LDS round trip.  Up to kBgMaxKT tile columns a
  // workgroup (the launcher splits K beyond).
  uint32_t ev[2][kBgEntRegs];
  uint32_t stride_rb[2] = {0u, 0u};
  if constexpr (!SRC_ROWMAJOR) {
    const TileEntry* table = reinterpret_cast<const TileEntry*>(P.src + kHeaderBytes);
#pragma unroll
    for (int rb = 0; rb < 2; rb++) {
      const TileEntry* row = table + (int64_t)(rb ? i1 : i0) * KT + j0;
#pragma unroll
      for (int q = 0; q < kBgEntRegs; q++) {
        const int j = min(64 * q + l, nt - 1);
        const u32x4 te = ld16(row + j);
        ev[rb][q] = (uint32_t)((((uint64_t)te[1] << 32) | te[0]) >> 8) | (te[2] << 30);
        if (q == 0) stride_rb[rb] = (uint32_t)__builtin_amdgcn_readfirstlane((int)te[3]);
      }
    }
    fill_sel48(s_sel, (int)threadIdx.x, kBgWaves * 64);
    __syncthreads();
  }
  // the entry of tile column jl (0 .. nt-1) of row-block rb
  auto entry = [&](int rb, int jl) -> uint32_t {
    uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)ev[rb][0], jl & 63);
#pragma unroll
    for (int q = 1; q < kBgEntRegs; q++)
      if ((jl >> 6) == q) e = (uint32_t)__builtin_amdgcn_readlane((int)ev[rb][q], jl & 63);
    return e;
  };

  // copies: wave w brings bands cb .. cb+3 of row-block cr (both slots of
  // each) and X rows 8 (kXC w + u) + l/8, u < kXC, the lane fetching the
  // source chunk whose swizzled position is l % 8; rows past M read row
  // M - 1 (their outputs are never stored)
  const int cr = w / (WAVES / 2), cb = kWB * (w % (WAVES / 2));
  const uint32_t cstride = stride_rb[cr];
  const uint16_t* xsrc[kXC];
#pragma unroll
  for (int u = 0; u < kXC; u++) {
    const int row = 8 * (kXC * w + u) + (l >> 3);
    const int gm = min(m0 + row, M - 1);
    xsrc[u] = P.X + (int64_t)gm * K + 8 * ((l & 7) ^ swz_f(row));
  }
  // row-major W: staged rows r = 0..255 (row-block i0, then i1), wave w
  // copying rows 64 w .. 64 w + 63 in 8-row chunks
  const uint16_t* wsrc[SRC_ROWMAJOR ? kWC : 1];
  if constexpr (SRC_ROWMAJOR) {
#pragma unroll
    for (int u = 0; u < kWC; u++) {
      const int r = 8 * (kWC * w + u) + (l >> 3);
      const int rb = r >> 7;
      const uint8_t* Wm = (FUSE && rb) ? P.src2 : P.src;
      const int ib = FUSE ? p : (rb ? i1 : i0);
      wsrc[u] = reinterpret_cast<const uint16_t*>(Wm) + ((int64_t)ib * kTile + (r & 127)) * K +
                8 * ((l & 7) ^ swz_f(r));
    }
  }
  const uint32_t w_lds = lds_addr(s_w), x_lds = lds_addr(s_x);

  auto issue = [&](int s) {
    const int st = s % kStages;
    const int jl = s >> 1, h = s & 1;
    const int col = (j0 + jl) * kTile + 64 * h;
    const uint32_t wb = w_lds + (uint32_t)(st * kBgWStage), xb = x_lds + (uint32_t)(st * kXStage);
#pragma unroll
    for (int u = 0; u < kXC; u++) dma16(xsrc[u] + col, xb + 1024u * (uint32_t)(kXC * w + u));
    if constexpr (SRC_ROWMAJOR) {
#pragma unroll
      for (int u = 0; u < kWC; u++) dma16(wsrc[u] + col, wb + 1024u * (uint32_t)(kWC * w + u));
    } else {
      const uint32_t e = entry(cr, jl);
      const uint8_t* piece = P.src + ((uint64_t)(e & 0x3fffffffu) << 8) + (uint64_t)cb * cstride;
      const uint32_t slot = wb + 1024u * (uint32_t)((cr * 8 + cb) * 2);
      if ((e >> 30) == 0) {
#pragma unroll
        for (int b = 0; b < kWB; b++) {
          const uint8_t* pb = piece + (uint64_t)b * cstride + 2048 * h + 16 * l;
          dma16(pb, slot + 2048u * b);
          dma16(pb + 1024, slot + 2048u * b + 1024u);
        }
      } else {
#pragma unroll
        for (int b = 0; b < kWB; b++) {
          const uint8_t* pb = piece + (uint64_t)b * cstride;
          dma16(pb + 1024 * h + 16 * l, slot + 2048u * b);
          dma4(pb + kSparseMetaOffset + 4 * l, slot + 2048u * b + 1024u);
        }
      }
    }
  };

  f32x4 acc[2][4][kNMB];
#pragma unroll
  for (int rb = 0; rb < 2; rb++)
#pragma unroll
    for (int b = 0; b < 4; b++)
#pragma unroll
      for (int c = 0; c < kNMB; c++) {
        acc[rb][b][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
        asm volatile("" : "+a"(acc[rb][b][c]));  // loop-carried in AGPRs, where the matrix instructions use them
      }

  auto w_stage = [&](int s) { return s_w + (s % kStages) * kBgWStage; };
  auto x_stage = [&](int s) { return s_x + (s % kStages) * kXStage; };
  // the kind of row-block rb's tile in step s (0 for row-major W)
  auto kind_of = [&](int s, int rb) -> uint32_t {
    if constexpr (SRC_ROWMAJOR) return 0u;
    return entry(rb, s >> 1) >> 30;
  };
  // B fragments of token block g of this wave from stage xs (the K halves
  // 0..31 and 32..63 of the 64-column step)
  auto read_blo = [&](const uint8_t* xs, int g) {
    return *reinterpret_cast<const u32x4*>(xs + swz(wm * kTok + 16 * g + (l & 15), hl));
  };
  auto read_bhi = [&](const uint8_t* xs, int g) {
    return *reinterpret_cast<const u32x4*>(xs + swz(wm * kTok + 16 * g + (l & 15), 4 + hl));
  };
  // row-block rb's A fragments of step s (tile kind k) into A.a[rb]
  auto read_a = [&](int s, int rb, uint32_t k, BigA& A) {
    const uint8_t* ws = w_stage(s);
#pragma unroll
    for (int b = 0; b < 4; b++) {
      if constexpr (SRC_ROWMAJOR) {
        const int r = rb * 128 + 16 * (4 * wn + b) + (l & 15);
        A.a[rb][b][0] = *reinterpret_cast<const u32x4*>(ws + swz(r, hl));
        A.a[rb][b][1] = *reinterpret_cast<const u32x4*>(ws + swz(r, 4 + hl));
      } else {
        const uint8_t* slot = ws + 1024 * ((rb * 8 + 4 * wn + b) * 2);
        A.a[rb][b][0] = *reinterpret_cast<const u32x4*>(slot + 16 * l);
        A.a[rb][b][1] = *reinterpret_cast<const u32x4*>(slot + 1024 + (k ? 16 * (l >> 2) : 16 * l));
      }
    }
  };
  // row-block rb's codes for step s (2:4: the lane's 16 bits of this 64-column
  // half; dense and 4:8: the dense halves' fixed code); a 4:8 band is rebuilt
  // into a dense piece's two halves first
  auto prologue = [&](int s, int rb, uint32_t k, BigA& A, uint32_t (&idx)[4]) {
    const int h = s & 1;
    // the previous step's last matrix instructions may still read their
    // code registers, which the ones computed here may reuse
    asm volatile("s_nop 7" ::: "memory");
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const u32x4 mc = A.a[rb][b][1];
      const uint32_t lo = (l & 1) ? mc[1] : mc[0], hi = (l & 1) ? mc[3] : mc[2];
      const uint32_t word = ((l & 2) ? hi : lo) >> (16 * h);
      if (k == 2) dense_halves48(A.a[rb][b][0], word & 0xffffu, s_sel, A.a[rb][b][0], A.a[rb][b][1]);
      idx[b] = k == 1 ? word : 0x4444u;
    }
  };

  // once this wave's reads of stage s are issued (s + 1 < n_steps): step
  // s + 1's copies have landed everywhere and nobody reads stage s any
  // more, which the copies of step s + 1 + kAhead then refill
  auto advance = [&](int s) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage s are done
    if (kAhead == 2 && s + 2 < n_steps)
      wait_copies<C::kCopies>();  // step s + 2's copies may stay in flight
    else
      wait_copies<0>();
    wg_barrier();
    if (s + 1 + kAhead < n_steps) issue(s + 1 + kAhead);
  };

  // One step.  A holds the step's A fragments on entry (read during the
  // previous step) and the next step's on exit; bl/bh[0] hold the B
  // fragments of token block 0.  Order, kept by scheduling barriers: within
  // a group, the first halves (one matrix instruction per row-block and
  // band) with the next group's B read after the second and fourth, then
  // the dense row-blocks' second halves; in the last group, after the
  // step's barrier, the next step's first B, then per row-block its
  // matrix instructions followed by the reads of its next A fragments (its
  // registers are free once its last instruction has issued).
  auto step = [&](int s, BigA& A, u32x4 (&bl)[2], u32x4 (&bh)[2]) {
    const uint8_t* xs = x_stage(s);
    const uint32_t k0 = kind_of(s, 0), k1 = kind_of(s, 1);
    const bool d0 = k0 != 1, d1 = k1 != 1;
    const bool more = s + 1 < n_steps;
    const int sn = more ? s + 1 : s;
    uint32_t idx[2][4];
#pragma unroll
    for (int g = 0; g < kNMB; g++) {
      const int c = g & 1, n = c ^ 1;
      const bool last = g + 1 == kNMB;
      if (last) {
        if (more) advance(s);
        if (more) {
          bl[n] = read_blo(x_stage(sn), 0);
          bh[n] = read_bhi(x_stage(sn), 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int rb = 0; rb < 2; rb++) {
        if constexpr (!SRC_ROWMAJOR) {
          if (g == 0) prologue(s, rb, rb ? k1 : k0, A, idx[rb]);
        }
#pragma unroll
        for (int b = 0; b < 4; b++) {
          if constexpr (SRC_ROWMAJOR) {
            mfma_acc<BF16>(acc[rb][b][g], A.a[rb][b][0], bl[c]);
          } else {
            smfmac_acc<BF16>(acc[rb][b][g], A.a[rb][b][0], bl[c], bh[c], idx[rb][b]);
          }
          if (!last && rb == 0 && b == 1) bl[n] = read_blo(xs, g + 1);
          if (!last && rb == 0 && b == 3) bh[n] = read_bhi(xs, g + 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (SRC_ROWMAJOR) {
#pragma unroll
          for (int b = 0; b < 4; b++) {
            mfma_acc<BF16>(acc[rb][b][g], A.a[rb][b][1], bh[c]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          if (rb ? d1 : d0) {
#pragma unroll
            for (int b = 0; b < 4; b++)
              smfmac_acc<BF16>(acc[rb][b][g], A.a[rb][b][1], bl[c], bh[c], 0xEEEEu);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (last && more) {
          read_a(sn, rb, kind_of(sn, rb), A);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  // ---- pipeline
#pragma unroll
  for (int s = 0; s < kAhead; s++) issue(s);  // n_steps >= 2 >= kAhead
  if (kAhead == 2)
    wait_copies<C::kCopies>();
  else
    wait_copies<0>();
  wg_barrier();
  if (kAhead < n_steps) issue(kAhead);
  BigA fa;
  u32x4 bl[2], bh[2];
  read_a(0, 0, kind_of(0, 0), fa);
  read_a(0, 1, kind_of(0, 1), fa);
  bl[0] = read_blo(x_stage(0), 0);
  bh[0] = read_bhi(x_stage(0), 0);
  for (int s = 0; s < n_steps; s += 2) {  // n_steps is even; kNMB is even, so B starts in buffer 0 each step
    step(s, fa, bl, bh);
    step(s + 1, fa, bl, bh);
  }

  acc_drain();
  // ---- epilogue: fp32 sums -> Y (rounded to nearest even for 16-bit Y),
  // fp32 partials of this K range, or the fused H = SiLU(gate) * up
  const int mw = m0 + wm * kTok + (l & 15);
  if constexpr (FUSE) {
    if (P.splits == 1) {
      const int F = P.N / 2;
#pragma unroll
      for (int g = 0; g < kNMB; g++) {
        const int m = mw + 16 * g;
        if (m < M) {
#pragma unroll
          for (int b = 0; b < 4; b++) {
            const int64_t n = (int64_t)p * kTile + 16 * (4 * wn + b) + 4 * hl;
            store4<BF16, OUT_F32>(P.Y, (int64_t)m * F + n, silu_mul(acc[0][b][g], acc[1][b][g]));
          }
        }
      }
      return;
    }
  }
  void* Yp = P.Y;
  if (P.splits > 1) Yp = reinterpret_cast<float*>(P.Y) + (int64_t)ks * P.M * P.N;
#pragma unroll
  for (int rb = 0; rb < 2; rb++) {
    if (rb == 1 && !second) break;
    const int i_rb = rb ? i1 : i0;
#pragma unroll
    for (int g = 0; g < kNMB; g++) {
      const int m = mw + 16 * g;
      if (m < M) {
#pragma unroll
        for (int b = 0; b < 4; b++) {
          const int64_t n = (int64_t)i_rb * kTile + 16 * (4 * wn + b) + 4 * hl;
          if (P.splits > 1)
            store4<BF16, true>(Yp, (int64_t)m * P.N + n, acc[rb][b][g]);
          else
            store4<BF16, OUT_F32>(Yp, (int64_t)m * P.N + n, acc[rb][b][g]);
        }
      }
    }
  }
}

template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32, bool FUSE, int BM, int WAVES>
hipError_t launch_prefill_big_bm(const PfArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(8 * a.per_xcd)), block(WAVES * 64);
  if (a.splits > 1)
    hipLaunchKernelGGL((k_prefill_big<BF16, SRC_ROWMAJOR, true, FUSE, BM, WAVES>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((k_prefill_big<BF16, SRC_ROWMAJOR, OUT_F32, FUSE, BM, WAVES>), grid, block, 0, s, a);
  return hipGetLastError();
}

// One launch of the big-tile kernel for the arguments a (a.Y is the fp32
// partial buffer when a.splits > 1; the caller reduces it).  waves: 4 (one
// a SIMD, widths 128, 192, 256) or 8 (two a SIMD, widths 128, 256).
hipError_t launch_prefill_big(bool bf16, bool rowmajor, bool out_f32, bool fuse, int bm, int waves, const PfArgs& a,
                              hipStream_t s) {
#define PATCH_BG(B, R, F, U)                                                                 \
  (waves == 8 ? (bm == 256   ? launch_prefill_big_bm<B, R, F, U, 256, 8>(a, s)              \
                 : bm == 128 ? launch_prefill_big_bm<B, R, F, U, 128, 8>(a, s)              \
                             : hipErrorInvalidValue)                                         \
              : (bm == 256   ? launch_prefill_big_bm<B, R, F, U, 256, 4>(a, s)              \
                 : bm == 192 ? launch_prefill_big_bm<B, R, F, U, 192, 4>(a, s)              \
                 : bm == 128 ? launch_prefill_big_bm<B, R, F, U, 128, 4>(a, s)              \
                             : hipErrorInvalidValue))
#define PATCH_BG2(B, R, F) (fuse ? PATCH_BG(B, R, F, true) : PATCH_BG(B, R, F, false))
  if (bf16) {
    if (rowmajor) return out_f32 ? PATCH_BG2(true, true, true) : PATCH_BG2(true, true, false);
    return out_f32 ? PATCH_BG2(true, false, true) : PATCH_BG2(true, false, false);
  }
  if (rowmajor) return out_f32 ? PATCH_BG2(false, true, true) : PATCH_BG2(false, true, false);
  return out_f32 ? PATCH_BG2(false, false, true) : PATCH_BG2(false, false, false);
#undef PATCH_BG2
#undef PATCH_BG
}

}  // namespace patch
