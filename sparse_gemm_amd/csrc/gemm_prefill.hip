// gemm_prefill.hip -- output-tiled hybrid GEMM for many tokens (M > 16).
//
// PATCH (arXiv 2509.23410), gist.science explainer, section 2 "Inference &
// Deployment": each tile runs on the dense matrix units or, when it is 2:4,
// on the sparse ones.  With M >= 512 the product is bound by the matrix
// cores.  A workgroup owns one 128-row tile row of W (row-block i) and 256
// columns of M, and keeps that 128 x 256 block of Y^T in fp32 accumulators:
//
//   * 4 waves in a 2 x 2 arrangement; wave (wn, wm) owns bands 4wn..4wn+3 of
//     the row-block (64 rows of W) and 128 columns of M: 4 x 8 accumulators
//     of 16 x 16;
//   * every wave of the workgroup sees the same tile kind at each step (one
//     row-block per workgroup), so the K loop is split into two loops: first
//     the row-block's dense tiles, then its 2:4 tiles (the tile table gives the
//     two lists).  A step covers 64 columns of K: half a dense tile (2 x
//     v_mfma_f32_16x16x32 deep) or one sparse slice (1 x
//     v_smfmac_f32_16x16x64 deep, half the matrix-core time);
//   * X[m0 .. m0+255][64 columns] is copied global -> LDS directly
//     (global_load_lds_dwordx4, no registers), double-buffered, its 16-byte
//     chunks XOR-swizzled by row so the B-operand reads hit distinct banks;
//   * W comes straight from the packed blob into A-operand registers (a 1 KB
//     fragment = one 16-byte load a lane), fetched one step ahead;
//   * workgroups are numbered so that each of the 8 XCDs gets a contiguous
//     run of output blocks (the M-blocks of a row-block share its W tiles in
//     that XCD's L2).
//
// With SRC_ROWMAJOR the same kernel reads plain row-major W with every tile
// dense: the same-shape dense baseline.
#include "device_common.h"

namespace patch {

constexpr int kPfBM = 256;                        // M columns of a workgroup block
constexpr int kPfRowBytes = 128;                  // one staged X row: 64 elements
constexpr int kPfBufBytes = kPfBM * kPfRowBytes;  // 32 KB per stage
constexpr int kPfMaxKT = 1024;

// Chunk position of 16-byte chunk c (0..7) of staged row r.  The XOR keeps the
// 16 rows read by one B-fragment load on distinct bank groups for both 32- and
// 64-bank LDS: bits (r0 ^ r3, r2, r1) of r.
__device__ __forceinline__ int swz_f(int r) { return (((r ^ (r >> 3)) & 1) << 2) | ((r >> 1) & 3); }
__device__ __forceinline__ int swz(int r, int c) { return r * kPfRowBytes + ((c ^ swz_f(r)) << 4); }

// 16 bytes per lane, global -> LDS without registers: lane l's chunk lands at
// LDS byte lds_base + 16*l (global_load_lds_dwordx4, M0 = LDS base).  Written
// as inline asm so the compiler does not order every later LDS read behind
// it; the kernel waits for these copies itself (vmcnt(0) before the barrier
// that publishes a stage).
// M0 is saved and restored around the copy, so the compiler's own use of M0
// is unaffected.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(gptr)
      : "memory");
}

// s_waitcnt vmcnt(0) as a real instruction (not inline asm), so the compiler's
// own wait-count tracking knows every vector-memory load has landed here.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

struct DenseA {
  u32x4 a[2][4];  // [slice in step][band]
};
struct SparseA {
  u32x4 a[4];        // [band]
  uint32_t meta[4];  // [band] both slices' index halves
  uint32_t shift;    // 16 * slice: moves this slice's half to bits 0..15
};

template <bool SRC_ROWMAJOR>
__device__ __forceinline__ void load_dense_step(DenseA& A, const uint8_t* __restrict__ src, uint64_t off, int64_t K,
                                                int i, int j, int half, int wn, int l) {
#pragma unroll
  for (int qq = 0; qq < 2; qq++) {
    const int q = 2 * half + qq;
#pragma unroll
    for (int bnd = 0; bnd < 4; bnd++) {
      const int band = 4 * wn + bnd;
      if constexpr (SRC_ROWMAJOR) {
        const uint16_t* W = reinterpret_cast<const uint16_t*>(src);
        A.a[qq][bnd] = ld16(W + ((int64_t)i * kTile + 16 * band + (l & 15)) * K + (int64_t)j * kTile + 32 * q +
                            8 * (l >> 4));
      } else {
        A.a[qq][bnd] = ld16(src + off + (q * 8 + band) * 1024 + 16 * l);
      }
    }
  }
}

__device__ __forceinline__ void load_sparse_step(SparseA& A, const uint8_t* __restrict__ src, uint64_t off, int q,
                                                 int wn, int l) {
#pragma unroll
  for (int bnd = 0; bnd < 4; bnd++) {
    const int band = 4 * wn + bnd;
    A.a[bnd] = ld16(src + off + (q * 8 + band) * 1024 + 16 * l);
    A.meta[bnd] = *reinterpret_cast<const uint32_t*>(src + off + kSparseValBytes + 4 * (64 * band + l));
  }
  A.shift = 16 * q;
}

template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32>
__global__ __launch_bounds__(256, 2) void k_prefill(const uint8_t* __restrict__ src, const uint16_t* __restrict__ X,
                                                    int M, int N, int K, void* __restrict__ Y, int n_mblk,
                                                    int n_tiles, int per_xcd) {
  const int id = blockIdx.x;
  const int t = (id & 7) * per_xcd + (id >> 3);
  if (t >= n_tiles) return;
  const int i = t / n_mblk, mb = t - (t / n_mblk) * n_mblk;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int wn = w >> 1, wm = w & 1;
  const int KT = K / kTile;
  const int m0 = mb * kPfBM;
  const int h = l >> 4;

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kPfBufBytes];
  __shared__ uint16_t s_list[2][kPfMaxKT];
  __shared__ int s_count[2];

  const TileEntry* table = reinterpret_cast<const TileEntry*>(src + kHeaderBytes) + (int64_t)i * KT;
  int nd, ns;
  if constexpr (SRC_ROWMAJOR) {
    nd = KT;
    ns = 0;
  } else {
    if (w == 0) {
      int base_d = 0, base_s = 0;
      for (int c0 = 0; c0 < KT; c0 += 64) {
        const int jj = c0 + l;
        const bool valid = jj < KT;
        const uint32_t kind = valid ? table[jj].kind : 0u;
        const bool sp = valid && kind != 0;
        const bool de = valid && kind == 0;
        const uint64_t bs = __ballot(sp), bd = __ballot(de);
        const uint64_t lt = (l == 0) ? 0ull : (~0ull >> (64 - l));
        if (de) s_list[0][base_d + __popcll(bd & lt)] = (uint16_t)jj;
        if (sp) s_list[1][base_s + __popcll(bs & lt)] = (uint16_t)jj;
        base_d += __popcll(bd);
        base_s += __popcll(bs);
      }
      if (l == 0) {
        s_count[0] = base_d;
        s_count[1] = base_s;
      }
    }
    __syncthreads();
    nd = s_count[0];
    ns = s_count[1];
  }
  const int n_steps = 2 * (nd + ns);

  // tile column of step s (dense tiles first, then sparse ones); the K range
  // of step s is columns 64*(s&1) .. +63 of that tile in both cases.
  auto step_tile = [&](int s) -> int {
    if constexpr (SRC_ROWMAJOR) {
      return s >> 1;
    } else {
      const int e = s >> 1;
      return e < nd ? (int)s_list[0][e] : (int)s_list[1][e - nd];
    }
  };

  // X stage of step s into buffer buf: 256 rows x 64 columns = 32 blocks of
  // 1 KB (8 rows); wave w fills blocks 8w .. 8w+7.  Lane l lands at row
  // 8*blk + l/8, chunk position l%8, so it fetches the source chunk whose
  // swizzled position is l%8.  Rows past M repeat row M-1 (never stored).
  auto issue_stage = [&](int s, int buf) {
    const int j = step_tile(s);
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)smem) + buf * kPfBufBytes;
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int blk = 8 * w + u;
      const int r = 8 * blk + (l >> 3);
      const int c = (l & 7) ^ swz_f(r);
      const int gm = min(m0 + r, M - 1);
      const uint16_t* g = X + (int64_t)gm * K + (int64_t)j * kTile + 64 * (s & 1) + 8 * c;
      lds_dma16(g, __builtin_amdgcn_readfirstlane(lds0 + 1024 * blk));
    }
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int a = 0; a < 4; a++)
#pragma unroll
    for (int c = 0; c < 8; c++) acc[a][c] = (f32x4){0.f, 0.f, 0.f, 0.f};

  if (n_steps > 0) {
    issue_stage(0, 0);
    wait_vmem_all();
    __syncthreads();
  }

  // ---- dense steps: s = 0 .. 2*nd-1
  if (nd > 0) {
    DenseA cur, nxt;
    {
      const int j = step_tile(0);
      load_dense_step<SRC_ROWMAJOR>(cur, src, SRC_ROWMAJOR ? 0 : table[j].offset, K, i, j, 0, wn, l);
      wait_vmem_all();
    }
    for (int s = 0; s < 2 * nd; s++) {
      const int buf = s & 1;
      const bool more_dense = s + 1 < 2 * nd;
      if (more_dense) {
        const int j = step_tile(s + 1);
        load_dense_step<SRC_ROWMAJOR>(nxt, src, SRC_ROWMAJOR ? 0 : table[j].offset, K, i, j, (s + 1) & 1, wn, l);
      }
      if (s + 1 < n_steps) issue_stage(s + 1, buf ^ 1);
      const uint8_t* xs = smem + buf * kPfBufBytes;
#pragma unroll
      for (int qq = 0; qq < 2; qq++) {
        u32x4 bf[8];
#pragma unroll
        for (int mblk = 0; mblk < 8; mblk++)
          bf[mblk] = *reinterpret_cast<const u32x4*>(xs + swz(wm * 128 + mblk * 16 + (l & 15), 4 * qq + h));
#pragma unroll
        for (int mblk = 0; mblk < 8; mblk++)
#pragma unroll
          for (int bnd = 0; bnd < 4; bnd++) acc[bnd][mblk] = mma_dense<BF16>(cur.a[qq][bnd], bf[mblk], acc[bnd][mblk]);
      }
      wait_vmem_all();
      __syncthreads();
      if (more_dense) cur = nxt;
    }
  }

  // ---- 2:4 steps: s = 2*nd .. n_steps-1
  if constexpr (!SRC_ROWMAJOR) {
    if (ns > 0) {
      SparseA cur, nxt;
      {
        const int j = step_tile(2 * nd);
        load_sparse_step(cur, src, table[j].offset, 0, wn, l);
        wait_vmem_all();
      }
      for (int s = 2 * nd; s < n_steps; s++) {
        const int buf = s & 1;
        const bool more = s + 1 < n_steps;
        if (more) {
          const int j = step_tile(s + 1);
          load_sparse_step(nxt, src, table[j].offset, (s + 1) & 1, wn, l);
          issue_stage(s + 1, buf ^ 1);
        }
        const uint8_t* xs = smem + buf * kPfBufBytes;
#pragma unroll
        for (int g4 = 0; g4 < 2; g4++) {
          u32x4 blo[4], bhi[4];
#pragma unroll
          for (int mm = 0; mm < 4; mm++) {
            const int row = wm * 128 + (4 * g4 + mm) * 16 + (l & 15);
            blo[mm] = *reinterpret_cast<const u32x4*>(xs + swz(row, h));
            bhi[mm] = *reinterpret_cast<const u32x4*>(xs + swz(row, 4 + h));
          }
#pragma unroll
          for (int mm = 0; mm < 4; mm++)
#pragma unroll
            for (int bnd = 0; bnd < 4; bnd++)
              acc[bnd][4 * g4 + mm] =
                  mma_sparse<BF16, 0>(cur.a[bnd], blo[mm], bhi[mm], acc[bnd][4 * g4 + mm], cur.meta[bnd] >> cur.shift);
        }
        wait_vmem_all();
        __syncthreads();
        if (more) cur = nxt;
      }
    }
  }

  // ---- epilogue: round and store Y[m][n .. n+3]
#pragma unroll
  for (int mblk = 0; mblk < 8; mblk++) {
    const int m = m0 + wm * 128 + mblk * 16 + (l & 15);
    if (m < M) {
#pragma unroll
      for (int bnd = 0; bnd < 4; bnd++) {
        const int64_t n = (int64_t)i * kTile + 16 * (4 * wn + bnd) + 4 * h;
        store4<BF16, OUT_F32>(Y, (int64_t)m * N + n, acc[bnd][mblk]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32>
static hipError_t launch_prefill_t(const void* src, const void* X, int64_t M, int64_t N, int64_t K, void* Y,
                                   hipStream_t s) {
  const int NT = (int)(N / kTile);
  const int n_mblk = (int)((M + kPfBM - 1) / kPfBM);
  const int n_tiles = NT * n_mblk;
  const int per_xcd = (n_tiles + 7) / 8;
  hipLaunchKernelGGL((k_prefill<BF16, SRC_ROWMAJOR, OUT_F32>), dim3((unsigned)(8 * per_xcd)), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(src), reinterpret_cast<const uint16_t*>(X), (int)M, (int)N,
                     (int)K, Y, n_mblk, n_tiles, per_xcd);
  return hipGetLastError();
}

hipError_t launch_prefill(bool bf16, bool rowmajor, bool out_f32, const void* src, const void* X, int64_t M, int64_t N,
                          int64_t K, void* Y, hipStream_t s) {
  if (bf16) {
    if (rowmajor) return out_f32 ? launch_prefill_t<true, true, true>(src, X, M, N, K, Y, s)
                                 : launch_prefill_t<true, true, false>(src, X, M, N, K, Y, s);
    return out_f32 ? launch_prefill_t<true, false, true>(src, X, M, N, K, Y, s)
                   : launch_prefill_t<true, false, false>(src, X, M, N, K, Y, s);
  }
  if (rowmajor) return out_f32 ? launch_prefill_t<false, true, true>(src, X, M, N, K, Y, s)
                               : launch_prefill_t<false, true, false>(src, X, M, N, K, Y, s);
  return out_f32 ? launch_prefill_t<false, false, true>(src, X, M, N, K, Y, s)
                 : launch_prefill_t<false, false, false>(src, X, M, N, K, Y, s);
}

}  // namespace patch
