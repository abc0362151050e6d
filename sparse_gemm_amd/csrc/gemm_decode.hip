// gemm_decode.hip -- weight-streaming hybrid GEMM for few tokens (M <= 16).
//
// PATCH (arXiv 2509.23410), gist.science explainer, section 2 "Inference &
// Deployment": dense tiles run on the dense matrix path and 2:4 tiles on the
// sparse one.  With M <= 16 the product is bound by the bytes of W, so the
// kernel streams each tile's packed bytes exactly once:
//
//   * one workgroup per 16-row band of W (N/16 workgroups) and all of K;
//     wave w of the workgroup's WAVES (1 to 8, by K and the grid) takes
//     the tile columns j = w, w+WAVES, ... of the band's row-block; its
//     tile-table entries arrive with one vector load and are read with
//     v_readlane (no list building, no barrier before the first weight
//     load); the 8 bands of a row-block run on one XCD, so the lines they
//     share sit in one L2;
//   * a tile's 16 x 128 band is 4 (dense) or 2 (sparse) 1 KB fragments that a
//     wave loads with one 16-byte load per lane each, straight into the A
//     operand registers; X (at most 16 rows) is read from L2 into the B
//     operand registers;
//   * both kinds run on v_smfmac_f32_16x16x64: a 2:4 tile is 2 of them (one
//     per 64-column slice, its own index codes), a dense tile 4 (each slice
//     as two halves with the fixed patterns (0,1) and (2,3));
//   * loads run DEPTH tiles ahead of the matrix instructions;
//   * the waves' fp32 partial sums are added in LDS in wave order (fixed, so
//     results are deterministic) and rounded to the output type.
//
// The same kernel with SRC_ROWMAJOR reads plain row-major W (every tile
// dense): that is the same-shape dense baseline.
#include "device_common.h"

namespace patch {


// Registers of one tile in flight.  Both kinds issue the same eight 16-byte
// loads (4 for X, 4 for W), so the wait counts the compiler derives stay
// exact whatever mix of kinds a wave meets:
//   dense : a[2q + e] = the band's half e of 64-column slice q (packed W), or
//           the row-major chunk of columns 32c + 8*(l/16) (dense baseline);
//   sparse: a[0], a[1] = value fragments of slices 0 and 1, a[2] = the
//           16 bytes of the band's codes holding this lane's word (word l & 3),
//           a[3] = the same chunk again (unused); 4:8 tiles alike (the
//           value fragments hold four kept values per group of eight, the
//           word four 8-bit position masks), rebuilt into a dense tile's
//           halves before the matrix instructions.
template <int MB>
struct DecodeFrag {
  u32x4 x[MB][4];  // B operand chunks of M block mb: X[16mb + m][k0 + 32c + 8h .. +7], c = 0..3
  u32x4 a[4];
  uint32_t kind;
};

// X is read through a buffer descriptor whose range ends with row M - 1:
// lanes whose X row is >= M (they only feed output columns that are never
// stored) get zeros from the range check, with no memory access, no
// predication (which would make the compiler wait for the load at once) and
// no hot spot on row 0 when M is 1.
// Q64 (64 x 64 execution tiles, format 4): `b` is the band within the
// entry's 64-row half and `kind` the entry's kind bits (bit q: 64-column
// slice q is 2:4); the piece holds slice 0, then slice 1 (2048 bytes dense,
// 1024 bytes 2:4), then the codes block if either slice is 2:4.  Slot
// registers: a[2q] = slice q's first fragment, a[2q + 1] = its second dense
// half, or, for a 2:4 slice, the codes chunk holding the lane's word.
template <bool SRC_ROWMAJOR, int MB, bool Q64 = false>
__device__ __forceinline__ void decode_load(DecodeFrag<MB>& f, const uint8_t* __restrict__ src, uint64_t off,
                                            uint32_t kind, uint32_t stride, __amdgpu_buffer_rsrc_t xr, int K,
                                            int i, int b, int j, int l) {
  const int h = l >> 4;
  const uint8_t* ap[4];
  if constexpr (SRC_ROWMAJOR) {
    const uint16_t* W = reinterpret_cast<const uint16_t*>(src);
    const uint8_t* wr = reinterpret_cast<const uint8_t*>(W + ((int64_t)i * kTile + 16 * b + (l & 15)) * K +
                                                         (int64_t)j * kTile + 8 * h);
#pragma unroll
    for (int c = 0; c < 4; c++) ap[c] = wr + 64 * c;
    f.kind = 0;
  } else if constexpr (Q64) {
    const uint8_t* pb = src + off + (uint64_t)b * stride;
    const uint32_t a1 = (kind & 1u) ? 1024u : 2048u;
    const uint8_t* mp = pb + a1 + ((kind & 2u) ? 1024u : 2048u) + 16 * (l >> 2);
    ap[0] = pb + 16 * l;
    ap[1] = (kind & 1u) ? mp : pb + 1024 + 16 * l;
    ap[2] = pb + a1 + 16 * l;
    ap[3] = (kind & 2u) ? mp : pb + a1 + 1024 + 16 * l;
    f.kind = kind;
  } else {
    // band b's piece of the tile: dense = blocks (slice 0, half 0/1), (slice
    // 1, half 0/1); 2:4 = value blocks of slices 0 and 1, then the codes
    const uint8_t* pb = src + off + (uint64_t)b * stride;
    const uint8_t* mp = pb + kSparseMetaOffset + 16 * (l >> 2);
    ap[0] = pb + 16 * l;
    ap[1] = pb + 1024 + 16 * l;
    ap[2] = kind ? mp : pb + 2048 + 16 * l;
    ap[3] = kind ? mp : pb + 3072 + 16 * l;
    f.kind = kind;
  }
#pragma unroll
  for (int mb = 0; mb < MB; mb++) {
    const uint32_t xo = ((uint32_t)(16 * mb + (l & 15)) * (uint32_t)K + (uint32_t)(j * kTile + 8 * h)) * 2u;
#pragma unroll
    for (int c = 0; c < 4; c++)
      f.x[mb][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (int)xo, 64 * c, 0));
  }
#pragma unroll
  for (int c = 0; c < 4; c++) f.a[c] = ld16(ap[c]);
}

// N48: the blob holds 4:8 tiles (their rebuild lives only in this
// instantiation: it costs the other kinds registers and occupancy).
template <bool BF16, bool SRC_ROWMAJOR, int MB, bool N48, bool Q64 = false>
__device__ __forceinline__ void decode_mma(DecodeFrag<MB>& f, f32x4 (&acc)[MB], int l, const u32x4* sel) {
  if constexpr (Q64) {
    // each 64-column slice on its own kind (f.kind is wave-uniform)
#pragma unroll
    for (int q = 0; q < 2; q++) {
      if ((f.kind >> q) & 1u) {
        const u32x4 mc = f.a[2 * q + 1];
        const uint32_t lo = (l & 1) ? mc[1] : mc[0], hi = (l & 1) ? mc[3] : mc[2];
        const uint32_t meta = (l & 2) ? hi : lo;
#pragma unroll
        for (int mb = 0; mb < MB; mb++) {
          if (q == 0)
            acc[mb] = mma_sparse<BF16, 0>(f.a[0], f.x[mb][0], f.x[mb][1], acc[mb], meta);
          else
            acc[mb] = mma_sparse<BF16, 1>(f.a[2], f.x[mb][2], f.x[mb][3], acc[mb], meta);
        }
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; mb++) {
          acc[mb] = mma_sparse<BF16, 0>(f.a[2 * q], f.x[mb][2 * q], f.x[mb][2 * q + 1], acc[mb], 0x4444u);
          acc[mb] = mma_sparse<BF16, 0>(f.a[2 * q + 1], f.x[mb][2 * q], f.x[mb][2 * q + 1], acc[mb], 0xEEEEu);
        }
      }
    }
  } else if constexpr (SRC_ROWMAJOR) {
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
      for (int c = 0; c < 4; c++) acc[mb] = mma_dense<BF16>(f.a[c], f.x[mb][c], acc[mb]);
  } else if (f.kind == 0 || (N48 && f.kind == 2)) {
    // dense, or 4:8 rebuilt in place into a dense piece's halves (values of
    // slice q in a[q], its two groups' masks in bits 16q .. 16q+15 of the
    // lane's word in the codes chunk a[2]); the slot is reloaded afterwards
    if constexpr (N48) {
      if (f.kind == 2) {
        // the mask word is read from a[3] (the same codes chunk as a[2]):
        // it is the slot's last load, so reading it makes the wait cover
        // every load of the slot before its registers are rewritten here
        const u32x4 mc = f.a[3], v0 = f.a[0], v1 = f.a[1];
        const uint32_t lo = (l & 1) ? mc[1] : mc[0], hi = (l & 1) ? mc[3] : mc[2];
        const uint32_t meta = (l & 2) ? hi : lo;
        dense_halves48(v0, meta & 0xffffu, sel, f.a[0], f.a[1]);
        dense_halves48(v1, meta >> 16, sel, f.a[2], f.a[3]);
      }
    }
    // slice q: halves with positions (0,1) (code 4) and (2,3) (code 14)
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
      for (int q = 0; q < 2; q++) {
        acc[mb] = mma_sparse<BF16, 0>(f.a[2 * q], f.x[mb][2 * q], f.x[mb][2 * q + 1], acc[mb], 0x4444u);
        acc[mb] = mma_sparse<BF16, 0>(f.a[2 * q + 1], f.x[mb][2 * q], f.x[mb][2 * q + 1], acc[mb], 0xEEEEu);
      }
  } else {
    // word l & 3 of the codes chunk, by two bit tests (plain selects; a
    // dynamic vector index would put the fragment array in scratch memory)
    const u32x4 mc = f.a[2];
    const uint32_t lo = (l & 1) ? mc[1] : mc[0], hi = (l & 1) ? mc[3] : mc[2];
    const uint32_t meta = (l & 2) ? hi : lo;
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
      // slice 0: logical K 0..63 of the tile -> B chunks 0 (K 8h..) and 1 (K 32+8h..)
      acc[mb] = mma_sparse<BF16, 0>(f.a[0], f.x[mb][0], f.x[mb][1], acc[mb], meta);
      // slice 1: logical K 64..127 -> B chunks 2 and 3
      acc[mb] = mma_sparse<BF16, 1>(f.a[1], f.x[mb][2], f.x[mb][3], acc[mb], meta);
    }
  }
}

// WAVES waves per workgroup (tile columns split between them); XCD_MAP puts
// the 8 bands of a row-block on one XCD (blocks are dealt to the 8 XCDs in
// turn), so lines they share -- the 2:4 metadata, X -- are fetched into one L2.
// FUSE: fused gate/up projection.  W is the row-block interleave of the gate
// (even row-blocks) and up (odd) matrices -- packed, or, with SRC_ROWMAJOR,
// two row-major matrices src (gate) and src2 (up); a workgroup takes band b
// of both row-blocks of pair q with twice the waves (the first WAVES on gate,
// the others on up) and writes H[m][128 q + ...] = SiLU(gate) * up, H being
// M x N/2.
// Q64: a blob of 64 x 64 execution tiles (format 4; not fused): band b of
// row-block i reads the entries of half-row-block 2i + b/4, band b mod 4.
template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32, int WAVES, int DEPTH, bool XCD_MAP, int MB, bool FUSE, bool N48,
          bool Q64 = false>
__global__ __launch_bounds__(WAVES * 64 * (FUSE ? 2 : 1)) void k_decode(const uint8_t* __restrict__ src,
                                                                         const uint8_t* __restrict__ src2,
                                                                         const uint16_t* __restrict__ X, int M, int N,
                                                                         int K, void* __restrict__ Y) {
  constexpr int kDecodeWaves = WAVES;
  constexpr int kAllWaves = WAVES * (FUSE ? 2 : 1);
  const int KT = K / kTile;
  const int bid = blockIdx.x;
  const int NB = FUSE ? N / kTile / 2 : N / kTile;  // row-blocks (fused: gate/up pairs)
  const int full = (NB / 8) * 64;  // blocks in complete groups of 8 row-blocks
  int q, b;                        // row-block (fused: pair) and 16-row band of W
  if (XCD_MAP && bid < full) {
    q = (bid & 7) + 8 * (bid >> 6);
    b = (bid >> 3) & 7;
  } else {
    q = bid >> 3;
    b = bid & 7;
  }
  const int wa = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = FUSE ? wa / WAVES : 0;  // fused: 0 gate, 1 up
  const int w = wa - g * WAVES;         // wave within its row-block
  const int l = threadIdx.x & 63;
  const int i = FUSE ? 2 * q + g : q;   // row-block of the (interleaved) matrix
  static_assert(!Q64 || (!SRC_ROWMAJOR && !FUSE && !N48), "64 x 64 execution tiles: packed W, not fused");
  const TileEntry* table =
      reinterpret_cast<const TileEntry*>(src + kHeaderBytes) + (int64_t)(Q64 ? 2 * i + (b >> 2) : i) * KT;
  const int bp = Q64 ? (b & 3) : b;  // the band's index inside its entries' pieces
  // row-major W: the matrix and row-block this wave reads
  const uint8_t* wsrc = SRC_ROWMAJOR && FUSE && g ? src2 : src;
  const int wi = SRC_ROWMAJOR && FUSE ? q : i;

  __shared__ f32x4 s_red[kAllWaves * MB][64];
  // X rows 0 .. M-1 (byte range M K 2, below 2^31 for M <= 128, K <= 65536)
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), (short)0, M * K * 2, 0x00020000);
  // 4:8 rebuild selectors (only in the instantiation for blobs with 4:8 tiles)
  __shared__ u32x4 s_sel[N48 ? 256 : 1];
  if constexpr (N48) {
    fill_sel48(s_sel, (int)threadIdx.x, kAllWaves * 64);
    __syncthreads();
  }

  // wave w takes tile columns j = w, w + WAVES, ... of its row-block (at
  // most 64 of them, which the launch guarantees).  Their table entries arrive with one
  // vector load (lane t holds the entry of the wave's t-th tile) and are read
  // with v_readlane.
  const int n_mine = (KT - w + kDecodeWaves - 1) / kDecodeWaves;
  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; mb++) acc[mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (n_mine > 0) {
    u32x4 ents = {0u, 0u, 0u, 0u};
    if constexpr (!SRC_ROWMAJOR) ents = ld16(table + w + kDecodeWaves * min(l, n_mine - 1));
    auto entry = [&](int t, uint64_t& off, uint32_t& kind, uint32_t& stride) {
      if constexpr (SRC_ROWMAJOR) {
        off = 0;
        kind = 0;
        stride = 0;
      } else {
        const int lane = t;
        off = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)ents[0], lane) |
              ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)ents[1], lane) << 32);
        kind = (uint32_t)__builtin_amdgcn_readlane((int)ents[2], lane);
        stride = (uint32_t)__builtin_amdgcn_readlane((int)ents[3], lane);
      }
    };
    DecodeFrag<MB> f[DEPTH];
#pragma unroll
    for (int s = 0; s < DEPTH; s++) {
      const int t = min(s, n_mine - 1);
      uint64_t off;
      uint32_t kind, stride;
      entry(t, off, kind, stride);
      decode_load<SRC_ROWMAJOR, MB, Q64>(f[s], SRC_ROWMAJOR ? wsrc : src, off, kind, stride, xr, K, wi, bp,
                                         w + kDecodeWaves * t, l);
    }
    // steady state: compute the DEPTH slots, refilling each with the tile
    // DEPTH further on (clamped to the last tile: a redundant, cached load)
    int t0 = 0;
    for (; t0 + DEPTH < n_mine; t0 += DEPTH) {
#pragma unroll
      for (int s = 0; s < DEPTH; s++) {
        decode_mma<BF16, SRC_ROWMAJOR, MB, N48, Q64>(f[s], acc, l, s_sel);
        const int tn = min(t0 + s + DEPTH, n_mine - 1);
        uint64_t off;
        uint32_t kind, stride;
        entry(tn, off, kind, stride);
        decode_load<SRC_ROWMAJOR, MB, Q64>(f[s], SRC_ROWMAJOR ? wsrc : src, off, kind, stride, xr, K, wi, bp,
                                           w + kDecodeWaves * tn, l);
      }
    }
    // last round: no refills
#pragma unroll
    for (int s = 0; s < DEPTH; s++)
      if (t0 + s < n_mine) decode_mma<BF16, SRC_ROWMAJOR, MB, N48, Q64>(f[s], acc, l, s_sel);
  }

  // ---- fixed-order reduction over waves (wave wa adds up M blocks wa,
  // wa + all waves, ...), then round and store
#pragma unroll
  for (int mb = 0; mb < MB; mb++) s_red[wa * MB + mb][l] = acc[mb];
  __syncthreads();
  for (int mb = wa; mb < MB; mb += kAllWaves) {
    f32x4 sum = s_red[mb][l];
#pragma unroll
    for (int ww = 1; ww < kDecodeWaves; ww++) sum += s_red[ww * MB + mb][l];
    const int m = 16 * mb + (l & 15);
    if constexpr (FUSE) {
      f32x4 up = s_red[(kDecodeWaves + 0) * MB + mb][l];
#pragma unroll
      for (int ww = 1; ww < kDecodeWaves; ww++) up += s_red[(kDecodeWaves + ww) * MB + mb][l];
      if (m < M) {
        const int64_t n = (int64_t)q * kTile + 16 * b + 4 * (l >> 4);
        store4<BF16, OUT_F32>(Y, (int64_t)m * (N / 2) + n, silu_mul(sum, up));
      }
    } else if (m < M) {
      const int64_t n = (int64_t)i * kTile + 16 * b + 4 * (l >> 4);
      store4<BF16, OUT_F32>(Y, (int64_t)m * N + n, sum);
    }
  }
}

template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32, bool FUSE, bool N48, int WAVES, int DEPTH, bool XCD_MAP, int MB,
          bool Q64>
static hipError_t launch_decode_v(const void* src, const void* src2, const void* X, int64_t M, int64_t N, int64_t K,
                                  void* Y, hipStream_t s) {
  const unsigned grid = (unsigned)(FUSE ? N / 32 : N / 16);
  hipLaunchKernelGGL((k_decode<BF16, SRC_ROWMAJOR, OUT_F32, WAVES, DEPTH, XCD_MAP, MB, FUSE, N48, Q64>), dim3(grid),
                     dim3(WAVES * 64 * (FUSE ? 2 : 1)), 0, s, reinterpret_cast<const uint8_t*>(src),
                     reinterpret_cast<const uint8_t*>(src2), reinterpret_cast<const uint16_t*>(X), (int)M, (int)N,
                     (int)K, Y);
  return hipGetLastError();
}

template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32, bool FUSE, bool N48, bool Q64 = false>
static hipError_t launch_decode_t(const void* src, const void* src2, const void* X, int64_t M, int64_t N, int64_t K,
                                  void* Y, hipStream_t s) {
  // Few waves a workgroup, several tiles in flight a wave: small workgroups
  // fill every CU several times over and keep starting while others drain,
  // which measured faster than 8 or 16 waves on the q_proj, gate_proj and
  // down_proj shapes.  A wave reads its table entries with one vector load,
  // so it may own at most 64 tile columns: larger K takes more waves.
  // (Fused gate/up: twice the waves, one set per matrix.)
  const int64_t KT = K / kTile;
#define PATCH_DV(W, D, MBK) \
  launch_decode_v<BF16, SRC_ROWMAJOR, OUT_F32, FUSE, N48, W, D, true, MBK, Q64>(src, src2, X, M, N, K, Y, s)
  if (M <= 16) {
    // Wide matrices, whose bands cover every CU at least twice: one wave a
    // band (gate_proj of LLaMA-2 7B, 11008 x 4096: 1-6% faster than two
    // waves; q_proj, 4096 x 4096 with one band a CU, is 30% slower so).
    if constexpr (!FUSE)
      if (KT <= 64 && N / 16 >= 2 * (int64_t)cu_count()) return PATCH_DV(1, 4, 1);
    if (KT <= 2 * 64) return PATCH_DV(2, 4, 1);
    if (KT <= 4 * 64) return PATCH_DV(4, 4, 1);
    return PATCH_DV(8, 2, 1);
  }
  // More tokens: MB column blocks of 16 per wave (X is re-read from L2 by
  // every band, which the 16 < M <= 128 range affords).
  if (KT <= 4 * 64) {
    if (M <= 32) return PATCH_DV(4, 2, 2);
    if (M <= 64) return PATCH_DV(4, 1, 4);
    return PATCH_DV(4, 1, 8);
  }
  if constexpr (FUSE) {
    return hipErrorInvalidValue;  // 16 waves with several blocks of M do not fit the registers
  } else {
    if (M <= 32) return PATCH_DV(8, 2, 2);
    if (M <= 64) return PATCH_DV(8, 1, 4);
    return PATCH_DV(8, 1, 8);
  }
#undef PATCH_DV
}

// Time model of this kernel for 16 < M <= 128, fitted to its measured times
// on the LLaMA-2 7B q_proj, gate_proj and down_proj shapes (10% rms error):
// a fixed cost, the weight bytes, and the X bytes every 16-row band re-reads
// from L2 (16 columns of M at a time).
double decode_estimate_us(int64_t M, int64_t N, int64_t K, double w_bytes) {
  const double mcols = 16.0 * (double)((M + 15) / 16);
  return 3.13 + w_bytes / 1.543e7 + (double)(N / 16) * mcols * (double)K * 2.0 / 9.30e6;
}

// src2 non-null: fused gate/up (see k_decode); Y is then H, M x N/2.
// n48: the packed blob holds 4:8 tiles; q64: it is a blob of 64 x 64
// execution tiles (format 4; packed, not fused).
hipError_t launch_decode(bool bf16, bool rowmajor, bool out_f32, const void* src, const void* src2, const void* X,
                         int64_t M, int64_t N, int64_t K, void* Y, bool n48, bool q64, hipStream_t s) {
  const bool fuse = src2 != nullptr;
  if (fuse && (N % (2 * kTile))) return hipErrorInvalidValue;
  if (q64) {
    if (rowmajor || fuse || n48) return hipErrorInvalidValue;
    if (bf16)
      return out_f32 ? launch_decode_t<true, false, true, false, false, true>(src, src2, X, M, N, K, Y, s)
                     : launch_decode_t<true, false, false, false, false, true>(src, src2, X, M, N, K, Y, s);
    return out_f32 ? launch_decode_t<false, false, true, false, false, true>(src, src2, X, M, N, K, Y, s)
                   : launch_decode_t<false, false, false, false, false, true>(src, src2, X, M, N, K, Y, s);
  }
#define PATCH_D(B, R, F, U, Q) launch_decode_t<B, R, F, U, Q>(src, src2, X, M, N, K, Y, s)
#define PATCH_D2(B, R, F) (fuse ? PATCH_D(B, R, F, true, false) : PATCH_D(B, R, F, false, false))
#define PATCH_D48(B, F) (fuse ? PATCH_D(B, false, F, true, true) : PATCH_D(B, false, F, false, true))
  if (!rowmajor && n48) {
    if (bf16) return out_f32 ? PATCH_D48(true, true) : PATCH_D48(true, false);
    return out_f32 ? PATCH_D48(false, true) : PATCH_D48(false, false);
  }
  if (bf16) {
    if (rowmajor) return out_f32 ? PATCH_D2(true, true, true) : PATCH_D2(true, true, false);
    return out_f32 ? PATCH_D2(true, false, true) : PATCH_D2(true, false, false);
  }
  if (rowmajor) return out_f32 ? PATCH_D2(false, true, true) : PATCH_D2(false, true, false);
  return out_f32 ? PATCH_D2(false, false, true) : PATCH_D2(false, false, false);
#undef PATCH_D48
#undef PATCH_D2
#undef PATCH_D
}

}  // namespace patch
