// gemm_decode.hip -- weight-streaming hybrid GEMM for few tokens (M <= 16).
//
// PATCH (arXiv 2509.23410), gist.science explainer, section 2 "Inference &
// Deployment": dense tiles run on the dense matrix path and 2:4 tiles on the
// sparse one.  With M <= 16 the product is bound by the bytes of W, so the
// kernel streams each tile's packed bytes exactly once:
//
//   * one workgroup per 16-row band of W (N/16 workgroups) and all of K;
//   * the workgroup first splits the band's row-block into a list of dense
//     and a list of sparse tiles (from the tile table), then its waves take
//     tiles round-robin from each list, so every wave gets an equal share of
//     each kind;
//   * a tile's 16 x 128 band is 4 (dense) or 2 (sparse) 1 KB fragments that a
//     wave loads with one 16-byte load per lane each, straight into the A
//     operand registers; X (at most 16 rows) is read from L2 into the B
//     operand registers, zero for rows >= M;
//   * dense: 4 x v_mfma_f32_16x16x32; sparse: 2 x v_smfmac_f32_16x16x64;
//   * loads run DEPTH tiles ahead of the matrix instructions;
//   * the waves' fp32 partial sums are added in LDS in wave order (fixed, so
//     results are deterministic) and rounded to the output type.
//
// The same kernel with SRC_ROWMAJOR reads plain row-major W (every tile
// dense): that is the same-shape dense baseline.
#include "device_common.h"

namespace patch {

constexpr int kDecodeWaves = 8;
constexpr int kDecodeMaxKT = 1024;  // K <= 131072

struct DecodeFrag {
  u32x4 x[4];  // B operand chunks: X[m][k0 + 32c + 8h .. +7], c = 0..3
  u32x4 a[4];  // A operand chunks (dense: 4 slices; sparse: 2 slices in a[0..1])
  uint32_t meta;
};

template <bool SRC_ROWMAJOR>
__device__ __forceinline__ void decode_load_dense(DecodeFrag& f, const uint8_t* __restrict__ src, uint64_t tile_off,
                                                  const uint16_t* __restrict__ X, int K, int M, int i, int b, int j,
                                                  int l) {
  const int m = l & 15, h = l >> 4;
  const bool mok = m < M;
  const uint16_t* xr = X + (int64_t)(mok ? m : 0) * K + (int64_t)j * kTile + 8 * h;
#pragma unroll
  for (int c = 0; c < 4; c++) f.x[c] = ld16_pred(xr + 32 * c, mok);
  if constexpr (SRC_ROWMAJOR) {
    const uint16_t* W = reinterpret_cast<const uint16_t*>(src);
    const uint16_t* wr = W + ((int64_t)i * kTile + 16 * b + m) * K + (int64_t)j * kTile + 8 * h;
#pragma unroll
    for (int c = 0; c < 4; c++) f.a[c] = ld16(wr + 32 * c);
  } else {
    const uint8_t* tp = src + tile_off + 1024 * b + 16 * l;
#pragma unroll
    for (int c = 0; c < 4; c++) f.a[c] = ld16(tp + 8192 * c);
  }
}

__device__ __forceinline__ void decode_load_sparse(DecodeFrag& f, const uint8_t* __restrict__ src, uint64_t tile_off,
                                                   const uint16_t* __restrict__ X, int K, int M, int b, int j, int l) {
  const int m = l & 15, h = l >> 4;
  const bool mok = m < M;
  const uint16_t* xr = X + (int64_t)(mok ? m : 0) * K + (int64_t)j * kTile + 8 * h;
#pragma unroll
  for (int c = 0; c < 4; c++) f.x[c] = ld16_pred(xr + 32 * c, mok);
  const uint8_t* tp = src + tile_off + 1024 * b + 16 * l;
  f.a[0] = ld16(tp);
  f.a[1] = ld16(tp + 8192);
  f.meta = *reinterpret_cast<const uint32_t*>(src + tile_off + kSparseValBytes + 4 * (64 * b + l));
}

template <bool BF16>
__device__ __forceinline__ f32x4 decode_mma_dense(const DecodeFrag& f, f32x4 acc) {
#pragma unroll
  for (int c = 0; c < 4; c++) acc = mma_dense<BF16>(f.a[c], f.x[c], acc);
  return acc;
}

template <bool BF16>
__device__ __forceinline__ f32x4 decode_mma_sparse(const DecodeFrag& f, f32x4 acc) {
  // slice 0: logical K 0..63 of the tile -> B chunks 0 (K 8h..) and 1 (K 32+8h..)
  acc = mma_sparse<BF16, 0>(f.a[0], f.x[0], f.x[1], acc, f.meta);
  // slice 1: logical K 64..127 -> B chunks 2 and 3
  acc = mma_sparse<BF16, 1>(f.a[1], f.x[2], f.x[3], acc, f.meta);
  return acc;
}

template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32, int DEPTH>
__global__ __launch_bounds__(kDecodeWaves * 64) void k_decode(const uint8_t* __restrict__ src,
                                                               const uint16_t* __restrict__ X, int M, int N, int K,
                                                               void* __restrict__ Y) {
  const int KT = K / kTile;
  const int band_g = blockIdx.x;  // 16-row band of W
  const int i = band_g >> 3, b = band_g & 7;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;

  __shared__ uint32_t s_list[2][kDecodeMaxKT];  // [0] dense tiles, [1] sparse tiles: (j << 0), offsets below
  __shared__ uint64_t s_off[2][kDecodeMaxKT];
  __shared__ int s_count[2];
  __shared__ f32x4 s_red[kDecodeWaves][64];

  int nd, ns;
  if constexpr (SRC_ROWMAJOR) {
    nd = KT;
    ns = 0;
  } else {
    // Split this row-block's tiles into a dense and a sparse list (in column order).
    const TileEntry* table = reinterpret_cast<const TileEntry*>(src + kHeaderBytes) + (int64_t)i * KT;
    if (w == 0) {
      int base_d = 0, base_s = 0;
      for (int c0 = 0; c0 < KT; c0 += 64) {
        const int jj = c0 + l;
        const bool valid = jj < KT;
        TileEntry e = {0, 0, 0};
        if (valid) e = table[jj];
        const bool sp = valid && e.kind != 0;
        const bool de = valid && e.kind == 0;
        const uint64_t bs = __ballot(sp), bd = __ballot(de);
        const uint64_t lt = (l == 0) ? 0ull : (~0ull >> (64 - l));
        if (de) {
          const int r = base_d + __popcll(bd & lt);
          s_list[0][r] = (uint32_t)jj;
          s_off[0][r] = e.offset;
        }
        if (sp) {
          const int r = base_s + __popcll(bs & lt);
          s_list[1][r] = (uint32_t)jj;
          s_off[1][r] = e.offset;
        }
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

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  // ---- dense tiles: wave w takes list entries w, w + 8, ...
  if (w < nd) {
    DecodeFrag f[DEPTH];
#pragma unroll
    for (int s = 0; s < DEPTH; s++) {
      const int e = min(w + s * kDecodeWaves, nd - 1);
      const int j = SRC_ROWMAJOR ? e : (int)s_list[0][e];
      const uint64_t off = SRC_ROWMAJOR ? 0 : s_off[0][e];
      decode_load_dense<SRC_ROWMAJOR>(f[s], src, off, X, K, M, i, b, j, l);
    }
    for (int base = w; base < nd; base += DEPTH * kDecodeWaves) {
#pragma unroll
      for (int s = 0; s < DEPTH; s++) {
        const int e = base + s * kDecodeWaves;
        if (e < nd) acc = decode_mma_dense<BF16>(f[s], acc);
        const int en = min(e + DEPTH * kDecodeWaves, nd - 1);
        const int j = SRC_ROWMAJOR ? en : (int)s_list[0][en];
        const uint64_t off = SRC_ROWMAJOR ? 0 : s_off[0][en];
        decode_load_dense<SRC_ROWMAJOR>(f[s], src, off, X, K, M, i, b, j, l);
      }
    }
  }
  // ---- sparse tiles
  if constexpr (!SRC_ROWMAJOR) {
    if (w < ns) {
      DecodeFrag f[DEPTH];
#pragma unroll
      for (int s = 0; s < DEPTH; s++) {
        const int e = min(w + s * kDecodeWaves, ns - 1);
        decode_load_sparse(f[s], src, s_off[1][e], X, K, M, b, (int)s_list[1][e], l);
      }
      for (int base = w; base < ns; base += DEPTH * kDecodeWaves) {
#pragma unroll
        for (int s = 0; s < DEPTH; s++) {
          const int e = base + s * kDecodeWaves;
          if (e < ns) acc = decode_mma_sparse<BF16>(f[s], acc);
          const int en = min(e + DEPTH * kDecodeWaves, ns - 1);
          decode_load_sparse(f[s], src, s_off[1][en], X, K, M, b, (int)s_list[1][en], l);
        }
      }
    }
  }

  // ---- fixed-order reduction over waves, then round and store
  s_red[w][l] = acc;
  __syncthreads();
  if (w == 0) {
    f32x4 sum = s_red[0][l];
#pragma unroll
    for (int ww = 1; ww < kDecodeWaves; ww++) sum += s_red[ww][l];
    const int m = l & 15;
    if (m < M) {
      const int64_t n = (int64_t)i * kTile + 16 * b + 4 * (l >> 4);
      store4<BF16, OUT_F32>(Y, (int64_t)m * N + n, sum);
    }
  }
}

template <bool BF16, bool SRC_ROWMAJOR, bool OUT_F32>
static hipError_t launch_decode_t(const void* src, const void* X, int64_t M, int64_t N, int64_t K, void* Y,
                                  hipStream_t s) {
  const unsigned grid = (unsigned)(N / 16);
  hipLaunchKernelGGL((k_decode<BF16, SRC_ROWMAJOR, OUT_F32, 2>), dim3(grid), dim3(kDecodeWaves * 64), 0, s,
                     reinterpret_cast<const uint8_t*>(src), reinterpret_cast<const uint16_t*>(X), (int)M, (int)N,
                     (int)K, Y);
  return hipGetLastError();
}

hipError_t launch_decode(bool bf16, bool rowmajor, bool out_f32, const void* src, const void* X, int64_t M, int64_t N,
                         int64_t K, void* Y, hipStream_t s) {
  if (bf16) {
    if (rowmajor) return out_f32 ? launch_decode_t<true, true, true>(src, X, M, N, K, Y, s)
                                 : launch_decode_t<true, true, false>(src, X, M, N, K, Y, s);
    return out_f32 ? launch_decode_t<true, false, true>(src, X, M, N, K, Y, s)
                   : launch_decode_t<true, false, false>(src, X, M, N, K, Y, s);
  }
  if (rowmajor) return out_f32 ? launch_decode_t<false, true, true>(src, X, M, N, K, Y, s)
                               : launch_decode_t<false, true, false>(src, X, M, N, K, Y, s);
  return out_f32 ? launch_decode_t<false, false, true>(src, X, M, N, K, Y, s)
                 : launch_decode_t<false, false, false>(src, X, M, N, K, Y, s);
}

}  // namespace patch
