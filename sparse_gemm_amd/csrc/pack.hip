// pack.hip -- dense W + tile map + 2:4 / 4:8 mask -> packed blob (format
// version 3, 128 x 128 execution tiles); dense W + quadrant map + 2:4 mask ->
// format version 4 (64 x 64 execution tiles, k_pack_q64 below).
//
// PATCH (arXiv 2509.23410), gist.science explainer, section 2 "Core
// Mechanism": every 128 x 128 tile of W is dense or 2:4 sparse; section 1
// "Problem Statement": a 2:4 group keeps two of four consecutive weights;
// section 2 "Pattern Selection": six possible patterns per group.
//
// Layout (the host writes the header and the tile table before this kernel
// runs): a piece is one 16-row band of one tile; inside a row-block each
// band's pieces of all tiles are back to back (band b of tile (i, j) at the
// table entry's offset + b * band_stride).  Lane l (row l%16 of the band,
// column group l/16) owns 16 bytes at 16*l of each 1 KB block of a piece:
//   dense piece (4096 B): blocks (q, e) at 2048*q + 1024*e hold, of the four
//       groups of four at columns 64*q + 16*(l/16) .. +15, the elements at
//       positions 2e and 2e+1 of each group (group order, then column order):
//       two halves that are 2:4 operands with the fixed patterns (0,1) and
//       (2,3);
//   2:4 piece (2304 B): block q at 1024*q holds the two kept values
//       (ascending column) of groups g = 16*q + 4*(l/16) + p, p = 0..3; then
//       at 2048 + 4*l the lane's word of codes i0 | i1 << 2 (bits 16*q + 4*p);
//   4:8 piece (2304 B; other N:M patterns, explainer section 5 "Future
//       Direction"): lane l's columns 64*q + 16*(l/16) .. +15 of slice q are
//       two groups of eight u = 0, 1; block q at 1024*q holds the four kept
//       values (ascending column) of group 0, then of group 1; at 2048 + 4*l
//       the lane's word whose byte 2q + u is group u's kept-position mask
//       (the sixteen columns a lane holds of a dense piece's two halves, which
//       the GEMM kernels rebuild in place).
// These are the lane orders of the A operand and index of
// v_smfmac_f32_16x16x64, for both tile kinds, so the GEMM kernels load each
// 1 KB fragment with one coalesced 16-byte load a lane, run dense and 2:4
// tiles on the same instruction, and a kernel that owns one band of a
// row-block streams one contiguous range.
#include "device_common.h"

namespace patch {

// grid: T * 4 workgroups of 256 threads; thread c = 256 * (blockIdx.x & 3)
// + threadIdx.x of tile t = blockIdx.x / 4 (c = 0 .. 1023) writes lane
// l = c & 63's share of 64-column slice q = c >> 9 of band (c >> 6) & 7, so
// every thread has work for every tile kind.
// The blob's matrix is assembled from up to kPackMaxSources row-major
// matrices of K columns (PackSources): concatenated by rows (several
// projections packed as one), or -- interleave -- row-block ib taken from
// source ib & 1, row-block ib / 2 (a fused gate/up projection).
__global__ __launch_bounds__(256) void k_pack(PackSources src, int K, int KT, uint8_t* __restrict__ blob) {
  const int t = blockIdx.x >> 2;
  const int c = ((blockIdx.x & 3) << 8) | threadIdx.x;
  const int q = c >> 9, band = (c >> 6) & 7, l = c & 63;
  const TileEntry e = reinterpret_cast<const TileEntry*>(blob + kHeaderBytes)[t];
  const int ib = t / KT, j = t - (t / KT) * KT;
  // source matrix and its row-block for blob row-block ib
  int si = 0, i = ib;
  if (src.interleave) {
    si = ib & 1;
    i = ib >> 1;
  } else {
    while (si + 1 < src.n && ib >= src.start[si + 1]) si++;
    i = ib - src.start[si];
  }
  const uint16_t* __restrict__ W = src.W[si];
  const uint8_t* __restrict__ mask = src.mask[si];
  const int64_t row = (int64_t)i * kTile + 16 * band + (l & 15);
  const int64_t col = (int64_t)j * kTile + 64 * q + 16 * (l >> 4);
  uint8_t* piece = blob + e.offset + (uint64_t)band * e.band_stride;
  if (e.kind == 0) {
    // 16 elements = 8 words of two; group g is words 2g (positions 0, 1) and
    // 2g+1 (positions 2, 3)
    const u32x4 w0 = ld16(W + row * K + col), w1 = ld16(W + row * K + col + 8);
    const u32x4 h0 = {w0[0], w0[2], w1[0], w1[2]};
    const u32x4 h1 = {w0[1], w0[3], w1[1], w1[3]};
    uint8_t* dst = piece + 2048 * q + 16 * l;
    st16(dst, h0);
    st16(dst + 1024, h1);
    return;
  }
  // slice q's half of the lane's codes word (bits 16q .. 16q+15)
  uint32_t meta = 0;
  bool bad = false;
  if (e.kind == 2) {
    // this lane's sixteen columns of slice q: groups u = 0, 1 of eight
    uint32_t vals[4];
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const u32x4 w = ld16(W + row * K + col + 8 * u);
      const uint2 mk = *reinterpret_cast<const uint2*>(mask + row * K + col + 8 * u);
      uint32_t kept[4] = {0u, 0u, 0u, 0u}, bits = 0;
      int n = 0;
#pragma unroll
      for (int p = 0; p < 8; p++) {
        const uint32_t mb = ((p < 4 ? mk.x : mk.y) >> (8 * (p & 3))) & 0xffu;
        const uint32_t v = (w[p >> 1] >> (16 * (p & 1))) & 0xffffu;
        if (mb) {
          if (n < 4) kept[n] = v;
          bits |= 1u << p;
          n++;
        }
      }
      bad |= (n != 4);
      vals[2 * u] = kept[0] | (kept[1] << 16);
      vals[2 * u + 1] = kept[2] | (kept[3] << 16);
      meta |= bits << (8 * u);
    }
    const u32x4 o = {vals[0], vals[1], vals[2], vals[3]};
    st16(piece + 1024 * q + 16 * l, o);
  } else {
    const u32x4 w0 = ld16(W + row * K + col), w1 = ld16(W + row * K + col + 8);
    const u32x4 m4 = ld16(mask + row * K + col);
    uint16_t wv[16];
#pragma unroll
    for (int d = 0; d < 4; d++) {
      wv[2 * d] = (uint16_t)(w0[d] & 0xffffu);
      wv[2 * d + 1] = (uint16_t)(w0[d] >> 16);
      wv[8 + 2 * d] = (uint16_t)(w1[d] & 0xffffu);
      wv[8 + 2 * d + 1] = (uint16_t)(w1[d] >> 16);
    }
    uint32_t outv[4];
#pragma unroll
    for (int p = 0; p < 4; p++) {
      const uint32_t mword = m4[p];  // mask bytes of group p (4 columns)
      uint32_t kept[2] = {0u, 0u};
      uint32_t pos[2] = {0u, 0u};
      int n = 0;
#pragma unroll
      for (int d = 0; d < 4; d++) {
        if ((mword >> (8 * d)) & 0xffu) {
          if (n < 2) {
            kept[n] = wv[4 * p + d];
            pos[n] = (uint32_t)d;
          }
          n++;
        }
      }
      bad |= (n != 2);
      outv[p] = kept[0] | (kept[1] << 16);
      meta |= (pos[0] | (pos[1] << 2)) << (4 * p);
    }
    const u32x4 o = {outv[0], outv[1], outv[2], outv[3]};
    st16(piece + 1024 * q + 16 * l, o);
  }
  // the two slices' threads write the two halves of the lane's word
  reinterpret_cast<uint16_t*>(piece + kSparseMetaOffset)[2 * l + q] = (uint16_t)meta;
  if (bad) atomicOr(reinterpret_cast<uint32_t*>(blob + kErrFlagOffset), 1u);
}

// Format 4 (64 x 64 execution tiles): grid = one workgroup of 256 threads
// per table entry (a 64-row half-row-block r and a tile column j); thread
// (band, l) writes lane l's share of band `band` (0..3) of the entry's
// piece: each 64-column slice q in order -- dense: two 1 KB halves holding
// positions (0,1) and (2,3) of each group of four (2048 bytes); 2:4: the kept
// values (1024 bytes) -- then, if either slice is 2:4, the lane's codes word
// (slice q's codes in bits 16q .. 16q+15) in the 256-byte block after them.
__global__ __launch_bounds__(256) void k_pack_q64(const uint16_t* __restrict__ W, const uint8_t* __restrict__ mask,
                                                  int K, int KC, uint8_t* __restrict__ blob) {
  const int t = blockIdx.x;
  const TileEntry e = reinterpret_cast<const TileEntry*>(blob + kHeaderBytes)[t];
  const int r = t / KC, j = t - (t / KC) * KC;
  const int band = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t row = (int64_t)r * 64 + 16 * band + (l & 15);
  uint8_t* piece = blob + e.offset + (uint64_t)band * e.band_stride;
  const uint32_t a1 = (e.kind & 1u) ? 1024u : 2048u;
  uint32_t meta = 0;
  bool bad = false;
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const int64_t col = (int64_t)j * kTile + 64 * q + 16 * (l >> 4);
    const u32x4 w0 = ld16(W + row * K + col), w1 = ld16(W + row * K + col + 8);
    uint8_t* part = piece + (q ? a1 : 0u);
    if (!((e.kind >> q) & 1u)) {
      const u32x4 h0 = {w0[0], w0[2], w1[0], w1[2]};
      const u32x4 h1 = {w0[1], w0[3], w1[1], w1[3]};
      st16(part + 16 * l, h0);
      st16(part + 1024 + 16 * l, h1);
      continue;
    }
    const u32x4 m4 = ld16(mask + row * K + col);
    uint32_t outv[4];
#pragma unroll
    for (int p = 0; p < 4; p++) {
      const uint32_t mword = m4[p];  // mask bytes of group p (4 columns)
      const u32x4& wsrc = p < 2 ? w0 : w1;
      const uint32_t wlo = wsrc[2 * (p & 1)], whi = wsrc[2 * (p & 1) + 1];  // positions 0,1 and 2,3
      uint32_t kept[2] = {0u, 0u}, pos[2] = {0u, 0u};
      int n = 0;
#pragma unroll
      for (int d = 0; d < 4; d++) {
        if ((mword >> (8 * d)) & 0xffu) {
          const uint32_t v = ((d < 2 ? wlo : whi) >> (16 * (d & 1))) & 0xffffu;
          if (n < 2) {
            kept[n] = v;
            pos[n] = (uint32_t)d;
          }
          n++;
        }
      }
      bad |= (n != 2);
      outv[p] = kept[0] | (kept[1] << 16);
      meta |= (pos[0] | (pos[1] << 2)) << (16 * q + 4 * p);
    }
    const u32x4 o = {outv[0], outv[1], outv[2], outv[3]};
    st16(part + 16 * l, o);
  }
  if (e.kind) {
    const uint32_t codes = a1 + ((e.kind & 2u) ? 1024u : 2048u);
    reinterpret_cast<uint32_t*>(piece + codes)[l] = meta;
  }
  if (bad) atomicOr(reinterpret_cast<uint32_t*>(blob + kErrFlagOffset), 1u);
}

hipError_t launch_pack_q64(const void* W, const uint8_t* mask, int64_t N, int64_t K, uint8_t* blob, hipStream_t s) {
  const int KC = (int)(K / kTile);
  const int64_t E = (N / 64) * KC;
  hipLaunchKernelGGL(k_pack_q64, dim3((unsigned)E), dim3(256), 0, s, reinterpret_cast<const uint16_t*>(W), mask,
                     (int)K, KC, blob);
  return hipGetLastError();
}

hipError_t launch_pack(const PackSources& src, int64_t N, int64_t K, uint8_t* blob, hipStream_t s) {
  const int KT = (int)(K / kTile);
  const int64_t T = (N / kTile) * KT;
  hipLaunchKernelGGL(k_pack, dim3((unsigned)(T * 4)), dim3(256), 0, s, src, (int)K, KT, blob);
  return hipGetLastError();
}

}  // namespace patch
