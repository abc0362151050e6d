// fine_mask.hip -- dense execution tiles of a mask learnt on finer tiles.
//
// PATCH's mask tiles can be as fine as 4 x 4 while the hardware executes
// 128 x 128 tiles (gist.science explainer, section 4 "Ablation Studies",
// "Tile Size").  An execution tile runs as 2:4 only if every fine tile in it
// is 2:4; otherwise it runs dense, and then it must hold W o E_fine: the
// weights its 2:4 fine tiles pruned become +0, the rest keep their bits.
// This kernel writes W o E_fine for the whole matrix (E_fine = 1 in dense
// fine tiles, the mask in 2:4 ones); patch_pack then stores the dense
// execution tiles from it and the 2:4 ones from the mask.
//
// HBM-bound elementwise: one thread per 8 weights of a row (16 bytes of W,
// 8 mask bytes, 16 bytes out); the fine-map bytes of its (at most two) fine
// tiles are shared by neighbouring threads and served by the caches.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace patch {
namespace {

constexpr int kFineThreads = 256;

__global__ __launch_bounds__(kFineThreads) void k_apply_fine_mask(int64_t n_chunks, int64_t K, int b1, int b2,
                                                                    const uint4* W,
                                                                    const uint8_t* __restrict__ fine_map,
                                                                    const uint2* __restrict__ mask,
                                                                    uint4* out) {  // may alias W
  const int64_t c = (int64_t)blockIdx.x * kFineThreads + threadIdx.x;  // chunk of 8 weights
  if (c >= n_chunks) return;
  const int64_t K8 = K / 8;
  const int64_t n = c / K8, k0 = 8 * (c - n * K8);
  const int64_t fKT = K / b2;
  const uint8_t* frow = fine_map + (n / b1) * fKT;
  // the two groups of four: k0..k0+3 and k0+4..k0+7 (b2 % 4 == 0, so each
  // group lies in one fine tile)
  const bool sp0 = frow[k0 / b2] != 0, sp1 = frow[(k0 + 4) / b2] != 0;
  uint4 w = W[c];
  const uint2 m = mask[c];
  uint32_t keep[8];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    keep[j] = !sp0 || ((m.x >> (8 * j)) & 0xffu) != 0;
    keep[4 + j] = !sp1 || ((m.y >> (8 * j)) & 0xffu) != 0;
  }
  uint32_t* wv = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint32_t lo = keep[2 * j] ? 0x0000ffffu : 0u, hi = keep[2 * j + 1] ? 0xffff0000u : 0u;
    wv[j] &= lo | hi;
  }
  out[c] = w;
}

}  // namespace

// N, K multiples of 128, b1 and b2 dividing 128 with b2 % 4 == 0 (checked by
// the caller); W, out 16-byte and mask 8-byte aligned.
hipError_t launch_apply_fine_mask(int64_t N, int64_t K, int b1, int b2, const void* W, const uint8_t* fine_map,
                                  const uint8_t* mask, void* out, hipStream_t s) {
  const int64_t n_chunks = N * K / 8;
  const int64_t blocks = (n_chunks + kFineThreads - 1) / kFineThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_apply_fine_mask, dim3((unsigned)blocks), dim3(kFineThreads), 0, s, n_chunks, K, b1, b2,
                     reinterpret_cast<const uint4*>(W), fine_map, reinterpret_cast<const uint2*>(mask),
                     reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace patch
