// sampler.hip -- forward hybrid-mask sampler.
//
// PATCH learns two distributions per weight matrix (gist.science explainer,
// section 2 "Methodology: PATCH", "Learnable Distributions"): per tile, dense
// vs 2:4, and per group of four weights inside 2:4 tiles, one of the six 2:4
// patterns; both are sampled with Gumbel-Softmax, and the final mask combines
// the dense option and the 2:4 option with the tile's weights (same section,
// "Hybrid Mask Generation").  This kernel is the forward pass of that
// sampler for 128 x 128 tiles: it produces the hard tile map and 2:4 mask
// that patch_pack consumes, and optionally the soft (differentiable) mask.
//
// Definitions (standard ones; the pages name Gumbel-Softmax only): a
// Gumbel(0, 1) sample from a uniform u in (0, 1) is g = -ln(-ln u); the soft
// sample of logits l_c at temperature tau is y_c = exp((l_c + g_c) / tau) /
// sum_j exp((l_j + g_j) / tau); the hard sample is the one-hot of
// argmax_c (l_c + g_c), the first class winning a tie.  Tile classes are
// (0 dense, 1 sparse); the six patterns are the kept position pairs in
// lexicographic order (0,1), (0,2), (0,3), (1,2), (1,3), (2,3).  The soft
// mask of the weight at position j of its group is y_dense + y_sparse *
// (sum of y_p over the patterns p that keep j).
//
// HBM-bound streaming: one thread per group of four weights.  A workgroup's
// 256 groups of six logits and six uniforms (2 x 6 KB, contiguous) come in
// with 16-byte loads into LDS, and each thread takes its 24-byte records from
// there; the tile's two logits and uniforms (shared by 32 groups of a row)
// are served by the caches; the thread writes the group's four mask bytes
// (one 4-byte store) and four soft values (one 16-byte store).
//
// Scores are float32.  In g = -ln(v), v = -ln(u), the inner logarithm needs
// small *relative* error (v is tiny for u near 1 and its relative error
// becomes g's absolute error), so it is the accurate logf; the outer one and
// the softmax exponentials only need small absolute error in the scores and
// probabilities, and run on the hardware's log2/exp2 approximations.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace patch {
namespace {

constexpr int kSamplerThreads = 256;
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float gumbel(float u) { return -kLn2 * __log2f(-logf(u)); }
__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

__global__ __launch_bounds__(kSamplerThreads) void k_sample_mask(int64_t n_groups, int64_t G, int64_t KT,
                                                                   const float* __restrict__ tile_logits,
                                                                   const float* __restrict__ tile_u,
                                                                   const float* __restrict__ pat_logits,
                                                                   const float* __restrict__ pat_u, float inv_tau,
                                                                   uint8_t* __restrict__ tile_map,
                                                                   uint8_t* __restrict__ mask,
                                                                   float* __restrict__ soft) {
  __shared__ float s_l[6 * kSamplerThreads], s_u[6 * kSamplerThreads];
  const int64_t base = (int64_t)blockIdx.x * kSamplerThreads;  // first group of the workgroup
  const int valid = (int)min((int64_t)kSamplerThreads, n_groups - base);
  // n_groups is a multiple of 32 (K / 4 is), so 6 * valid floats are whole 16-byte chunks
  const int n4 = valid * 6 / 4;
  const float4* gl = reinterpret_cast<const float4*>(pat_logits + 6 * base);
  const float4* gu = reinterpret_cast<const float4*>(pat_u + 6 * base);
  for (int i = threadIdx.x; i < n4; i += kSamplerThreads) {
    reinterpret_cast<float4*>(s_l)[i] = gl[i];
    reinterpret_cast<float4*>(s_u)[i] = gu[i];
  }
  __syncthreads();
  if ((int)threadIdx.x >= valid) return;
  const int64_t gi = base + threadIdx.x;  // group n * G + g
  const int64_t n = gi / G, g = gi - n * G;

  // pattern scores l_p + g_p
  const float2* lp = reinterpret_cast<const float2*>(s_l + 6 * threadIdx.x);
  const float2* up = reinterpret_cast<const float2*>(s_u + 6 * threadIdx.x);
  float s[6];
#pragma unroll
  for (int c = 0; c < 3; c++) {
    const float2 l = lp[c], u = up[c];
    s[2 * c] = l.x + gumbel(u.x);
    s[2 * c + 1] = l.y + gumbel(u.y);
  }
  int best = 0;
  float smax = s[0];
#pragma unroll
  for (int c = 1; c < 6; c++)
    if (s[c] > smax) {
      smax = s[c];
      best = c;
    }
  // kept pair of pattern `best`: first positions 0 0 0 1 1 2, second 1 2 3 2 3 3
  const int a = (0x211000 >> (4 * best)) & 15, b = (0x332321 >> (4 * best)) & 15;
  *reinterpret_cast<uint32_t*>(mask + 4 * gi) = (1u << (8 * a)) | (1u << (8 * b));

  // the tile's two scores (row n, columns 4g..4g+3 lie in tile (n/128, g/32))
  const bool writer = (n & 127) == 0 && (g & 31) == 0;
  if (!writer && !soft) return;
  const int64_t t = (n >> 7) * KT + (g >> 5);
  const float2 tl = reinterpret_cast<const float2*>(tile_logits)[t];
  const float2 tu = reinterpret_cast<const float2*>(tile_u)[t];
  const float sd = tl.x + gumbel(tu.x), ss = tl.y + gumbel(tu.y);
  if (writer) tile_map[t] = ss > sd ? 1 : 0;
  if (!soft) return;

  const float tmax = fmaxf(sd, ss);
  const float ed = fast_exp((sd - tmax) * inv_tau), es = fast_exp((ss - tmax) * inv_tau);
  const float rt = __frcp_rn(ed + es);
  const float y_dense = ed * rt, y_sparse = es * rt;
  float e[6], sum = 0.f;
#pragma unroll
  for (int c = 0; c < 6; c++) {
    e[c] = fast_exp((s[c] - smax) * inv_tau);
    sum += e[c];
  }
  const float r = __frcp_rn(sum);
  // position j is kept by: 0 -> patterns 0 1 2; 1 -> 0 3 4; 2 -> 1 3 5; 3 -> 2 4 5
  const float q0 = (e[0] + e[1] + e[2]) * r, q1 = (e[0] + e[3] + e[4]) * r;
  const float q2 = (e[1] + e[3] + e[5]) * r, q3 = (e[2] + e[4] + e[5]) * r;
  float4 out;
  out.x = y_dense + y_sparse * q0;
  out.y = y_dense + y_sparse * q1;
  out.z = y_dense + y_sparse * q2;
  out.w = y_dense + y_sparse * q3;
  reinterpret_cast<float4*>(soft)[gi] = out;
}

}  // namespace

// N, K: multiples of 128 (checked by the caller); pointers as documented for
// patch_sample_mask; soft may be null.
hipError_t launch_sample_mask(int64_t N, int64_t K, const float* tile_logits, const float* tile_u,
                              const float* pat_logits, const float* pat_u, float tau, uint8_t* tile_map,
                              uint8_t* mask, float* soft, hipStream_t s) {
  const int64_t G = K / 4, n_groups = N * G;
  const int64_t blocks = (n_groups + kSamplerThreads - 1) / kSamplerThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sample_mask, dim3((unsigned)blocks), dim3(kSamplerThreads), 0, s, n_groups, G, K / 128,
                     tile_logits, tile_u, pat_logits, pat_u, 1.0f / tau, tile_map, mask, soft);
  return hipGetLastError();
}

}  // namespace patch
