// probe.hip -- measurement probes: the ceilings the GEMM kernels are
// compared with, measured on the device they run on (the datasheet gives
// 8 TB/s of HBM and 2.5 PFLOP/s of dense bf16 matrix math; what one launch
// of a given size can reach is lower and is what these kernels measure).
// They compute nothing of the method and are not called by the GEMM path.
#include "device_common.h"
#include "prefill_common.h"

namespace patch {

// Streams n16 16-byte chunks once, grid-stride, four loads in flight a lane;
// the chunks are folded into one word a lane, stored only if it equals a
// constant (so the loads cannot be dropped and almost nothing is written).
__global__ __launch_bounds__(256) void k_probe_read(const u32x4* __restrict__ src, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= src[i];
  const uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (v == 0x9e3779b9u) sink[blockIdx.x] = v;
}

// KIND 0: v_mfma_f32_16x16x32_bf16, 1: v_smfmac_f32_16x16x64_bf16,
// 2: v_mfma_f32_32x32x16_bf16, 3: v_smfmac_f32_32x32x32_bf16.  Eight
// independent accumulator chains a wave, operands in registers.
typedef float f32x16 __attribute__((ext_vector_type(16)));
template <int KIND>
__global__ __launch_bounds__(256) void k_probe_mma(int iters, float* __restrict__ sink) {
  const uint32_t l = threadIdx.x & 63;
  // small bf16 values (1.0 + lane/64 in the high half of each word)
  const uint32_t v = 0x3f803f80u + (l << 16) + l;
  const u32x4 a = {v, v ^ 1u, v ^ 2u, v ^ 3u};
  const u32x8 b = {v, v ^ 4u, v ^ 5u, v ^ 6u, v ^ 7u, v ^ 8u, v ^ 9u, v ^ 10u};
  const int idx = (int)(0x4444u + l);
  // distinct A operands a chain, so no two chains compute the same values
  // (the compiler would merge them into one dependent chain)
  u32x4 aj[8];
#pragma unroll
  for (int j = 0; j < 8; j++) aj[j] = a ^ (uint32_t)(j * 0x00010001u);
  float s = 0.f;
  if constexpr (KIND < 2) {
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; j++) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int j = 0; j < 8; j++) {
        if constexpr (KIND == 0)
          // written out: for this loop the compiler's allocation of the
          // builtin's accumulators adds register copies every iteration
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                       : "+a"(acc[j])
                       : "v"(aj[j]), "v"((u32x4){b[0], b[1], b[2], b[3]}));
        else
          acc[j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, aj[j]),
                                                             __builtin_bit_cast(bf16x16, b), acc[j], idx, 0, 0);
      }
      // keep each chain in its own registers (without this the allocator
      // rotates the accumulators through copies every iteration)
#pragma unroll
      for (int j = 0; j < 8; j++) {
        if constexpr (KIND == 0)
          asm volatile("" : "+a"(acc[j]));
        else
          asm volatile("" : "+v"(acc[j]));
      }
    }
#pragma unroll
    for (int j = 0; j < 8; j++) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  } else {
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int c = 0; c < 16; c++) acc[j][c] = 0.f;
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if constexpr (KIND == 2)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, aj[j]),
                                                           __builtin_bit_cast(bf16x8, (u32x4){b[0], b[1], b[2], b[3]}),
                                                           acc[j], 0, 0, 0);
        else
          acc[j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8, aj[j]),
                                                             __builtin_bit_cast(bf16x16, b), acc[j], idx, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if constexpr (KIND == 2)
          asm volatile("" : "+a"(acc[j]));
        else
          asm volatile("" : "+v"(acc[j]));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int c = 0; c < 16; c++) s += acc[j][c];
  }
  if (s == 1234.5f) sink[blockIdx.x] = s;
}

// Global -> LDS copy rate with the copy instruction the prefill kernels use:
// 8 waves a workgroup, each issuing 7 copies of 1 KB an iteration (16 bytes a
// lane) into one of two LDS slots, waiting for the previous iteration's
// copies (vmcnt) and meeting at a barrier, as the prefill kernels' copy ring
// does.  Workgroup g copies from its window of `window` bytes (a power of
// two) at offset (g * window) mod src_bytes, cycling through it: a few windows in all stay
// in the L2s after the first pass, windows that add up to more than the L2s
// are served from past them.  The LDS is read once at the end (a word
// stored only if it equals a constant), so the copies cannot be dropped.
constexpr int kProbeCopies = 7;
__global__ __launch_bounds__(512) void k_probe_copy(const uint8_t* __restrict__ src, int64_t src_bytes,
                                                    int64_t window, int iters, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[2 * kProbeCopies * 8 * 1024];
  const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint8_t* win = src + ((int64_t)blockIdx.x * window) % src_bytes;
  const uint32_t base = lds_addr(buf);
  for (int it = 0; it < iters; it++) {
    const uint32_t slot = base + (uint32_t)((it & 1) * kProbeCopies * 8 * 1024);
#pragma unroll
    for (int j = 0; j < kProbeCopies; j++) {
      const int64_t c = ((int64_t)it * kProbeCopies + j) * 8 + w;
      dma16(win + ((c << 10) & (window - 1)) + 16 * l, slot + (uint32_t)((j * 8 + w) * 1024));
    }
    wait_copies<kProbeCopies>();  // the previous iteration's copies have landed
    wg_barrier();
  }
  wait_copies<0>();
  __syncthreads();
  if (buf[threadIdx.x] == 0x77 && buf[threadIdx.x + 1] == 0x78) sink[blockIdx.x] = 1u;
}

uint64_t probe_copy_bytes(int iters, int workgroups) {
  return (uint64_t)kProbeCopies * 8u * 1024u * (uint64_t)iters * (uint64_t)workgroups;
}

hipError_t launch_probe_copy(const void* src, uint64_t src_bytes, uint64_t window, int iters, int workgroups,
                             void* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_probe_copy, dim3((unsigned)workgroups), dim3(512), 0, s, reinterpret_cast<const uint8_t*>(src),
                     (int64_t)src_bytes, (int64_t)window, iters, reinterpret_cast<uint32_t*>(sink));
  return hipGetLastError();
}

// Flops (dense-equivalent for the sparse instructions) one launch executes.
uint64_t probe_mma_flops(int kind, int iters, int workgroups) {
  // per instruction: 16x16x32 and 32x32x16 dense = 16384 / 32768; the sparse
  // ones cover twice the K of their dense counterparts
  static const uint64_t per_instr[4] = {2ull * 16 * 16 * 32, 2ull * 16 * 16 * 64, 2ull * 32 * 32 * 16,
                                        2ull * 32 * 32 * 32};
  static const uint64_t chains[4] = {8, 8, 4, 4};
  return per_instr[kind] * chains[kind] * (uint64_t)iters * 4ull * (uint64_t)workgroups;
}

hipError_t launch_probe_read(const void* src, uint64_t bytes, void* sink, uint64_t sink_bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t grid = n16 / (256 * 4);
  grid = grid < 1 ? 1 : (grid > 8192 ? 8192 : grid);
  if ((uint64_t)grid * 4u > sink_bytes) grid = (int64_t)(sink_bytes / 4u);
  if (grid < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_probe_read, dim3((unsigned)grid), dim3(256), 0, s, reinterpret_cast<const u32x4*>(src), n16,
                     reinterpret_cast<uint32_t*>(sink));
  return hipGetLastError();
}

hipError_t launch_probe_mma(int kind, int iters, int workgroups, void* sink, hipStream_t s) {
  float* out = reinterpret_cast<float*>(sink);
  const dim3 g((unsigned)workgroups), b(256);
  switch (kind) {
    case 0: hipLaunchKernelGGL(k_probe_mma<0>, g, b, 0, s, iters, out); break;
    case 1: hipLaunchKernelGGL(k_probe_mma<1>, g, b, 0, s, iters, out); break;
    case 2: hipLaunchKernelGGL(k_probe_mma<2>, g, b, 0, s, iters, out); break;
    case 3: hipLaunchKernelGGL(k_probe_mma<3>, g, b, 0, s, iters, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace patch
