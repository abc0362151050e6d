// prefill_common.h -- pieces shared by the prefill (many-token) kernels:
// launch arguments, the swizzled LDS layout of staged rows, global -> LDS
// copies and barriers.
#pragma once

#include "device_common.h"

namespace patch {

constexpr int kPfRowBytes = 128;  // one staged row of X (or row-major W): 64 elements
constexpr int kPfMaxKT = 1024;    // tile columns a workgroup keeps entries of

// Chunk position of 16-byte chunk c (0..7) of staged row r.  The XOR keeps the
// 16 rows read by one B-fragment load on distinct bank groups for both 32- and
// 64-bank LDS: bits (r0 ^ r3, r2, r1) of r.
__device__ __forceinline__ int swz_f(int r) { return (((r ^ (r >> 3)) & 1) << 2) | ((r >> 1) & 3); }
__device__ __forceinline__ int swz(int r, int c) { return r * kPfRowBytes + ((c ^ swz_f(r)) << 4); }

// Workgroup barrier without the fences __syncthreads adds (they would wait
// for every load in flight); callers wait for what they need first.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Raw buffer descriptor: byte addressing from `base`, loads at offsets >=
// `bytes` return zero (word 3 = the gfx9-family raw-buffer format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

struct PfArgs {
  const uint8_t* src;
  const uint8_t* src2;  // fused gate/up with row-major W: the up matrix (src is gate)
  const uint16_t* X;
  void* Y;
  int M, N, K, NT, KT, n_mblk, n_pairs;
  int mg;       // M-blocks per group (the output blocks are ordered group-major)
  int splits;   // K ranges; above 1, Y is the fp32 partial buffer [splits][M][N]
  int kt_split; // tile columns per K range
  int n_blocks, per_xcd;
  // Tail split (tail_s > 1; splits = 1): the first n_full blocks (8 * an
  // XCD's share) run whole; the n_tail blocks after them run in tail_s K
  // ranges of kt_split tile columns, tail_per of them an XCD.  Range k > 0
  // of tail block b hands its fp32 sums to range 0 through slot
  // b * (tail_s - 1) + k - 1 of part (256 x BM floats each, in the lanes'
  // order) and the flag of the same index: it stores token there, which
  // is this launch's own (nonzero) value; range 0 waits for the token and
  // sets the flag back to 0, so every completed launch leaves its flags at
  // 0 and no other launch's value can pass for its own.
  int n_full, n_tail, tail_s, tail_per;
  float* part;
  uint64_t* flags;
  uint64_t token;
  // what range 0 waits for (token, except in tests of the bounded wait) and
  // how many polls it makes before it gives up
  uint64_t wait_token;
  int wait_polls;
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// 16 bytes a lane, global -> LDS: lane l's bytes land at LDS byte lds + 16 l
// (M0 holds the LDS base; it is saved and restored around the copy).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(g)
      : "memory");
}
// 4 bytes a lane, global -> LDS: lane l's bytes land at LDS byte lds + 4 l.
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(g)
      : "memory");
}
// N copies global -> LDS issued back to back in one block (M0 saved once):
// copy k moves lane l's 16 bytes (W16) or 4 bytes from the global address
// src[k] + voff[k] (src[k] wave-uniform, in SGPRs; voff[k] the lane's byte
// offset) to LDS byte lds + k * LS + 16 l (4 l).  The address arithmetic
// stays scalar: one 64-bit scalar add per copy where a per-lane pointer
// would cost two vector adds.  M0 is only ever moved into (s_mov leaves
// SCC alone, which the compiler may keep live across the block).
template <int N, int LS, bool W16>
__device__ __forceinline__ void dma_n(const uint8_t* const (&src)[N], const uint32_t (&voff)[N], uint32_t lds) {
  static_assert(N >= 1 && N <= 4, "1 to 4 copies");
  const uint32_t m1 = lds + (uint32_t)LS, m2 = lds + 2u * (uint32_t)LS, m3 = lds + 3u * (uint32_t)LS;
  uint32_t saved;
  if constexpr (N == 1) {
    if constexpr (W16)
      asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                   : "=&s"(saved) : "s"(lds), "v"(voff[0]), "s"(src[0]) : "memory");
    else
      asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
                   : "=&s"(saved) : "s"(lds), "v"(voff[0]), "s"(src[0]) : "memory");
  } else if constexpr (N == 2) {
    if constexpr (W16)
      asm volatile(
          "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
          "global_load_lds_dwordx4 %3, %5\n\ts_mov_b32 m0, %2\n\t"
          "global_load_lds_dwordx4 %4, %6\n\ts_mov_b32 m0, %0"
          : "=&s"(saved) : "s"(lds), "s"(m1), "v"(voff[0]), "v"(voff[1]), "s"(src[0]), "s"(src[1]) : "memory");
    else
      asm volatile(
          "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
          "global_load_lds_dword %3, %5\n\ts_mov_b32 m0, %2\n\t"
          "global_load_lds_dword %4, %6\n\ts_mov_b32 m0, %0"
          : "=&s"(saved) : "s"(lds), "s"(m1), "v"(voff[0]), "v"(voff[1]), "s"(src[0]), "s"(src[1]) : "memory");
  } else if constexpr (N == 3) {
    if constexpr (W16)
      asm volatile(
          "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
          "global_load_lds_dwordx4 %4, %7\n\ts_mov_b32 m0, %2\n\t"
          "global_load_lds_dwordx4 %5, %8\n\ts_mov_b32 m0, %3\n\t"
          "global_load_lds_dwordx4 %6, %9\n\ts_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(lds), "s"(m1), "s"(m2), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "s"(src[0]), "s"(src[1]),
            "s"(src[2])
          : "memory");
    else
      asm volatile(
          "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
          "global_load_lds_dword %4, %7\n\ts_mov_b32 m0, %2\n\t"
          "global_load_lds_dword %5, %8\n\ts_mov_b32 m0, %3\n\t"
          "global_load_lds_dword %6, %9\n\ts_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(lds), "s"(m1), "s"(m2), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "s"(src[0]), "s"(src[1]),
            "s"(src[2])
          : "memory");
  } else {
    if constexpr (W16)
      asm volatile(
          "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
          "global_load_lds_dwordx4 %5, %9\n\ts_mov_b32 m0, %2\n\t"
          "global_load_lds_dwordx4 %6, %10\n\ts_mov_b32 m0, %3\n\t"
          "global_load_lds_dwordx4 %7, %11\n\ts_mov_b32 m0, %4\n\t"
          "global_load_lds_dwordx4 %8, %12\n\ts_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(lds), "s"(m1), "s"(m2), "s"(m3), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]),
            "s"(src[0]), "s"(src[1]), "s"(src[2]), "s"(src[3])
          : "memory");
    else
      asm volatile(
          "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
          "global_load_lds_dword %5, %9\n\ts_mov_b32 m0, %2\n\t"
          "global_load_lds_dword %6, %10\n\ts_mov_b32 m0, %3\n\t"
          "global_load_lds_dword %7, %11\n\ts_mov_b32 m0, %4\n\t"
          "global_load_lds_dword %8, %12\n\ts_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(lds), "s"(m1), "s"(m2), "s"(m3), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]),
            "s"(src[0]), "s"(src[1]), "s"(src[2]), "s"(src[3])
          : "memory");
  }
}

template <int N>
__device__ __forceinline__ void wait_copies() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace patch
