// device_common.h -- vector types, fragment loads and matrix-core wrappers
// shared by the gfx950 kernels of the hybrid tile-sparse GEMM.
//
// Matrix-core operand layouts used throughout (checked on gfx950 against a
// CPU model for every lane and every 2:4 pattern before any kernel was
// written):
//   v_mfma_f32_16x16x32_{bf16,f16}:  A lane l = row l%16, K 8*(l/16)+t (t<8);
//                                    B lane l = col l%16, K 8*(l/16)+t;
//                                    D lane l, reg r = row 4*(l/16)+r, col l%16.
//   v_smfmac_f32_16x16x64_{bf16,f16}: A lane l = row l%16, 8 stored values
//                                    covering logical K 16*(l/16) .. +15, value
//                                    v in the group of four v/2, its position
//                                    in that group = index bits [2v+1:2v] of
//                                    the 16-bit half selected by ABID;
//                                    B lane l = col l%16, regs 0..7 = K
//                                    8*(l/16)+t, regs 8..15 = K 32+8*(l/16)+t
//                                    (two stacked 16x16x32 B fragments);
//                                    D as for the dense instruction.
#pragma once

#include <hip/hip_runtime.h>

#include "pack_sources.h"
#include <stdint.h>

#include <atomic>

namespace patch {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 128;             // execution tile edge (N and K)
constexpr int kHeaderBytes = 256;
constexpr int kErrFlagOffset = 252;    // reserved header word used by pack to report a bad mask

// A 16-byte chunk loaded by one lane.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 ld16_pred(const void* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? *reinterpret_cast<const u32x4*>(p) : z;
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Dense 16x16x32 step: acc += A(16x32) * B(32x16).
template <bool BF16>
__device__ __forceinline__ f32x4 mma_dense(u32x4 a, u32x4 b, f32x4 acc) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc, 0,
                                                  0, 0);
  }
}

// 2:4 sparse 16x16x64 step: acc += A_sparse(16x64, 8 stored values a lane) * B(64x16).
// b_lo covers logical K 8h..8h+7, b_hi covers 32+8h..32+8h+7 (h = lane/16).
// ABID selects which 16-bit half of `idx` holds this step's 2-bit positions.
template <bool BF16, int ABID>
__device__ __forceinline__ f32x4 mma_sparse(u32x4 a, u32x4 b_lo, u32x4 b_hi, f32x4 acc, uint32_t idx) {
  u32x8 b = {b_lo[0], b_lo[1], b_lo[2], b_lo[3], b_hi[0], b_hi[1], b_hi[2], b_hi[3]};
  if constexpr (BF16) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x16, b),
                                                     acc, (int)idx, 0, ABID);
  } else {
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x16, b), acc,
                                                    (int)idx, 0, ABID);
  }
}

// Store four consecutive outputs Y[row][n..n+3] of one accumulator lane.
// 16-bit outputs are rounded to nearest even (v_cvt_pk_bf16_f32 /
// v_cvt_f16_f32 round to nearest even on gfx950).
template <bool BF16, bool OUT_F32>
__device__ __forceinline__ void store4(void* Y, int64_t elem_off, f32x4 v) {
  if constexpr (OUT_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(Y) + elem_off) = v;
  } else if constexpr (BF16) {
    bf16x4 o = __builtin_convertvector(v, bf16x4);
    *reinterpret_cast<bf16x4*>(reinterpret_cast<uint16_t*>(Y) + elem_off) = o;
  } else {
    f16x4 o = __builtin_convertvector(v, f16x4);
    *reinterpret_cast<f16x4*>(reinterpret_cast<uint16_t*>(Y) + elem_off) = o;
  }
}

constexpr int kDensePieceBytes = 4096;   // one 16-row band of a dense tile
constexpr int kSparsePieceBytes = 2304;  // one band of a 2:4 tile: 2048 of values, 256 of codes
constexpr int kSparseMetaOffset = 2048;  // codes after the values in a 2:4 piece

// One tile-table entry of the packed blob.  Band b's piece of the tile
// starts at offset + b * band_stride.
// SiLU(x) = x / (1 + e^-x), the gate activation of the LLaMA MLP, and the
// gated product SiLU(g) * u, in fp32.
__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }
__device__ __forceinline__ f32x4 silu_mul(f32x4 g, f32x4 u) {
  f32x4 h;
#pragma unroll
  for (int c = 0; c < 4; c++) h[c] = silu_f(g[c]) * u[c];
  return h;
}

// Rebuilding a 4:8 group (four of eight consecutive weights kept): its four
// kept 16-bit values in ascending column order sit in two words (v01 =
// values 0 and 1, v23 = values 2 and 3), i.e. value k in bytes 2k, 2k+1 of
// the byte pool {v23 : v01} that v_perm_b32 selects from (selector bytes
// 0-3 pick v01's bytes, 4-7 v23's, 0x0c a zero byte).  sel48(m) are the four
// selector words that turn the pool into the group's eight elements in
// column order for the position mask m: element p takes the lowest value
// not yet placed if bit p is set, else zero.  Kernels keep sel48 of every
// byte in a 4 KB LDS table, so a group costs one LDS read and four perms.
__device__ __forceinline__ u32x4 sel48(uint32_t m) {
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  uint32_t k = 0;
#pragma unroll
  for (int p = 0; p < 8; p++) {
    const uint32_t kept = (m >> p) & 1u;
    const uint32_t s = kept ? ((2u * k) | ((2u * k + 1u) << 8)) : 0x0c0cu;
    w[p >> 1] |= s << (16 * (p & 1));
    k += kept;
  }
  return (u32x4){w[0], w[1], w[2], w[3]};
}
__device__ __forceinline__ u32x4 expand48(uint32_t v01, uint32_t v23, u32x4 sel) {
  return (u32x4){__builtin_amdgcn_perm(v23, v01, sel[0]), __builtin_amdgcn_perm(v23, v01, sel[1]),
                 __builtin_amdgcn_perm(v23, v01, sel[2]), __builtin_amdgcn_perm(v23, v01, sel[3])};
}
// Fill a 256-entry selector table (every thread of the workgroup calls it;
// the caller synchronises before reading).
__device__ __forceinline__ void fill_sel48(u32x4* table, int tid, int nthreads) {
  for (int m = tid; m < 256; m += nthreads) table[m] = sel48((uint32_t)m);
}

// A lane's sixteen columns of a 4:8 tile's 64-column slice (two groups of
// eight: values v = group 0's four then group 1's four, masks m16 = group 0
// in bits 0-7, group 1 in bits 8-15) -> the lane's chunks of a dense
// piece's two halves: h0 = positions (0,1), h1 = positions (2,3) of each
// group of four, the fixed-pattern operands a dense tile runs on.
__device__ __forceinline__ void dense_halves48(u32x4 v, uint32_t m16, const u32x4* table, u32x4& h0, u32x4& h1) {
  const u32x4 x0 = expand48(v[0], v[1], table[m16 & 0xffu]), x1 = expand48(v[2], v[3], table[(m16 >> 8) & 0xffu]);
  h0 = (u32x4){x0[0], x0[2], x1[0], x1[2]};
  h1 = (u32x4){x0[1], x0[3], x1[1], x1[3]};
}

struct TileEntry {
  uint64_t offset;       // byte offset of the tile's band-0 piece from the blob start
  uint32_t kind;         // 0 dense, 1 sparse
  uint32_t band_stride;  // bytes from one band's pieces to the next in this row-block
};

// Number of compute units of the current device, read once per device (the
// cache is atomic: GEMM calls may come from several host threads).
inline int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace patch
