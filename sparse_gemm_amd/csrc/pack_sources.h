// pack_sources.h -- where the pack kernel reads the rows of a blob's matrix
// from (shared by the kernel and the host side of the C ABI).
#pragma once
#include <cstdint>

namespace patch {

// n row-major sources of K columns: concatenated by rows (source s holds the
// blob's row-blocks start[s] .. start[s+1]-1: several projections packed as
// one), or interleaved row-block by row-block (n = 2: row-block i of the
// blob from source i & 1, its row-block i / 2: a fused gate/up projection).
constexpr int kPackMaxSources = 8;
struct PackSources {
  const uint16_t* W[kPackMaxSources];
  const uint8_t* mask[kPackMaxSources];
  int start[kPackMaxSources + 1];
  int n;
  int interleave;
};

}  // namespace patch
