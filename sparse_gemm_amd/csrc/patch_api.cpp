// patch_api.cpp -- host side of the C ABI declared in include/patch.h:
// argument validation, the packed header and tile table, kernel selection.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "pack_sources.h"
#include "patch.h"

namespace patch {
hipError_t launch_pack(const PackSources& src, int64_t N, int64_t K, uint8_t* blob, hipStream_t s);
hipError_t launch_pack_q64(const void* W, const uint8_t* mask, int64_t N, int64_t K, uint8_t* blob, hipStream_t s);
hipError_t launch_decode(bool bf16, bool rowmajor, bool out_f32, const void* src, const void* src2, const void* X,
                         int64_t M, int64_t N, int64_t K, void* Y, bool n48, bool q64, hipStream_t s);
hipError_t launch_prefill(bool bf16, bool rowmajor, bool out_f32, const void* src, const void* src2, const void* X,
                          int64_t M, int64_t N, int64_t K, void* Y, void* ws, uint64_t ws_bytes, int force_bm,
                          bool force_lds, int force_big, bool q64, hipStream_t s);
uint64_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K, bool rowmajor);
double prefill_estimate_us(int64_t M, int64_t N, int64_t K, bool rowmajor, uint64_t ws_bytes);
void tail_wait_test(int polls);
double decode_estimate_us(int64_t M, int64_t N, int64_t K, double w_bytes);
hipError_t launch_sample_mask(int64_t N, int64_t K, const float* tile_logits, const float* tile_u,
                              const float* pat_logits, const float* pat_u, float tau, uint8_t* tile_map,
                              uint8_t* mask, float* soft, hipStream_t s);
hipError_t launch_apply_fine_mask(int64_t N, int64_t K, int b1, int b2, const void* W, const uint8_t* fine_map,
                                  const uint8_t* mask, void* out, hipStream_t s);
hipError_t launch_probe_read(const void* src, uint64_t bytes, void* sink, uint64_t sink_bytes, hipStream_t s);
hipError_t launch_probe_mma(int kind, int iters, int workgroups, void* sink, hipStream_t s);
uint64_t probe_mma_flops(int kind, int iters, int workgroups);
hipError_t launch_probe_copy(const void* src, uint64_t src_bytes, uint64_t window, int iters, int workgroups,
                             void* sink, hipStream_t s);
uint64_t probe_copy_bytes(int iters, int workgroups);
}  // namespace patch

namespace {

constexpr uint32_t kMagic = 0x48435450u;  // "PTCH"
constexpr uint32_t kVersion = 3;     // 128 x 128 execution tiles
constexpr uint32_t kVersionQ64 = 4;  // 64 x 64 execution tiles
constexpr int64_t kQuad = 64;        // their edge
constexpr int64_t kTile = 128;
constexpr uint64_t kDenseBytes = 32768;
constexpr uint64_t kSparseBytes = 18432;
constexpr uint64_t kDensePiece = 4096;   // one 16-row band of a dense tile
constexpr uint64_t kSparsePiece = 2304;  // one band of a 2:4 tile: values + codes
constexpr int64_t kMaxDim = int64_t(1) << 20;  // N, K upper bound (int32 indexing inside kernels)
constexpr int64_t kMaxKT = 1024;              // prefill kernel's per-workgroup tile lists
constexpr int64_t kDecodeMaxK = 65536;        // decode kernel: <= 64 tile columns per wave
constexpr int64_t kDecodeMaxM = 128;          // decode kernel: <= 8 blocks of 16 columns of M
constexpr int64_t kDecodeAutoM = 16;          // AUTO: always decode up to here
constexpr uint64_t kErrFlagOffset = 252;
// the prefill kernels keep a tile's piece offset / 256 in 30 bits
constexpr uint64_t kMaxBlobBytes = uint64_t(1) << 38;

thread_local std::string g_err;

patch_status fail(patch_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

}  // namespace

namespace patch {
patch_status set_last_error(patch_status s, const char* msg) {
  g_err = msg;
  return s;
}
}  // namespace patch

namespace {

patch_status hip_fail(hipError_t e, const char* what) {
  return fail(PATCH_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

patch_status check_nk(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N % kTile || K % kTile)
    return fail(PATCH_ERR_SHAPE, "N=%lld K=%lld must be positive multiples of 128", (long long)N, (long long)K);
  if (N > kMaxDim || K > kMaxDim || K / kTile > kMaxKT)
    return fail(PATCH_ERR_SHAPE, "N=%lld K=%lld exceed the supported maximum (%lld, K/128 <= %lld)", (long long)N,
                (long long)K, (long long)kMaxDim, (long long)kMaxKT);
  return PATCH_OK;
}

patch_status check_dtype(patch_dtype dt) {
  if (dt != PATCH_F16 && dt != PATCH_BF16) return fail(PATCH_ERR_INVALID_ARG, "dtype %d is not F16 or BF16", (int)dt);
  return PATCH_OK;
}

patch_status check_ydtype(patch_dtype in, patch_dtype y) {
  if (y != in && y != PATCH_F32)
    return fail(PATCH_ERR_INVALID_ARG, "y_dtype %d must equal the input dtype %d or be F32", (int)y, (int)in);
  return PATCH_OK;
}

// Format 4: bytes of one band piece of a table entry with kind bits kb
// (bit q: 64-column slice q is 2:4), and of the whole blob for a quadrant map.
uint64_t q64_piece(uint32_t kb) { return (kb & 1u ? 1024u : 2048u) + (kb & 2u ? 1024u : 2048u) + (kb ? 256u : 0u); }

patch_status check_desc_q64(const patch_packed_desc* d) {
  if (d->tile_n != kQuad || d->tile_k != kQuad) return fail(PATCH_ERR_INVALID_ARG, "descriptor version/tile mismatch");
  if (check_dtype((patch_dtype)d->dtype)) return PATCH_ERR_INVALID_ARG;
  patch_status s = check_nk(d->N, d->K);
  if (s) return s;
  const uint64_t Tq = (uint64_t)d->nt_n * d->nt_k, E = (uint64_t)(d->N / kQuad) * (uint64_t)(d->K / kTile);
  // the data take 8192 bytes a dense quadrant, 4096 a 2:4 one and 1024 a
  // table entry with a 2:4 slice (at most one per 2:4 quadrant)
  const uint64_t base = d->data_offset + 8192u * (Tq - d->n_sparse) + 4096u * d->n_sparse;
  if (d->nt_n != d->N / kQuad || d->nt_k != d->K / kQuad || d->n_sparse > Tq || d->n_48 != 0 ||
      d->table_offset != 256 || d->data_offset != round_up(256 + 16 * E, 256) || d->total_bytes < base ||
      d->total_bytes > base + 1024u * std::min<uint64_t>(d->n_sparse, E) || (d->total_bytes - base) % 1024u)
    return fail(PATCH_ERR_INVALID_ARG, "inconsistent descriptor");
  if (d->total_bytes >= kMaxBlobBytes)
    return fail(PATCH_ERR_UNSUPPORTED, "blob of %llu bytes exceeds the supported %llu",
                (unsigned long long)d->total_bytes, (unsigned long long)kMaxBlobBytes);
  return PATCH_OK;
}

patch_status check_desc(const patch_packed_desc* d) {
  if (!d) return fail(PATCH_ERR_INVALID_ARG, "null descriptor");
  if (d->version == kVersionQ64) return check_desc_q64(d);
  if (d->version != kVersion || d->tile_n != kTile || d->tile_k != kTile)
    return fail(PATCH_ERR_INVALID_ARG, "descriptor version/tile mismatch");
  if (check_dtype((patch_dtype)d->dtype)) return PATCH_ERR_INVALID_ARG;
  patch_status s = check_nk(d->N, d->K);
  if (s) return s;
  const uint64_t T = (uint64_t)d->nt_n * d->nt_k;
  if (d->nt_n != d->N / kTile || d->nt_k != d->K / kTile || d->n_sparse > T || d->n_48 > d->n_sparse ||
      d->table_offset != 256 ||
      d->data_offset != round_up(256 + 16 * T, 256) ||
      d->total_bytes != d->data_offset + kDenseBytes * (T - d->n_sparse) + kSparseBytes * d->n_sparse)
    return fail(PATCH_ERR_INVALID_ARG, "inconsistent descriptor");
  if (d->total_bytes >= kMaxBlobBytes)
    return fail(PATCH_ERR_UNSUPPORTED, "blob of %llu bytes exceeds the supported %llu",
                (unsigned long long)d->total_bytes, (unsigned long long)kMaxBlobBytes);
  return PATCH_OK;
}

void put32(uint8_t* p, uint32_t v) { std::memcpy(p, &v, 4); }
void put64(uint8_t* p, uint64_t v) { std::memcpy(p, &v, 8); }

}  // namespace

extern "C" {

int32_t patch_abi_version(void) { return 5; }

patch_status patch_sample_mask(int64_t N, int64_t K, const float* tile_logits_dev, const float* tile_u_dev,
                               const float* pat_logits_dev, const float* pat_u_dev, float tau, uint8_t* tile_map_dev,
                               uint8_t* mask_dev, float* soft_dev, void* stream) {
  patch_status s;
  if ((s = check_nk(N, K))) return s;
  if (!tile_logits_dev || !tile_u_dev || !pat_logits_dev || !pat_u_dev || !tile_map_dev || !mask_dev)
    return fail(PATCH_ERR_INVALID_ARG, "null pointer argument");
  auto aligned = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
  if (!aligned(tile_logits_dev, 8) || !aligned(tile_u_dev, 8) || !aligned16(pat_logits_dev) ||
      !aligned16(pat_u_dev) || !aligned(mask_dev, 4) || (soft_dev && !aligned16(soft_dev)))
    return fail(PATCH_ERR_INVALID_ARG,
                "tile logits and uniforms must be 8-byte, pattern logits, uniforms and soft 16-byte, and the mask "
                "4-byte aligned");
  if (!std::isfinite(tau) || !(tau > 0.0f)) return fail(PATCH_ERR_INVALID_ARG, "tau must be finite and > 0");
  hipError_t e = patch::launch_sample_mask(N, K, tile_logits_dev, tile_u_dev, pat_logits_dev, pat_u_dev, tau,
                                           tile_map_dev, mask_dev, soft_dev, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launch sampler");
  return PATCH_OK;
}

namespace {
patch_status check_fine(int64_t N, int64_t K, int64_t b1, int64_t b2) {
  patch_status s = check_nk(N, K);
  if (s) return s;
  if (b1 <= 0 || b2 <= 0 || kTile % b1 || kTile % b2 || b2 % 4)
    return fail(PATCH_ERR_SHAPE, "fine tiles %lld x %lld must divide 128 (columns a multiple of 4)", (long long)b1,
                (long long)b2);
  return PATCH_OK;
}
}  // namespace

patch_status patch_exec_tile_map(int64_t N, int64_t K, int64_t b1, int64_t b2, const uint8_t* fine_map_host,
                                 uint8_t* exec_map_host, int64_t* n_sparse_out) {
  patch_status s = check_fine(N, K, b1, b2);
  if (s) return s;
  if (!fine_map_host || !exec_map_host) return fail(PATCH_ERR_INVALID_ARG, "null tile map");
  const int64_t fKT = K / b2, KT = K / kTile, rn = kTile / b1, rk = kTile / b2;
  int64_t n_sparse = 0;
  for (int64_t i = 0; i < N / kTile; i++)
    for (int64_t j = 0; j < KT; j++) {
      bool all = true;
      for (int64_t a = 0; a < rn && all; a++) {
        const uint8_t* row = fine_map_host + (i * rn + a) * fKT + j * rk;
        for (int64_t b = 0; b < rk; b++)
          if (!row[b]) {
            all = false;
            break;
          }
      }
      exec_map_host[i * KT + j] = all ? 1 : 0;
      n_sparse += all;
    }
  if (n_sparse_out) *n_sparse_out = n_sparse;
  return PATCH_OK;
}

patch_status patch_apply_fine_mask(patch_dtype dtype, int64_t N, int64_t K, int64_t b1, int64_t b2, const void* W_dev,
                                   const uint8_t* fine_map_dev, const uint8_t* mask_dev, void* W_out_dev,
                                   void* stream) {
  patch_status s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_fine(N, K, b1, b2))) return s;
  if (!W_dev || !fine_map_dev || !mask_dev || !W_out_dev) return fail(PATCH_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(W_dev) || !aligned16(W_out_dev) || (reinterpret_cast<uintptr_t>(mask_dev) & 7u))
    return fail(PATCH_ERR_INVALID_ARG, "W and W_out must be 16-byte and the mask 8-byte aligned");
  hipError_t e = patch::launch_apply_fine_mask(N, K, (int)b1, (int)b2, W_dev, fine_map_dev, mask_dev, W_out_dev,
                                               reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launch apply_fine_mask");
  return PATCH_OK;
}

const char* patch_status_string(patch_status s) {
  switch (s) {
    case PATCH_OK: return "ok";
    case PATCH_ERR_INVALID_ARG: return "invalid argument";
    case PATCH_ERR_SHAPE: return "unsupported shape";
    case PATCH_ERR_MASK: return "mask does not keep exactly two of four in a sparse tile";
    case PATCH_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case PATCH_ERR_UNSUPPORTED: return "unsupported";
    case PATCH_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* patch_last_error(void) { return g_err.c_str(); }

patch_status patch_probe_stream_read(const void* src_dev, uint64_t bytes, void* sink_dev, uint64_t sink_bytes,
                                     void* stream) {
  if (!src_dev || !sink_dev || !aligned16(src_dev)) return fail(PATCH_ERR_INVALID_ARG, "null or unaligned pointer");
  if (bytes == 0 || bytes % 16) return fail(PATCH_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (sink_bytes < 4) return fail(PATCH_ERR_INVALID_ARG, "sink needs at least 4 bytes");
  hipError_t e = patch::launch_probe_read(src_dev, bytes, sink_dev, sink_bytes, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launch stream-read probe");
  return PATCH_OK;
}

void patch_debug_tail_wait(int32_t polls) { patch::tail_wait_test((int)polls); }

patch_status patch_probe_copy_rate(const void* src_dev, uint64_t src_bytes, uint64_t window_bytes, int32_t iters,
                                   int32_t workgroups, void* sink_dev, uint64_t sink_bytes, void* stream) {
  if (!src_dev || !sink_dev || !aligned16(src_dev) || iters < 1 || workgroups < 1)
    return fail(PATCH_ERR_INVALID_ARG, "probe_copy_rate: null or unaligned pointer, iters or workgroups < 1");
  if (window_bytes < 1024 || (window_bytes & (window_bytes - 1)) || src_bytes < window_bytes ||
      src_bytes % window_bytes)
    return fail(PATCH_ERR_INVALID_ARG, "probe_copy_rate: window must be a power of two >= 1 KB dividing src_bytes");
  if (sink_bytes < 4ull * (uint64_t)workgroups) return fail(PATCH_ERR_INVALID_ARG, "probe_copy_rate: sink too small");
  hipError_t e = patch::launch_probe_copy(src_dev, src_bytes, window_bytes, iters, workgroups, sink_dev,
                                          reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launch copy probe");
  return PATCH_OK;
}

uint64_t patch_probe_copy_bytes(int32_t iters, int32_t workgroups) {
  if (iters < 1 || workgroups < 1) return 0;
  return patch::probe_copy_bytes(iters, workgroups);
}

uint64_t patch_probe_matrix_flops(int32_t kind, int32_t iters, int32_t workgroups) {
  if (kind < 0 || kind > 3 || iters < 1 || workgroups < 1) return 0;
  return patch::probe_mma_flops(kind, iters, workgroups);
}

patch_status patch_probe_matrix_rate(int32_t kind, int32_t iters, int32_t workgroups, void* sink_dev, void* stream) {
  if (kind < 0 || kind > 3) return fail(PATCH_ERR_INVALID_ARG, "kind %d outside 0..3", (int)kind);
  if (iters < 1 || workgroups < 1) return fail(PATCH_ERR_INVALID_ARG, "iters and workgroups must be >= 1");
  if (!sink_dev) return fail(PATCH_ERR_INVALID_ARG, "null sink");
  hipError_t e = patch::launch_probe_mma(kind, iters, workgroups, sink_dev, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launch matrix-rate probe");
  return PATCH_OK;
}

uint64_t patch_packed_bytes(patch_dtype dtype, int64_t N, int64_t K, const uint8_t* tile_map_host) {
  if (check_dtype(dtype) || check_nk(N, K) || !tile_map_host) return 0;
  const int64_t T = (N / kTile) * (K / kTile);
  uint64_t ns = 0;
  for (int64_t t = 0; t < T; t++) {
    if (tile_map_host[t] > 2) return 0;  // 0 dense, 1 2:4, 2 4:8
    ns += tile_map_host[t] != 0;
  }
  return round_up(256 + 16 * (uint64_t)T, 256) + kDenseBytes * (uint64_t)(T - (int64_t)ns) + kSparseBytes * ns;
}

}  // extern "C"

extern "C" uint64_t patch_packed_bytes_q64(patch_dtype dtype, int64_t N, int64_t K, const uint8_t* quad_map_host) {
  if (check_dtype(dtype) || check_nk(N, K) || !quad_map_host) return 0;
  const int64_t R = N / kQuad, KQ = K / kQuad, KC = K / kTile;
  uint64_t total = round_up(256 + 16 * (uint64_t)(R * KC), 256);
  for (int64_t r = 0; r < R; r++)
    for (int64_t j = 0; j < KC; j++) {
      const uint8_t a = quad_map_host[r * KQ + 2 * j], b = quad_map_host[r * KQ + 2 * j + 1];
      if (a > 1 || b > 1) return 0;  // 0 dense, 1 2:4
      total += 4 * q64_piece((uint32_t)a | ((uint32_t)b << 1));
    }
  return total;
}

// Pack the N x K matrix assembled from the sources (see PackSources);
// tile_map_host is the map of the assembled matrix.
static patch_status pack_common(patch_dtype dtype, int64_t N, int64_t K, const patch::PackSources& src,
                                const uint8_t* tile_map_host, void* packed_dev, uint64_t packed_bytes,
                                patch_packed_desc* desc_out, void* stream) {
  patch_status s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_nk(N, K))) return s;
  if (!tile_map_host || !packed_dev || !desc_out) return fail(PATCH_ERR_INVALID_ARG, "null pointer argument");
  for (int i = 0; i < src.n; i++) {
    if (!src.W[i] || !src.mask[i]) return fail(PATCH_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(src.W[i]) || !aligned16(src.mask[i]))
      return fail(PATCH_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  }
  if (!aligned16(packed_dev)) return fail(PATCH_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const int64_t NT = N / kTile, KT = K / kTile, T = NT * KT;
  for (int64_t t = 0; t < T; t++)
    if (tile_map_host[t] > 2)
      return fail(PATCH_ERR_INVALID_ARG, "tile map byte %d at tile %lld (0 dense, 1 2:4, 2 4:8)", (int)tile_map_host[t],
                  (long long)t);
  const uint64_t need = patch_packed_bytes(dtype, N, K, tile_map_host);
  if (need >= kMaxBlobBytes) return fail(PATCH_ERR_UNSUPPORTED, "blob of %llu bytes too large", (unsigned long long)need);
  if (packed_bytes < need)
    return fail(PATCH_ERR_BUFFER_TOO_SMALL, "packed buffer %llu < %llu bytes", (unsigned long long)packed_bytes,
                (unsigned long long)need);

  // header + tile table, built on the host
  const uint64_t data_off = round_up(256 + 16 * (uint64_t)T, 256);
  std::vector<uint8_t> head(data_off, 0);
  // Row-block i: 8 bands of S_i bytes, band b holding its piece of every
  // tile in order; an entry holds the offset of the tile's band-0 piece, its
  // kind and S_i.
  uint32_t ns = 0, n48 = 0;
  uint64_t rb = data_off;
  for (int64_t i = 0; i < NT; i++) {
    uint64_t stride = 0;
    for (int64_t j = 0; j < KT; j++) stride += tile_map_host[i * KT + j] ? kSparsePiece : kDensePiece;
    uint64_t prefix = 0;
    for (int64_t j = 0; j < KT; j++) {
      const int64_t t = i * KT + j;
      const uint32_t kind = tile_map_host[t];  // 0 dense, 1 2:4, 2 4:8
      put64(&head[256 + 16 * t], rb + prefix);
      put32(&head[256 + 16 * t + 8], kind);
      put32(&head[256 + 16 * t + 12], (uint32_t)stride);
      prefix += kind ? kSparsePiece : kDensePiece;
      ns += kind != 0;
      n48 += kind == 2;
    }
    rb += 8 * stride;
  }
  put32(&head[0], kMagic);
  put32(&head[4], kVersion);
  put32(&head[8], (uint32_t)dtype);
  put32(&head[12], (uint32_t)kTile);
  put32(&head[16], (uint32_t)kTile);
  put32(&head[20], (uint32_t)N);
  put32(&head[24], (uint32_t)K);
  put32(&head[28], (uint32_t)NT);
  put32(&head[32], (uint32_t)KT);
  put32(&head[36], ns);
  put64(&head[40], 256);
  put64(&head[48], data_off);
  put64(&head[56], need - data_off);
  put64(&head[64], need);
  put32(&head[72], n48);

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(packed_dev, head.data(), head.size(), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(header)");
  e = patch::launch_pack(src, N, K, reinterpret_cast<uint8_t*>(packed_dev), st);
  if (e != hipSuccess) return hip_fail(e, "launch pack");
  uint32_t flag = 0;
  e = hipMemcpyAsync(&flag, reinterpret_cast<uint8_t*>(packed_dev) + kErrFlagOffset, 4, hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(flag)");
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  if (flag)
    return fail(PATCH_ERR_MASK,
                "a group inside a 2:4 (4:8) tile does not keep exactly two of four (four of eight) weights");

  patch_packed_desc d;
  d.version = kVersion;
  d.dtype = (uint32_t)dtype;
  d.tile_n = d.tile_k = (uint32_t)kTile;
  d.N = (uint32_t)N;
  d.K = (uint32_t)K;
  d.nt_n = (uint32_t)NT;
  d.nt_k = (uint32_t)KT;
  d.n_sparse = ns;
  d.n_48 = n48;
  d.table_offset = 256;
  d.data_offset = data_off;
  d.total_bytes = need;
  *desc_out = d;
  return PATCH_OK;
}

extern "C" patch_status patch_pack_q64(patch_dtype dtype, int64_t N, int64_t K, const void* W_dev,
                                      const uint8_t* quad_map_host, const uint8_t* mask_dev, void* packed_dev,
                                      uint64_t packed_bytes, patch_packed_desc* desc_out, void* stream) {
  patch_status s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_nk(N, K))) return s;
  if (!W_dev || !quad_map_host || !mask_dev || !packed_dev || !desc_out)
    return fail(PATCH_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(W_dev) || !aligned16(mask_dev) || !aligned16(packed_dev))
    return fail(PATCH_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const int64_t R = N / kQuad, KQ = K / kQuad, KC = K / kTile;
  for (int64_t t = 0; t < R * KQ; t++)
    if (quad_map_host[t] > 1)
      return fail(PATCH_ERR_INVALID_ARG, "quadrant map byte %d at quadrant %lld (0 dense, 1 2:4)",
                  (int)quad_map_host[t], (long long)t);
  const uint64_t need = patch_packed_bytes_q64(dtype, N, K, quad_map_host);
  if (need >= kMaxBlobBytes) return fail(PATCH_ERR_UNSUPPORTED, "blob of %llu bytes too large", (unsigned long long)need);
  if (packed_bytes < need)
    return fail(PATCH_ERR_BUFFER_TOO_SMALL, "packed buffer %llu < %llu bytes", (unsigned long long)packed_bytes,
                (unsigned long long)need);

  // header + table, built on the host: half-row-block r takes 4 bands of
  // S_r bytes, band b holding its piece of every tile column in order
  const uint64_t data_off = round_up(256 + 16 * (uint64_t)(R * KC), 256);
  std::vector<uint8_t> head(data_off, 0);
  uint32_t ns = 0;
  uint64_t hb = data_off;
  for (int64_t r = 0; r < R; r++) {
    uint64_t stride = 0;
    for (int64_t j = 0; j < KC; j++)
      stride += q64_piece((uint32_t)quad_map_host[r * KQ + 2 * j] | ((uint32_t)quad_map_host[r * KQ + 2 * j + 1] << 1));
    uint64_t prefix = 0;
    for (int64_t j = 0; j < KC; j++) {
      const int64_t t = r * KC + j;
      const uint32_t kb = (uint32_t)quad_map_host[r * KQ + 2 * j] | ((uint32_t)quad_map_host[r * KQ + 2 * j + 1] << 1);
      put64(&head[256 + 16 * t], hb + prefix);
      put32(&head[256 + 16 * t + 8], kb);
      put32(&head[256 + 16 * t + 12], (uint32_t)stride);
      prefix += q64_piece(kb);
      ns += (kb & 1u) + (kb >> 1);
    }
    hb += 4 * stride;
  }
  put32(&head[0], kMagic);
  put32(&head[4], kVersionQ64);
  put32(&head[8], (uint32_t)dtype);
  put32(&head[12], (uint32_t)kQuad);
  put32(&head[16], (uint32_t)kQuad);
  put32(&head[20], (uint32_t)N);
  put32(&head[24], (uint32_t)K);
  put32(&head[28], (uint32_t)R);
  put32(&head[32], (uint32_t)KQ);
  put32(&head[36], ns);
  put64(&head[40], 256);
  put64(&head[48], data_off);
  put64(&head[56], need - data_off);
  put64(&head[64], need);
  put32(&head[72], 0);

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(packed_dev, head.data(), head.size(), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(header)");
  e = patch::launch_pack_q64(W_dev, mask_dev, N, K, reinterpret_cast<uint8_t*>(packed_dev), st);
  if (e != hipSuccess) return hip_fail(e, "launch pack_q64");
  uint32_t flag = 0;
  e = hipMemcpyAsync(&flag, reinterpret_cast<uint8_t*>(packed_dev) + kErrFlagOffset, 4, hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(flag)");
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  if (flag) return fail(PATCH_ERR_MASK, "a group inside a 2:4 quadrant does not keep exactly two of four weights");

  patch_packed_desc d;
  d.version = kVersionQ64;
  d.dtype = (uint32_t)dtype;
  d.tile_n = d.tile_k = (uint32_t)kQuad;
  d.N = (uint32_t)N;
  d.K = (uint32_t)K;
  d.nt_n = (uint32_t)R;
  d.nt_k = (uint32_t)KQ;
  d.n_sparse = ns;
  d.n_48 = 0;
  d.table_offset = 256;
  d.data_offset = data_off;
  d.total_bytes = need;
  *desc_out = d;
  return PATCH_OK;
}

// The tile map of the row-block interleave of two F x K matrices.
static std::vector<uint8_t> interleave_maps(int64_t F, int64_t K, const uint8_t* map_g, const uint8_t* map_u) {
  const int64_t FT = F / kTile, KT = K / kTile;
  std::vector<uint8_t> m((size_t)(2 * FT * KT));
  for (int64_t i = 0; i < FT; i++)
    for (int64_t j = 0; j < KT; j++) {
      m[(size_t)((2 * i) * KT + j)] = map_g[i * KT + j];
      m[(size_t)((2 * i + 1) * KT + j)] = map_u[i * KT + j];
    }
  return m;
}

extern "C" {

patch_status patch_pack(patch_dtype dtype, int64_t N, int64_t K, const void* W_dev, const uint8_t* tile_map_host,
                        const uint8_t* mask_dev, void* packed_dev, uint64_t packed_bytes,
                        patch_packed_desc* desc_out, void* stream) {
  patch::PackSources src{};
  src.W[0] = reinterpret_cast<const uint16_t*>(W_dev);
  src.mask[0] = mask_dev;
  src.start[0] = 0;
  src.start[1] = (int)(N / kTile);
  src.n = 1;
  src.interleave = 0;
  return pack_common(dtype, N, K, src, tile_map_host, packed_dev, packed_bytes, desc_out, stream);
}

// Row-concatenation of count matrices with the same K: sizes and the
// concatenated tile map (empty on invalid arguments).
static std::vector<uint8_t> concat_maps(int32_t count, const int64_t* N_host, int64_t K,
                                        const uint8_t* const* maps_host, int64_t* N_total) {
  std::vector<uint8_t> m;
  *N_total = 0;
  if (count < 1 || count > patch::kPackMaxSources || !N_host || !maps_host || K <= 0 || K % kTile) return m;
  const int64_t KT = K / kTile;
  for (int32_t i = 0; i < count; i++) {
    if (N_host[i] <= 0 || N_host[i] % kTile || !maps_host[i]) return std::vector<uint8_t>();
    *N_total += N_host[i];
  }
  if (*N_total > kMaxDim) return std::vector<uint8_t>();
  for (int32_t i = 0; i < count; i++) m.insert(m.end(), maps_host[i], maps_host[i] + (N_host[i] / kTile) * KT);
  return m;
}

uint64_t patch_packed_bytes_concat(patch_dtype dtype, int32_t count, const int64_t* N_host, int64_t K,
                                   const uint8_t* const* tile_maps_host) {
  int64_t N = 0;
  const std::vector<uint8_t> m = concat_maps(count, N_host, K, tile_maps_host, &N);
  if (m.empty()) return 0;
  return patch_packed_bytes(dtype, N, K, m.data());
}

patch_status patch_pack_concat(patch_dtype dtype, int32_t count, const int64_t* N_host, int64_t K,
                               const void* const* W_dev, const uint8_t* const* tile_maps_host,
                               const uint8_t* const* masks_dev, void* packed_dev, uint64_t packed_bytes,
                               patch_packed_desc* desc_out, void* stream) {
  if (!W_dev || !masks_dev) return fail(PATCH_ERR_INVALID_ARG, "null pointer argument");
  if (count < 1 || count > patch::kPackMaxSources)
    return fail(PATCH_ERR_INVALID_ARG, "count=%d must be 1 .. %d", (int)count, patch::kPackMaxSources);
  int64_t N = 0;
  const std::vector<uint8_t> m = concat_maps(count, N_host, K, tile_maps_host, &N);
  if (m.empty()) return fail(PATCH_ERR_SHAPE, "every N must be a positive multiple of 128, K too, sum within range");
  patch::PackSources src{};
  src.n = count;
  src.interleave = 0;
  src.start[0] = 0;
  for (int32_t i = 0; i < count; i++) {
    src.W[i] = reinterpret_cast<const uint16_t*>(W_dev[i]);
    src.mask[i] = masks_dev[i];
    src.start[i + 1] = src.start[i] + (int)(N_host[i] / kTile);
  }
  return pack_common(dtype, N, K, src, m.data(), packed_dev, packed_bytes, desc_out, stream);
}

uint64_t patch_packed_bytes_gate_up(patch_dtype dtype, int64_t F, int64_t K, const uint8_t* map_g_host,
                                    const uint8_t* map_u_host) {
  if (check_dtype(dtype) || F <= 0 || F % kTile || check_nk(2 * F, K) || !map_g_host || !map_u_host) return 0;
  const std::vector<uint8_t> m = interleave_maps(F, K, map_g_host, map_u_host);
  return patch_packed_bytes(dtype, 2 * F, K, m.data());
}

patch_status patch_pack_gate_up(patch_dtype dtype, int64_t F, int64_t K, const void* Wg_dev, const void* Wu_dev,
                                const uint8_t* map_g_host, const uint8_t* map_u_host, const uint8_t* mask_g_dev,
                                const uint8_t* mask_u_dev, void* packed_dev, uint64_t packed_bytes,
                                patch_packed_desc* desc_out, void* stream) {
  patch_status s;
  if (F <= 0 || F % kTile) return fail(PATCH_ERR_SHAPE, "F=%lld must be a positive multiple of 128", (long long)F);
  if ((s = check_nk(2 * F, K))) return s;
  if (!map_g_host || !map_u_host) return fail(PATCH_ERR_INVALID_ARG, "null pointer argument");
  const std::vector<uint8_t> m = interleave_maps(F, K, map_g_host, map_u_host);
  patch::PackSources src{};
  src.n = 2;
  src.interleave = 1;
  src.W[0] = reinterpret_cast<const uint16_t*>(Wg_dev);
  src.W[1] = reinterpret_cast<const uint16_t*>(Wu_dev);
  src.mask[0] = mask_g_dev;
  src.mask[1] = mask_u_dev;
  return pack_common(dtype, 2 * F, K, src, m.data(), packed_dev, packed_bytes, desc_out, stream);
}

patch_status patch_desc_from_header(const void* header_host, uint64_t header_bytes, patch_packed_desc* desc_out) {
  if (!header_host || !desc_out) return fail(PATCH_ERR_INVALID_ARG, "null pointer argument");
  // the descriptor's fields end with n_48 at bytes 72..75
  if (header_bytes < 76) return fail(PATCH_ERR_BUFFER_TOO_SMALL, "header needs at least 76 bytes");
  const uint8_t* h = reinterpret_cast<const uint8_t*>(header_host);
  uint32_t u[10];
  uint64_t v[4];
  std::memcpy(u, h, 40);
  std::memcpy(v, h + 40, 32);
  if (u[0] != kMagic) return fail(PATCH_ERR_INVALID_ARG, "bad magic");
  patch_packed_desc d;
  d.version = u[1];
  d.dtype = u[2];
  d.tile_n = u[3];
  d.tile_k = u[4];
  d.N = u[5];
  d.K = u[6];
  d.nt_n = u[7];
  d.nt_k = u[8];
  d.n_sparse = u[9];
  std::memcpy(&d.n_48, h + 72, 4);
  d.table_offset = v[0];
  d.data_offset = v[1];
  d.total_bytes = v[3];
  if (v[2] != d.total_bytes - d.data_offset) return fail(PATCH_ERR_INVALID_ARG, "inconsistent data size");
  patch_status s = check_desc(&d);
  if (s) return s;
  *desc_out = d;
  return PATCH_OK;
}

static uint64_t workspace_for(int64_t M, int64_t N, int64_t K, bool rowmajor) {
  if (M <= 0 || M > (int64_t)0x7fffffff || N <= 0 || K <= 0 || N % kTile || K % kTile || N > kMaxDim || K > kMaxDim ||
      K / kTile > kMaxKT)
    return 0;
  return patch::prefill_workspace_bytes(M, N, K, rowmajor);
}

uint64_t patch_gemm_workspace_bytes(const patch_packed_desc* desc, int64_t M) {
  if (!desc) return 0;
  return workspace_for(M, desc->N, desc->K, false);
}

uint64_t patch_dense_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) { return workspace_for(M, N, K, true); }

// src2 non-null: the fused gate/up product H = SiLU(X Wg^T) * (X Wu^T), N = 2F
// (row-major: src = Wg, src2 = Wu; packed: src2 = src, the interleaved blob);
// Y is then H, M x F.
static patch_status gemm_common(bool rowmajor, patch_dtype dt, int64_t M, int64_t N, int64_t K, const void* src,
                                const void* src2, uint64_t w_bytes, const void* X_dev, void* Y_dev,
                                patch_dtype y_dtype, void* ws, uint64_t ws_bytes, int32_t variant, void* stream,
                                bool has48 = false, bool q64 = false) {
  patch_status s;
  if ((s = check_ydtype(dt, y_dtype))) return s;
  if (M < 0 || M > (int64_t)0x7fffffff) return fail(PATCH_ERR_INVALID_ARG, "M=%lld out of range", (long long)M);
  if (variant < PATCH_VARIANT_AUTO || variant > PATCH_VARIANT_PREFILL_BIG8_W256)
    return fail(PATCH_ERR_INVALID_ARG, "unknown variant %d", (int)variant);
  if (has48 && variant >= PATCH_VARIANT_PREFILL_W64 && variant <= PATCH_VARIANT_PREFILL_W256)
    return fail(PATCH_ERR_UNSUPPORTED, "the register-staged prefill variants run dense and 2:4 tiles only");
  if (q64 && ((variant >= PATCH_VARIANT_PREFILL_W64 && variant <= PATCH_VARIANT_PREFILL_W256) ||
              variant >= PATCH_VARIANT_PREFILL_BIG))
    return fail(PATCH_ERR_UNSUPPORTED,
                "a blob of 64 x 64 execution tiles runs on the decode and LDS-staged prefill kernels only");
  if (q64 && src2) return fail(PATCH_ERR_UNSUPPORTED, "the fused gate/up product takes 128 x 128 execution tiles");
  if (variant == PATCH_VARIANT_DECODE && M > kDecodeMaxM)
    return fail(PATCH_ERR_INVALID_ARG, "decode variant needs M <= %lld (M=%lld)", (long long)kDecodeMaxM, (long long)M);
  if (M == 0) return PATCH_OK;
  if (!src || !X_dev || !Y_dev) return fail(PATCH_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(src) || !aligned16(X_dev) || !aligned16(Y_dev) || (src2 && !aligned16(src2)))
    return fail(PATCH_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const bool fuse = src2 != nullptr;
  if (fuse && N % (2 * kTile)) return fail(PATCH_ERR_SHAPE, "fused gate/up needs an even number of row-blocks");
  // the fused decode kernel runs twice the waves: with more than one block of
  // 16 tokens it needs K <= 32768
  const bool fused_decode_ok = !fuse || M <= 16 || K <= 32768;
  if (variant == PATCH_VARIANT_DECODE && !fused_decode_ok)
    return fail(PATCH_ERR_UNSUPPORTED, "fused decode needs M <= 16 or K <= 32768");
  if (ws_bytes > 0 && (!ws || !aligned16(ws)))
    return fail(PATCH_ERR_INVALID_ARG, "workspace must be non-null and 16-byte aligned when workspace_bytes > 0");
  if (variant == PATCH_VARIANT_DECODE && K > kDecodeMaxK)
    return fail(PATCH_ERR_UNSUPPORTED, "decode variant needs K <= %lld (K=%lld)", (long long)kDecodeMaxK, (long long)K);
  // AUTO: decode for up to 16 tokens; up to 128, whichever kernel's time
  // model is lower (the prefill one for the split the workspace allows).
  bool decode = variant == PATCH_VARIANT_DECODE;
  if (variant == PATCH_VARIANT_AUTO && K <= kDecodeMaxK && M <= kDecodeMaxM && fused_decode_ok)
    decode = M <= kDecodeAutoM || patch::decode_estimate_us(M, N, K, (double)w_bytes) <=
                                      patch::prefill_estimate_us(M, N, K, rowmajor, ws ? ws_bytes : 0);
  const bool bf16 = dt == PATCH_BF16, f32out = y_dtype == PATCH_F32;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  static const int kForceBm[17] = {0, 0, 0, 64, 128, 192, 256, 128, 192, 256, 64, 0, 128, 192, 256, 128, 256};
  const int big = variant >= PATCH_VARIANT_PREFILL_BIG8_W128 ? 8 : variant >= PATCH_VARIANT_PREFILL_BIG ? 4 : 0;
  const bool lds = variant >= PATCH_VARIANT_PREFILL_W128_LDS && variant <= PATCH_VARIANT_PREFILL_W64_LDS;
  hipError_t e = decode ? patch::launch_decode(bf16, rowmajor, f32out, src, src2, X_dev, M, N, K, Y_dev, has48, q64,
                                               st)
                        : patch::launch_prefill(bf16, rowmajor, f32out, src, src2, X_dev, M, N, K, Y_dev, ws,
                                                ws_bytes, kForceBm[variant], lds, big, q64, st);
  if (e != hipSuccess) return hip_fail(e, decode ? "launch decode" : "launch prefill");
  return PATCH_OK;
}

patch_status patch_gemm_ex(const patch_packed_desc* desc, const void* packed_dev, const void* X_dev, int64_t M,
                           void* Y_dev, patch_dtype y_dtype, void* workspace_dev, uint64_t workspace_bytes,
                           int32_t variant, void* stream) {
  patch_status s = check_desc(desc);
  if (s) return s;
  return gemm_common(false, (patch_dtype)desc->dtype, M, desc->N, desc->K, packed_dev, nullptr,
                     desc->total_bytes - desc->data_offset, X_dev, Y_dev, y_dtype, workspace_dev, workspace_bytes,
                     variant, stream, desc->n_48 > 0, desc->version == kVersionQ64);
}

patch_status patch_gemm(const patch_packed_desc* desc, const void* packed_dev, const void* X_dev, int64_t M,
                        void* Y_dev, patch_dtype y_dtype, void* workspace_dev, uint64_t workspace_bytes,
                        void* stream) {
  return patch_gemm_ex(desc, packed_dev, X_dev, M, Y_dev, y_dtype, workspace_dev, workspace_bytes,
                       PATCH_VARIANT_AUTO, stream);
}

patch_status patch_dense_gemm_ex(patch_dtype dtype, int64_t M, int64_t N, int64_t K, const void* X_dev,
                                 const void* W_dev, void* Y_dev, patch_dtype y_dtype, void* workspace_dev,
                                 uint64_t workspace_bytes, int32_t variant, void* stream) {
  patch_status s;
  if ((s = check_dtype(dtype))) return s;
  if ((s = check_nk(N, K))) return s;
  return gemm_common(true, dtype, M, N, K, W_dev, nullptr, (uint64_t)(N * K * 2), X_dev, Y_dev, y_dtype,
                     workspace_dev, workspace_bytes, variant, stream);
}

patch_status patch_dense_gemm(patch_dtype dtype, int64_t M, int64_t N, int64_t K, const void* X_dev,
                              const void* W_dev, void* Y_dev, patch_dtype y_dtype, void* workspace_dev,
                              uint64_t workspace_bytes, void* stream) {
  return patch_dense_gemm_ex(dtype, M, N, K, X_dev, W_dev, Y_dev, y_dtype, workspace_dev, workspace_bytes,
                             PATCH_VARIANT_AUTO, stream);
}

uint64_t patch_gemm_swiglu_workspace_bytes(const patch_packed_desc* desc, int64_t M) {
  if (!desc || desc->nt_n % 2) return 0;
  return workspace_for(M, desc->N, desc->K, false);
}

uint64_t patch_dense_gemm_swiglu_workspace_bytes(int64_t M, int64_t F, int64_t K) {
  if (F <= 0 || F % kTile) return 0;
  return workspace_for(M, 2 * F, K, true);
}

patch_status patch_gemm_swiglu(const patch_packed_desc* desc, const void* packed_dev, const void* X_dev, int64_t M,
                               void* H_dev, patch_dtype h_dtype, void* workspace_dev, uint64_t workspace_bytes,
                               int32_t variant, void* stream) {
  patch_status s = check_desc(desc);
  if (s) return s;
  if (desc->version == kVersionQ64)
    return fail(PATCH_ERR_UNSUPPORTED, "the fused gate/up product takes 128 x 128 execution tiles");
  if (desc->nt_n % 2) return fail(PATCH_ERR_SHAPE, "a gate/up blob has an even number of row-blocks");
  return gemm_common(false, (patch_dtype)desc->dtype, M, desc->N, desc->K, packed_dev, packed_dev,
                     desc->total_bytes - desc->data_offset, X_dev, H_dev, h_dtype, workspace_dev, workspace_bytes,
                     variant, stream, desc->n_48 > 0);
}

patch_status patch_dense_gemm_swiglu(patch_dtype dtype, int64_t M, int64_t F, int64_t K, const void* X_dev,
                                     const void* Wg_dev, const void* Wu_dev, void* H_dev, patch_dtype h_dtype,
                                     void* workspace_dev, uint64_t workspace_bytes, int32_t variant, void* stream) {
  patch_status s;
  if ((s = check_dtype(dtype))) return s;
  if (F <= 0 || F % kTile) return fail(PATCH_ERR_SHAPE, "F=%lld must be a positive multiple of 128", (long long)F);
  if ((s = check_nk(2 * F, K))) return s;
  if (!Wu_dev) return fail(PATCH_ERR_INVALID_ARG, "null pointer argument");
  return gemm_common(true, dtype, M, 2 * F, K, Wg_dev, Wu_dev, (uint64_t)(2 * F * K * 2), X_dev, H_dev, h_dtype,
                     workspace_dev, workspace_bytes, variant, stream);
}

}  // extern "C"
