/*
 * oracle.c -- CPU oracle for the PATCH hybrid tile-sparse GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  The product
 * path (the HIP library and its Python binding) never calls it, and it shares
 * no code, header, table or constant generator with that path.
 *
 * What it computes (sources: "PATCH: Learnable Tile-level Hybrid Sparsity for
 * LLMs", arXiv 2509.23410; pages: the arXiv abstract, and the gist.science
 * explainer, section "2. Methodology: PATCH"):
 *
 *   - A weight matrix W (N x K, row-major, N = output features, K = input
 *     features) is partitioned into tiles of b1 x b2 (tile_n x tile_k).
 *     (gist.science explainer, section 2, "Core Mechanism".)
 *   - Each tile is either dense (keeps every weight) or 2:4 sparse (in every
 *     group of four consecutive weights, two are kept).
 *     (same section; section 1 "Problem Statement" defines the 2:4 rule.)
 *   - At inference the tile choice is hard: the effective mask E is 1 in
 *     dense tiles and the supplied 2:4 mask in sparse tiles.  The explainer
 *     calls the mask a weighted combination of the dense and the 2:4 option;
 *     with a hard 0/1 weight that combination is exactly this selection.
 *   - The product is Y = X * (W o E)^T, X being M x K.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *   - the groups of four run along K (the reduction dimension) inside a row;
 *   - a tile-map byte != 0 marks a sparse tile; a mask byte != 0 marks "keep";
 *   - the mask inside dense tiles is ignored and not validated;
 *   - a sparse-tile group whose mask does not keep exactly two positions is an
 *     error (ORACLE_ERR_MASK);
 *   - kept values are stored bit-exactly (a kept -0.0 stays -0.0).
 *
 * Arithmetic: every product of two binary16/bfloat16 values is exact in
 * binary64 (11x11 or 8x8 significand bits), and the sum runs over k in
 * ascending order in binary64, so the result does not depend on the number
 * of threads (OpenMP splits the work over output rows n only).
 *
 * The packed formats are the repository's own (version 3: 128 x 128
 * execution tiles; version 4: 64 x 64 ones): the pages fix only the tile
 * shape (128 x 128 execution tiles, gist.science explainer, section 4
 * "Ablation Studies", which also finds smaller tiles give finer control),
 * the six 2:4 patterns (section 2, "Pattern Selection") and nothing about
 * bytes.  oracle_pack() and oracle_pack_q64() write them from their written
 * definitions, restated next to each function.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_SHAPE 2
#define ORACLE_ERR_MASK 3
#define ORACLE_ERR_SMALL 4

#define ORACLE_F16 0
#define ORACLE_BF16 1

/* Number of OpenMP threads oracle_gemm_f64 runs on (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------------------
 * Element decoding, written from the IEEE 754-2008 binary16 definition and the
 * bfloat16 definition (the upper 16 bits of an IEEE binary32).
 * ------------------------------------------------------------------------- */
double oracle_f16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

double oracle_bf16_to_double(uint16_t b) {
  int sign = (b >> 15) & 1;
  int e = (b >> 7) & 0xff;
  int f = b & 0x7f;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -133); /* subnormal: f * 2^-7 * 2^-126 */
  } else if (e == 255) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(128 + f), e - 134); /* (1 + f/128) * 2^(e-127) */
  }
  return sign ? -v : v;
}

static double decode(uint16_t bits, int dtype) {
  return dtype == ORACLE_F16 ? oracle_f16_to_double(bits) : oracle_bf16_to_double(bits);
}

/* Round a binary64 value to the nearest bfloat16 / binary16 (ties to even).
 * Used only to measure the rounding floor of a 16-bit output. */
static uint16_t round_to_bits(double v, int mant_bits, int emin, int emax, int ebias, int expbits) {
  uint16_t sign = 0;
  if (signbit(v)) { sign = 1; v = -v; }
  uint16_t out;
  if (isnan(v)) {
    out = (uint16_t)(((1u << expbits) - 1) << mant_bits | (1u << (mant_bits - 1)));
  } else if (isinf(v)) {
    out = (uint16_t)(((1u << expbits) - 1) << mant_bits);
  } else if (v == 0.0) {
    out = 0;
  } else {
    int e;
    frexp(v, &e); /* v = m * 2^e, m in [0.5, 1) -> unbiased exponent e-1 */
    int ue = e - 1;
    if (ue < emin) ue = emin; /* subnormal range shares the minimum exponent */
    /* quantum = 2^(ue - mant_bits) */
    double q = ldexp(1.0, ue - mant_bits);
    double n = v / q;           /* exact: q is a power of two */
    double r = nearbyint(n);    /* default rounding mode: to nearest, ties even */
    double rv = r * q;
    /* re-derive exponent after rounding (may carry into the next binade) */
    if (rv == 0.0) {
      out = 0; /* underflow to zero keeps the sign below */
    } else if (rv >= ldexp(1.0, emax + 1)) {
      out = (uint16_t)(((1u << expbits) - 1) << mant_bits);
    } else {
      int e2;
      frexp(rv, &e2);
      int ue2 = e2 - 1;
      if (ue2 < emin) { /* subnormal */
        uint32_t frac = (uint32_t)(rv / ldexp(1.0, emin - mant_bits));
        out = (uint16_t)frac;
      } else {
        uint32_t frac = (uint32_t)(rv / ldexp(1.0, ue2 - mant_bits)) - (1u << mant_bits);
        out = (uint16_t)(((uint32_t)(ue2 + ebias) << mant_bits) | frac);
      }
    }
  }
  return (uint16_t)(out | (sign << 15));
}

uint16_t oracle_double_to_bf16(double v) { return round_to_bits(v, 7, -126, 127, 127, 8); }
uint16_t oracle_double_to_f16(double v) { return round_to_bits(v, 10, -14, 15, 15, 5); }

/* ---------------------------------------------------------------------------
 * Validation and the effective mask (gist.science explainer, section 2,
 * "Core Mechanism" and "Hybrid Mask Generation").
 * ------------------------------------------------------------------------- */
static int check_shape(int64_t N, int64_t K, int64_t tn, int64_t tk) {
  if (N <= 0 || K <= 0 || tn <= 0 || tk <= 0) return ORACLE_ERR_ARG;
  if (N % tn != 0 || K % tk != 0 || tk % 4 != 0) return ORACLE_ERR_SHAPE;
  return ORACLE_OK;
}

/* Tile kinds (tile-map bytes): 0 dense, 1 2:4 (two kept in every group of
 * four consecutive weights along K), 2 4:8 (four kept in every group of
 * eight).  4:8 is one of the "other N:M patterns" the explainer's section 5
 * "Significance" names as future work (the framework is pattern-agnostic);
 * any other byte is an error (ORACLE_ERR_ARG).
 * Returns ORACLE_ERR_MASK if a group inside a 2:4 or 4:8 tile does not keep
 * exactly half its positions; *bad_row / *bad_group receive the first one
 * (the group index counts groups of that tile's kind from column 0). */
int oracle_validate(int64_t N, int64_t K, int64_t tn, int64_t tk, const uint8_t* tile_map,
                    const uint8_t* mask, int64_t* bad_row, int64_t* bad_group) {
  int rc = check_shape(N, K, tn, tk);
  if (rc) return rc;
  int64_t KT = K / tk;
  for (int64_t t = 0; t < (N / tn) * KT; t++) {
    if (tile_map[t] > 2) return ORACLE_ERR_ARG;
    if (tile_map[t] == 2 && tk % 8) return ORACLE_ERR_SHAPE;
  }
  for (int64_t n = 0; n < N; n++) {
    for (int64_t k0 = 0; k0 < K;) {
      const int kind = tile_map[(n / tn) * KT + k0 / tk];
      const int gs = kind == 2 ? 8 : 4; /* group size */
      if (kind) {                       /* dense tile: mask not read */
        int kept = 0;
        for (int d = 0; d < gs; d++) kept += mask[n * K + k0 + d] != 0;
        if (kept != gs / 2) {
          if (bad_row) *bad_row = n;
          if (bad_group) *bad_group = k0 / gs;
          return ORACLE_ERR_MASK;
        }
      }
      k0 += gs;
    }
  }
  return ORACLE_OK;
}

/* E[n][k] = 1 in dense tiles, (mask != 0) in 2:4 and 4:8 tiles. */
int oracle_effective_mask(int64_t N, int64_t K, int64_t tn, int64_t tk, const uint8_t* tile_map,
                          const uint8_t* mask, uint8_t* E) {
  int rc = check_shape(N, K, tn, tk);
  if (rc) return rc;
  int64_t KT = K / tk;
  for (int64_t n = 0; n < N; n++)
    for (int64_t k = 0; k < K; k++) {
      int sparse = tile_map[(n / tn) * KT + k / tk] != 0;
      E[n * K + k] = sparse ? (mask[n * K + k] != 0) : 1;
    }
  return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * The GEMM: Y[m][n] = sum_k X[m][k] * W[n][k] * E[n][k], fp64, k ascending.
 * X: M x K element bits, W: N x K element bits, Y: M x N doubles.
 * ------------------------------------------------------------------------- */
int oracle_gemm_f64(int dtype, int64_t M, int64_t N, int64_t K, int64_t tn, int64_t tk,
                    const uint16_t* X, const uint16_t* W, const uint8_t* tile_map, const uint8_t* mask,
                    double* Y) {
  if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return ORACLE_ERR_ARG;
  if (M < 0) return ORACLE_ERR_ARG;
  int rc = oracle_validate(N, K, tn, tk, tile_map, mask, NULL, NULL);
  if (rc) return rc;
  if (M == 0) return ORACLE_OK;
  int64_t KT = K / tk;
  double* Xd = (double*)malloc(sizeof(double) * (size_t)(M * K));
  if (!Xd) return ORACLE_ERR_ARG;
  for (int64_t i = 0; i < M * K; i++) Xd[i] = decode(X[i], dtype);
  int fail = 0;
#pragma omp parallel
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)K);
    if (!w) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; n++) {
      if (!w) continue;
      /* masked row: W_eff[n][k] = W[n][k] where kept, +0 elsewhere */
      for (int64_t k = 0; k < K; k++) {
        int sparse = tile_map[(n / tn) * KT + k / tk] != 0;
        int keep = sparse ? (mask[n * K + k] != 0) : 1;
        w[k] = keep ? decode(W[n * K + k], dtype) : 0.0;
      }
      for (int64_t m = 0; m < M; m++) {
        const double* x = Xd + m * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++) acc += x[k] * w[k];
        Y[m * N + n] = acc;
      }
    }
    free(w);
  }
  free(Xd);
  return fail ? ORACLE_ERR_ARG : ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * The LLaMA MLP's gated product, the step on either side of the gate and up
 * projections.  The pages evaluate PATCH on LLaMA-2 models (gist.science
 * explainer, section 4 "Experimental Results"); the MLP of that architecture
 * computes H = SiLU(X Wg^T) * (X Wu^T) elementwise before the down
 * projection, with SiLU(x) = x * sigmoid(x) = x / (1 + e^-x).  Neither formula
 * is on the pages; both are the architecture's standard definitions.
 * ------------------------------------------------------------------------- */
double oracle_silu(double x) { return x / (1.0 + exp(-x)); }

/* H[m][f] = SiLU(Yg[m][f]) * Yu[m][f], Yg = X (Wg o Eg)^T and Yu = X (Wu o Eu)^T
 * each computed by oracle_gemm_f64; X: M x K, Wg and Wu: F x K, H: M x F. */
int oracle_swiglu_f64(int dtype, int64_t M, int64_t F, int64_t K, int64_t tn, int64_t tk, const uint16_t* X,
                      const uint16_t* Wg, const uint16_t* Wu, const uint8_t* map_g, const uint8_t* map_u,
                      const uint8_t* mask_g, const uint8_t* mask_u, double* H) {
  if (M < 0 || F < 0) return ORACLE_ERR_ARG;
  if (M == 0 || F == 0) return ORACLE_OK;
  double* yg = (double*)malloc(sizeof(double) * (size_t)(M * F));
  double* yu = (double*)malloc(sizeof(double) * (size_t)(M * F));
  int rc = (yg && yu) ? ORACLE_OK : ORACLE_ERR_ARG;
  if (!rc) rc = oracle_gemm_f64(dtype, M, F, K, tn, tk, X, Wg, map_g, mask_g, yg);
  if (!rc) rc = oracle_gemm_f64(dtype, M, F, K, tn, tk, X, Wu, map_u, mask_u, yu);
  if (!rc)
    for (int64_t i = 0; i < M * F; i++) H[i] = oracle_silu(yg[i]) * yu[i];
  free(yg);
  free(yu);
  return rc;
}

/* Round an fp64 result to the 16-bit output type (RNE) -- used to measure the
 * error floor that any 16-bit output must carry. */
void oracle_round_f64(int dtype, int64_t n, const double* in, uint16_t* out) {
  for (int64_t i = 0; i < n; i++)
    out[i] = dtype == ORACLE_F16 ? oracle_double_to_f16(in[i]) : oracle_double_to_bf16(in[i]);
}

/* ---------------------------------------------------------------------------
 * Packed format, version 3 (the repository's own format; restated here).
 *
 * Tile edge b = 128 in both directions; NT = N/128, KT = K/128, T = NT*KT.
 * Little-endian.  All bytes not written below are zero.
 *
 * Header, 256 bytes at offset 0:
 *   u32 magic 0x48435450, u32 version 3, u32 dtype (0 f16, 1 bf16),
 *   u32 tile_n 128, u32 tile_k 128, u32 N, u32 K, u32 NT, u32 KT,
 *   u32 n_sparse (2:4 and 4:8 tiles), u64 table_offset (= 256),
 *   u64 data_offset, u64 data_bytes, u64 total_bytes, u32 n_48 (the 4:8
 *   tiles among them) at byte 72.
 * Data at data_offset = round_up(256 + 16*T, 256).
 *
 * A "band" is 16 consecutive rows of a row-block (b = 0..7); a "piece" is
 * one band of one tile: 4096 bytes for a dense tile, 2304 for a sparse one.
 * Row-block i takes 8 * S_i bytes, S_i = sum over its tiles of the piece
 * sizes (the band stride); row-blocks follow each other.  Inside row-block
 * i, band b's pieces of tiles j = 0 .. KT-1 are back to back, and band b
 * starts S_i bytes after band b-1.
 * Tile table at 256: T entries of 16 bytes, tile (i, j) at index i*KT + j:
 *   u64 byte offset (from the start of the blob) of the tile's band-0 piece,
 *   u32 kind (0 dense, 1 2:4, 2 4:8), u32 S_i.
 * So band b's piece of tile (i, j) starts at entry offset + b * S_i.
 *
 * Inside a piece a "lane" is a number l = 0..63 with row-in-band
 * r = l mod 16 and column group h = l / 16; a chunk is 16 bytes, lane l's
 * chunk of a 1024-byte block sits at byte 16*l.
 *
 * Dense piece: blocks (q, e) at byte 2048*q + 1024*e, q = 0, 1 (64-column
 *   slice), e = 0, 1 (half).  Lane l of block (q, e) holds, of row
 *   16*band + r and the four groups of four g = 0..3 at columns
 *   64*q + 16*h .. +15, the elements at positions 2e and 2e+1: element
 *   2*g + u (u = 0, 1) is column 64*q + 16*h + 4*g + 2*e + u.  (Each half is
 *   a 2:4 operand with the fixed pattern (0,1) or (2,3), so a dense tile runs
 *   on the same sparse matrix instruction as a 2:4 tile.)
 * 4:8 piece (2304 bytes, like a 2:4 one): lane l owns, in 64-column slice
 *   q (q = 0, 1), columns 64*q + 16*h .. +15 of row 16*band + r -- two
 *   groups of eight, u = 0 (columns 64*q + 16*h + 0..7) and u = 1 (+8..15).
 *   Values: block q at byte 1024*q; lane l's 16 bytes at 1024*q + 16*l hold
 *   the four kept elements (ascending column) of group u = 0, then the four
 *   of group u = 1.  Masks at byte 2048: a u32 per lane at 2048 + 4*l whose
 *   byte 2*q + u has bit p set iff column 64*q + 16*h + 8*u + p of the row
 *   is kept.  (Lane l's sixteen columns are those it holds of a dense
 *   piece's two halves, so a kernel rebuilds a dense tile's operands from
 *   them without moving data between lanes.)
 * Sparse (2:4) piece: groups of four columns g = 0..31 (columns 4g..4g+3).
 *   Values: block q (q = 0, 1) at byte 1024*q; lane l holds, for p = 0..3
 *   and group g = 16*q + 4*h + p, the two kept elements of row 16*band + r in
 *   ascending column order -- 8 elements, 16 bytes.
 *   Metadata at byte 2048: a u32 per lane l at 2048 + 4*l.  Bits
 *   16*q + 4*p .. +3 hold the code of group g = 16*q + 4*h + p of that row;
 *   code = i0 | (i1 << 2), i0 < i1 the positions (0..3) of the two kept
 *   elements inside the group.
 * ------------------------------------------------------------------------- */
#define PT_B 128
#define PT_DENSE_BYTES 32768u
#define PT_SPARSE_BYTES 18432u
#define PT_DENSE_PIECE 4096u
#define PT_SPARSE_PIECE 2304u

static uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

uint64_t oracle_packed_bytes(int64_t N, int64_t K, const uint8_t* tile_map) {
  if (N <= 0 || K <= 0 || N % PT_B || K % PT_B) return 0;
  int64_t T = (N / PT_B) * (K / PT_B);
  uint64_t ns = 0;
  for (int64_t t = 0; t < T; t++) ns += tile_map[t] != 0;
  return round_up(256 + 16 * (uint64_t)T, 256) + PT_DENSE_BYTES * (uint64_t)(T - (int64_t)ns) +
         PT_SPARSE_BYTES * ns;
}

static void put32(uint8_t* p, uint32_t v) {
  for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static void put64(uint8_t* p, uint64_t v) {
  for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static void put16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)v;
  p[1] = (uint8_t)(v >> 8);
}

int oracle_pack(int dtype, int64_t N, int64_t K, const uint16_t* W, const uint8_t* tile_map,
                const uint8_t* mask, uint8_t* out, uint64_t out_bytes) {
  if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return ORACLE_ERR_ARG;
  if (N <= 0 || K <= 0) return ORACLE_ERR_ARG;
  if (N % PT_B || K % PT_B) return ORACLE_ERR_SHAPE;
  int rc = oracle_validate(N, K, PT_B, PT_B, tile_map, mask, NULL, NULL);
  if (rc) return rc;
  uint64_t total = oracle_packed_bytes(N, K, tile_map);
  if (out_bytes < total) return ORACLE_ERR_SMALL;
  memset(out, 0, (size_t)total);
  int64_t NT = N / PT_B, KT = K / PT_B, T = NT * KT;
  uint32_t ns = 0, n48 = 0;
  for (int64_t t = 0; t < T; t++) {
    ns += tile_map[t] != 0;
    n48 += tile_map[t] == 2;
  }
  uint64_t data_off = round_up(256 + 16 * (uint64_t)T, 256);
  put32(out + 0, 0x48435450u);
  put32(out + 4, 3);
  put32(out + 8, (uint32_t)dtype);
  put32(out + 12, PT_B);
  put32(out + 16, PT_B);
  put32(out + 20, (uint32_t)N);
  put32(out + 24, (uint32_t)K);
  put32(out + 28, (uint32_t)NT);
  put32(out + 32, (uint32_t)KT);
  put32(out + 36, ns);
  put64(out + 40, 256);
  put64(out + 48, data_off);
  put64(out + 56, total - data_off);
  put64(out + 64, total);
  put32(out + 72, n48);

  uint64_t rb = data_off;  /* start of the current row-block */
  for (int64_t i = 0; i < NT; i++) {
    uint64_t stride = 0;     /* S_i */
    for (int64_t j = 0; j < KT; j++) stride += tile_map[i * KT + j] ? PT_SPARSE_PIECE : PT_DENSE_PIECE;
    uint64_t prefix = 0;     /* offset of tile j's piece inside a band */
    for (int64_t j = 0; j < KT; j++) {
      int64_t t = i * KT + j;
      int sparse = tile_map[t] != 0;
      put64(out + 256 + 16 * t, rb + prefix);
      put32(out + 256 + 16 * t + 8, (uint32_t)tile_map[t]);
      put32(out + 256 + 16 * t + 12, (uint32_t)stride);
      for (int band = 0; band < 8; band++) {
        uint8_t* piece = out + rb + (uint64_t)band * stride + prefix;
        if (!sparse) {
          for (int q = 0; q < 2; q++)
            for (int e = 0; e < 2; e++)
              for (int l = 0; l < 64; l++)
                for (int g = 0; g < 4; g++)
                  for (int u = 0; u < 2; u++) {
                    int64_t row = i * PT_B + 16 * band + (l % 16);
                    int64_t col = j * PT_B + 64 * q + 16 * (l / 16) + 4 * g + 2 * e + u;
                    put16(piece + 2048 * q + 1024 * e + 16 * l + 2 * (2 * g + u), W[row * K + col]);
                  }
        } else if (tile_map[t] == 2) {
          for (int l = 0; l < 64; l++) {
            int64_t row = i * PT_B + 16 * band + (l % 16);
            for (int q = 0; q < 2; q++)
              for (int u = 0; u < 2; u++) {
                int64_t c0 = j * PT_B + 64 * q + 16 * (l / 16) + 8 * u;
                int s = 0;
                uint8_t bits = 0;
                for (int p = 0; p < 8; p++)
                  if (mask[row * K + c0 + p]) {
                    put16(piece + 1024 * q + 16 * l + 8 * u + 2 * s, W[row * K + c0 + p]);
                    bits |= (uint8_t)(1u << p);
                    s++;
                  }
                piece[2048 + 4 * l + 2 * q + u] = bits;
              }
          }
        } else {
          for (int q = 0; q < 2; q++)
            for (int l = 0; l < 64; l++) {
              int64_t row = i * PT_B + 16 * band + (l % 16);
              for (int p = 0; p < 4; p++) {
                int g = 16 * q + 4 * (l / 16) + p;
                int64_t c0 = j * PT_B + 4 * g;
                int s = 0;
                int pos[2] = {0, 0};
                for (int d = 0; d < 4; d++)
                  if (mask[row * K + c0 + d]) {
                    put16(piece + 1024 * q + 16 * l + 2 * (2 * p + s), W[row * K + c0 + d]);
                    pos[s] = d;
                    s++;
                  }
                uint32_t code = (uint32_t)pos[0] | ((uint32_t)pos[1] << 2);
                uint8_t* meta = piece + 2048 + 4 * l;
                uint32_t word = (uint32_t)meta[0] | ((uint32_t)meta[1] << 8) | ((uint32_t)meta[2] << 16) |
                                ((uint32_t)meta[3] << 24);
                word |= code << (16 * q + 4 * p);
                put32(meta, word);
              }
            }
        }
      }
      prefix += sparse ? PT_SPARSE_PIECE : PT_DENSE_PIECE;
    }
    rb += 8 * stride;
  }
  return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Packed format version 4: 64 x 64 execution tiles (the repository's own
 * layout).  The explainer's section 4 "Ablation Studies" ("Tile Size") finds
 * the method robust across tile sizes, the smaller ones giving finer
 * control, while execution wants large tiles; this format lets every 64 x 64
 * quadrant of a 128 x 128 tile be dense or 2:4 on its own.  Only dense and
 * 2:4 (no 4:8).  N and K multiples of 128.  Little-endian; all bytes not
 * written below are zero.
 *
 * Input: a quadrant map of (N/64) x (K/64) bytes, quadrant (R, C) -- rows
 * 64R .. 64R+63, columns 64C .. 64C+63 -- at R*(K/64) + C: 0 dense, 1 2:4.
 *
 * Header, 256 bytes at offset 0, as in version 3 except: version 4,
 *   tile_n = tile_k = 64, NT = N/64, KT = K/64 (the quadrant map's shape),
 *   n_sparse = the 2:4 quadrants, n_48 = 0.
 * A "half-row-block" r (r = 0 .. N/64 - 1) is rows 64r .. 64r+63; with
 * KC = K/128 tile columns, a "cell" (r, j) is its columns 128j .. 128j+127:
 * two quadrants, slice q = 0, 1 being quadrant (r, 2j + q).  Its kind bits
 * are k = sparse(r, 2j) | sparse(r, 2j+1) << 1.
 * Table at 256: N/64 * KC entries of 16 bytes, cell (r, j) at r*KC + j:
 *   u64 byte offset of the cell's band-0 piece, u32 kind bits k, u32 S_r.
 * Data at data_offset = round_up(256 + 16 * (N/64) * KC, 256).
 *
 * A "band" is 16 rows of a half-row-block (b = 0..3, rows 64r + 16b ..);
 * a "piece" is one band of one cell.  A piece holds the cell's two slices
 * in order, a dense slice taking 2048 bytes and a 2:4 slice 1024, followed,
 * if either slice is 2:4, by a 256-byte codes block: piece size
 * P(k) = (k&1 ? 1024 : 2048) + (k&2 ? 1024 : 2048) + (k ? 256 : 0), i.e.
 * 4096 (both dense), 3328 (one of each), 2304 (both 2:4).  Slice 1 starts at
 * A1 = (k&1 ? 1024 : 2048), the codes block at A1 + (k&2 ? 1024 : 2048).
 * S_r = sum over j of P(k(r, j)); half-row-block r takes 4 * S_r bytes,
 * half-row-blocks follow each other; inside r, band b's pieces of cells
 * j = 0 .. KC-1 lie back to back and band b starts S_r bytes after band b-1.
 *
 * Lanes l = 0..63 as in version 3 (row-in-band l mod 16, column group
 * h = l / 16, 16 bytes at 16 l of a 1 KB block).  For a slice q at byte A
 * of the piece:
 *   dense: blocks e = 0, 1 at A + 1024 e; lane l holds, of the row's four
 *     groups of four at columns 128j + 64q + 16h .. +15, the elements at
 *     positions 2e and 2e+1 (element 2g + u = column 128j + 64q + 16h +
 *     4g + 2e + u) -- version 3's dense block (q, e);
 *   2:4: the block at A; lane l holds, for p = 0..3, the two kept elements
 *     (ascending column) of group G = 16q + 4h + p (columns 128j + 4G ..
 *     +3) -- version 3's 2:4 value block q -- and the lane's u32 at
 *     codes + 4 l holds, in bits 16q + 4p .. +3, that group's code
 *     i0 | i1 << 2 (bits of a dense slice stay zero).
 * So a piece with k = 0 or 3 is byte for byte a version-3 dense or 2:4
 * piece, and a quadrant map constant on every 128 x 128 tile gives the same
 * data bytes as version 3 (only the header and table differ).
 * ------------------------------------------------------------------------- */
#define PQ_B 64

static uint64_t q64_piece(int k) { return (k & 1 ? 1024u : 2048u) + (k & 2 ? 1024u : 2048u) + (k ? 256u : 0u); }

uint64_t oracle_packed_bytes_q64(int64_t N, int64_t K, const uint8_t* quad_map) {
  if (N <= 0 || K <= 0 || N % PT_B || K % PT_B) return 0;
  int64_t R = N / PQ_B, KC = K / PT_B, KQ = K / PQ_B;
  uint64_t total = round_up(256 + 16 * (uint64_t)(R * KC), 256);
  for (int64_t r = 0; r < R; r++)
    for (int64_t j = 0; j < KC; j++) {
      int k = (quad_map[r * KQ + 2 * j] != 0) | ((quad_map[r * KQ + 2 * j + 1] != 0) << 1);
      total += 4 * q64_piece(k);
    }
  return total;
}

int oracle_pack_q64(int dtype, int64_t N, int64_t K, const uint16_t* W, const uint8_t* quad_map,
                    const uint8_t* mask, uint8_t* out, uint64_t out_bytes) {
  if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return ORACLE_ERR_ARG;
  if (N <= 0 || K <= 0) return ORACLE_ERR_ARG;
  if (N % PT_B || K % PT_B) return ORACLE_ERR_SHAPE;
  int64_t R = N / PQ_B, KC = K / PT_B, KQ = K / PQ_B;
  for (int64_t t = 0; t < R * KQ; t++)
    if (quad_map[t] > 1) return ORACLE_ERR_ARG; /* dense and 2:4 only */
  int rc = oracle_validate(N, K, PQ_B, PQ_B, quad_map, mask, NULL, NULL);
  if (rc) return rc;
  uint64_t total = oracle_packed_bytes_q64(N, K, quad_map);
  if (out_bytes < total) return ORACLE_ERR_SMALL;
  memset(out, 0, (size_t)total);
  uint32_t ns = 0;
  for (int64_t t = 0; t < R * KQ; t++) ns += quad_map[t] != 0;
  uint64_t data_off = round_up(256 + 16 * (uint64_t)(R * KC), 256);
  put32(out + 0, 0x48435450u);
  put32(out + 4, 4);
  put32(out + 8, (uint32_t)dtype);
  put32(out + 12, PQ_B);
  put32(out + 16, PQ_B);
  put32(out + 20, (uint32_t)N);
  put32(out + 24, (uint32_t)K);
  put32(out + 28, (uint32_t)R);
  put32(out + 32, (uint32_t)KQ);
  put32(out + 36, ns);
  put64(out + 40, 256);
  put64(out + 48, data_off);
  put64(out + 56, total - data_off);
  put64(out + 64, total);
  put32(out + 72, 0);

  uint64_t hb = data_off; /* start of the current half-row-block */
  for (int64_t r = 0; r < R; r++) {
    uint64_t stride = 0; /* S_r */
    for (int64_t j = 0; j < KC; j++)
      stride += q64_piece((quad_map[r * KQ + 2 * j] != 0) | ((quad_map[r * KQ + 2 * j + 1] != 0) << 1));
    uint64_t prefix = 0; /* offset of cell j's piece inside a band */
    for (int64_t j = 0; j < KC; j++) {
      int kb = (quad_map[r * KQ + 2 * j] != 0) | ((quad_map[r * KQ + 2 * j + 1] != 0) << 1);
      uint8_t* ent = out + 256 + 16 * (r * KC + j);
      put64(ent, hb + prefix);
      put32(ent + 8, (uint32_t)kb);
      put32(ent + 12, (uint32_t)stride);
      uint64_t a1 = kb & 1 ? 1024 : 2048;
      uint64_t codes = a1 + (kb & 2 ? 1024 : 2048);
      for (int band = 0; band < 4; band++) {
        uint8_t* piece = out + hb + (uint64_t)band * stride + prefix;
        for (int q = 0; q < 2; q++) {
          uint8_t* part = piece + (q ? a1 : 0);
          int sparse = (kb >> q) & 1;
          for (int l = 0; l < 64; l++) {
            int64_t row = r * PQ_B + 16 * band + (l % 16);
            int h = l / 16;
            if (!sparse) {
              for (int e = 0; e < 2; e++)
                for (int g = 0; g < 4; g++)
                  for (int u = 0; u < 2; u++) {
                    int64_t col = j * PT_B + 64 * q + 16 * h + 4 * g + 2 * e + u;
                    put16(part + 1024 * e + 16 * l + 2 * (2 * g + u), W[row * K + col]);
                  }
            } else {
              for (int p = 0; p < 4; p++) {
                int G = 16 * q + 4 * h + p;
                int64_t c0 = j * PT_B + 4 * G;
                int s = 0, pos[2] = {0, 0};
                for (int d = 0; d < 4; d++)
                  if (mask[row * K + c0 + d]) {
                    put16(part + 16 * l + 2 * (2 * p + s), W[row * K + c0 + d]);
                    pos[s++] = d;
                  }
                uint8_t* cw = piece + codes + 4 * l;
                uint32_t word = (uint32_t)cw[0] | ((uint32_t)cw[1] << 8) | ((uint32_t)cw[2] << 16) |
                                ((uint32_t)cw[3] << 24);
                word |= ((uint32_t)pos[0] | ((uint32_t)pos[1] << 2)) << (16 * q + 4 * p);
                put32(cw, word);
              }
            }
          }
        }
      }
      prefix += q64_piece(kb);
    }
    hb += 4 * stride;
  }
  return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Forward hybrid-mask sampler (gist.science explainer, section 2 "Methodology:
 * PATCH", "Learnable Distributions"): a learnable two-way distribution per
 * tile decides dense vs 2:4, sampled with Gumbel-Softmax; inside 2:4 tiles a
 * second learnable distribution picks one of the six 2:4 patterns per group
 * of four; the final mask combines the dense option and the 2:4 option with
 * the tile's weights.
 *
 * Definitions used (standard, not on the pages): a Gumbel(0, 1) sample from
 * a uniform u in (0, 1) is g = -ln(-ln u); the Gumbel-Softmax sample of
 * logits l_i at temperature tau is y_i = exp((l_i + g_i) / tau) /
 * sum_j exp((l_j + g_j) / tau), and its hard (straight-through forward)
 * value is the one-hot of argmax_i (l_i + g_i).
 *
 * Readings (not on the pages): the tile classes are (0 dense, 1 sparse); the
 * six patterns are the kept position pairs in lexicographic order (0,1),
 * (0,2), (0,3), (1,2), (1,3), (2,3); the soft mask of a weight at position
 * j of its group in tile t is y_dense(t) + y_sparse(t) * sum over patterns p
 * holding j of y_p(group); the hard outputs are the tile map (1 where the
 * sparse class wins) and, in every group (the pack reads it only inside 2:4
 * tiles), the kept pair of the winning pattern.  The uniforms are inputs (the
 * caller draws them).  Hard decisions are taken on float32 scores
 * l + (-logf(-logf(u))), the first index winning a tie -- the precision the
 * GPU sampler decides in; the soft values are computed in binary64.
 * ------------------------------------------------------------------------- */
static const int kPatternPairs[6][2] = {{0, 1}, {0, 2}, {0, 3}, {1, 2}, {1, 3}, {2, 3}};

double oracle_gumbel_f64(double u) { return -log(-log(u)); }
float oracle_gumbel_f32(float u) { return -logf(-logf(u)); }

/* Gumbel-Softmax over n (1..8) classes: y[0..n) soft (binary64); returns the
 * hard argmax (float32 scores). */
int oracle_gumbel_softmax(int n, const float* logit, const float* u, double tau, double* y) {
  if (n < 1 || n > 8 || !(tau > 0.0)) return -1;
  int best = 0;
  float best_s = logit[0] + oracle_gumbel_f32(u[0]);
  for (int i = 1; i < n; i++) {
    const float s = logit[i] + oracle_gumbel_f32(u[i]);
    if (s > best_s) {
      best_s = s;
      best = i;
    }
  }
  if (y) {
    double z[8], zmax = -INFINITY, sum = 0.0;
    for (int i = 0; i < n; i++) {
      z[i] = ((double)logit[i] + oracle_gumbel_f64((double)u[i])) / tau;
      if (z[i] > zmax) zmax = z[i];
    }
    for (int i = 0; i < n; i++) {
      z[i] = exp(z[i] - zmax);
      sum += z[i];
    }
    for (int i = 0; i < n; i++) y[i] = z[i] / sum;
  }
  return best;
}

/* The hybrid mask of an N x K weight with tiles of tn x tk (tk % 4 == 0):
 *   tile_logits, tile_u: [N/tn][K/tk][2] (class 0 dense, 1 sparse);
 *   pat_logits, pat_u:   [N][K/4][6] (the six patterns above);
 * outputs tile_map [N/tn][K/tk] (1 = sparse), mask [N][K] (1 = keep, the
 * winning pattern of every group), soft [N][K] (binary64; may be NULL). */
int oracle_sample_mask(int64_t N, int64_t K, int64_t tn, int64_t tk, const float* tile_logits, const float* tile_u,
                       const float* pat_logits, const float* pat_u, double tau, uint8_t* tile_map, uint8_t* mask,
                       double* soft) {
  if (N < 0 || K < 0 || tn <= 0 || tk <= 0 || tk % 4 || N % tn || K % tk || !(tau > 0.0)) return ORACLE_ERR_SHAPE;
  const int64_t KT = K / tk, G = K / 4;
  for (int64_t i = 0; i < N / tn; i++)
    for (int64_t j = 0; j < KT; j++) {
      const int64_t t = i * KT + j;
      tile_map[t] = (uint8_t)oracle_gumbel_softmax(2, tile_logits + 2 * t, tile_u + 2 * t, tau, NULL);
    }
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; n++) {
    for (int64_t g = 0; g < G; g++) {
      double yp[6], yt[2];
      const int64_t o = (n * G + g) * 6;
      const int p = oracle_gumbel_softmax(6, pat_logits + o, pat_u + o, tau, yp);
      for (int j = 0; j < 4; j++)
        mask[n * K + 4 * g + j] = (uint8_t)(j == kPatternPairs[p][0] || j == kPatternPairs[p][1]);
      if (soft) {
        const int64_t t = (n / tn) * KT + (4 * g) / tk;
        oracle_gumbel_softmax(2, tile_logits + 2 * t, tile_u + 2 * t, tau, yt);
        for (int j = 0; j < 4; j++) {
          double q = 0.0;
          for (int c = 0; c < 6; c++)
            if (j == kPatternPairs[c][0] || j == kPatternPairs[c][1]) q += yp[c];
          soft[n * K + 4 * g + j] = yt[0] + yt[1] * q;
        }
      }
    }
  }
  return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Mask tiles finer than the execution tile (gist.science explainer, section 4
 * "Ablation Studies", "Tile Size": PATCH works across tile sizes, 4 x 4 being
 * the finest control, while the hardware executes larger tiles, 128 x 128).
 *
 * Reading (not on the pages): the model was trained with the fine effective
 * mask E_fine (oracle_effective_mask at the fine tile size), so inference
 * must compute X (W o E_fine)^T exactly.  An execution tile runs as 2:4 only
 * if every fine tile inside it is 2:4 (then its 2:4 mask is the fine one);
 * otherwise it runs dense on W o E_fine -- the weights its 2:4 fine tiles
 * pruned stored as +0.
 * ------------------------------------------------------------------------- */

/* exec_map[i][j] (N/en x K/ek) = 1 iff every fine tile (b1 x b2) inside
 * execution tile (i, j) is 2:4 in fine_map (N/b1 x K/b2). */
int oracle_exec_map(int64_t N, int64_t K, int64_t b1, int64_t b2, int64_t en, int64_t ek, const uint8_t* fine_map,
                    uint8_t* exec_map) {
  if (check_shape(N, K, b1, b2) || check_shape(N, K, en, ek) || en % b1 || ek % b2) return ORACLE_ERR_SHAPE;
  const int64_t fKT = K / b2, eKT = K / ek;
  for (int64_t i = 0; i < N / en; i++)
    for (int64_t j = 0; j < eKT; j++) {
      int all = 1;
      for (int64_t fi = i * (en / b1); fi < (i + 1) * (en / b1); fi++)
        for (int64_t fj = j * (ek / b2); fj < (j + 1) * (ek / b2); fj++) all &= fine_map[fi * fKT + fj] != 0;
      exec_map[i * eKT + j] = (uint8_t)all;
    }
  return ORACLE_OK;
}

/* W_out = W o E_fine as element bits: a kept weight's bits unchanged, a
 * pruned one +0 (bits 0). */
int oracle_apply_fine_mask(int64_t N, int64_t K, int64_t b1, int64_t b2, const uint16_t* W, const uint8_t* fine_map,
                           const uint8_t* mask, uint16_t* W_out) {
  int rc = check_shape(N, K, b1, b2);
  if (rc) return rc;
  uint8_t* E = (uint8_t*)malloc((size_t)(N * K));
  if (!E) return ORACLE_ERR_ARG;
  rc = oracle_effective_mask(N, K, b1, b2, fine_map, mask, E);
  if (!rc)
    for (int64_t i = 0; i < N * K; i++) W_out[i] = E[i] ? W[i] : (uint16_t)0;
  free(E);
  return rc;
}
