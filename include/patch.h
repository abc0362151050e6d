/*
 * patch.h -- C ABI of the MI355X (gfx950) hybrid tile-sparse GEMM library.
 *
 * The method: PATCH, "Learnable Tile-level Hybrid Sparsity for LLMs"
 * (arXiv 2509.23410).  A weight matrix W (N x K) is cut into tiles; every
 * tile is either dense or 2:4 sparse (two kept weights in every four
 * consecutive ones), which gives an overall sparsity anywhere between 0% and
 * 50% (arXiv abstract; gist.science explainer, section 2 "Methodology:
 * PATCH", "Core Mechanism").  Dense tiles run on dense matrix units and 2:4
 * tiles on the sparse matrix path (same explainer, "Inference &
 * Deployment"); execution tiles are 128 x 128 (section 4, "Ablation
 * Studies").  This library computes Y = X * (W o E)^T on one GPU, with E the
 * effective mask: 1 inside dense tiles, the 2:4 mask inside sparse tiles.
 *
 * Conventions for every entry point:
 *   - Matrices are row-major with the last index contiguous: W is N x K
 *     (output features x input features, the layout of a linear layer's
 *     weight), X is M x K, Y is M x N.  Elements are IEEE binary16 (PATCH_F16)
 *     or bfloat16 (PATCH_BF16); Y may also be binary32 (PATCH_F32).
 *   - "_dev" pointers are device memory on the current HIP device, owned by
 *     the caller, 16-byte aligned.  "_host" pointers are host memory.  The
 *     library allocates no device memory and keeps no pointer after return.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     GEMM calls are asynchronous on that stream; patch_pack synchronises it.
 *   - Errors are returned as patch_status; nothing is thrown.  On an error
 *     found on the host nothing is launched and no output is written.
 *     patch_last_error() returns a thread-local description of the last
 *     failure on the calling thread.
 *   - N and K must be positive multiples of 128 (else PATCH_ERR_SHAPE).
 *     M >= 0; M == 0 is a no-op returning PATCH_OK.
 */
#ifndef PATCH_H
#define PATCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PATCH_OK = 0,
  PATCH_ERR_INVALID_ARG = 1,      /* null/unaligned pointer, bad dtype, M < 0, bad descriptor */
  PATCH_ERR_SHAPE = 2,            /* N or K not a positive multiple of 128, or too large */
  PATCH_ERR_MASK = 3,             /* a group of four inside a sparse tile does not keep exactly 2 */
  PATCH_ERR_BUFFER_TOO_SMALL = 4, /* packed buffer or workspace smaller than required */
  PATCH_ERR_UNSUPPORTED = 5,      /* valid request this build does not implement */
  PATCH_ERR_HIP = 6               /* a HIP runtime call failed; see patch_last_error() */
} patch_status;

typedef enum { PATCH_F16 = 0, PATCH_BF16 = 1, PATCH_F32 = 2 } patch_dtype;

/* GEMM variant selection for patch_gemm_ex (patch_gemm uses PATCH_VARIANT_AUTO). */
typedef enum {
  PATCH_VARIANT_AUTO = 0,    /* decode for M <= 16 (K <= 65536); for 16 < M <= 128 the
                                kernel whose time model is lower (prefill's for the K
                                split the workspace passed allows); prefill otherwise */
  PATCH_VARIANT_DECODE = 1,  /* W-streaming kernel; valid for 1 <= M <= 128, K <= 65536
                                (else PATCH_ERR_INVALID_ARG / PATCH_ERR_UNSUPPORTED) */
  PATCH_VARIANT_PREFILL = 2, /* output-tiled MFMA kernel, W and X staged through LDS;
                                any M >= 1; splits K when the output blocks cannot fill
                                the GPU and the workspace allows */
  /* The prefill kernel at one M-block width and staging (K split as its
   * cost model decides for that width, within the workspace passed): for
   * tests and measurements that must run every kernel on the same shapes;
   * the register-staged ones run dense and 2:4 tiles only (a blob with 4:8
   * tiles: PATCH_ERR_UNSUPPORTED). */
  PATCH_VARIANT_PREFILL_W64 = 3,      /* registers, 64 columns of M a workgroup */
  PATCH_VARIANT_PREFILL_W128 = 4,     /* registers, 128 */
  PATCH_VARIANT_PREFILL_W192 = 5,     /* registers, 192 */
  PATCH_VARIANT_PREFILL_W256 = 6,     /* registers, 256 */
  PATCH_VARIANT_PREFILL_W128_LDS = 7, /* W and X staged through LDS, 128 */
  PATCH_VARIANT_PREFILL_W192_LDS = 8, /* W and X staged through LDS, 192 */
  PATCH_VARIANT_PREFILL_W256_LDS = 9, /* W and X staged through LDS, 256 */
  PATCH_VARIANT_PREFILL_W64_LDS = 10, /* W and X staged through LDS, 64 */
  /* The prefill kernel whose waves each hold a 128-row register tile of
   * both row-blocks of their pair (W and X staged through LDS), with 4
   * waves (one a SIMD): its own choice of width, or 128, 192 or 256
   * columns of M a workgroup; with 8 waves (two a SIMD): 128 or 256. */
  PATCH_VARIANT_PREFILL_BIG = 11,
  PATCH_VARIANT_PREFILL_BIG_W128 = 12,
  PATCH_VARIANT_PREFILL_BIG_W192 = 13,
  PATCH_VARIANT_PREFILL_BIG_W256 = 14,
  PATCH_VARIANT_PREFILL_BIG8_W128 = 15,
  PATCH_VARIANT_PREFILL_BIG8_W256 = 16
} patch_variant;

/* Host-side mirror of the packed blob's header (format version 3). */
typedef struct {
  uint32_t version;   /* 3 (128 x 128 execution tiles) or 4 (64 x 64, patch_pack_q64) */
  uint32_t dtype;     /* PATCH_F16 or PATCH_BF16 */
  uint32_t tile_n;    /* 128 (version 4: 64) */
  uint32_t tile_k;    /* 128 (version 4: 64) */
  uint32_t N, K;      /* matrix shape */
  uint32_t nt_n;      /* N / tile_n */
  uint32_t nt_k;      /* K / tile_k */
  uint32_t n_sparse;  /* number of compressed tiles (2:4 and 4:8; version 4: 2:4 quadrants) */
  uint32_t n_48;      /* number of 4:8 tiles among them (header byte 72; version 4: 0) */
  uint64_t table_offset; /* 256 */
  uint64_t data_offset;  /* round_up(256 + 16 * entries, 256); entries = nt_n * nt_k
                            (version 4: (N / 64) * (K / 128)) */
  uint64_t total_bytes;  /* size of the whole blob */
} patch_packed_desc;

/* ABI version of this header (incremented on any incompatible change). */
int32_t patch_abi_version(void);

/*
 * Size in bytes of the packed blob for a tile map (PATCH "tile-level
 * assignment", gist.science explainer, section 2 "Core Mechanism"):
 *   round_up(256 + 16*T, 256) + 32768 * n_dense + 18432 * n_sparse,
 * T = (N/128)*(K/128), n_sparse the 2:4 and 4:8 tiles.  tile_map_host: T
 * bytes, row-block-major (tile (i, j) at i*(K/128) + j): 0 dense, 1 2:4,
 * 2 4:8.  Returns 0 if the arguments are invalid (dtype, shape, null map, a
 * map byte above 2).
 */
uint64_t patch_packed_bytes(patch_dtype dtype, int64_t N, int64_t K, const uint8_t* tile_map_host);

/*
 * Pack dense W plus a tile map and a 2:4 (or 4:8) mask into the blob
 * (format version 3): a 256-byte header, a 16-byte-per-tile table (data
 * offset, kind, band stride) and the tile data.  A 2:4 tile keeps, for every
 * group of four consecutive weights along K, the two kept values plus a
 * 4-bit code i0 | i1 << 2 (2 bits per kept value); a dense tile keeps all
 * 128 x 128 values, each 64-column slice stored as two halves holding
 * positions (0,1) and (2,3) of every group of four.  A tile is stored as
 * eight pieces, one per 16-row band (4096 bytes dense, 2304 bytes 2:4 or 4:8);
 * within a row-block the pieces of one band for all its tiles lie back to
 * back, so band b of a tile sits at the tile's offset + b * band stride.
 * Pieces are laid out in the lane order of the sparse matrix instruction's
 * operands, which then runs both kinds (a dense half is a 2:4 operand with a
 * fixed code).  The 2:4 rule: gist.science explainer, section 1 "Problem
 * Statement"; the six patterns: section 2 "Pattern Selection".
 *
 * A 4:8 tile (another N:M pattern, explainer section 5 "Significance",
 * "Future Direction") keeps four of every eight consecutive weights along K.
 * A band piece takes 2304 bytes, as a 2:4 one.  In each 64-column slice q a
 * lane l owns columns 64q + 16(l/16) .. +15, which are two groups of eight
 * u = 0, 1: the 1 KB block at 1024q holds, at 16l, the four kept values
 * (ascending column) of group 0 and then of group 1; the lane's 32-bit word
 * at 2048 + 4l holds group u's 8-bit position mask in byte 2q + u.  Those
 * sixteen columns are exactly the lane's share of a dense piece's two
 * halves, so the GEMM kernels rebuild the halves in registers and run them
 * on the sparse instruction with the dense tile's fixed codes: 4:8 tiles
 * take a 2:4 tile's bytes and a dense tile's matrix-core time.
 *
 *   W_dev          N x K elements of `dtype`, row-major, device.
 *   tile_map_host  T bytes on the host: 0 dense, 1 2:4, 2 4:8 (other
 *                  values: PATCH_ERR_INVALID_ARG).
 *   mask_dev       N x K bytes on the device, nonzero = keep.  Read only
 *                  inside 2:4 and 4:8 tiles (ignored in dense tiles).
 *   packed_dev     output, device, at least patch_packed_bytes() bytes.
 *   desc_out       host descriptor of the result (written on success only).
 *
 * Synchronises `stream` (to report PATCH_ERR_MASK: a 2:4 group not keeping
 * two of four, or a 4:8 group not keeping four of eight).  On PATCH_ERR_MASK the
 * blob contents are undefined.  The blob is immutable afterwards and may be
 * shared by any number of concurrent GEMM calls.
 */
patch_status patch_pack(patch_dtype dtype, int64_t N, int64_t K, const void* W_dev, const uint8_t* tile_map_host,
                        const uint8_t* mask_dev, void* packed_dev, uint64_t packed_bytes,
                        patch_packed_desc* desc_out, void* stream);

/*
 * 64 x 64 execution tiles (format version 4).  The explainer's section 4
 * "Ablation Studies" ("Tile Size") finds the method robust across tile
 * sizes, smaller tiles giving finer control, while execution wants larger
 * tiles.  Here every 64 x 64 quadrant of a 128 x 128 tile is dense or 2:4 on
 * its own, so a mask chosen on 64 x 64 tiles runs as it is (where the
 * 128 x 128 policy, patch_exec_tile_map, runs a tile as 2:4 only if all its
 * quadrants are).  Dense and 2:4 only (no 4:8); N and K multiples of 128.
 *
 *   quad_map_host  (N/64) x (K/64) bytes on the host, quadrant (R, C) --
 *                  rows 64R.., columns 64C.. -- at R*(K/64) + C: 0 dense,
 *                  1 2:4 (other values: PATCH_ERR_INVALID_ARG).
 *
 * Layout: a table entry per 64-row half-row-block r and 128-column tile
 * column j (at r*(K/128) + j): u64 offset of its band-0 piece, u32 kind bits
 * k (bit q set: the 64-column slice q, quadrant (r, 2j + q), is 2:4), u32
 * the half-row-block's band stride.  A piece (16 rows) holds slice 0 then
 * slice 1 -- 2048 bytes dense (version 3's dense blocks), 1024 bytes 2:4
 * (version 3's value block) -- then, if k != 0, a 256-byte codes block (lane
 * l's u32 at 4l, slice q's codes in bits 16q..16q+15): 4096, 3328 or 2304
 * bytes.  Size: round_up(256 + 16 * entries, 256) + 8192 per dense quadrant
 * + 4096 per 2:4 quadrant + 1024 per entry with k != 0.
 *
 * patch_packed_bytes_q64 returns that size (0 for invalid arguments);
 * patch_pack_q64 takes W and the mask as patch_pack does (the mask read only
 * inside 2:4 quadrants), synchronises `stream`, and reports PATCH_ERR_MASK
 * for a 2:4-quadrant group not keeping two of four.  patch_gemm,
 * patch_gemm_ex (AUTO, DECODE, PREFILL and the LDS-staged PREFILL_W*_LDS
 * variants; the others return PATCH_ERR_UNSUPPORTED) and
 * patch_gemm_noalloc run such a blob; the fused gate/up product does not.
 */
uint64_t patch_packed_bytes_q64(patch_dtype dtype, int64_t N, int64_t K, const uint8_t* quad_map_host);
patch_status patch_pack_q64(patch_dtype dtype, int64_t N, int64_t K, const void* W_dev,
                            const uint8_t* quad_map_host, const uint8_t* mask_dev, void* packed_dev,
                            uint64_t packed_bytes, patch_packed_desc* desc_out, void* stream);

/* Parse a blob header already copied to the host (for reloading a saved blob).
 * header_bytes must be at least 76 (the descriptor's fields end with n_48 at
 * bytes 72..75; else PATCH_ERR_BUFFER_TOO_SMALL).  Checks magic, version,
 * dtype, tile shape and that the sizes agree. */
patch_status patch_desc_from_header(const void* header_host, uint64_t header_bytes, patch_packed_desc* desc_out);

/*
 * Device workspace bytes the prefill kernel can use for this M: when its
 * output blocks alone cannot fill the GPU (few tokens or few row-blocks) it
 * splits K into ranges, writes each range's fp32 partial sums to the
 * workspace ([splits][M][N] floats) and adds them in range order in a
 * second kernel on the same stream, so results do not depend on timing.
 * When the blocks fill whole rounds of the GPU with a few left over (the
 * tail split), only those few are cut into K ranges, which hand their fp32
 * sums (256 x width floats a block and range) and a flag each through the
 * workspace to the block's first range, which adds them in range order.
 * 0 when no split is wanted.  A smaller workspace only means fewer ranges
 * (none below two planes of M*N floats) or no tail split.  The workspace is
 * scratch owned by the call: its contents need no initialisation and are
 * undefined after; calls that run concurrently need distinct workspaces.
 */
uint64_t patch_gemm_workspace_bytes(const patch_packed_desc* desc, int64_t M);

/* The same for patch_dense_gemm on an N x K weight (same kernels and shape
 * choice as patch_gemm, every tile dense). */
uint64_t patch_dense_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * Hybrid GEMM: Y = X * (W o E)^T from the packed blob -- the inference-time
 * product of a PATCH layer, whose dense tiles run on dense matrix units and
 * whose 2:4 tiles run on the sparse path (gist.science explainer, section 2
 * "Methodology: PATCH", "Inference & Deployment"; E as in "Core
 * Mechanism": 1 in dense tiles, the 2:4 mask in sparse ones).  Both tile
 * kinds run on v_smfmac_f32_16x16x64 (bf16/f16): a 2:4 slice once with its
 * packed codes, a dense slice as its two fixed-pattern halves; accumulation
 * is fp32; a 16-bit Y is rounded to nearest even.
 *
 *   desc        descriptor from patch_pack / patch_desc_from_header.
 *   packed_dev  the blob (device).
 *   X_dev       M x K elements of desc->dtype (device).
 *   Y_dev       M x N elements of y_dtype (device), y_dtype in {desc->dtype, PATCH_F32}.
 *   workspace   device scratch of workspace_bytes (16-byte aligned), or NULL
 *               with workspace_bytes = 0; see patch_gemm_workspace_bytes().
 * Asynchronous on `stream`.
 */
patch_status patch_gemm(const patch_packed_desc* desc, const void* packed_dev, const void* X_dev, int64_t M,
                        void* Y_dev, patch_dtype y_dtype, void* workspace_dev, uint64_t workspace_bytes,
                        void* stream);

/* patch_gemm with an explicit kernel variant (patch_variant); used by tests to
 * run both kernels on the same shapes. */
patch_status patch_gemm_ex(const patch_packed_desc* desc, const void* packed_dev, const void* X_dev, int64_t M,
                           void* Y_dev, patch_dtype y_dtype, void* workspace_dev, uint64_t workspace_bytes,
                           int32_t variant, void* stream);

/*
 * Same-shape dense baseline: Y = X * W^T from plain row-major W (N x K) --
 * the dense layer PATCH's speedups are measured against (gist.science
 * explainer, section 4 "Experimental Results", "Speedup & Efficiency"), with
 * the same kernels and tiling as patch_gemm, every tile dense, on the dense
 * matrix instruction.  Arguments as patch_gemm, with W_dev N x K elements of
 * `dtype` in place of the blob.
 */
patch_status patch_dense_gemm(patch_dtype dtype, int64_t M, int64_t N, int64_t K, const void* X_dev,
                              const void* W_dev, void* Y_dev, patch_dtype y_dtype, void* workspace_dev,
                              uint64_t workspace_bytes, void* stream);

/* patch_dense_gemm with an explicit kernel variant (patch_variant). */
patch_status patch_dense_gemm_ex(patch_dtype dtype, int64_t M, int64_t N, int64_t K, const void* X_dev,
                                 const void* W_dev, void* Y_dev, patch_dtype y_dtype, void* workspace_dev,
                                 uint64_t workspace_bytes, int32_t variant, void* stream);

/*
 * Several projections of the same input in one launch (e.g. attention's q,
 * k and v): pack the row-concatenation of count (1 .. 8) matrices with the
 * same K -- matrix i is N_host[i] x K (a multiple of 128), with its own tile
 * map (host) and mask (device), arguments per matrix as patch_pack -- into
 * one format-3 blob with N = sum of N_host.  patch_gemm on it returns the
 * projections side by side: Y = [Y_0 | Y_1 | ...], M x N.
 */
uint64_t patch_packed_bytes_concat(patch_dtype dtype, int32_t count, const int64_t* N_host, int64_t K,
                                   const uint8_t* const* tile_maps_host);
patch_status patch_pack_concat(patch_dtype dtype, int32_t count, const int64_t* N_host, int64_t K,
                               const void* const* W_dev, const uint8_t* const* tile_maps_host,
                               const uint8_t* const* masks_dev, void* packed_dev, uint64_t packed_bytes,
                               patch_packed_desc* desc_out, void* stream);

/*
 * Fused gate/up projection of the LLaMA MLP (the pages evaluate PATCH on
 * LLaMA-2 models, gist.science explainer, section 4 "Experimental Results";
 * that architecture's MLP is down(SiLU(gate(x)) * up(x))):
 *   H = SiLU(X (Wg o Eg)^T) * (X (Wu o Eu)^T)   elementwise, H is M x F,
 * SiLU(x) = x / (1 + e^-x), all in fp32 before one rounding of H.
 *
 * patch_pack_gate_up packs the two F x K matrices into ONE blob of the
 * row-block interleave of Wg and Wu (N = 2F: row-block 2i holds Wg's
 * row-block i, 2i+1 holds Wu's; the same format version 3, tile maps and
 * masks interleaved the same way), so one GEMM launch reads both and a
 * workgroup holds matching gate and up sums for its epilogue.  Arguments as
 * patch_pack, per matrix; F a positive multiple of 128.  A plain patch_gemm
 * on this blob returns the two projections interleaved by 128 columns.
 */
uint64_t patch_packed_bytes_gate_up(patch_dtype dtype, int64_t F, int64_t K, const uint8_t* map_g_host,
                                    const uint8_t* map_u_host);
patch_status patch_pack_gate_up(patch_dtype dtype, int64_t F, int64_t K, const void* Wg_dev, const void* Wu_dev,
                                const uint8_t* map_g_host, const uint8_t* map_u_host, const uint8_t* mask_g_dev,
                                const uint8_t* mask_u_dev, void* packed_dev, uint64_t packed_bytes,
                                patch_packed_desc* desc_out, void* stream);

/*
 * H from a gate/up blob (desc->N = 2F).  H_dev: M x F of h_dtype (the blob's
 * dtype or PATCH_F32); workspace and variant as patch_gemm_ex (the fused
 * decode kernel runs twice the waves and so needs M <= 16 or K <= 32768,
 * else PATCH_ERR_UNSUPPORTED; AUTO then takes the prefill kernel, whose K
 * split adds the ranges' partial sums before SiLU).  Asynchronous.
 */
uint64_t patch_gemm_swiglu_workspace_bytes(const patch_packed_desc* desc, int64_t M);
patch_status patch_gemm_swiglu(const patch_packed_desc* desc, const void* packed_dev, const void* X_dev, int64_t M,
                               void* H_dev, patch_dtype h_dtype, void* workspace_dev, uint64_t workspace_bytes,
                               int32_t variant, void* stream);

/* Same-shape dense baseline of the fused projection from two plain
 * row-major F x K matrices Wg_dev and Wu_dev (every tile dense). */
uint64_t patch_dense_gemm_swiglu_workspace_bytes(int64_t M, int64_t F, int64_t K);
patch_status patch_dense_gemm_swiglu(patch_dtype dtype, int64_t M, int64_t F, int64_t K, const void* X_dev,
                                     const void* Wg_dev, const void* Wu_dev, void* H_dev, patch_dtype h_dtype,
                                     void* workspace_dev, uint64_t workspace_bytes, int32_t variant, void* stream);

/*
 * Forward hybrid-mask sampler (gist.science explainer, section 2
 * "Methodology: PATCH": tile selection and pattern selection are learnable
 * distributions sampled with Gumbel-Softmax; the final mask combines the
 * dense and the 2:4 option).  For an N x K weight with 128 x 128 tiles
 * (N, K positive multiples of 128):
 *   tile_logits_dev, tile_u_dev: float32 [N/128][K/128][2], class 0 dense,
 *     class 1 sparse (8-byte aligned);
 *   pat_logits_dev, pat_u_dev: float32 [N][K/4][6], the six kept position
 *     pairs of a group in lexicographic order (0,1) (0,2) (0,3) (1,2) (1,3)
 *     (2,3) (16-byte aligned);
 *   the u arrays hold the sampler's uniforms, each in the open interval
 *     (0, 1) (the caller draws them; other values give IEEE inf/NaN scores);
 *   tau: the temperature, finite and > 0.
 * With g = -ln(-ln u) per class (float32), outputs (caller-owned device
 * memory, row-major):
 *   tile_map_dev uint8 [N/128][K/128]: 1 where l_sparse + g > l_dense + g'
 *     (a 2:4 tile), else 0 -- the tile map patch_pack takes (after a copy
 *     to the host);
 *   mask_dev uint8 [N][K] (4-byte aligned): 1 at the two positions of the
 *     pattern with the largest l_p + g_p (first on a tie) in every group --
 *     the 2:4 mask patch_pack takes;
 *   soft_dev float32 [N][K] (16-byte aligned) or NULL: y_dense + y_sparse *
 *     (sum of y_p over the patterns keeping the position), y = softmax of
 *     (l + g) / tau over the tile's two classes and over the group's six
 *     patterns.
 * Asynchronous on `stream`.  Errors: PATCH_ERR_SHAPE (N, K), PATCH_ERR_INVALID_ARG
 * (null or misaligned pointers, tau not finite and positive).
 */
patch_status patch_sample_mask(int64_t N, int64_t K, const float* tile_logits_dev, const float* tile_u_dev,
                               const float* pat_logits_dev, const float* pat_u_dev, float tau, uint8_t* tile_map_dev,
                               uint8_t* mask_dev, float* soft_dev, void* stream);

/*
 * Mask tiles finer than the 128 x 128 execution tile (gist.science
 * explainer, section 4 "Ablation Studies", "Tile Size": the mask can be
 * learnt on tiles as fine as 4 x 4; the hardware executes 128 x 128).  The
 * result must stay X (W o E_fine)^T, E_fine the effective mask at the fine
 * tile size (1 in dense fine tiles, the 2:4 mask in 2:4 ones).  Policy: an
 * execution tile runs as 2:4 only if every fine tile in it is 2:4 (its 2:4
 * mask is then the fine one); otherwise it runs dense on W o E_fine.
 *
 * Fine tiles are b1 x b2 (rows x columns), b1 and b2 dividing 128, b2 a
 * multiple of 4; the fine map is uint8 [N/b1][K/b2], nonzero = 2:4.
 *
 * patch_exec_tile_map (host only): exec_map_host uint8 [N/128][K/128] = 1
 * where every fine tile is 2:4; *n_sparse_out (may be NULL) receives their
 * number.  Errors: PATCH_ERR_SHAPE, PATCH_ERR_INVALID_ARG (null maps).
 *
 * patch_apply_fine_mask: W_out_dev = W o E_fine as element bits (kept weights
 * unchanged, pruned ones +0), N x K row-major 16-bit elements of dtype; W_dev
 * and W_out_dev 16-byte aligned (they may be the same buffer), mask_dev uint8
 * [N][K] 8-byte aligned, fine_map_dev the fine map in device memory.  The
 * groups of the 2:4 fine tiles are applied as given (patch_pack validates
 * the ones its 2:4 execution tiles store).  Asynchronous.  Then
 * patch_pack(W_out, exec map, mask) packs the layer.
 */
patch_status patch_exec_tile_map(int64_t N, int64_t K, int64_t b1, int64_t b2, const uint8_t* fine_map_host,
                                 uint8_t* exec_map_host, int64_t* n_sparse_out);
patch_status patch_apply_fine_mask(patch_dtype dtype, int64_t N, int64_t K, int64_t b1, int64_t b2, const void* W_dev,
                                   const uint8_t* fine_map_dev, const uint8_t* mask_dev, void* W_out_dev,
                                   void* stream);

/*
 * patch_gemm without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The prefill kernel's K split and tail
 * split -- the only scratch the GEMM path uses: fp32 partial sums of the K
 * ranges, written before they are read, and the tail split's flags, which
 * each launch leaves at 0; nothing to clear -- go to a device array of
 * patch_noalloc_scratch_bytes() bytes (64 MiB) that the
 * library holds on every device it runs on until the process ends.
 * Arguments and results as patch_gemm, same kernels and launch shapes.
 * Errors: as patch_gemm; PATCH_ERR_BUFFER_TOO_SMALL if this shape's launch
 * wants more scratch than the array holds (patch_gemm_workspace_bytes(desc,
 * M) > patch_noalloc_scratch_bytes()), checked on the host before anything
 * is launched; PATCH_ERR_HIP if the array's address cannot be had.  Calls
 * that overlap on one device share the array and race: serialize them.
 * The call allocates nothing (no hipMalloc, no library allocation).
 */
uint64_t patch_noalloc_scratch_bytes(void);
patch_status patch_gemm_noalloc(const patch_packed_desc* desc, const void* packed_dev, const void* X_dev, int64_t M,
                                void* Y_dev, patch_dtype y_dtype, void* stream);

/*
 * For tests of the prefill kernel's bounded wait.  In the tail split (the
 * output blocks left over after whole rounds of the GPU, cut into K ranges
 * that hand their fp32 sums to the block's first range through the
 * workspace) the first range polls a flag per range a bounded number of
 * times.  polls > 0: in the launches that follow, the first range waits for
 * a flag value that no range stores and gives up after that many polls,
 * marking its block's outputs NaN -- the path a range that never arrives
 * would take, forced from the host so a test can see the launch end;
 * polls <= 0: back to normal (the default).  Process-wide, for tests only.
 */
void patch_debug_tail_wait(int32_t polls);

/*
 * Measurement probes.  They compute nothing of the method; they measure, on
 * the device the GEMMs run on, the ceilings the GEMM kernels are compared
 * with (the datasheet peaks -- 8 TB/s HBM, 2.5 PFLOP/s dense bf16 matrix
 * math, twice that for 2:4 sparse instructions -- are upper bounds that one
 * launch of a given size does not reach).  Both are asynchronous on
 * `stream`; the caller times them.
 *
 * patch_probe_stream_read: reads `bytes` (a multiple of 16) of src_dev once
 * with 16-byte loads and writes at most a few words of sink_dev (scratch of
 * sink_bytes, at least 4; it bounds the grid: sink_bytes / 4 workgroups).
 * Errors: PATCH_ERR_INVALID_ARG (null or unaligned pointers, bytes not a
 * positive multiple of 16, sink_bytes < 4).
 *
 * patch_probe_matrix_rate: `workgroups` workgroups of 4 waves, each wave
 * issuing `iters` rounds of independent matrix instructions of one kind on
 * register operands: kind 0 v_mfma_f32_16x16x32_bf16, 1
 * v_smfmac_f32_16x16x64_bf16, 2 v_mfma_f32_32x32x16_bf16, 3
 * v_smfmac_f32_32x32x32_bf16.  sink_dev: scratch of 4 * workgroups bytes.
 * patch_probe_matrix_flops returns the flops one such launch executes
 * (dense-equivalent for the sparse kinds: 2 x rows x columns x logical K per
 * instruction), 0 for bad arguments.  Errors: PATCH_ERR_INVALID_ARG (kind
 * outside 0..3, iters or workgroups < 1, null sink).
 *
 * patch_probe_copy_rate: the global -> LDS copy rate of the prefill kernels'
 * copy instruction (global_load_lds, 16 bytes a lane): `workgroups`
 * workgroups of 8 waves, each wave copying 7 KB an iteration for `iters`
 * iterations into a two-slot LDS ring (wait for the previous iteration's
 * copies, then a barrier).  Workgroup g reads its window of window_bytes (a
 * power of two) at offset (g * window_bytes) mod src_bytes of src_dev,
 * cycling through it: few distinct windows (src_bytes within the L2s)
 * measure copies from L2, windows adding up to more than the L2s copies
 * from past them.  sink_dev:
 * scratch of at least 4 * workgroups bytes.  patch_probe_copy_bytes returns
 * the bytes one launch copies (0 for bad arguments).  Errors:
 * PATCH_ERR_INVALID_ARG (null or unaligned pointers, iters or workgroups <
 * 1, window_bytes not a power of two of at least 1024 dividing src_bytes,
 * sink too small).
 */
patch_status patch_probe_stream_read(const void* src_dev, uint64_t bytes, void* sink_dev, uint64_t sink_bytes,
                                     void* stream);
patch_status patch_probe_copy_rate(const void* src_dev, uint64_t src_bytes, uint64_t window_bytes, int32_t iters,
                                   int32_t workgroups, void* sink_dev, uint64_t sink_bytes, void* stream);
uint64_t patch_probe_copy_bytes(int32_t iters, int32_t workgroups);
patch_status patch_probe_matrix_rate(int32_t kind, int32_t iters, int32_t workgroups, void* sink_dev, void* stream);
uint64_t patch_probe_matrix_flops(int32_t kind, int32_t iters, int32_t workgroups);

const char* patch_status_string(patch_status s);
const char* patch_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PATCH_H */
