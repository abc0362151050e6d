"""ctypes marshalling for the C oracle (test infrastructure only)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F16, BF16 = 0, 1
_DT = {"f16": F16, "bf16": BF16, F16: F16, BF16: BF16}
_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_ERRS = {1: "invalid argument", 2: "shape not a multiple of the tile", 3: "mask: a sparse group does not keep exactly 2",
         4: "buffer too small"}


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle error {code}: {_ERRS.get(code, '?')}")
        self.code = code


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain C, OpenMP, IEEE arithmetic)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_validate.argtypes = [I64, I64, I64, I64, P, P, P, P]
    lib.oracle_validate.restype = ctypes.c_int
    lib.oracle_effective_mask.argtypes = [I64, I64, I64, I64, P, P, P]
    lib.oracle_effective_mask.restype = ctypes.c_int
    lib.oracle_gemm_f64.argtypes = [ctypes.c_int, I64, I64, I64, I64, I64, P, P, P, P, P]
    lib.oracle_gemm_f64.restype = ctypes.c_int
    lib.oracle_round_f64.argtypes = [ctypes.c_int, I64, P, P]
    lib.oracle_round_f64.restype = None
    lib.oracle_packed_bytes.argtypes = [I64, I64, P]
    lib.oracle_packed_bytes.restype = ctypes.c_uint64
    lib.oracle_pack.argtypes = [ctypes.c_int, I64, I64, P, P, P, P, ctypes.c_uint64]
    lib.oracle_pack.restype = ctypes.c_int
    lib.oracle_packed_bytes_q64.argtypes = [I64, I64, P]
    lib.oracle_packed_bytes_q64.restype = ctypes.c_uint64
    lib.oracle_pack_q64.argtypes = [ctypes.c_int, I64, I64, P, P, P, P, ctypes.c_uint64]
    lib.oracle_pack_q64.restype = ctypes.c_int
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_swiglu_f64.argtypes = [ctypes.c_int, I64, I64, I64, I64, I64, P, P, P, P, P, P, P, P]
    lib.oracle_swiglu_f64.restype = ctypes.c_int
    lib.oracle_gumbel_f64.argtypes = [ctypes.c_double]
    lib.oracle_gumbel_f64.restype = ctypes.c_double
    lib.oracle_gumbel_f32.argtypes = [ctypes.c_float]
    lib.oracle_gumbel_f32.restype = ctypes.c_float
    lib.oracle_gumbel_softmax.argtypes = [ctypes.c_int, P, P, ctypes.c_double, P]
    lib.oracle_gumbel_softmax.restype = ctypes.c_int
    lib.oracle_sample_mask.argtypes = [I64, I64, I64, I64, P, P, P, P, ctypes.c_double, P, P, P]
    lib.oracle_sample_mask.restype = ctypes.c_int
    lib.oracle_exec_map.argtypes = [I64, I64, I64, I64, I64, I64, P, P]
    lib.oracle_exec_map.restype = ctypes.c_int
    lib.oracle_apply_fine_mask.argtypes = [I64, I64, I64, I64, P, P, P, P]
    lib.oracle_apply_fine_mask.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint16)


def _u8(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint8)


def num_threads() -> int:
    return int(load().oracle_num_threads())


def f16_to_double(bits: int) -> float:
    return load().oracle_f16_to_double(int(bits))


def bf16_to_double(bits: int) -> float:
    return load().oracle_bf16_to_double(int(bits))


def validate(N, K, tile_map, mask, tile_n=128, tile_k=128):
    """Returns None if valid, else (row, group) of the first bad sparse group."""
    lib = load()
    tm, mk = _u8(tile_map), _u8(mask)
    r = ctypes.c_int64(-1)
    g = ctypes.c_int64(-1)
    rc = lib.oracle_validate(N, K, tile_n, tile_k, _p(tm), _p(mk), ctypes.byref(r), ctypes.byref(g))
    if rc == 3:
        return (r.value, g.value)
    if rc:
        raise OracleError(rc)
    return None


def effective_mask(N, K, tile_map, mask, tile_n=128, tile_k=128) -> np.ndarray:
    lib = load()
    tm, mk = _u8(tile_map), _u8(mask)
    E = np.zeros((N, K), dtype=np.uint8)
    rc = lib.oracle_effective_mask(N, K, tile_n, tile_k, _p(tm), _p(mk), _p(E))
    if rc:
        raise OracleError(rc)
    return E


def gemm_f64(dtype, X, W, tile_map, mask, tile_n=128, tile_k=128) -> np.ndarray:
    """Y = X (W o E)^T in fp64; X (M, K) and W (N, K) are 16-bit patterns."""
    lib = load()
    X, W = _u16(X), _u16(W)
    M, K = X.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError("K mismatch")
    tm, mk = _u8(tile_map), _u8(mask)
    Y = np.zeros((M, N), dtype=np.float64)
    rc = lib.oracle_gemm_f64(_DT[dtype], M, N, K, tile_n, tile_k, _p(X), _p(W), _p(tm), _p(mk), _p(Y))
    if rc:
        raise OracleError(rc)
    return Y


def round_f64(dtype, Y: np.ndarray) -> np.ndarray:
    """fp64 -> 16-bit patterns with round-to-nearest-even."""
    lib = load()
    Y = np.ascontiguousarray(Y, dtype=np.float64)
    out = np.zeros(Y.shape, dtype=np.uint16)
    lib.oracle_round_f64(_DT[dtype], Y.size, _p(Y), _p(out))
    return out


def packed_bytes(N, K, tile_map) -> int:
    return int(load().oracle_packed_bytes(N, K, _p(_u8(tile_map))))


def pack(dtype, W, tile_map, mask) -> np.ndarray:
    """The format-1 blob as a uint8 array."""
    lib = load()
    W = _u16(W)
    N, K = W.shape
    tm, mk = _u8(tile_map), _u8(mask)
    nbytes = lib.oracle_packed_bytes(N, K, _p(tm))
    if nbytes == 0:
        raise OracleError(2)
    out = np.zeros(nbytes, dtype=np.uint8)
    rc = lib.oracle_pack(_DT[dtype], N, K, _p(W), _p(tm), _p(mk), _p(out), nbytes)
    if rc:
        raise OracleError(rc)
    return out


def packed_bytes_q64(N, K, quad_map) -> int:
    """Size of the format-4 blob (64 x 64 execution tiles) for a (N/64, K/64) quadrant map."""
    qm = _u8(quad_map)
    if N % 128 or K % 128 or qm.shape != (N // 64, K // 64):
        return 0
    return int(load().oracle_packed_bytes_q64(N, K, _p(qm)))


def pack_q64(dtype, W, quad_map, mask) -> np.ndarray:
    """The format-4 blob (64 x 64 execution tiles, quadrant map 0 dense / 1
    2:4) as a uint8 array."""
    lib = load()
    W = _u16(W)
    N, K = W.shape
    qm, mk = _u8(quad_map), _u8(mask)
    if qm.shape != (N // 64, K // 64):
        raise OracleError(2)
    nbytes = lib.oracle_packed_bytes_q64(N, K, _p(qm))
    if nbytes == 0:
        raise OracleError(2)
    out = np.zeros(nbytes, dtype=np.uint8)
    rc = lib.oracle_pack_q64(_DT[dtype], N, K, _p(W), _p(qm), _p(mk), _p(out), nbytes)
    if rc:
        raise OracleError(rc)
    return out


def silu(x: float) -> float:
    return load().oracle_silu(float(x))


def swiglu_f64(dtype, X, Wg, Wu, map_g, map_u, mask_g, mask_u, tile_n=128, tile_k=128) -> np.ndarray:
    """H = SiLU(X (Wg o Eg)^T) * (X (Wu o Eu)^T) in fp64 (the LLaMA MLP's gated
    product); X (M, K), Wg and Wu (F, K) are 16-bit patterns."""
    lib = load()
    X, Wg, Wu = _u16(X), _u16(Wg), _u16(Wu)
    M, K = X.shape
    F, K2 = Wg.shape
    if K != K2 or Wu.shape != Wg.shape:
        raise ValueError("shape mismatch")
    H = np.zeros((M, F), dtype=np.float64)
    rc = lib.oracle_swiglu_f64(_DT[dtype], M, F, K, tile_n, tile_k, _p(X), _p(Wg), _p(Wu), _p(_u8(map_g)),
                               _p(_u8(map_u)), _p(_u8(mask_g)), _p(_u8(mask_u)), _p(H))
    if rc:
        raise OracleError(rc)
    return H


def interleave_gate_up(A_g: np.ndarray, A_u: np.ndarray, rows_per_block: int) -> np.ndarray:
    """Rows of A_g and A_u interleaved by blocks of rows_per_block: block 2i is
    A_g's block i, block 2i+1 is A_u's (the row order the fused gate/up blob
    is packed in).  A pure permutation of rows, used for weights (128-row
    blocks), tile maps (one row per row-block) and masks."""
    if A_g.shape != A_u.shape or A_g.shape[0] % rows_per_block:
        raise ValueError("shape mismatch")
    nb = A_g.shape[0] // rows_per_block
    g = A_g.reshape(nb, rows_per_block, *A_g.shape[1:])
    u = A_u.reshape(nb, rows_per_block, *A_u.shape[1:])
    return np.stack([g, u], axis=1).reshape(2 * A_g.shape[0], *A_g.shape[1:])


# ---------------------------------------------------------------------------- hybrid-mask sampler
# Forward Gumbel-Softmax sampler (gist.science explainer, section 2
# "Methodology: PATCH", "Learnable Distributions"); definitions and readings
# are restated in oracle.c next to oracle_sample_mask.
PATTERN_PAIRS = ((0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3))


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def gumbel(u: float) -> float:
    """-ln(-ln u) in binary64."""
    return load().oracle_gumbel_f64(float(u))


def gumbel_softmax(logits, u, tau: float):
    """(soft probabilities in binary64, hard argmax on float32 scores)."""
    logits, u = _f32(logits), _f32(u)
    y = np.zeros(logits.size, dtype=np.float64)
    best = load().oracle_gumbel_softmax(int(logits.size), _p(logits), _p(u), float(tau), _p(y))
    if best < 0:
        raise OracleError(1)
    return y, best


def sample_mask(tile_logits, tile_u, pat_logits, pat_u, tau: float, tile_n: int = 128, tile_k: int = 128,
                soft: bool = True):
    """tile_logits, tile_u: [N/tn, K/tk, 2]; pat_logits, pat_u: [N, K/4, 6].
    Returns (tile_map uint8 [N/tn, K/tk], mask uint8 [N, K], soft float64
    [N, K] or None)."""
    pat_logits, pat_u = _f32(pat_logits), _f32(pat_u)
    tile_logits, tile_u = _f32(tile_logits), _f32(tile_u)
    N, G = pat_logits.shape[0], pat_logits.shape[1]
    K = 4 * G
    assert pat_logits.shape == (N, G, 6) and pat_u.shape == pat_logits.shape
    assert tile_logits.shape == (N // tile_n, K // tile_k, 2) and tile_u.shape == tile_logits.shape
    tmap = np.zeros((N // tile_n, K // tile_k), dtype=np.uint8)
    mask = np.zeros((N, K), dtype=np.uint8)
    out = np.zeros((N, K), dtype=np.float64) if soft else None
    rc = load().oracle_sample_mask(N, K, tile_n, tile_k, _p(tile_logits), _p(tile_u), _p(pat_logits), _p(pat_u),
                                   float(tau), _p(tmap), _p(mask), _p(out) if soft else None)
    if rc:
        raise OracleError(rc)
    return tmap, mask, out


# ---------------------------------------------------------------------------- fine mask tiles
# Mask tiles finer than the 128 x 128 execution tile (gist.science explainer,
# section 4 "Ablation Studies", "Tile Size"); the reading is restated in
# oracle.c next to oracle_exec_map.
def exec_map(N, K, fine_map, b1, b2, en=128, ek=128) -> np.ndarray:
    """Execution tile map: 1 iff every fine tile inside is 2:4."""
    fm = _u8(fine_map)
    assert fm.shape == (N // b1, K // b2)
    out = np.zeros((N // en, K // ek), dtype=np.uint8)
    rc = load().oracle_exec_map(N, K, b1, b2, en, ek, _p(fm), _p(out))
    if rc:
        raise OracleError(rc)
    return out


def apply_fine_mask(W, fine_map, mask, b1, b2) -> np.ndarray:
    """W o E_fine as element bits (pruned weights +0)."""
    W = _u16(W)
    N, K = W.shape
    fm, mk = _u8(fine_map), _u8(mask)
    out = np.zeros_like(W)
    rc = load().oracle_apply_fine_mask(N, K, b1, b2, _p(W), _p(fm), _p(mk), _p(out))
    if rc:
        raise OracleError(rc)
    return out
