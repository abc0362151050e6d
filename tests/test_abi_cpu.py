"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any GPU call."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
from sparse_gemm_amd import inputs, patch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "patch.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(patch_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(patch.LIB_PATH)
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(patch.EXPORTS)
    assert patch.load().patch_abi_version() == 4


def test_packed_bytes_matches_oracle_closed_form():
    for frac in (0.0, 0.5, 1.0):
        p = inputs.make_custom("bf16", 384, 640, 1, "exact", frac, "top2")
        assert patch.packed_bytes(torch.bfloat16, 384, 640, p.tile_map) == oracle.packed_bytes(384, 640, p.tile_map)


@pytest.mark.parametrize("N,K", [(100, 256), (256, 100), (0, 256), (256, -128), (128, 128 * 1025)])
def test_bad_shapes_rejected(N, K):
    lib = patch.load()
    tm = np.zeros(max(1, (max(N, 0) // 128) * (max(K, 0) // 128)), np.uint8)
    assert lib.patch_packed_bytes(1, N, K, tm.ctypes.data_as(ctypes.c_void_p)) == 0
    d = patch.Desc()
    rc = lib.patch_pack(1, N, K, ctypes.c_void_p(16), tm.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(16),
                        ctypes.c_void_p(16), 1 << 40, ctypes.byref(d), None)
    assert patch.STATUS[rc] == "PATCH_ERR_SHAPE"
    rc = lib.patch_dense_gemm(1, 4, N, K, ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), 1, None, 0,
                              None)
    assert patch.STATUS[rc] == "PATCH_ERR_SHAPE"
    assert "multiple" in lib.patch_last_error().decode() or "exceed" in lib.patch_last_error().decode()


def test_bad_arguments_rejected_before_launch():
    lib = patch.load()
    tm = np.zeros(4, np.uint8)
    d = patch.Desc()
    V = ctypes.c_void_p
    tmp = tm.ctypes.data_as(V)
    # bad dtype
    assert patch.STATUS[lib.patch_pack(7, 256, 256, V(16), tmp, V(16), V(16), 1 << 20, ctypes.byref(d), None)] == \
        "PATCH_ERR_INVALID_ARG"
    # null pointers
    assert patch.STATUS[lib.patch_pack(1, 256, 256, None, tmp, V(16), V(16), 1 << 20, ctypes.byref(d), None)] == \
        "PATCH_ERR_INVALID_ARG"
    # unaligned pointer
    assert patch.STATUS[lib.patch_pack(1, 256, 256, V(18), tmp, V(16), V(16), 1 << 20, ctypes.byref(d), None)] == \
        "PATCH_ERR_INVALID_ARG"
    # blob too small
    need = lib.patch_packed_bytes(1, 256, 256, tmp)
    assert patch.STATUS[lib.patch_pack(1, 256, 256, V(16), tmp, V(16), V(16), need - 1, ctypes.byref(d), None)] == \
        "PATCH_ERR_BUFFER_TOO_SMALL"
    # dense gemm: y dtype must be the input dtype or F32
    assert patch.STATUS[lib.patch_dense_gemm(1, 4, 256, 256, V(16), V(16), V(16), 0, None, 0, None)] == \
        "PATCH_ERR_INVALID_ARG"
    # M < 0, decode variant with M > 128, unknown variant
    assert patch.STATUS[lib.patch_dense_gemm(1, -1, 256, 256, V(16), V(16), V(16), 1, None, 0, None)] == \
        "PATCH_ERR_INVALID_ARG"
    assert patch.STATUS[lib.patch_dense_gemm_ex(1, 129, 256, 256, V(16), V(16), V(16), 1, None, 0, 1, None)] == \
        "PATCH_ERR_INVALID_ARG"
    for bad_variant in (11, 12, -1):
        assert patch.STATUS[lib.patch_dense_gemm_ex(1, 4, 256, 256, V(16), V(16), V(16), 1, None, 0, bad_variant,
                                                    None)] == "PATCH_ERR_INVALID_ARG"
    # a workspace size without a workspace, or an unaligned one
    assert patch.STATUS[lib.patch_dense_gemm_ex(1, 4, 256, 256, V(16), V(16), V(16), 1, None, 64, 2, None)] == \
        "PATCH_ERR_INVALID_ARG"
    assert patch.STATUS[lib.patch_dense_gemm_ex(1, 4, 256, 256, V(16), V(16), V(16), 1, V(24), 64, 2, None)] == \
        "PATCH_ERR_INVALID_ARG"
    # the decode kernel serves K <= 65536 only
    assert patch.STATUS[lib.patch_dense_gemm_ex(1, 4, 256, 65536 + 128, V(16), V(16), V(16), 1, None, 0, 1, None)] == \
        "PATCH_ERR_UNSUPPORTED"
    # M == 0 is a no-op that launches nothing (valid on a machine without a GPU)
    assert lib.patch_dense_gemm(1, 0, 256, 256, V(16), V(16), V(16), 1, None, 0, None) == 0


def test_desc_from_oracle_header_and_gemm_checks():
    p = inputs.make_custom("bf16", 256, 384, 2, "bernoulli", 0.5, "top2")
    blob = oracle.pack("bf16", p.w, p.tile_map, p.mask)
    d = patch.desc_from_header(blob[:256].tobytes())
    assert (d.version, d.dtype, d.N, d.K, d.nt_n, d.nt_k) == (3, 1, 256, 384, 2, 3)
    assert d.n_sparse == int(p.tile_map.sum()) and d.total_bytes == blob.size
    lib = patch.load()
    assert lib.patch_gemm_workspace_bytes(ctypes.byref(d), 2048) == 0
    # M = 0 no-op on a valid descriptor
    assert lib.patch_gemm(ctypes.byref(d), ctypes.c_void_p(16), ctypes.c_void_p(16), 0, ctypes.c_void_p(16), 1,
                          None, 0, None) == 0
    # corrupted headers are rejected
    bad = bytearray(blob[:256].tobytes())
    bad[0] ^= 1
    with pytest.raises(patch.PatchError):
        patch.desc_from_header(bytes(bad))
    bad = bytearray(blob[:256].tobytes())
    bad[64] ^= 0x10  # total_bytes
    with pytest.raises(patch.PatchError):
        patch.desc_from_header(bytes(bad))
    d.n_sparse += 1  # descriptor no longer matches its sizes
    assert patch.STATUS[lib.patch_gemm(ctypes.byref(d), ctypes.c_void_p(16), ctypes.c_void_p(16), 4,
                                       ctypes.c_void_p(16), 1, None, 0, None)] == "PATCH_ERR_INVALID_ARG"


def test_workspace_query_host_logic():
    """The workspace query is host logic: K is split only when the output
    blocks cannot fill the GPU, into whole M x N fp32 planes, never more
    bytes than 2 * N * K, and nothing for invalid shapes."""
    lib = patch.load()
    ws = lambda M, N, K: int(lib.patch_dense_gemm_workspace_bytes(M, N, K))
    assert ws(2048, 11008, 4096) == 0  # 43 row-block pairs x 8+ M-blocks fill the GPU
    for M, N, K in [(128, 4096, 4096), (64, 4096, 11008), (17, 512, 4096), (300, 384, 4096)]:
        b = ws(M, N, K)
        assert b > 0 and b % (M * N * 4) == 0 and b <= 2 * N * K, (M, N, K, b)
        assert b // (M * N * 4) <= K // 256  # at least two tile columns a range
    for bad in [(0, 4096, 4096), (-1, 4096, 4096), (16, 100, 4096), (16, 4096, 100), (16, 4096, 128 * 1025)]:
        assert ws(*bad) == 0, bad


@pytest.mark.parametrize("b1,b2", [(1, 4), (4, 4), (16, 16), (32, 64), (64, 128), (128, 128)])
def test_exec_tile_map_matches_oracle(b1, b2):
    """Host logic of patch_exec_tile_map (no GPU): the execution map of a
    fine map equals the oracle's, byte for byte."""
    rng = np.random.default_rng(b1 * 1000 + b2)
    N, K = 384, 512
    fm = inputs.gen_fine_map(rng, N, K, b1, b2, 0.4, 0.8)
    got = patch.exec_tile_map(N, K, fm, b1, b2)
    assert np.array_equal(got, oracle.exec_map(N, K, fm, b1, b2))


def test_exec_tile_map_rejects_bad_tiles():
    lib = patch.load()
    fm = np.ones(4096, dtype=np.uint8)
    out = np.zeros(16, dtype=np.uint8)
    P = ctypes.c_void_p
    for b1, b2, want in ((3, 4, 2), (4, 2, 2), (4, 6, 2), (256, 128, 2), (0, 4, 2), (4, 4, 0)):
        assert lib.patch_exec_tile_map(256, 256, b1, b2, P(fm.ctypes.data), P(out.ctypes.data), None) == want
    assert lib.patch_exec_tile_map(256, 256, 4, 4, None, P(out.ctypes.data), None) == 1
    assert lib.patch_exec_tile_map(200, 256, 4, 4, P(fm.ctypes.data), P(out.ctypes.data), None) == 2
