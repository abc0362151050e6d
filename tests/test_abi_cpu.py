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
V = ctypes.c_void_p


def _declared():
    src = open(os.path.join(ROOT, "include", "patch.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(patch_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(patch.LIB_PATH)
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(patch.EXPORTS)
    assert patch.load().patch_abi_version() == 5


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
    for bad_variant in (17, 18, -1):
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
    bytes than 2 * N * K, or -- the tail split -- for the blocks left over
    after whole rounds, into one slot of fp32 sums a block and range; nothing
    for invalid shapes."""
    lib = patch.load()
    ws = lambda M, N, K: int(lib.patch_dense_gemm_workspace_bytes(M, N, K))
    # 43 row-block pairs x 8 M-blocks of 256: a round of 256 blocks, the 88
    # left over in two K ranges (the tail split): a slot of 256 x 256 fp32
    # sums for each, then their 8-byte flags (rounded to 256 bytes)
    assert ws(2048, 11008, 4096) == 88 * 256 * 256 * 4 + 768
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


def test_desc_from_header_needs_76_bytes():
    """The descriptor's last field (n_48) is at header bytes 72..75: a shorter
    buffer is rejected instead of read past its end."""
    p = inputs.make_custom("bf16", 256, 384, 3, "bernoulli", 0.5, "top2")
    blob = oracle.pack("bf16", p.w, p.tile_map, p.mask)
    assert patch.desc_from_header(bytes(blob[:76].tobytes())).N == 256
    for n in (72, 75):
        with pytest.raises(patch.PatchError) as e:
            patch.desc_from_header(bytes(blob[:n].tobytes()))
        assert e.value.name == "PATCH_ERR_BUFFER_TOO_SMALL"


def _fake_packed(N=256, K=384, dtype=1):
    d = patch.Desc()
    d.version, d.dtype, d.tile_n, d.tile_k, d.N, d.K = 3, dtype, 128, 128, N, K
    d.nt_n, d.nt_k = N // 128, K // 128
    d.table_offset, d.data_offset = 256, 256 + 256
    d.total_bytes = 512 + 32768 * d.nt_n * d.nt_k
    return patch.PackedWeight(torch.zeros(d.total_bytes, dtype=torch.uint8), d)


def test_binding_rejects_bad_tensors_before_any_call():
    """The C ABI takes raw pointers, so the binding checks shapes, dtypes,
    layout and device before calling it (no GPU is touched here: every case
    fails in the binding)."""
    pw = _fake_packed()
    bf = torch.bfloat16
    X = torch.zeros(4, 384, dtype=bf)
    cases = [
        (lambda: patch.gemm(torch.zeros(4, 256, dtype=bf), pw), "K = 384"),          # X has the wrong K
        (lambda: patch.gemm(torch.zeros(4, 384, dtype=torch.float16), pw), "bfloat16"),  # X dtype != blob dtype
        (lambda: patch.gemm(torch.zeros(384, 8, dtype=bf).t(), pw), "contiguous"),   # transposed view
        (lambda: patch.gemm(torch.zeros(4, 768, dtype=bf)[:, ::2], pw), "contiguous"),  # strided view
        (lambda: patch.gemm(torch.zeros(384, dtype=bf), pw), "2-D"),
        (lambda: patch.gemm(X, pw, out_dtype=torch.float32, out=torch.zeros(4, 256, dtype=bf)), "float32"),
        (lambda: patch.gemm(X, pw, out=torch.zeros(4, 128, dtype=bf)), "shape"),
        (lambda: patch.gemm(X, pw, out=torch.zeros(256, 4, dtype=bf).t()), "contiguous"),
        (lambda: patch.gemm(X, pw, out_dtype=torch.float16), "out_dtype"),
        (lambda: patch.gemm(X, pw), "device"),                                       # all checks pass but the device
        (lambda: patch.gemm(X, patch.PackedWeight(pw.blob[:100], pw.desc)), "smaller"),
        (lambda: patch.dense_gemm(X, torch.zeros(256, 256, dtype=bf)), "K = 256"),
        (lambda: patch.dense_gemm(X, torch.zeros(256, 384, dtype=torch.float16)), "bfloat16"),
        (lambda: patch.dense_gemm(X, torch.zeros(384, 256, dtype=bf).t()), "contiguous"),
        (lambda: patch.dense_gemm(X, torch.zeros(256, 384, dtype=bf), out=torch.zeros(4, 255, dtype=bf)), "shape"),
        (lambda: patch.gemm_swiglu(X, pw, out=torch.zeros(4, 256, dtype=bf)), "shape"),  # H is M x N/2
        (lambda: patch.dense_gemm_swiglu(X, torch.zeros(128, 384, dtype=bf), torch.zeros(256, 384, dtype=bf)),
         "shape"),
        (lambda: patch.pack(torch.zeros(256, 384, dtype=bf), np.zeros((2, 3), np.uint8),
                            torch.zeros(256, 384, dtype=torch.int8)), "uint8"),
        (lambda: patch.pack(torch.zeros(256, 384, dtype=bf), np.zeros((2, 3), np.uint8),
                            torch.zeros(256, 383, dtype=torch.uint8)), "shape"),
        (lambda: patch.pack(torch.zeros(256, 384, dtype=bf), np.zeros((3, 2), np.uint8),
                            torch.zeros(256, 384, dtype=torch.uint8)), "tile map"),
        (lambda: patch.pack(torch.zeros(256, 384, dtype=torch.float32), np.zeros((2, 3), np.uint8),
                            torch.zeros(256, 384, dtype=torch.uint8)), "float16 or bfloat16"),
        (lambda: patch.pack(torch.zeros(256, 384, dtype=bf), np.zeros((2, 3), np.uint8),
                            torch.zeros(256, 384, dtype=torch.uint8)), "device"),
    ]
    for fn, text in cases:
        with pytest.raises(ValueError) as e:
            fn()
        assert text in str(e.value), (text, str(e.value))


# ---------------------------------------------------------------- 64 x 64 execution tiles (format 4)
def test_packed_bytes_q64_matches_oracle():
    lib = patch.load()
    for seed, (s_exec, p_sub) in enumerate(((0.0, 0.0), (0.3, 0.5), (1.0, 1.0), (0.0, 0.7))):
        p = inputs.make_fine("bf16", 384, 640, 64, 64, 30 + seed, s_exec=s_exec, p_sub=p_sub)
        want = oracle.packed_bytes_q64(384, 640, p.tile_map)
        assert patch.packed_bytes_q64(torch.bfloat16, 384, 640, p.tile_map) == want
        qm = np.ascontiguousarray(p.tile_map)
        assert lib.patch_packed_bytes_q64(0, 384, 640, qm.ctypes.data_as(ctypes.c_void_p)) == want
    bad = np.zeros((6, 10), np.uint8)
    bad[1, 3] = 2  # 4:8 is not a quadrant kind
    assert lib.patch_packed_bytes_q64(1, 384, 640, bad.ctypes.data_as(ctypes.c_void_p)) == 0
    assert patch.packed_bytes_q64(torch.bfloat16, 384, 640, np.zeros((3, 5), np.uint8)) == 0  # wrong map shape
    assert lib.patch_packed_bytes_q64(1, 320, 640, np.zeros((5, 10), np.uint8).ctypes.data_as(ctypes.c_void_p)) == 0


def test_pack_q64_host_checks_before_any_device_work():
    lib = patch.load()
    qm = np.zeros((4, 4), np.uint8)
    qm[0, 0] = 3
    d = patch.Desc()
    rc = lib.patch_pack_q64(1, 256, 256, V(16), qm.ctypes.data_as(ctypes.c_void_p), V(16), V(16), 1 << 40,
                            ctypes.byref(d), None)
    assert patch.STATUS[rc] == "PATCH_ERR_INVALID_ARG"
    qm[0, 0] = 1
    rc = lib.patch_pack_q64(1, 256, 256, V(16), qm.ctypes.data_as(ctypes.c_void_p), V(16), V(16), 1024,
                            ctypes.byref(d), None)
    assert patch.STATUS[rc] == "PATCH_ERR_BUFFER_TOO_SMALL"
    rc = lib.patch_pack_q64(1, 256, 256, V(8), qm.ctypes.data_as(ctypes.c_void_p), V(16), V(16), 1 << 40,
                            ctypes.byref(d), None)
    assert patch.STATUS[rc] == "PATCH_ERR_INVALID_ARG"  # unaligned W


def test_desc_from_oracle_q64_header_and_gemm_checks():
    p = inputs.make_fine("bf16", 256, 384, 64, 64, 33, s_exec=0.3, p_sub=0.5)
    blob = oracle.pack_q64("bf16", p.w, p.tile_map, p.mask)
    d = patch.desc_from_header(blob[:256].tobytes())
    assert (d.version, d.dtype, d.tile_n, d.tile_k, d.N, d.K, d.nt_n, d.nt_k, d.n_48) == (4, 1, 64, 64, 256, 384,
                                                                                           4, 6, 0)
    assert d.n_sparse == int(p.tile_map.sum()) and d.total_bytes == blob.size
    lib = patch.load()
    assert lib.patch_gemm(ctypes.byref(d), V(16), V(16), 0, V(16), 1, None, 0, None) == 0  # M = 0 no-op
    # the register-staged and big-tile variants and the fused product reject it before any device work
    for v in (3, 6, 11, 16):
        assert patch.STATUS[lib.patch_gemm_ex(ctypes.byref(d), V(16), V(16), 64, V(16), 1, None, 0, v,
                                              None)] == "PATCH_ERR_UNSUPPORTED"
    assert patch.STATUS[lib.patch_gemm_swiglu(ctypes.byref(d), V(16), V(16), 64, V(16), 1, None, 0, 0,
                                              None)] == "PATCH_ERR_UNSUPPORTED"
    bad = bytearray(blob[:256].tobytes())
    bad[64] ^= 0x04  # total_bytes off by 1 KiB * 4: no longer a multiple of the step or out of range
    bad[56] ^= 0x04
    with pytest.raises(patch.PatchError):
        patch.desc_from_header(bytes(bad))
    d.n_48 = 1
    assert patch.STATUS[lib.patch_gemm(ctypes.byref(d), V(16), V(16), 4, V(16), 1, None, 0,
                                       None)] == "PATCH_ERR_INVALID_ARG"


def test_probe_copy_rate_host_checks():
    """The global -> LDS copy probe: its byte count in closed form (7 copies of
    1 KB a wave, 8 waves a workgroup, per iteration) and every argument check
    taken before any launch."""
    lib = patch.load()
    V = ctypes.c_void_p
    assert lib.patch_probe_copy_bytes(3, 5) == 7 * 8 * 1024 * 3 * 5
    assert lib.patch_probe_copy_bytes(0, 5) == 0 and lib.patch_probe_copy_bytes(3, 0) == 0
    bad = [
        (None, 1 << 20, 1 << 18, 10, 4, V(16), 64),        # null source
        (V(16), 1 << 20, 1 << 18, 10, 4, None, 64),        # null sink
        (V(24), 1 << 20, 1 << 18, 10, 4, V(16), 64),       # unaligned source
        (V(16), 1 << 20, 1000, 10, 4, V(16), 64),          # window not a multiple of 1 KB
        (V(16), 3 << 20, 3 << 10, 10, 4, V(16), 64),       # window not a power of two
        (V(16), 3 << 18, 1 << 19, 10, 4, V(16), 64),       # window does not divide the source
        (V(16), 1 << 20, 1 << 21, 10, 4, V(16), 64),       # window larger than the source
        (V(16), 1 << 20, 1 << 18, 0, 4, V(16), 64),        # no iterations
        (V(16), 1 << 20, 1 << 18, 10, 0, V(16), 64),       # no workgroups
        (V(16), 1 << 20, 1 << 18, 10, 32, V(16), 64),      # sink smaller than 4 bytes a workgroup
    ]
    for args in bad:
        assert patch.STATUS[lib.patch_probe_copy_rate(*args, None)] == "PATCH_ERR_INVALID_ARG", args
