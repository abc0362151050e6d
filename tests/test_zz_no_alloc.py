"""patch_gemm_noalloc: the hybrid GEMM with the library's own device scratch
(for callers that cannot allocate).  Checked against patch_gemm (the entry
point it is a variant of) and the oracle, on two calls in a row, the second
with fewer tokens; and its size limit on the host."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from sparse_gemm_amd import inputs, patch
from tests.gpu_util import assert_close, dev_bits, dev_u8


def test_noalloc_rejects_scratch_beyond_its_size():
    """A shape whose launch wants more scratch than the library holds is
    refused on the host, before any pointer is touched (no GPU needed)."""
    lib = patch.load()
    cap = int(lib.patch_noalloc_scratch_bytes())
    assert cap == 64 << 20
    d = patch.Desc()
    d.version, d.dtype, d.tile_n, d.tile_k, d.N, d.K = 3, 1, 128, 128, 32768, 65536
    d.nt_n, d.nt_k = 256, 512
    M = 7886
    want = int(lib.patch_gemm_workspace_bytes(ctypes.byref(d), M))
    assert want > cap
    V = ctypes.c_void_p
    rc = lib.patch_gemm_noalloc(ctypes.byref(d), V(256), V(256), M, V(256), 1, None)
    assert patch.STATUS[rc] == "PATCH_ERR_BUFFER_TOO_SMALL"
    assert "scratch" in lib.patch_last_error().decode()


@pytest.mark.gpu
def test_noalloc_matches_gemm_two_calls():
    assert torch.cuda.is_available(), "GPU test"
    torch.cuda.set_device(0)
    lib = patch.load()
    # 512 x 4096: the prefill launch splits K at these token counts, so the
    # scratch holds the partial sums
    N, K = 512, 4096
    p = inputs.make_custom("bf16", N, K, 31, "bernoulli", 0.5, "top2")
    pw = patch.pack(dev_bits(p.w, "bf16"), p.tile_map, dev_u8(p.mask))
    for M in (160, 64, 4):  # the second call smaller than the first, then a decode-sized one
        want = int(lib.patch_gemm_workspace_bytes(ctypes.byref(pw.desc), M))
        assert want > 0 or M <= 16, (M, want)  # (the query answers for the prefill kernel at any M)
        Xb = inputs.make_custom_x("bf16", M, K, 32 + M)
        X = dev_bits(Xb, "bf16")
        ref = oracle.gemm_f64("bf16", Xb, p.w, p.tile_map, p.mask)
        for od in (torch.bfloat16, torch.float32):
            y_ref = patch.gemm(X, pw, out_dtype=od)
            y = torch.full((M, N), 7.0, dtype=od, device="cuda")
            patch.gemm_noalloc(X, pw, out=y)
            torch.cuda.synchronize()
            f32 = od == torch.float32
            # the same kernels and K ranges as patch_gemm: identical results
            assert torch.equal(y, y_ref), (M, od)
            assert_close(y, y_ref.double().cpu().numpy(), f32=f32, what=f"noalloc vs gemm M={M} {od}")
            assert_close(y, ref, f32=f32, what=f"noalloc vs oracle M={M} {od}")
