"""GPU parity of the fine-mask-tile path (patch_exec_tile_map,
patch_apply_fine_mask, then patch_pack and patch_gemm) against the CPU
oracle, through the C ABI.

PATCH's mask can be learnt on tiles as fine as 4 x 4 while execution needs
128 x 128 tiles (gist.science explainer, section 4 "Ablation Studies", "Tile
Size").  Policy: a 128 x 128 tile runs as 2:4 only if all its fine tiles are
2:4, else dense on W o E_fine.  Bars: W o E_fine and the packed blob are
bit-exact with the oracle; the GEMM meets the hybrid GEMM's tolerance against
the oracle's product on the fine tiles, X (W o E_fine)^T.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from sparse_gemm_amd import inputs, patch
from tests.gpu_util import assert_close, dev_bits, dev_u8

pytestmark = pytest.mark.gpu

TILES = [(1, 4), (4, 4), (8, 16), (16, 16), (32, 64), (64, 64), (128, 128)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    patch.load()
    torch.cuda.set_device(0)


@pytest.mark.parametrize("b1,b2", TILES)
def test_apply_fine_mask_bit_exact(b1, b2):
    N, K = 384, 640
    p = inputs.make_fine("bf16", N, K, b1, b2, 10 + b1 + b2)
    p.w[:4, :16] = 0x8000  # kept -0 stays -0
    out = patch.apply_fine_mask(dev_bits(p.w, "bf16"), dev_u8(p.tile_map), dev_u8(p.mask), b1, b2)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.apply_fine_mask(p.w, p.tile_map, p.mask, b1, b2))


def test_apply_fine_mask_in_place_and_f16():
    N, K, b1, b2 = 256, 384, 16, 32
    p = inputs.make_fine("f16", N, K, b1, b2, 3)
    W = dev_bits(p.w, "f16")
    patch.apply_fine_mask(W, dev_u8(p.tile_map), dev_u8(p.mask), b1, b2, out=W)
    torch.cuda.synchronize()
    got = W.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.apply_fine_mask(p.w, p.tile_map, p.mask, b1, b2))


@pytest.mark.parametrize("b1,b2", TILES)
@pytest.mark.parametrize("M", [1, 16, 100])
def test_pack_fine_and_gemm(b1, b2, M):
    """pack_fine: blob equal to the oracle's pack of (W o E_fine, its
    execution map, mask); the GEMM on it equals the fine-tiled product."""
    N, K = 384, 640
    p = inputs.make_fine("bf16", N, K, b1, b2, 20 + b1 + b2, s_exec=0.5)
    pw = patch.pack_fine(dev_bits(p.w, "bf16"), p.tile_map, dev_u8(p.mask), b1, b2)
    torch.cuda.synchronize()
    em = oracle.exec_map(N, K, p.tile_map, b1, b2)
    ref_blob = oracle.pack("bf16", oracle.apply_fine_mask(p.w, p.tile_map, p.mask, b1, b2), em, p.mask)
    assert np.array_equal(pw.blob.cpu().numpy(), ref_blob)
    assert pw.desc.n_sparse == int(em.sum())
    Xb = inputs.make_custom_x("bf16", M, K, 30 + M)
    ref = oracle.gemm_f64("bf16", Xb, p.w, p.tile_map, p.mask, tile_n=b1, tile_k=b2)
    assert_close(patch.gemm(dev_bits(Xb, "bf16"), pw), ref, what=f"{b1}x{b2} M={M}")
    assert_close(patch.gemm(dev_bits(Xb, "bf16"), pw, out_dtype=torch.float32), ref, f32=True,
                 what=f"{b1}x{b2} M={M} f32")


def test_pack_fine_llama_q_proj():
    """LLaMA-2-7B q_proj shape with 32 x 32 mask tiles: blob bit-exact, the
    GEMM at M = 16 on every output."""
    N, K, b1, b2 = 4096, 4096, 32, 32
    p = inputs.make_fine("bf16", N, K, b1, b2, 7, s_exec=0.5, p_sub=0.9)
    pw = patch.pack_fine(dev_bits(p.w, "bf16"), p.tile_map, dev_u8(p.mask), b1, b2)
    torch.cuda.synchronize()
    em = oracle.exec_map(N, K, p.tile_map, b1, b2)
    assert 0 < em.sum() < em.size
    ref_blob = oracle.pack("bf16", oracle.apply_fine_mask(p.w, p.tile_map, p.mask, b1, b2), em, p.mask)
    assert np.array_equal(pw.blob.cpu().numpy(), ref_blob)
    Xb = inputs.make_custom_x("bf16", 16, K, 8)
    ref = oracle.gemm_f64("bf16", Xb, p.w, p.tile_map, p.mask, tile_n=b1, tile_k=b2)
    assert_close(patch.gemm(dev_bits(Xb, "bf16"), pw), ref, what="q_proj 32x32")


def test_apply_fine_mask_rejects_bad_arguments():
    lib = patch.load()
    p = inputs.make_fine("bf16", 128, 256, 4, 4, 1)
    W, fm, mk = dev_bits(p.w, "bf16"), dev_u8(p.tile_map), dev_u8(p.mask)
    out = torch.empty(128 * 256 + 8, dtype=torch.bfloat16, device="cuda")
    P = ctypes.c_void_p
    s = P(patch._stream())

    def call(dt=1, N=128, K=256, b1=4, b2=4, w=W.data_ptr(), o=out.data_ptr(), m=mk.data_ptr()):
        return lib.patch_apply_fine_mask(dt, N, K, b1, b2, P(w), P(fm.data_ptr()), P(m), P(o), s)

    assert call() == 0
    assert call(dt=2) == 1                     # F32 is not a weight type
    assert call(b1=3) == 2 and call(b2=6) == 2 and call(N=100) == 2
    assert call(o=out.data_ptr() + 2) == 1     # W_out not 16-byte aligned
    assert call(m=mk.data_ptr() + 4) == 1      # mask not 8-byte aligned
    assert call(w=0) == 1
    torch.cuda.synchronize()
