"""GPU parity of 4:8 tiles (four of every eight consecutive weights kept along
K) against the CPU oracle, through the C ABI.

4:8 is one of the "other N:M patterns" the gist.science explainer's section
5 "Significance" ("Future Direction") says the method extends to.  A 4:8
tile is the third tile kind (tile-map byte 2) next to dense (0) and 2:4 (1):
the pack stores four values and an 8-bit position mask per group, and the
GEMM kernels rebuild each lane's group of the dense 16x16x32 operand in
registers.  Bars as for the other kinds: blob bit-exact, GEMM within the
hybrid GEMM's tolerance (fp32 output 1e-5), exact on small integers and on
identity X.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_gemm_amd import inputs, patch
from tests.gpu_util import assert_close, dev_bits, dev_u8, host_f64

pytestmark = pytest.mark.gpu

LDS_KERNELS = ["prefill_w64_lds", "prefill_w128_lds", "prefill_w192_lds", "prefill_w256_lds", "prefill_big_w128",
               "prefill_big_w192", "prefill_big_w256", "prefill_big8_w128", "prefill_big8_w256"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    patch.load()
    torch.cuda.set_device(0)


def _pack(p):
    W = dev_bits(p.w, p.dtype)
    return patch.pack(W, p.tile_map, dev_u8(p.mask)), W


@pytest.mark.parametrize("N,K,f24,f48,mk", [(128, 128, 0.0, 1.0, "top"), (384, 640, 0.3, 0.4, "top"),
                                            (384, 640, 0.3, 0.4, "uniform"), (256, 1152, 0.0, 0.6, "uniform")])
def test_pack_48_bit_exact(N, K, f24, f48, mk):
    p = inputs.make_mixed("bf16", N, K, N + K, f24, f48, mk)
    pw, _ = _pack(p)
    torch.cuda.synchronize()
    assert np.array_equal(pw.blob.cpu().numpy(), oracle.pack("bf16", p.w, p.tile_map, p.mask))
    assert pw.desc.n_48 == int((p.tile_map == 2).sum()) and pw.desc.n_sparse == int((p.tile_map != 0).sum())


def test_pack_48_llama_q_proj_bit_exact():
    p = inputs.make_mixed("bf16", 4096, 4096, 3, 0.25, 0.5)
    pw, _ = _pack(p)
    torch.cuda.synchronize()
    assert np.array_equal(pw.blob.cpu().numpy(), oracle.pack("bf16", p.w, p.tile_map, p.mask))


def test_pack_48_rejects_bad_masks_and_map_bytes():
    p = inputs.make_mixed("bf16", 128, 256, 4, 0.0, 1.0)
    W = dev_bits(p.w, "bf16")
    for bad in (3, 5):
        m = p.mask.copy()
        m[7, 8:16] = 0
        m[7, 8:8 + bad] = 1
        with pytest.raises(patch.PatchError) as e:
            patch.pack(W, p.tile_map, dev_u8(m))
        assert e.value.name == "PATCH_ERR_MASK"
    with pytest.raises(patch.PatchError) as e:
        patch.pack(W, np.array([[3, 0]], np.uint8), dev_u8(p.mask))
    assert e.value.name == "PATCH_ERR_INVALID_ARG"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M", [1, 4, 16, 17, 64, 100, 128, 300])
def test_gemm_48_small(dtype, M):
    """384 x 640 with all three kinds: auto / decode / prefill, 16-bit and
    fp32 output."""
    p = inputs.make_mixed(dtype, 384, 640, 5, 0.3, 0.4, "uniform")
    pw, _ = _pack(p)
    Xb = inputs.make_custom_x(dtype, M, 640, 40 + M)
    X = dev_bits(Xb, dtype)
    ref = oracle.gemm_f64(dtype, Xb, p.w, p.tile_map, p.mask)
    for v in ["auto", "prefill"] + (["decode"] if M <= 128 else []):
        assert_close(patch.gemm(X, pw, variant=v), ref, what=f"{dtype} M={M} {v}")
        assert_close(patch.gemm(X, pw, out_dtype=torch.float32, variant=v), ref, f32=True,
                     what=f"{dtype} M={M} {v} f32")


@pytest.mark.parametrize("variant", LDS_KERNELS)
def test_gemm_48_every_lds_kernel(variant):
    """Every LDS-staged prefill kernel, with and without a K split, on
    640 x 1152 (a lone middle row-block)."""
    N, K = 640, 1152
    p = inputs.make_mixed("bf16", N, K, 6, 0.3, 0.4)
    pw, _ = _pack(p)
    ws = torch.empty(2 * N * K, dtype=torch.uint8, device="cuda")
    for M in (17, 300, 700):
        Xb = inputs.make_custom_x("bf16", M, K, 50 + M)
        ref = oracle.gemm_f64("bf16", Xb, p.w, p.tile_map, p.mask)
        for w in (ws, None):
            assert_close(patch.gemm(dev_bits(Xb, "bf16"), pw, variant=variant, workspace=w), ref,
                         what=f"{variant} M={M}")


@pytest.mark.parametrize("variant", ["decode", "prefill"] + LDS_KERNELS)
def test_gemm_48_exact_small_integers(variant):
    """f16 small integers, fp32 output: exact (every product and sum is an
    integer below 2^24), so each kept value meets its own X column."""
    rng = np.random.default_rng(7)
    N, K, M = 256, 768, 16 if variant == "decode" else 150
    p = inputs.make_mixed("f16", N, K, 8, 0.3, 0.5, "uniform")
    p.w = inputs.to_bits(rng.integers(-3, 4, (N, K)).astype(np.float64), "f16")
    Xb = inputs.to_bits(rng.integers(-3, 4, (M, K)).astype(np.float64), "f16")
    pw, _ = _pack(p)
    ws = torch.empty(2 * N * K, dtype=torch.uint8, device="cuda")
    y = patch.gemm(dev_bits(Xb, "f16"), pw, out_dtype=torch.float32, variant=variant, workspace=ws)
    assert np.array_equal(host_f64(y), oracle.gemm_f64("f16", Xb, p.w, p.tile_map, p.mask))


def test_gemm_48_identity_x():
    """X = identity rows: Y^T = W o E exactly, every kept position in every
    lane slot (decode with 1 and 8 blocks of 16 tokens, prefill)."""
    N, K = 256, 384
    p = inputs.make_mixed("bf16", N, K, 9, 0.0, 1.0, "uniform")
    pw, _ = _pack(p)
    E = oracle.effective_mask(N, K, p.tile_map, p.mask)
    WE = inputs.bits_to_f32(np.where(E != 0, p.w, 0).astype(np.uint16), "bf16").astype(np.float64)
    eye = inputs.to_bits(np.eye(K), "bf16")
    for v in ["prefill"] + LDS_KERNELS:
        y = patch.gemm(dev_bits(eye, "bf16"), pw, out_dtype=torch.float32, variant=v)
        assert np.array_equal(host_f64(y), WE.T), v
    for rows in (16, 128):
        for k0 in range(0, K, rows):
            y = patch.gemm(dev_bits(eye[k0:k0 + rows], "bf16"), pw, out_dtype=torch.float32, variant="decode")
            assert np.array_equal(host_f64(y), WE.T[k0:k0 + rows])


@pytest.mark.parametrize("M", [1, 16, 2048])
def test_gemm_48_llama_shapes(M):
    """LLaMA-2-7B gate_proj shape with 2:4 and 4:8 tiles: every output at
    M <= 16, sampled rows at M = 2048."""
    p = inputs.make_mixed("bf16", 11008, 4096, 10, 0.25, 0.5)
    pw, _ = _pack(p)
    Xb = inputs.make_custom_x("bf16", M, 4096, 11)
    y = patch.gemm(dev_bits(Xb, "bf16"), pw)
    if M <= 16:
        assert_close(y, oracle.gemm_f64("bf16", Xb, p.w, p.tile_map, p.mask), what=f"M={M}")
    else:
        rows = np.unique(np.linspace(0, M - 1, 20).astype(np.int64))
        ref = oracle.gemm_f64("bf16", Xb[rows], p.w, p.tile_map, p.mask)
        assert_close(y[torch.from_numpy(rows).cuda()], ref, what="M=2048 sampled")


def test_swiglu_48():
    """The fused gate/up projection on gate and up weights with 4:8 tiles."""
    F, K = 384, 640
    g = inputs.make_mixed("bf16", F, K, 12, 0.3, 0.4)
    u = inputs.make_mixed("bf16", F, K, 13, 0.2, 0.5)
    pw = patch.pack_gate_up(dev_bits(g.w, "bf16"), dev_bits(u.w, "bf16"), g.tile_map, u.tile_map, dev_u8(g.mask),
                            dev_u8(u.mask))
    for M in (1, 16, 300):
        Xb = inputs.make_custom_x("bf16", M, K, 70 + M)
        ref = oracle.swiglu_f64("bf16", Xb, g.w, u.w, g.tile_map, u.tile_map, g.mask, u.mask)
        for v in ("auto", "prefill") + (("decode",) if M <= 16 else ()):
            assert_close(patch.gemm_swiglu(dev_bits(Xb, "bf16"), pw, out_dtype=torch.float32, variant=v), ref,
                         f32=True, what=f"M={M} {v}")


def test_register_variants_reject_48_blobs():
    p = inputs.make_mixed("bf16", 256, 256, 14, 0.0, 1.0)
    pw, _ = _pack(p)
    X = dev_bits(inputs.make_custom_x("bf16", 64, 256, 1), "bf16")
    for v in ("prefill_w64", "prefill_w128", "prefill_w192", "prefill_w256"):
        with pytest.raises(patch.PatchError) as e:
            patch.gemm(X, pw, variant=v)
        assert e.value.name == "PATCH_ERR_UNSUPPORTED"
    q = inputs.make_mixed("bf16", 256, 256, 15, 1.0, 0.0)  # no 4:8 tiles: allowed
    pq, _ = _pack(q)
    assert_close(patch.gemm(X, pq, variant="prefill_w64"),
                 oracle.gemm_f64("bf16", inputs.make_custom_x("bf16", 64, 256, 1), q.w, q.tile_map, q.mask),
                 what="2:4 blob on the register kernel")
