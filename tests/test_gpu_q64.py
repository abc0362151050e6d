"""GPU parity of 64 x 64 execution tiles (packed format 4), through the C ABI.

The explainer (gist.science, section 4 "Ablation Studies", "Tile Size")
finds PATCH robust across tile sizes, smaller tiles giving finer control,
while execution wants larger tiles.  Format 4 lets every 64 x 64 quadrant of
a 128 x 128 tile be dense or 2:4 on its own; the decode kernel and the
LDS-staged prefill kernel run it.

Bars: the GPU-packed blob is bit-exact with oracle.pack_q64; the GEMM meets
the hybrid GEMM's tolerance (tests/gpu_util.py) against the fp64 oracle's
product with the 64 x 64 tile map; small-integer inputs with a float32
output match exactly; a quadrant map constant on every 128 x 128 tile gives
the same output bits as the 128 x 128 format (the same matrix instructions
in the same order).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from sparse_gemm_amd import inputs, patch
from tests.gpu_util import assert_close, dev_bits, dev_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    patch.load()
    torch.cuda.set_device(0)


def _problem(dtype, N, K, seed, s_exec=0.3, p_sub=0.5):
    """Weights with a 64 x 64 quadrant map (tile_map, N/64 x K/64): with
    probability s_exec a 128 x 128 tile is 2:4 in all four quadrants, else
    each quadrant is 2:4 with probability p_sub; a uniformly drawn 2:4
    pattern in every group."""
    return inputs.make_fine(dtype, N, K, 64, 64, seed, s_exec=s_exec, p_sub=p_sub)


def _pack(p):
    W = dev_bits(p.w, p.dtype)
    return patch.pack_q64(W, p.tile_map, dev_u8(p.mask)), W


def _ref(p, X):
    return oracle.gemm_f64(p.dtype, X, p.w, p.tile_map, p.mask, tile_n=64, tile_k=64)


PACK_CASES = [
    ("mixed_bf16_256x384", "bf16", 256, 384, 1, 0.3, 0.5),
    ("mixed_f16_384x640", "f16", 384, 640, 2, 0.2, 0.5),
    ("single_tile_f16", "f16", 128, 128, 3, 0.0, 0.5),
    ("all_dense", "bf16", 256, 256, 4, 0.0, 0.0),
    ("all_sparse", "bf16", 256, 256, 5, 1.0, 1.0),
    ("q_proj_4096", "bf16", 4096, 4096, 6, 0.25, 0.5),
]


@pytest.mark.parametrize("name,dtype,N,K,seed,s_exec,p_sub", PACK_CASES, ids=[c[0] for c in PACK_CASES])
def test_pack_q64_bit_exact(name, dtype, N, K, seed, s_exec, p_sub):
    p = _problem(dtype, N, K, seed, s_exec, p_sub)
    pw, _ = _pack(p)
    torch.cuda.synchronize()
    got = pw.blob.cpu().numpy()
    ref = oracle.pack_q64(dtype, p.w, p.tile_map, p.mask)
    assert got.size == ref.size == pw.nbytes
    diff = np.flatnonzero(got != ref)
    assert diff.size == 0, f"{name}: {diff.size} bytes differ, first at {diff[:8]}"
    assert pw.desc.version == 4 and pw.n_sparse == int(p.tile_map.sum())


def test_pack_q64_rejects_illegal_mask_on_gpu():
    p = _problem("bf16", 256, 256, 7, 1.0, 1.0)
    mask = p.mask.copy()
    mask[130, 64:68] = [1, 1, 1, 0]  # quadrant (2, 1): 2:4
    with pytest.raises(patch.PatchError) as e:
        patch.pack_q64(dev_bits(p.w, "bf16"), p.tile_map, dev_u8(mask))
    assert e.value.name == "PATCH_ERR_MASK"
    qm = p.tile_map.copy()
    qm[2, 1] = 0  # the same group inside a dense quadrant is ignored
    pw = patch.pack_q64(dev_bits(p.w, "bf16"), qm, dev_u8(mask))
    torch.cuda.synchronize()
    assert np.array_equal(pw.blob.cpu().numpy(), oracle.pack_q64("bf16", p.w, qm, mask))


GEMM_M = [1, 3, 16, 17, 64, 100, 128, 129, 300]
VARIANTS = ["auto", "prefill", "prefill_w64_lds", "prefill_w128_lds", "prefill_w192_lds", "prefill_w256_lds"]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M", GEMM_M)
def test_gemm_q64(dtype, M):
    """384 x 640 (6 x 10 quadrants, every kind pair), every M edge, the
    decode and every LDS-staged variant, both output types."""
    p = _problem(dtype, 384, 640, 11 + M)
    cells = p.tile_map.reshape(6, 5, 2)
    kinds = set((cells[..., 0] + 2 * cells[..., 1]).ravel().tolist())
    assert kinds == {0, 1, 2, 3}  # both-dense, either mixed order, both-2:4 cells
    pw, _ = _pack(p)
    Xb = inputs.make_custom_x(dtype, M, 640, M)
    X = dev_bits(Xb, dtype)
    ref = _ref(p, Xb)
    for v in VARIANTS + (["decode"] if M <= 128 else []):
        y = patch.gemm(X, pw, variant=v)
        assert_close(y, ref, what=f"{dtype} M={M} {v} kinds={sorted(kinds)}")
        y32 = patch.gemm(X, pw, out_dtype=torch.float32, variant=v)
        assert_close(y32, ref, f32=True, what=f"{dtype} M={M} {v} f32")


@pytest.mark.parametrize("M", [1, 16, 100, 300])
def test_gemm_q64_small_integers_exact(M):
    """Small integers (exact in bf16, products and sums exact in fp32): the
    float32 output equals the oracle exactly, for all four kind pairs of a
    cell."""
    N, K = 256, 512
    rng = np.random.default_rng(21 + M)
    qm = np.array([[0, 1, 1, 0, 1, 1, 0, 0], [1, 0, 0, 1, 1, 1, 0, 0],
                   [1, 1, 0, 0, 0, 1, 1, 0], [0, 0, 1, 1, 1, 0, 0, 1]], np.uint8)
    p = _problem("bf16", N, K, 12)
    wv = rng.integers(-3, 4, (N, K)).astype(np.float32)
    xv = rng.integers(-3, 4, (M, K)).astype(np.float32)
    w = (wv.view(np.uint32) >> 16).astype(np.uint16)
    x = (xv.view(np.uint32) >> 16).astype(np.uint16)
    pw = patch.pack_q64(dev_bits(w, "bf16"), qm, dev_u8(p.mask))
    ref = oracle.gemm_f64("bf16", x, w, qm, p.mask, tile_n=64, tile_k=64)
    X = dev_bits(x, "bf16")
    for v in ["auto", "prefill"] + (["decode"] if M <= 128 else []):
        y = patch.gemm(X, pw, out_dtype=torch.float32, variant=v).cpu().numpy().astype(np.float64)
        assert np.array_equal(y, ref), f"M={M} {v}"


@pytest.mark.parametrize("M", [1, 16, 100, 300])
def test_q64_tile_constant_map_matches_128_format(M):
    """A quadrant map constant on every 128 x 128 tile: the same output bits
    as the 128 x 128 blob of the same weights."""
    N, K = 384, 640
    p = inputs.make_custom("bf16", N, K, 13, "bernoulli", 0.5, "uniform")
    qm = np.kron(p.tile_map, np.ones((2, 2), np.uint8))
    W, mk = dev_bits(p.w, "bf16"), dev_u8(p.mask)
    p3, p4 = patch.pack(W, p.tile_map, mk), patch.pack_q64(W, qm, mk)
    X = dev_bits(inputs.make_custom_x("bf16", M, K, 5), "bf16")
    for v in ["auto", "prefill"] + (["decode"] if M <= 128 else []):
        y3 = patch.gemm(X, p3, out_dtype=torch.float32, variant=v)
        y4 = patch.gemm(X, p4, out_dtype=torch.float32, variant=v)
        assert torch.equal(y3, y4), f"M={M} {v}"


def test_gemm_q64_split_and_no_workspace():
    """K split into ranges (workspace) and no split (no workspace): both
    within tolerance of the oracle."""
    p = _problem("bf16", 256, 4096, 14)
    pw, _ = _pack(p)
    Xb = inputs.make_custom_x("bf16", 64, 4096, 3)
    X = dev_bits(Xb, "bf16")
    ref = _ref(p, Xb)
    assert_close(patch.gemm(X, pw, variant="prefill"), ref, what="split")
    assert_close(patch.gemm(X, pw, variant="prefill", workspace=None), ref, what="no workspace")


def test_gemm_q64_noalloc_matches():
    p = _problem("bf16", 256, 512, 15)
    pw, _ = _pack(p)
    X = dev_bits(inputs.make_custom_x("bf16", 200, 512, 4), "bf16")
    y = patch.gemm(X, pw, out_dtype=torch.float32, variant="auto")
    out = torch.empty_like(y)
    patch.gemm_noalloc(X, pw, out)
    assert torch.equal(y, out)


@pytest.mark.parametrize("M,sample", [(1, None), (16, None), (2048, 48)])
def test_gemm_q64_llama_gate_proj(M, sample):
    """LLaMA-2-7B gate_proj shape (11008 x 4096) with a 64 x 64 quadrant map
    (about half of the quadrants 2:4): decode at M = 1 and 16, prefill at
    M = 2048 checked on 48 sampled rows of X."""
    N, K = 11008, 4096
    p = _problem("bf16", N, K, 16, 0.3, 0.5)
    pw, _ = _pack(p)
    Xb = inputs.make_custom_x("bf16", M, K, 6)
    y = patch.gemm(dev_bits(Xb, "bf16"), pw)
    rows = np.arange(M) if sample is None else np.random.default_rng(7).choice(M, sample, replace=False)
    ref = _ref(p, Xb[rows])
    assert_close(y[torch.from_numpy(rows).cuda()], ref, what=f"gate_proj M={M}")


def test_q64_unsupported_paths():
    """The register-staged and big-tile prefill variants and the fused
    gate/up product reject a blob of 64 x 64 execution tiles."""
    p = _problem("bf16", 256, 256, 17)
    pw, _ = _pack(p)
    X = dev_bits(inputs.make_custom_x("bf16", 256, 256, 2), "bf16")
    for v in ["prefill_w64", "prefill_w256", "prefill_big", "prefill_big8_w256"]:
        with pytest.raises(patch.PatchError) as e:
            patch.gemm(X, pw, variant=v)
        assert e.value.name == "PATCH_ERR_UNSUPPORTED", v
    lib = patch.load()
    H = torch.empty((256, 128), dtype=torch.bfloat16, device="cuda")
    rc = lib.patch_gemm_swiglu(ctypes.byref(pw.desc), pw.blob.data_ptr(), X.data_ptr(), 256, H.data_ptr(),
                               1, None, 0, 0, None)
    assert rc == 5  # PATCH_ERR_UNSUPPORTED


def test_q64_deterministic_and_graph_replays_match_eager():
    """64 x 64 tiles through decode, the split-K prefill and the unsplit
    prefill: two eager runs are bitwise equal, and the same calls captured in
    a HIP graph and replayed three times (eager work and synchronisations in
    between) equal the eager results bit for bit."""
    p = _problem("bf16", 512, 4096, 18)
    pw, _ = _pack(p)
    X4 = dev_bits(inputs.make_custom_x("bf16", 4, 4096, 21), "bf16")
    X128 = dev_bits(inputs.make_custom_x("bf16", 128, 4096, 22), "bf16")
    X600 = dev_bits(inputs.make_custom_x("bf16", 600, 4096, 23), "bf16")
    outs = [torch.empty((4, 512), dtype=torch.bfloat16, device="cuda"),
            torch.empty((128, 512), dtype=torch.float32, device="cuda"),
            torch.empty((600, 512), dtype=torch.bfloat16, device="cuda")]

    def run():
        patch.gemm(X4, pw, out=outs[0])
        patch.gemm(X128, pw, out_dtype=torch.float32, variant="prefill", out=outs[1])
        patch.gemm(X600, pw, variant="prefill_w192_lds", out=outs[2], workspace=None)

    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    run()
    torch.cuda.synchronize()
    for a, b in zip(outs, eager):
        assert torch.equal(a, b), "repeat"
    assert int(patch.load().patch_gemm_workspace_bytes(ctypes.byref(pw.desc), 128)) > 0  # the split path
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for o in outs:
            o.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), f"replay {rep}"
        other = patch.gemm(X128, pw)  # eager work between replays
        torch.cuda.synchronize()
        assert other.shape == (128, 512)
