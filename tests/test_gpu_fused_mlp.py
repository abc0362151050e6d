"""GPU parity of the fused projections against the CPU oracle, through the C
ABI: the gate/up projection H = SiLU(X Wg^T) * (X Wu^T) (the LLaMA MLP's
gated product; the pages evaluate PATCH on LLaMA-2 models, gist.science
explainer, section 4 "Experimental Results"), and several projections of
one input packed as one (attention's q, k, v).

Bars: the packed blob is bit-exact with the oracle's pack of the row-block
interleave of gate and up.  A 16-bit H is compared with the fp64 oracle
against its own rounding floor: H is a product of two sums, heavier-tailed
than a GEMM output, and on small outputs rounding the exact H to bf16 alone
can cost more than the plain GEMM's fixed 2e-3 (2.3e-3 relative Frobenius
for one token of a 384-wide H).  So a 16-bit H must be within that floor
(computed per case from the oracle) plus 5e-4 relative Frobenius -- room
for fp32 accumulation and the fp32 SiLU, about 1e-6 each, while a
truncating epilogue (twice the floor) fails -- and its max error within
max(1e-2, floor + 5e-3) of max|H_ref|.  An fp32 H is held to 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_gemm_amd import inputs, patch
from tests.gpu_util import assert_close, dev_bits, dev_u8, errors, host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    patch.load()
    torch.cuda.set_device(0)


def _pair(F, K, seed, map_kind="bernoulli", fraction=0.5, mask_kind="uniform", dtype="bf16"):
    g = inputs.make_custom(dtype, F, K, seed, map_kind, fraction, mask_kind, key=41)
    u = inputs.make_custom(dtype, F, K, seed, map_kind, fraction, mask_kind, key=42)
    return g, u


def _pack_pair(g, u):
    pw = patch.pack_gate_up(dev_bits(g.w, g.dtype), dev_bits(u.w, u.dtype), g.tile_map, u.tile_map, dev_u8(g.mask),
                            dev_u8(u.mask))
    return pw


def check_h(y: torch.Tensor, ref: np.ndarray, dtype: str, what: str = ""):
    """A 16-bit H against the fp64 oracle, with the bar set by the rounding
    floor of the exact H (see the module docstring)."""
    yh = host_f64(y)
    assert yh.shape == ref.shape and np.all(np.isfinite(yh)), what
    floor_rel, floor_max = errors(inputs.bits_to_f32(oracle.round_f64(dtype, ref), dtype).astype(np.float64), ref)
    rel, mx = errors(yh, ref)
    assert rel <= floor_rel + 5e-4 and mx <= max(1e-2, floor_max + 5e-3), (
        f"{what}: rel-Frobenius {rel:.3e} (floor {floor_rel:.3e}), max {mx:.3e} (floor {floor_max:.3e})")


def _ref(g, u, Xb, rows=None):
    Xs = Xb if rows is None else Xb[rows]
    return oracle.swiglu_f64(g.dtype, Xs, g.w, u.w, g.tile_map, u.tile_map, g.mask, u.mask)


def _oracle_blob(g, u):
    W = oracle.interleave_gate_up(g.w, u.w, 128)
    tm = oracle.interleave_gate_up(g.tile_map, u.tile_map, 1)
    mk = oracle.interleave_gate_up(g.mask, u.mask, 128)
    return oracle.pack(g.dtype, W, tm, mk)


@pytest.mark.parametrize("F,K,seed", [(128, 128, 1), (384, 640, 2), (256, 384, 3)])
def test_pack_gate_up_bit_exact(F, K, seed):
    g, u = _pair(F, K, seed)
    pw = _pack_pair(g, u)
    torch.cuda.synchronize()
    got = pw.blob.cpu().numpy()
    ref = _oracle_blob(g, u)
    assert got.size == ref.size and np.array_equal(got, ref)
    assert pw.N == 2 * F and pw.n_sparse == int(g.tile_map.sum() + u.tile_map.sum())


def test_pack_gate_up_llama7b_bit_exact():
    cfg = inputs.CONFIGS["sweep"]
    g, u = inputs.make_weights(cfg, 4, 2), inputs.make_weights(cfg, 5, 2)  # gate_proj, up_proj at s = 0.5
    pw = _pack_pair(g, u)
    torch.cuda.synchronize()
    assert np.array_equal(pw.blob.cpu().numpy(), _oracle_blob(g, u))


def test_pack_gate_up_rejects_illegal_mask():
    g, u = _pair(256, 256, 4, "sparse", 1.0, "top2")
    mask = u.mask.copy()
    mask[100, 8:12] = [1, 1, 1, 0]
    with pytest.raises(patch.PatchError) as e:
        patch.pack_gate_up(dev_bits(g.w, "bf16"), dev_bits(u.w, "bf16"), g.tile_map, u.tile_map, dev_u8(g.mask),
                           dev_u8(mask))
    assert e.value.name == "PATCH_ERR_MASK"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M", [1, 4, 16, 17, 64, 100, 128, 129, 300])
def test_swiglu_small_ragged(dtype, M):
    """384 x 640 gate and up (3 gate/up row-block pairs, 5 tile columns),
    every M edge, auto / decode / prefill, 16-bit and fp32 H; the dense
    baseline on the same weights with all tiles dense."""
    F, K = 384, 640
    g, u = _pair(F, K, 5, dtype=dtype)
    pw = _pack_pair(g, u)
    Xb = inputs.make_custom_x(dtype, M, K, 50 + M)
    X = dev_bits(Xb, dtype)
    ref = _ref(g, u, Xb)
    for v in ["auto", "prefill"] + (["decode"] if M <= 128 else []):
        check_h(patch.gemm_swiglu(X, pw, variant=v), ref, dtype, what=f"{dtype} M={M} {v}")
        assert_close(patch.gemm_swiglu(X, pw, out_dtype=torch.float32, variant=v), ref, f32=True,
                     what=f"{dtype} M={M} {v} f32")
    gd, ud = _pair(F, K, 5, "dense", 0.0, "top2", dtype=dtype)
    ref_d = _ref(gd, ud, Xb)
    Wg, Wu = dev_bits(gd.w, dtype), dev_bits(ud.w, dtype)
    for v in ["auto", "prefill"] + (["decode"] if M <= 128 else []):
        check_h(patch.dense_gemm_swiglu(X, Wg, Wu, variant=v), ref_d, dtype, what=f"dense {dtype} M={M} {v}")


PREFILL_KERNELS = ["prefill_w64", "prefill_w128", "prefill_w192", "prefill_w256", "prefill_w128_lds", "prefill_w192_lds",
                   "prefill_w256_lds", "prefill_w64_lds", "prefill_big_w128", "prefill_big_w192", "prefill_big_w256", "prefill_big8_w128", "prefill_big8_w256"]


@pytest.mark.parametrize("variant", PREFILL_KERNELS)
def test_swiglu_every_prefill_kernel(variant):
    """Every prefill kernel with the fused epilogue (unsplit: gate and up sums
    meet in LDS) and with a K split (the ordered reduction applies SiLU), on
    640 x 1152 gate and up (5 pairs, 9 tile columns), packed and dense."""
    F, K = 640, 1152
    g, u = _pair(F, K, 6)
    pw = _pack_pair(g, u)
    gd, ud = _pair(F, K, 6, "dense", 0.0, "top2")
    Wg, Wu = dev_bits(gd.w, "bf16"), dev_bits(ud.w, "bf16")
    ws = torch.empty(4 * F * K, dtype=torch.uint8, device="cuda")
    for M in (17, 300, 700):
        Xb = inputs.make_custom_x("bf16", M, K, 60 + M)
        X = dev_bits(Xb, "bf16")
        ref, ref_d = _ref(g, u, Xb), _ref(gd, ud, Xb)
        for w in (ws, None):
            tag = f"{variant} M={M} ws={'yes' if w is not None else 'no'}"
            check_h(patch.gemm_swiglu(X, pw, variant=variant, workspace=w), ref, "bf16", what=tag)
            assert_close(patch.gemm_swiglu(X, pw, out_dtype=torch.float32, variant=variant, workspace=w), ref,
                         f32=True, what=tag + " f32")
            check_h(patch.dense_gemm_swiglu(X, Wg, Wu, variant=variant, workspace=w), ref_d, "bf16", what="dense " + tag)


def test_swiglu_identity_x():
    """X = identity rows: H^T = SiLU(Wg o Eg) * (Wu o Eu); with fp32 output
    each element is one fp32 SiLU of an exact product, so it matches the
    oracle to fp32 rounding of the SiLU (rtol 1e-6)."""
    F, K = 256, 384
    g, u = _pair(F, K, 7)
    pw = _pack_pair(g, u)
    eye = inputs.to_bits(np.eye(K), "bf16")
    ref = _ref(g, u, eye)
    y = patch.gemm_swiglu(dev_bits(eye, "bf16"), pw, out_dtype=torch.float32, variant="prefill")
    np.testing.assert_allclose(host_f64(y), ref, rtol=1e-6, atol=1e-30)
    for rows in (16, 128):
        for k0 in range(0, K, rows):
            y = patch.gemm_swiglu(dev_bits(eye[k0:k0 + rows], "bf16"), pw, out_dtype=torch.float32, variant="decode")
            np.testing.assert_allclose(host_f64(y), ref[k0:k0 + rows], rtol=1e-6, atol=1e-30)


def test_swiglu_long_k_decode_limits():
    """The fused decode kernel takes M <= 16 at any K up to 65536, and more
    tokens only up to K = 32768 (AUTO then runs the prefill kernel)."""
    F, K = 128, 65536
    g, u = _pair(F, K, 8)
    pw = _pack_pair(g, u)
    for M in (1, 16, 17):
        Xb = inputs.make_custom_x("bf16", M, K, 70 + M)
        ref = _ref(g, u, Xb)
        X = dev_bits(Xb, "bf16")
        check_h(patch.gemm_swiglu(X, pw), ref, "bf16", what=f"auto M={M}")
        if M <= 16:
            check_h(patch.gemm_swiglu(X, pw, variant="decode"), ref, "bf16", what=f"decode M={M}")
        else:
            with pytest.raises(patch.PatchError) as e:
                patch.gemm_swiglu(X, pw, variant="decode")
            assert e.value.name == "PATCH_ERR_UNSUPPORTED"


@pytest.mark.parametrize("M", [1, 16, 2048])
def test_swiglu_llama7b_mlp(M):
    """LLaMA-2-7B gate_proj and up_proj (11008 x 4096 each, s = 0.5): every
    output at M = 1 and 16, sampled rows at M = 2048; deterministic."""
    cfg = inputs.CONFIGS["sweep"]
    g, u = inputs.make_weights(cfg, 4, 2), inputs.make_weights(cfg, 5, 2)
    pw = _pack_pair(g, u)
    Xb = inputs.make_x(cfg, M, g.K, matrix_index=4)
    X = dev_bits(Xb, "bf16")
    h = patch.gemm_swiglu(X, pw)
    h2 = patch.gemm_swiglu(X, pw)
    assert torch.equal(h, h2)
    if M <= 16:
        check_h(h, _ref(g, u, Xb), "bf16", what=f"M={M}")
    else:
        rows = np.unique(np.linspace(0, M - 1, 24).astype(np.int64))
        check_h(h[torch.from_numpy(rows).cuda()], _ref(g, u, Xb, rows), "bf16", what=f"M={M} sampled")


# ------------------------------------------------------------------ several projections in one blob
def _concat_oracle_blob(ps):
    W = np.concatenate([p.w for p in ps])
    tm = np.concatenate([p.tile_map for p in ps])
    mk = np.concatenate([p.mask for p in ps])
    return oracle.pack(ps[0].dtype, W, tm, mk)


def _pack_concat(ps):
    return patch.pack_concat([dev_bits(p.w, p.dtype) for p in ps], [p.tile_map for p in ps],
                             [dev_u8(p.mask) for p in ps])


def test_pack_concat_bit_exact():
    ps = [inputs.make_custom("bf16", n, 640, 80 + n, "bernoulli", 0.5, "uniform") for n in (128, 384, 256)]
    pw = _pack_concat(ps)
    torch.cuda.synchronize()
    assert pw.N == 768 and np.array_equal(pw.blob.cpu().numpy(), _concat_oracle_blob(ps))


def test_pack_concat_llama7b_qkv_bit_exact():
    cfg = inputs.CONFIGS["sweep"]
    ps = [inputs.make_weights(cfg, mi, 2) for mi in (0, 1, 2)]  # q_proj, k_proj, v_proj at s = 0.5
    pw = _pack_concat(ps)
    torch.cuda.synchronize()
    assert np.array_equal(pw.blob.cpu().numpy(), _concat_oracle_blob(ps))


@pytest.mark.parametrize("M", [1, 16, 64, 300])
def test_concat_gemm_is_the_projections_side_by_side(M):
    ps = [inputs.make_custom("bf16", n, 640, 90 + n, "bernoulli", 0.5, "uniform") for n in (256, 128, 384)]
    pw = _pack_concat(ps)
    Xb = inputs.make_custom_x("bf16", M, 640, 95 + M)
    ref = np.concatenate([oracle.gemm_f64("bf16", Xb, p.w, p.tile_map, p.mask) for p in ps], axis=1)
    X = dev_bits(Xb, "bf16")
    for v in ["auto", "prefill"] + (["decode"] if M <= 128 else []):
        assert_close(patch.gemm(X, pw, variant=v), ref, what=f"M={M} {v}")


def test_pack_concat_rejects_bad_arguments():
    p = inputs.make_custom("bf16", 128, 256, 99, "bernoulli", 0.5, "uniform")
    W, mk = dev_bits(p.w, "bf16"), dev_u8(p.mask)
    with pytest.raises(ValueError):
        patch.pack_concat([W], [p.tile_map, p.tile_map], [mk])
    with pytest.raises(patch.PatchError):
        patch.pack_concat([W] * 9, [p.tile_map] * 9, [mk] * 9)
