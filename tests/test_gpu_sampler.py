"""GPU parity of the forward hybrid-mask sampler (patch_sample_mask) against
the CPU oracle, through the C ABI.

The sampler follows the gist.science explainer, section 2 "Methodology:
PATCH", "Learnable Distributions": Gumbel-Softmax tile selection (dense vs
2:4) and pattern selection (one of the six 2:4 patterns), and the soft mask
combining the dense and the 2:4 option.

Bars.  Hard outputs (tile map, mask) are integers decided by float32 scores
l + g, g = -ln(-ln u), on both sides; the two sides' logf may differ by an
ulp, so a decision is compared exactly where the oracle's binary64 scores
separate the winner from the runner-up by more than 1e-4 (the float32 score
error is below 4e-6 for |l| + |g| < 32), and elsewhere the GPU's choice must
be one of the classes within 1e-4 of the best (such near-ties must stay rare:
below 0.1% of the decisions).  Soft values: a float32 score error ds moves a
softmax probability by at most ds / (4 tau) per class, two classes at a time,
so |soft_gpu - soft_oracle| <= 1e-5 / tau + 1e-6.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from sparse_gemm_amd import inputs, patch
from tests.gpu_util import assert_close, dev_bits, dev_u8, host_f64

pytestmark = pytest.mark.gpu

MARGIN = 1e-4
PAIR_INDEX = {pair: p for p, pair in enumerate(oracle.PATTERN_PAIRS)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    patch.load()
    torch.cuda.set_device(0)


def _dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _scores(l: np.ndarray, u: np.ndarray) -> np.ndarray:
    return l.astype(np.float64) - np.log(-np.log(u.astype(np.float64)))


def check_decisions(got: np.ndarray, scores: np.ndarray, what: str):
    """got: chosen class per decision; scores: [..., C] binary64."""
    got = got.reshape(-1)
    sc = scores.reshape(got.size, -1)
    best = sc.max(axis=1)
    top2 = np.partition(sc, -2, axis=1)[:, -2]
    unique = best - top2 > MARGIN
    ref = sc.argmax(axis=1)
    bad = unique & (got != ref)
    assert not bad.any(), f"{what}: {int(bad.sum())} decisions differ, first at {int(np.argmax(bad))}"
    amb = ~unique
    if amb.any():
        chosen = sc[np.arange(got.size), got]
        assert np.all(best[amb] - chosen[amb] <= MARGIN), what
    assert amb.sum() <= max(2, got.size // 1000), f"{what}: {int(amb.sum())} near-ties"


def mask_patterns(mask: np.ndarray) -> np.ndarray:
    """Pattern index per group of a uint8 [N, K] mask; every group must keep
    exactly two positions."""
    N, K = mask.shape
    g = mask.reshape(N, K // 4, 4)
    assert np.all(g.sum(axis=2) == 2) and np.all(g <= 1), "every group keeps exactly two positions"
    first = g.argmax(axis=2)
    second = 3 - g[:, :, ::-1].argmax(axis=2)
    code = np.full((4, 4), -1)
    for (a, b), p in PAIR_INDEX.items():
        code[a, b] = p
    return code[first, second]


def run_and_check(N, K, seed, tau, soft=True, **kw):
    s = inputs.make_sampler_inputs(N, K, seed, **kw)
    tmap, mask, sf = patch.sample_mask(_dev(s.tile_logits), _dev(s.tile_u), _dev(s.pat_logits), _dev(s.pat_u), tau,
                                       soft=soft)
    torch.cuda.synchronize()
    tmap, mask = tmap.cpu().numpy(), mask.cpu().numpy()
    what = f"N={N} K={K} seed={seed} tau={tau}"
    check_decisions(tmap, _scores(s.tile_logits, s.tile_u), what + " tile map")
    check_decisions(mask_patterns(mask), _scores(s.pat_logits, s.pat_u), what + " patterns")
    r_map, r_mask, r_soft = oracle.sample_mask(s.tile_logits, s.tile_u, s.pat_logits, s.pat_u, tau, soft=soft)
    if soft:
        err = np.abs(host_f64(sf) - r_soft)
        assert err.max() <= 1e-5 / tau + 1e-6, f"{what}: soft max error {err.max():.3e}"
    else:
        assert sf is None
    return s, tmap, mask, r_map, r_mask


@pytest.mark.parametrize("N,K", [(128, 128), (256, 384), (384, 640)])
@pytest.mark.parametrize("tau", [0.25, 1.0, 4.0])
def test_sampler_small(N, K, tau):
    run_and_check(N, K, 1 + N + K, tau)


def test_sampler_without_soft_output():
    """soft = NULL: the same tile map and mask."""
    s = inputs.make_sampler_inputs(256, 512, 2)
    args = (_dev(s.tile_logits), _dev(s.tile_u), _dev(s.pat_logits), _dev(s.pat_u), 0.5)
    a = patch.sample_mask(*args, soft=True)
    b = patch.sample_mask(*args, soft=False)
    assert b[2] is None
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_sampler_deterministic():
    s = inputs.make_sampler_inputs(384, 640, 3)
    args = (_dev(s.tile_logits), _dev(s.tile_u), _dev(s.pat_logits), _dev(s.pat_u), 0.7)
    a, b = patch.sample_mask(*args), patch.sample_mask(*args)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("N,K", [(4096, 4096), (11008, 4096)])
def test_sampler_llama7b_shapes(N, K):
    """LLaMA-2-7B q_proj and gate_proj shapes, every output."""
    run_and_check(N, K, 4, 0.5, sparse_bias=0.4)


def test_sampler_extreme_inputs():
    """Uniforms at the ends of the drawn range (2^-24 and 1 - 2^-24, g from
    about -2.8 to 16.6) and logits of +-30: finite outputs, the same
    decisions."""
    N, K = 128, 256
    rng = np.random.default_rng(9)
    s = inputs.make_sampler_inputs(N, K, 5)
    ends = np.float32([2.0 ** -24, 1 - 2.0 ** -24])
    s.pat_u = ends[rng.integers(0, 2, s.pat_u.shape)]
    s.tile_u = ends[rng.integers(0, 2, s.tile_u.shape)]
    s.pat_logits = np.float32(30.0) * np.sign(s.pat_logits)
    tmap, mask, sf = patch.sample_mask(_dev(s.tile_logits), _dev(s.tile_u), _dev(s.pat_logits), _dev(s.pat_u), 1.0)
    torch.cuda.synchronize()
    assert torch.isfinite(sf).all()
    # ties are exact here (equal logits and equal uniforms): the first index wins on both sides
    r_map, r_mask, r_soft = oracle.sample_mask(s.tile_logits, s.tile_u, s.pat_logits, s.pat_u, 1.0)
    assert np.array_equal(mask.cpu().numpy(), r_mask)
    assert np.array_equal(tmap.cpu().numpy(), r_map)
    assert np.abs(host_f64(sf) - r_soft).max() <= 1e-5 + 1e-6


def test_sampled_mask_packs_and_multiplies():
    """The sampler's hard outputs feed the inference path: pack them (the map
    copied to the host) and multiply; the blob equals the oracle's pack of
    the same map and mask byte for byte, the GEMM matches the oracle, and
    the sparsity is 0.5 x the fraction of 2:4 tiles."""
    N, K, M = 384, 640, 33
    s, tmap, mask, _, _ = run_and_check(N, K, 6, 1.0, sparse_bias=0.5)
    p = inputs.make_custom("bf16", N, K, 6, "dense", 0.0, "top2")
    W = dev_bits(p.w, "bf16")
    pw = patch.pack(W, tmap, dev_u8(mask))
    torch.cuda.synchronize()
    assert np.array_equal(pw.blob.cpu().numpy(), oracle.pack("bf16", p.w, tmap, mask))
    E = oracle.effective_mask(N, K, tmap, mask)
    assert (E == 0).sum() * tmap.size * 2 == N * K * int(tmap.sum())
    Xb = inputs.make_custom_x("bf16", M, K, 60)
    assert_close(patch.gemm(dev_bits(Xb, "bf16"), pw), oracle.gemm_f64("bf16", Xb, p.w, tmap, mask), what="gemm")


def test_sampler_rejects_bad_arguments():
    lib = patch.load()
    s = inputs.make_sampler_inputs(128, 256, 7)
    tl, tu, pl, pu = _dev(s.tile_logits), _dev(s.tile_u), _dev(s.pat_logits), _dev(s.pat_u)
    for tau in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(patch.PatchError) as e:
            patch.sample_mask(tl, tu, pl, pu, tau)
        assert e.value.name == "PATCH_ERR_INVALID_ARG"
    tmap = torch.empty((1, 2), dtype=torch.uint8, device="cuda")
    mask = torch.empty((128, 256), dtype=torch.uint8, device="cuda")
    soft = torch.empty(128 * 256 + 4, dtype=torch.float32, device="cuda")
    P = ctypes.c_void_p

    def call(N=128, K=256, ptrs=None, soft_ptr=soft.data_ptr()):
        p = ptrs or [tl.data_ptr(), tu.data_ptr(), pl.data_ptr(), pu.data_ptr()]
        return lib.patch_sample_mask(N, K, P(p[0]), P(p[1]), P(p[2]), P(p[3]), ctypes.c_float(1.0),
                                     P(tmap.data_ptr()), P(mask.data_ptr()), P(soft_ptr), P(patch._stream()))

    assert call() == 0
    assert call(soft_ptr=0) == 0
    assert call(soft_ptr=soft.data_ptr() + 4) == 1       # soft not 16-byte aligned
    assert call(N=100) == 2 and call(K=0) == 2
    assert call(ptrs=[0, tu.data_ptr(), pl.data_ptr(), pu.data_ptr()]) == 1
    assert call(ptrs=[tl.data_ptr(), tu.data_ptr(), pl.data_ptr() + 4, pu.data_ptr()]) == 1
    torch.cuda.synchronize()
