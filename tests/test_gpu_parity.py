"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Pages: PATCH (arXiv 2509.23410), gist.science explainer, section 2 "Core
Mechanism" (dense or 2:4 tiles), "Inference & Deployment" (dense tiles on dense
kernels, 2:4 tiles on the sparse path), section 4 "Ablation Studies" (128 x
128 execution tiles).

Bars: the packed blob is bit-exact with the oracle's; a GEMM with a 16-bit
output is within relative Frobenius 2e-3 and max error 1e-2 * max|Y_ref| of
the fp64 oracle (tests/gpu_util.py); cases whose exact result is
representable (identity X, small integers with a float32 output) must match
exactly.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from sparse_gemm_amd import inputs, patch
from tests.gpu_util import assert_close, dev_bits, dev_u8, host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    patch.load()
    torch.cuda.set_device(0)


def _pack(p):
    W = dev_bits(p.w, p.dtype)
    return patch.pack(W, p.tile_map, dev_u8(p.mask)), W


def _ref(p, X, rows=None):
    Xs = X if rows is None else X[rows]
    return oracle.gemm_f64(p.dtype, Xs, p.w, p.tile_map, p.mask)


# ------------------------------------------------------------------ pack
PACK_CASES = [
    ("tiny_seed0", lambda: inputs.make_weights(inputs.CONFIGS["tiny"], 0, 0, seed=0)),
    ("tiny_seed1", lambda: inputs.make_weights(inputs.CONFIGS["tiny"], 0, 0, seed=1)),
    ("tiny_all_dense", lambda: inputs.make_weights(inputs.CONFIGS["tiny"], 0, 0, map_kind="dense")),
    ("tiny_all_sparse", lambda: inputs.make_weights(inputs.CONFIGS["tiny"], 0, 0, map_kind="sparse")),
    ("single_tile_sparse_bf16", lambda: inputs.make_custom("bf16", 128, 128, 3, "sparse", 1.0, "uniform")),
    ("single_tile_dense_f16", lambda: inputs.make_custom("f16", 128, 128, 3, "dense", 0.0, "top2")),
    ("ragged_384x640", lambda: inputs.make_custom("bf16", 384, 640, 4, "bernoulli", 0.5, "uniform")),
    ("decode_q_proj", lambda: inputs.make_weights(inputs.CONFIGS["decode"], 0, 0)),
]


@pytest.mark.parametrize("name,make", PACK_CASES, ids=[c[0] for c in PACK_CASES])
def test_pack_bit_exact(name, make):
    p = make()
    pw, _ = _pack(p)
    torch.cuda.synchronize()
    got = pw.blob.cpu().numpy()
    ref = oracle.pack(p.dtype, p.w, p.tile_map, p.mask)
    assert got.size == ref.size
    diff = np.flatnonzero(got != ref)
    assert diff.size == 0, f"{name}: {diff.size} bytes differ, first at {diff[:8]}"
    assert pw.n_sparse == int(p.tile_map.sum())


@pytest.mark.parametrize("mi", [0, 1])
def test_pack_bit_exact_prefill_mlp_and_13b(mi):
    for cfg in ("prefill_mlp", "imbalanced_13b"):
        p = inputs.make_weights(inputs.CONFIGS[cfg], mi, 0)
        pw, _ = _pack(p)
        torch.cuda.synchronize()
        got = pw.blob.cpu().numpy()
        ref = oracle.pack(p.dtype, p.w, p.tile_map, p.mask)
        assert np.array_equal(got, ref), cfg


def test_pack_rejects_illegal_mask_on_gpu():
    p = inputs.make_custom("bf16", 256, 256, 5, "sparse", 1.0, "top2")
    mask = p.mask.copy()
    mask[200, 4 * 40:4 * 40 + 4] = [1, 1, 1, 0]
    with pytest.raises(patch.PatchError) as e:
        patch.pack(dev_bits(p.w, "bf16"), p.tile_map, dev_u8(mask))
    assert e.value.name == "PATCH_ERR_MASK"
    # the same bad group inside a dense tile is ignored
    tm = p.tile_map.copy()
    tm[1, 1] = 0
    pw = patch.pack(dev_bits(p.w, "bf16"), tm, dev_u8(mask))
    torch.cuda.synchronize()
    assert np.array_equal(pw.blob.cpu().numpy(), oracle.pack("bf16", p.w, tm, mask))


# ------------------------------------------------------------------ GEMM, small shapes
SMALL_M = [1, 2, 3, 4, 7, 15, 16, 17, 31, 33, 48, 64, 65, 100, 128, 129, 255, 256, 257, 300]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M", SMALL_M)
def test_gemm_small_ragged(dtype, M):
    """384 x 640 (3 x 5 tiles, random map), every M edge, every variant, both
    output types."""
    p = inputs.make_custom(dtype, 384, 640, 7, "bernoulli", 0.5, "top2")
    assert 0 < p.tile_map.sum() < p.tile_map.size
    pw, _ = _pack(p)
    Xb = inputs.make_custom_x(dtype, M, 640, M)
    X = dev_bits(Xb, dtype)
    ref = _ref(p, Xb)
    variants = ["auto", "prefill"] + (["decode"] if M <= 128 else [])
    for v in variants:
        y = patch.gemm(X, pw, variant=v)
        assert_close(y, ref, what=f"{dtype} M={M} {v}")
        y32 = patch.gemm(X, pw, out_dtype=torch.float32, variant=v)
        assert_close(y32, ref, f32=True, what=f"{dtype} M={M} {v} f32")


def test_empty_m():
    """M = 0: every variant returns an empty product and launches nothing
    (the boundary accepts it before looking at the pointers)."""
    p = inputs.make_custom("bf16", 384, 640, 7, "bernoulli", 0.5, "top2")
    pw, W = _pack(p)
    X = torch.empty((0, 640), dtype=torch.bfloat16, device="cuda")
    for v in ("auto", "decode", "prefill", "prefill_w64_lds", "prefill_w256"):
        for od in (None, torch.float32):
            y = patch.gemm(X, pw, out_dtype=od, variant=v)
            assert tuple(y.shape) == (0, 384), v
    assert tuple(patch.dense_gemm(X, W).shape) == (0, 384)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M", [1, 16, 17, 300])
def test_dense_baseline_small(dtype, M):
    p = inputs.make_custom(dtype, 384, 640, 8, "dense", 0.0, "top2")
    W = dev_bits(p.w, dtype)
    Xb = inputs.make_custom_x(dtype, M, 640, M + 1)
    X = dev_bits(Xb, dtype)
    ref = _ref(p, Xb)
    for v in ["auto", "prefill"] + (["decode"] if M <= 128 else []):
        assert_close(patch.dense_gemm(X, W, variant=v), ref, what=f"dense {dtype} M={M} {v}")
        assert_close(patch.dense_gemm(X, W, out_dtype=torch.float32, variant=v), ref, f32=True,
                     what=f"dense {dtype} M={M} {v} f32")


@pytest.mark.parametrize("M", [5, 16, 64, 300])
def test_all_dense_map_matches_dense_baseline(M):
    """An all-dense tile map computes the same products as the dense baseline
    (packed dense tiles run as two fixed-pattern halves on the sparse
    instruction, the baseline on the dense one), so with fp32 output the two
    agree to fp32 accumulation-order rounding, and both match the oracle."""
    p = inputs.make_custom("bf16", 256, 512, 9, "dense", 0.0, "top2")
    pw, W = _pack(p)
    Xb = inputs.make_custom_x("bf16", M, 512, 3)
    X = dev_bits(Xb, "bf16")
    ref = _ref(p, Xb)
    for v in ["prefill"] + (["decode"] if M <= 128 else []):
        a = patch.gemm(X, pw, out_dtype=torch.float32, variant=v)
        b = patch.dense_gemm(X, W, out_dtype=torch.float32, variant=v)
        assert_close(a, ref, f32=True, what=f"hybrid all-dense M={M} {v}")
        assert_close(b, ref, f32=True, what=f"dense M={M} {v}")
        scale = float(b.abs().max())
        assert float((a - b).abs().max()) <= 1e-5 * scale, v


@pytest.mark.parametrize("K", [16384, 16512, 32768, 32896, 65536])
def test_decode_long_k(K):
    """The decode kernel splits a band's tile columns over 2, 4 or 8 waves by
    K (each wave may own at most 64 of them): both sides of every switch,
    the largest K, and M on both sides of each column-block count."""
    p = inputs.make_custom("bf16", 256, K, 14, "bernoulli", 0.5, "uniform")
    pw, W = _pack(p)
    Xb = inputs.make_custom_x("bf16", 128, K, 15)
    ref = _ref(p, Xb)
    pd = inputs.make_custom("bf16", 256, K, 14, "dense", 0.0, "top2")
    ref_d = _ref(pd, Xb)
    for M in (1, 16, 17, 33, 64, 65, 128):
        X = dev_bits(Xb[:M], "bf16")
        assert_close(patch.gemm(X, pw, variant="decode"), ref[:M], what=f"K={K} M={M}")
        assert_close(patch.dense_gemm(X, W, variant="decode"), ref_d[:M], what=f"dense K={K} M={M}")


@pytest.mark.parametrize("M", [520, 1061, 1500])
def test_prefill_m_groups(M):
    """Prefill orders its output blocks by groups of M-blocks (two groups at
    these M, the last one short when the M-blocks are odd) over an odd
    number of row-blocks (a lone middle row-block): every output against the
    oracle."""
    p = inputs.make_custom("bf16", 640, 384, 16, "bernoulli", 0.5, "uniform")
    pw, _ = _pack(p)
    Xb = inputs.make_custom_x("bf16", M, 384, 17)
    ref = _ref(p, Xb)
    X = dev_bits(Xb, "bf16")
    assert_close(patch.gemm(X, pw, variant="prefill"), ref, what=f"M={M}")
    assert_close(patch.gemm(X, pw, out_dtype=torch.float32, variant="prefill"), ref, f32=True, what=f"M={M} f32")


@pytest.mark.parametrize("N,K", [(512, 4096), (256, 2688), (384, 4096)])
@pytest.mark.parametrize("M", [17, 64, 128, 200, 300])
def test_prefill_split_k(N, K, M):
    """Few output blocks: prefill splits K into ranges (the last one short
    where the tile count does not divide) and adds the fp32 partials in range
    order in a second kernel.  Every output against the oracle with the
    workspace the library asks for, with a workspace of two planes (fewer
    ranges) and with none (no split); the dense baseline takes the same
    path."""
    lib = patch.load()
    p = inputs.make_custom("bf16", N, K, 18, "bernoulli", 0.5, "uniform")
    pw, W = _pack(p)
    Xb = inputs.make_custom_x("bf16", M, K, 19)
    X = dev_bits(Xb, "bf16")
    ref = _ref(p, Xb)
    need = int(lib.patch_gemm_workspace_bytes(ctypes.byref(pw.desc), M))
    assert need > 0 and need % (M * N * 4) == 0, need
    two = torch.empty(2 * M * N * 4, dtype=torch.uint8, device="cuda")
    for ws in ("auto", two, None):
        tag = ws if isinstance(ws, str) or ws is None else "two planes"
        assert_close(patch.gemm(X, pw, variant="prefill", workspace=ws), ref, what=f"M={M} ws={tag}")
        assert_close(patch.gemm(X, pw, out_dtype=torch.float32, variant="prefill", workspace=ws), ref, f32=True,
                     what=f"M={M} ws={tag} f32")
    pd = inputs.make_custom("bf16", N, K, 18, "dense", 0.0, "top2")
    assert_close(patch.dense_gemm(X, W, variant="prefill"), _ref(pd, Xb), what=f"dense M={M}")
    # AUTO with the workspace takes the split prefill path for M > 16, and is
    # deterministic run to run
    a = patch.gemm(X, pw, out_dtype=torch.float32)
    b = patch.gemm(X, pw, out_dtype=torch.float32)
    assert torch.equal(a, b)
    assert_close(a, ref, f32=True, what=f"auto M={M}")


PREFILL_KERNELS = ["prefill_w64", "prefill_w128", "prefill_w192", "prefill_w256", "prefill_w128_lds", "prefill_w192_lds",
                   "prefill_w256_lds", "prefill_w64_lds", "prefill_big_w128", "prefill_big_w192", "prefill_big_w256", "prefill_big8_w128", "prefill_big8_w256"]
BIG_KERNELS = ["prefill_big_w128", "prefill_big_w192", "prefill_big_w256", "prefill_big8_w128", "prefill_big8_w256"]


@pytest.mark.parametrize("variant", PREFILL_KERNELS)
def test_prefill_every_kernel(variant):
    """Every prefill kernel (M-block width 64/128/192/256, W and X staged
    through registers or through LDS) on the same shape: 640 x 1152 (a lone middle
    row-block, 9 tile columns so K ranges come out uneven), M from below one
    block to several, with a workspace of 2 N K bytes (K split as that
    width's model decides) and with none; packed and dense baseline; every
    output against the oracle."""
    N, K = 640, 1152
    p = inputs.make_custom("bf16", N, K, 24, "bernoulli", 0.5, "uniform")
    pw, W = _pack(p)
    pd = inputs.make_custom("bf16", N, K, 24, "dense", 0.0, "top2")
    ws = torch.empty(2 * N * K, dtype=torch.uint8, device="cuda")
    for M in (17, 100, 300, 700):
        Xb = inputs.make_custom_x("bf16", M, K, 25 + M)
        X = dev_bits(Xb, "bf16")
        ref, ref_d = _ref(p, Xb), _ref(pd, Xb)
        for w in (ws, None):
            tag = f"{variant} M={M} ws={'yes' if w is not None else 'no'}"
            assert_close(patch.gemm(X, pw, variant=variant, workspace=w), ref, what=tag)
            assert_close(patch.gemm(X, pw, out_dtype=torch.float32, variant=variant, workspace=w), ref, f32=True,
                         what=tag + " f32")
            assert_close(patch.dense_gemm(X, W, variant=variant, workspace=w), ref_d, what="dense " + tag)


@pytest.mark.parametrize("variant", PREFILL_KERNELS)
def test_prefill_every_kernel_f16_exact(variant):
    """f16, small integers, fp32 output: every kernel equals the oracle
    exactly (any fp32 summation order is exact here)."""
    rng = np.random.default_rng(26)
    N, K, M = 384, 768, 150
    p = inputs.make_custom("f16", N, K, 27, "bernoulli", 0.5, "uniform")
    p.w = inputs.to_bits(rng.integers(-2, 3, (N, K)).astype(np.float64), "f16")
    Xb = inputs.to_bits(rng.integers(-2, 3, (M, K)).astype(np.float64), "f16")
    pw, W = _pack(p)
    ref = _ref(p, Xb)
    ws = torch.empty(2 * N * K, dtype=torch.uint8, device="cuda")
    y = patch.gemm(dev_bits(Xb, "f16"), pw, out_dtype=torch.float32, variant=variant, workspace=ws)
    assert np.array_equal(host_f64(y), ref), variant


@pytest.mark.parametrize("variant", [v for v in PREFILL_KERNELS if v.endswith("_lds") or "big" in v])
def test_prefill_lds_short_k(variant):
    """The LDS-staged kernels at one to three tile columns (two to six
    64-column steps: the pipeline's first step is also its last-but-one or
    last), with and without a K split, packed and row-major W."""
    for K in (128, 256, 384):
        N = 384
        p = inputs.make_custom("bf16", N, K, 40 + K, "bernoulli", 0.5, "uniform")
        pw, W = _pack(p)
        pd = inputs.make_custom("bf16", N, K, 40 + K, "dense", 0.0, "top2")
        ws = torch.empty(2 * N * K, dtype=torch.uint8, device="cuda")
        for M in (40, 300):
            Xb = inputs.make_custom_x("bf16", M, K, 50 + M)
            X = dev_bits(Xb, "bf16")
            for w in (ws, None):
                tag = f"{variant} K={K} M={M} ws={'yes' if w is not None else 'no'}"
                assert_close(patch.gemm(X, pw, variant=variant, workspace=w), _ref(p, Xb), what=tag)
                assert_close(patch.dense_gemm(X, W, variant=variant, workspace=w), _ref(pd, Xb), what="dense " + tag)


# Shapes with a little over 256 output blocks at one width, so that the
# LDS-staged kernel at that width runs a round of whole blocks and cuts the
# few left over into K ranges (the tail split), and one with fewer blocks
# than a round and a long K, all of whose blocks run in two ranges:
# (variant, N, K, M).  N = 640 has a lone middle row-block; the M values
# leave a ragged last M-block.
TAIL_CASES = [("prefill_w64_lds", 640, 1152, 5750),     # 270 blocks: 14 left over, 3 ranges
              ("prefill_w128_lds", 1536, 1152, 5450),   # 258: 2 left over, 3 ranges
              ("prefill_w192_lds", 1536, 2048, 8371),   # 264: 8 left over, 8 ranges
              ("prefill_w256_lds", 1536, 1152, 14800),  # 348: 92 left over, 2 ranges
              ("prefill_w256_lds", 1536, 8192, 2000)]   # 48: no whole round, 2 ranges of 32 tile columns


@pytest.mark.parametrize("variant,N,K,M", TAIL_CASES)
def test_prefill_tail_split(variant, N, K, M):
    """The tail split: the blocks left over after the whole rounds run in K
    ranges, each range handing its fp32 sums to the block's first range
    through the workspace.  2:4 + dense blob, row-major dense W, a 2:4 + 4:8
    + dense blob and a 64 x 64 tile blob, bf16 and fp32 outputs, on sampled
    rows against the oracle (every output column, so every block of the
    sampled rows); a workspace with room for the slots (64 MB of arbitrary
    bytes: each launch's flags carry its own token, and the first range
    sets them back to 0); repeated calls equal bit for bit; without a
    workspace the data-parallel launch runs."""
    rows = _sampled_rows(M, n=32, seed=M)
    # rows in the last M-blocks too, where the left-over blocks are
    rows = np.unique(np.concatenate([rows, np.arange(M - 300, M, 37)]))
    sel = torch.from_numpy(rows).cuda()
    Xb = inputs.make_custom_x("bf16", M, K, 70 + M)
    X = dev_bits(Xb, "bf16")
    p = inputs.make_custom("bf16", N, K, 71, "bernoulli", 0.5, "uniform")
    pw, W = _pack(p)
    # a workspace of arbitrary bytes: the flags need no initialisation
    ws = torch.randint(0, 256, (64 << 20,), dtype=torch.uint8, device="cuda")
    ref = _ref(p, Xb, rows)
    tag = f"{variant} N={N} K={K} M={M}"
    a = patch.gemm(X, pw, out_dtype=torch.float32, variant=variant, workspace=ws)
    b = patch.gemm(X, pw, out_dtype=torch.float32, variant=variant, workspace=ws)
    assert torch.equal(a, b), tag
    assert_close(a[sel], ref, f32=True, what=tag + " f32")
    assert_close(patch.gemm(X, pw, variant=variant, workspace=ws)[sel], ref, what=tag)
    assert_close(patch.gemm(X, pw, variant=variant, workspace=None)[sel], ref, what=tag + " no workspace")
    pd = inputs.make_custom("bf16", N, K, 71, "dense", 0.0, "top2")
    assert_close(patch.dense_gemm(X, W, variant=variant, workspace=ws)[sel], _ref(pd, Xb, rows), what="dense " + tag)
    pm = inputs.make_mixed("bf16", N, K, 72, 0.3, 0.4, "uniform")
    pwm, _ = _pack(pm)
    assert_close(patch.gemm(X, pwm, variant=variant, workspace=ws)[sel], _ref(pm, Xb, rows), what="4:8 " + tag)
    pq = inputs.make_fine("bf16", N, K, 64, 64, 73, s_exec=0.3, p_sub=0.5)
    pwq = patch.pack_q64(dev_bits(pq.w, "bf16"), pq.tile_map, dev_u8(pq.mask))
    assert_close(patch.gemm(X, pwq, variant=variant, workspace=ws)[sel],
                 oracle.gemm_f64("bf16", Xb[rows], pq.w, pq.tile_map, pq.mask, tile_n=64, tile_k=64),
                 what="64x64 tiles " + tag)


def test_tail_split_bounded_wait():
    """The tail split's bounded wait, forced from the host: with
    patch_debug_tail_wait(64) the first K range of every left-over block
    waits for a flag value no range stores, gives up after 64 polls and
    marks its block's outputs NaN.  The launch ends; the NaN outputs are
    exactly the left-over blocks (whole 256-column M-blocks x 128-row
    row-blocks, two row-blocks a block: 2 x 92 of them here); every other
    output matches the oracle; and the next launch, back to normal on the
    same workspace, is correct everywhere."""
    variant, N, K, M = TAIL_CASES[3]  # 348 blocks: a round of 256, 92 left over in two ranges
    p = inputs.make_custom("bf16", N, K, 76, "bernoulli", 0.5, "uniform")
    pw, _ = _pack(p)
    Xb = inputs.make_custom_x("bf16", M, K, 77)
    X = dev_bits(Xb, "bf16")
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    rows = np.unique(np.concatenate([_sampled_rows(M, n=40, seed=7), np.arange(0, M, 256)]))
    ref = _ref(p, Xb, rows)
    try:
        patch.debug_tail_wait(64)
        y = patch.gemm(X, pw, out_dtype=torch.float32, variant=variant, workspace=ws)
        torch.cuda.synchronize()
    finally:
        patch.debug_tail_wait(0)
    nan = torch.isnan(y).cpu().numpy()
    n_mb, nt = (M + 255) // 256, N // 128
    cells = np.zeros((n_mb, nt))
    for mb in range(n_mb):
        for i in range(nt):
            cells[mb, i] = nan[mb * 256:(mb + 1) * 256, i * 128:(i + 1) * 128].mean()
    assert set(np.unique(cells)) <= {0.0, 1.0}, "NaN outputs must form whole blocks"
    assert int(cells.sum()) == 2 * 92, int(cells.sum())
    got = host_f64(y[torch.from_numpy(rows).cuda()])
    fin = ~np.isnan(got)
    assert fin.any()
    scale = float(np.abs(ref).max())
    assert float(np.abs(got[fin] - ref[fin]).max()) <= 1e-2 * scale
    y2 = patch.gemm(X, pw, out_dtype=torch.float32, variant=variant, workspace=ws)
    assert not bool(torch.isnan(y2).any())
    assert_close(y2[torch.from_numpy(rows).cuda()], ref, f32=True, what="after the forced wait")


def test_tail_split_graph_replays():
    """Tail-split launches captured in a HIP graph (the graph holds one token
    per launch, so every replay relies on the previous one having set its
    flags back to 0): one with a whole round and left-over blocks, one
    without, replayed four times with eager tail-split launches on the same
    workspace and synchronisations in between; every replay equals the eager
    result bit for bit."""
    cases = []
    for variant, N, K, M in (TAIL_CASES[3], TAIL_CASES[4]):
        p = inputs.make_custom("bf16", N, K, 74, "bernoulli", 0.5, "uniform")
        pw, _ = _pack(p)
        X = dev_bits(inputs.make_custom_x("bf16", M, K, 75 + M), "bf16")
        cases.append((variant, pw, X, torch.empty((M, N), dtype=torch.float32, device="cuda")))
    ws = torch.randint(0, 256, (64 << 20,), dtype=torch.uint8, device="cuda")

    def run():
        for variant, pw, X, out in cases:
            patch.gemm(X, pw, out_dtype=torch.float32, variant=variant, workspace=ws, out=out)

    run()
    torch.cuda.synchronize()
    eager = [c[3].clone() for c in cases]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        for c in cases:
            c[3].fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        for c, e in zip(cases, eager):
            assert torch.equal(c[3], e), f"replay {rep} {c[0]}"
        run()  # eager tail-split launches (fresh tokens) on the same workspace
        torch.cuda.synchronize()
        for c, e in zip(cases, eager):
            assert torch.equal(c[3], e), f"eager after replay {rep} {c[0]}"


# ------------------------------------------------------------------ exact cases
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_identity_x_gives_masked_weights_exactly(dtype):
    """X = rows of the identity: every output is one product w * 1, exact in
    any precision, so Y^T == W o E bit for bit.  This pins every metadata
    position of every lane for both variants."""
    p = inputs.make_custom(dtype, 256, 384, 10, "bernoulli", 0.5, "uniform")
    pw, _ = _pack(p)
    E = oracle.effective_mask(p.N, p.K, p.tile_map, p.mask)
    Weff = np.where(E != 0, inputs.bits_to_f32(p.w, dtype), 0.0).astype(np.float64)
    eye = inputs.to_bits(np.eye(p.K), dtype)
    # prefill: all K rows at once, every prefill kernel staged through LDS
    for v in ["prefill", "prefill_w64_lds"] + BIG_KERNELS:
        y = patch.gemm(dev_bits(eye, dtype), pw, variant=v)
        assert np.array_equal(host_f64(y).T, Weff), v
    # decode: 16 rows at a time (one block of M), then 128 (eight blocks)
    for rows in (16, 128):
        for k0 in range(0, p.K, rows):
            y = patch.gemm(dev_bits(eye[k0:k0 + rows], dtype), pw, variant="decode")
            assert np.array_equal(host_f64(y).T, Weff[:, k0:k0 + rows]), (rows, k0)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M", [3, 16, 40, 128, 200])
def test_small_integers_exact_in_f32(dtype, M):
    """|x|, |w| <= 2 and K <= 4096: every partial sum is an integer below 2^24,
    so any fp32 summation order is exact and must equal the oracle."""
    rng = np.random.default_rng(M)
    N, K = 256, 1024
    p = inputs.make_custom(dtype, N, K, 11, "bernoulli", 0.5, "uniform")
    p.w = inputs.to_bits(rng.integers(-2, 3, (N, K)).astype(np.float64), dtype)
    Xb = inputs.to_bits(rng.integers(-2, 3, (M, K)).astype(np.float64), dtype)
    pw, _ = _pack(p)
    ref = _ref(p, Xb)
    for v in ["prefill"] + BIG_KERNELS + (["decode"] if M <= 128 else []):
        y = patch.gemm(dev_bits(Xb, dtype), pw, out_dtype=torch.float32, variant=v)
        assert np.array_equal(host_f64(y), ref), v


def test_six_patterns_every_lane_slot():
    """Each of the six patterns in every group of a full tile, with X = ones on
    one column at a time."""
    N = K = 128
    rng = np.random.default_rng(5)
    w = inputs.to_bits(rng.integers(1, 8, (N, K)).astype(np.float64), "bf16")
    pat = (np.arange(N)[:, None] + np.arange(K // 4)[None, :]) % 6
    mask = np.zeros((N, K // 4, 4), np.uint8)
    np.put_along_axis(mask, inputs.PATTERNS[pat], 1, axis=-1)
    mask = mask.reshape(N, K)
    tm = np.ones((1, 1), np.uint8)
    pw = patch.pack(dev_bits(w, "bf16"), tm, dev_u8(mask))
    eye = inputs.to_bits(np.eye(K), "bf16")
    ref = oracle.gemm_f64("bf16", eye, w, tm, mask)
    for v in ["prefill"] + BIG_KERNELS:
        y = patch.gemm(dev_bits(eye, "bf16"), pw, out_dtype=torch.float32, variant=v)
        assert np.array_equal(host_f64(y), ref), v
    for rows in (16, 32, 64, 128):
        for k0 in range(0, K, rows):
            y = patch.gemm(dev_bits(eye[k0:k0 + rows], "bf16"), pw, out_dtype=torch.float32, variant="decode")
            assert np.array_equal(host_f64(y), ref[k0:k0 + rows]), (rows, k0)


# ------------------------------------------------------------------ robustness
def test_output_guard_bands_untouched():
    p = inputs.make_custom("bf16", 384, 640, 12, "bernoulli", 0.5, "top2")
    pw, _ = _pack(p)
    for M in (7, 70, 300):
        X = dev_bits(inputs.make_custom_x("bf16", M, 640, 1), "bf16")
        for v in ["prefill"] + (["decode"] if M <= 128 else []):
            pad = 4096
            buf = torch.full((M * 384 + 2 * pad,), 12345.0, dtype=torch.float32, device="cuda")
            y = buf[pad:pad + M * 384].view(M, 384)
            patch.gemm(X, pw, out_dtype=torch.float32, variant=v, out=y)
            torch.cuda.synchronize()
            assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[pad + M * 384:] == 12345.0), v


def test_blob_guard_bands_untouched():
    p = inputs.make_custom("bf16", 256, 384, 13, "bernoulli", 0.5, "top2")
    n = oracle.packed_bytes(p.N, p.K, p.tile_map)
    pad = 4096
    buf = torch.full((n + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    pw = patch.pack(dev_bits(p.w, "bf16"), p.tile_map, dev_u8(p.mask), out=buf[pad:pad + n])
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 0xA5) and torch.all(buf[pad + n:] == 0xA5)
    assert np.array_equal(pw.blob.cpu().numpy(), oracle.pack("bf16", p.w, p.tile_map, p.mask))


def test_deterministic_repeat():
    p = inputs.make_weights(inputs.CONFIGS["decode"], 0, 0)
    pw, _ = _pack(p)
    for M in (16, 128, 512):
        X = dev_bits(inputs.make_x(inputs.CONFIGS["decode"], M, p.K), "bf16")
        a = patch.gemm(X, pw, out_dtype=torch.float32)
        b = patch.gemm(X, pw, out_dtype=torch.float32)
        assert torch.equal(a, b), M


def test_graph_replays_match_eager():
    """The GEMM calls can be captured in a HIP graph (the bench times them
    that way): decode, split-K prefill (with its workspace from the graph's
    pool) and the dense baseline in one graph, replayed three times with
    other eager GEMMs and synchronisations in between; every replay must
    equal the eager results bit for bit (the kernels are deterministic)."""
    p = inputs.make_custom("bf16", 512, 4096, 20, "bernoulli", 0.5, "uniform")
    pw, W = _pack(p)
    X4 = dev_bits(inputs.make_custom_x("bf16", 4, 4096, 21), "bf16")
    X128 = dev_bits(inputs.make_custom_x("bf16", 128, 4096, 22), "bf16")
    Xo = dev_bits(inputs.make_custom_x("bf16", 64, 4096, 23), "bf16")
    outs = [torch.empty((4, 512), dtype=torch.bfloat16, device="cuda"),
            torch.empty((128, 512), dtype=torch.float32, device="cuda"),
            torch.empty((128, 512), dtype=torch.bfloat16, device="cuda")]

    def run():
        patch.gemm(X4, pw, out=outs[0])
        patch.gemm(X128, pw, out_dtype=torch.float32, variant="prefill", out=outs[1])
        patch.dense_gemm(X128, W, variant="prefill", out=outs[2])

    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
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
        other = patch.gemm(Xo, pw, variant="prefill")  # eager work between replays
        torch.cuda.synchronize()
        assert other.shape == (64, 512)


# ------------------------------------------------------------------ the named workloads
def test_config_tiny_all_seeds():
    cfg = inputs.CONFIGS["tiny"]
    for seed in range(6):
        p = inputs.make_weights(cfg, 0, 0, seed=seed)
        pw, _ = _pack(p)
        Xb = inputs.make_x(cfg, 16, p.K, seed=seed)
        ref = _ref(p, Xb)
        for v in ("auto", "decode", "prefill"):
            assert_close(patch.gemm(dev_bits(Xb, "f16"), pw, variant=v), ref, what=f"tiny seed {seed} {v}")


def test_config_decode_q_proj_full():
    cfg = inputs.CONFIGS["decode"]
    p = inputs.make_weights(cfg, 0, 0)
    assert p.tile_map.sum() == 512
    pw, W = _pack(p)
    for M in cfg.Ms:
        Xb = inputs.make_x(cfg, M, p.K)
        X = dev_bits(Xb, "bf16")
        ref = _ref(p, Xb)
        assert_close(patch.gemm(X, pw), ref, what=f"decode M={M}")
        assert_close(patch.gemm(X, pw, out_dtype=torch.float32), ref, f32=True, what=f"decode M={M} f32")


def _sampled_rows(M, n=24, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, size=min(M, n), replace=False)]))
    return rows


@pytest.mark.parametrize("mi", [0, 1])
def test_config_prefill_mlp_sampled(mi):
    cfg = inputs.CONFIGS["prefill_mlp"]
    p = inputs.make_weights(cfg, mi, 0)
    assert p.tile_map.sum() == 2202
    pw, _ = _pack(p)
    M = cfg.Ms[0]
    Xb = inputs.make_x(cfg, M, p.K, matrix_index=mi)
    y = patch.gemm(dev_bits(Xb, "bf16"), pw)
    rows = _sampled_rows(M)
    assert_close(y[torch.from_numpy(rows).cuda()], _ref(p, Xb, rows), what=f"prefill_mlp {cfg.matrices[mi].name}")


@pytest.mark.parametrize("mi", [0, 1])
def test_config_imbalanced_13b_sampled(mi):
    cfg = inputs.CONFIGS["imbalanced_13b"]
    p = inputs.make_weights(cfg, mi, 0)
    NT = p.N // 128
    assert np.all(p.tile_map[:NT // 2] == 0) and np.all(p.tile_map[NT // 2:] == 1)
    pw, _ = _pack(p)
    M = cfg.Ms[0]
    Xb = inputs.make_x(cfg, M, p.K, matrix_index=mi)
    y = patch.gemm(dev_bits(Xb, "bf16"), pw)
    rows = _sampled_rows(M, seed=mi)
    assert_close(y[torch.from_numpy(rows).cuda()], _ref(p, Xb, rows), what=f"13b {cfg.matrices[mi].name}")


@pytest.mark.parametrize("mi", range(7))
def test_config_sweep_sampled(mi):
    """Sparsity sweep, every one of its seven independently seeded
    LLaMA-2-7B matrices (q, k, v, o, gate, up, down), at every sparse-tile
    fraction: the packed blob equals the oracle's byte for byte, and the GEMM
    at every M of the sweep is within tolerance on sampled output rows."""
    cfg = inputs.CONFIGS["sweep"]
    base = None
    for si, frac in enumerate(cfg.fractions):
        p = inputs.make_weights(cfg, mi, si, reuse=base)
        base = base or p
        assert p.tile_map.sum() == int(np.round(frac * p.tile_map.size))
        pw, _ = _pack(p)
        blob = pw.blob.cpu().numpy()
        want = oracle.pack("bf16", p.w, p.tile_map, p.mask)
        assert blob.size == want.size and np.array_equal(blob, want), f"sweep {cfg.matrices[mi].name} s={frac} blob"
        for M in cfg.Ms:
            Xb = inputs.make_x(cfg, M, p.K, matrix_index=mi)
            y = patch.gemm(dev_bits(Xb, "bf16"), pw)
            rows = _sampled_rows(M, n=8, seed=si)
            assert_close(y[torch.from_numpy(rows).cuda()], _ref(p, Xb, rows),
                         what=f"sweep {cfg.matrices[mi].name} s={frac} M={M}")
