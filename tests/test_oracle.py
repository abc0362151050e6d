"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test names what pins it: a library routine or textbook special case, an
exact invariant stated by the pages, brute force on tiny inputs, or a
hand-worked example of the byte format.  Page citations refer to PATCH
(arXiv 2509.23410): the arXiv abstract, and the gist.science explainer
sections "1. Problem Statement", "2. Methodology: PATCH" and
"4. Experimental Results".
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
from sparse_gemm_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- element codecs
def test_f16_decode_all_patterns_match_numpy():
    """binary16 decoding: every one of the 65536 patterns against numpy's
    float16 -> float64 conversion (library routine)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_all_patterns_match_torch():
    """bfloat16 decoding: all 65536 patterns against torch's bfloat16 -> float64."""
    import torch

    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_round_to_f16_matches_numpy_rne():
    """fp64 -> binary16 rounding against numpy (direct RNE), with exact ties."""
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 6, 20000),
        # exact halfway cases between adjacent binary16 values
        (np.arange(1, 4000, dtype=np.float64) + 0.5) * 2.0 ** -10,
        (np.arange(1, 400, dtype=np.float64) + 0.5) * 2.0 ** -24,  # subnormal ties
        np.array([65504.0, 65519.99, 65520.0, -65520.0, 0.0, -0.0, 1e-9, -1e-9]),
    ])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    got = oracle.round_f64("f16", v)
    assert np.array_equal(got, ref)


def test_round_to_bf16_matches_torch_rne():
    """fp64 -> bfloat16 rounding against torch's float32 -> bfloat16 (RNE), on
    values exactly representable in float32 so torch's route is exact."""
    import torch

    rng = np.random.default_rng(2)
    f32 = (rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000)).astype(np.float32)
    ties = ((rng.integers(0, 1 << 16, 5000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    f32 = np.concatenate([f32, ties, np.array([3.3895314e38, -3.3895314e38, 0.0, -0.0], np.float32)])
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_f64("bf16", f32.astype(np.float64))
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- effective mask
def _problem(N, K, kind, frac, dtype="bf16", seed=0, mask="top2"):
    return inputs.make_custom(dtype, N, K, seed, kind, frac, mask)


def test_effective_mask_two_of_four_in_sparse_tiles_one_in_dense():
    """S2: in a 2:4 tile every group of four keeps exactly two (explainer
    section 1, '2:4 ... two non-zero values per four elements'); a dense tile
    keeps everything (section 2, 'remain dense (0% sparsity)')."""
    p = _problem(512, 384, "bernoulli", 0.5, seed=3)
    E = oracle.effective_mask(p.N, p.K, p.tile_map, p.mask)
    tm = np.repeat(np.repeat(p.tile_map, 128, 0), 128, 1).astype(bool)
    groups = E.reshape(p.N, p.K // 4, 4).sum(-1)
    gsparse = tm.reshape(p.N, p.K // 4, 4)[..., 0]
    assert np.all(groups[gsparse] == 2)
    assert np.all(E[~tm] == 1)
    assert 0 < p.tile_map.sum() < p.tile_map.size


@pytest.mark.parametrize("frac", [0.0, 0.25, 0.5, 0.75, 1.0])
def test_sparsity_is_half_the_sparse_tile_fraction(frac):
    """S3: overall sparsity = 0.5 x (fraction of sparse tiles), exactly, which
    spans 0%..50% (abstract: 'continuous sparsity ratio between 0% and 50%')."""
    p = _problem(512, 512, "exact", frac, seed=4)
    E = oracle.effective_mask(p.N, p.K, p.tile_map, p.mask)
    zeros = int((E == 0).sum())
    T = p.tile_map.size
    n_sparse = int(p.tile_map.sum())
    assert n_sparse == int(np.round(frac * T))
    # zeros / (N K) == 0.5 * n_sparse / T, compared as exact rationals
    assert zeros * 2 * T == n_sparse * p.N * p.K


def test_mask_in_dense_tiles_is_ignored_and_not_validated():
    p = _problem(256, 256, "exact", 0.5, seed=5)
    mask = p.mask.copy()
    dense_i, dense_j = np.argwhere(p.tile_map == 0)[0]
    mask[dense_i * 128:(dense_i + 1) * 128, dense_j * 128:(dense_j + 1) * 128] = 0  # illegal, but dense
    assert oracle.validate(p.N, p.K, p.tile_map, mask) is None
    X = inputs.make_custom_x("bf16", 8, 256, 1)
    assert np.array_equal(oracle.gemm_f64("bf16", X, p.w, p.tile_map, mask),
                          oracle.gemm_f64("bf16", X, p.w, p.tile_map, p.mask))


@pytest.mark.parametrize("keep", [(0,), (0, 1, 2), (), (0, 1, 2, 3)])
def test_illegal_sparse_group_is_rejected(keep):
    p = _problem(256, 256, "sparse", 1.0, seed=6)
    mask = p.mask.copy()
    mask[37, 4 * 9:4 * 9 + 4] = 0
    for d in keep:
        mask[37, 4 * 9 + d] = 1
    assert oracle.validate(p.N, p.K, p.tile_map, mask) == (37, 9)
    with pytest.raises(oracle.OracleError):
        oracle.gemm_f64("bf16", np.zeros((1, 256), np.uint16), p.w, p.tile_map, mask)
    with pytest.raises(oracle.OracleError):
        oracle.pack("bf16", p.w, p.tile_map, mask)


# ---------------------------------------------------------------- the GEMM
def test_all_dense_map_equals_numpy_matmul():
    """S1: with an all-dense tile map the method is a plain GEMM; against
    numpy.matmul in float64 (library routine) to 1e-12 relative."""
    for dtype in ("bf16", "f16"):
        p = _problem(256, 384, "dense", 0.0, dtype=dtype, seed=7)
        X = inputs.make_custom_x(dtype, 33, 384, 2)
        Y = oracle.gemm_f64(dtype, X, p.w, p.tile_map, p.mask)
        Xf = inputs.bits_to_f32(X, dtype).astype(np.float64)
        Wf = inputs.bits_to_f32(p.w, dtype).astype(np.float64)
        ref = Xf @ Wf.T
        np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_all_sparse_map_equals_numpy_matmul_of_masked_weights():
    """Uniform 2:4 special case: every tile sparse, so Y = X (W o mask)^T with
    the mask applied by numpy (library matmul of the masked matrix)."""
    p = _problem(256, 256, "sparse", 1.0, seed=8, mask="uniform")
    X = inputs.make_custom_x("bf16", 16, 256, 3)
    Y = oracle.gemm_f64("bf16", X, p.w, p.tile_map, p.mask)
    Wf = inputs.bits_to_f32(p.w, "bf16").astype(np.float64) * (p.mask != 0)
    ref = inputs.bits_to_f32(X, "bf16").astype(np.float64) @ Wf.T
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def _int_bits(vals, dtype):
    return inputs.to_bits(np.asarray(vals, dtype=np.float64), dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_brute_force_8x8_all_tile_maps(dtype):
    """S4: 8 x 8 weights with 4 x 4 tiles (the pages' finest tile, section 4
    'Tile Size'), all 16 tile maps, integer-valued X and W in -3..3.  A second
    formulation sums only over the two kept positions of each group, read from
    the six-pattern table, and must agree exactly."""
    rng = np.random.default_rng(11)
    M, N, K = 5, 8, 8
    Xi = rng.integers(-3, 4, (M, K))
    Wi = rng.integers(-3, 4, (N, K))
    X, W = _int_bits(Xi, dtype), _int_bits(Wi, dtype)
    pats = rng.integers(0, 6, (N, K // 4))
    mask = np.zeros((N, K), np.uint8)
    for n in range(N):
        for g in range(K // 4):
            for d in inputs.PATTERNS[pats[n, g]]:
                mask[n, 4 * g + d] = 1
    for bitsmap in range(16):
        tmap = np.array([(bitsmap >> b) & 1 for b in range(4)], np.uint8).reshape(2, 2)
        Y = oracle.gemm_f64(dtype, X, W, tmap, mask, tile_n=4, tile_k=4)
        ref = np.zeros((M, N), dtype=np.int64)
        for m in range(M):
            for n in range(N):
                s = 0
                for g in range(K // 4):
                    if tmap[n // 4, (4 * g) // 4]:
                        for d in inputs.PATTERNS[pats[n, g]]:
                            s += Xi[m, 4 * g + d] * Wi[n, 4 * g + d]
                    else:
                        for d in range(4):
                            s += Xi[m, 4 * g + d] * Wi[n, 4 * g + d]
                ref[m, n] = s
        assert np.array_equal(Y, ref.astype(np.float64)), bitsmap


def test_identity_x_recovers_masked_weights():
    """With X = identity rows, Y^T is W o E exactly (one product per output)."""
    p = _problem(256, 256, "bernoulli", 0.5, seed=9)
    X = inputs.to_bits(np.eye(256), "bf16")
    Y = oracle.gemm_f64("bf16", X, p.w, p.tile_map, p.mask)
    E = oracle.effective_mask(p.N, p.K, p.tile_map, p.mask)
    Wf = inputs.bits_to_f32(p.w, "bf16").astype(np.float64) * E
    assert np.array_equal(Y.T, Wf)


def test_six_patterns_each_select_their_columns():
    """Each of the six 2:4 patterns (section 2 'Pattern Selection') keeps its two
    columns: with W = 1 and X = one-hot columns, Y reads back the pattern."""
    for pi, (a, b) in enumerate(inputs.PATTERNS):
        N = K = 128
        W = inputs.to_bits(np.ones((N, K)), "bf16")
        mask = np.zeros((N, K), np.uint8)
        mask[:, a::4] = 1
        mask[:, b::4] = 1
        X = inputs.to_bits(np.eye(K)[:4], "bf16")
        Y = oracle.gemm_f64("bf16", X, W, np.ones((1, 1), np.uint8), mask)
        expect = np.zeros((4, N))
        expect[a] = 1
        expect[b] = 1
        assert np.array_equal(Y, expect), pi


def test_oracle_result_independent_of_thread_count():
    import subprocess
    import sys
    code = ("import numpy as np, oracle; from sparse_gemm_amd import inputs;"
            "p = inputs.make_custom('bf16', 384, 256, 1, 'bernoulli', 0.5, 'top2');"
            "X = inputs.make_custom_x('bf16', 7, 256, 1);"
            "print(oracle.gemm_f64('bf16', X, p.w, p.tile_map, p.mask).tobytes().hex()[:4000])")
    outs = []
    for t in ("1", "5"):
        env = dict(os.environ, OMP_NUM_THREADS=t)
        outs.append(subprocess.check_output([sys.executable, "-c", code], env=env,
                                            cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
    assert outs[0] == outs[1]


# ---------------------------------------------------------------- packed format
def _golden(name):
    kv = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            kv[k] = int(v, 0)
    return kv


def test_pack_hand_worked_example():
    g = _golden("pack_format_example.txt")
    N, K = 128, 256
    W = np.full((N, K), 0x3F80, np.uint16)
    W[g["dense.row"], g["dense.col"]] = g["dense.bits"]
    W[g["dense2.row"], g["dense2.col"]] = g["dense2.bits"]
    W[g["sparse.row"], g["sparse.col"]] = g["sparse.bits"]
    mask = np.zeros((N, K), np.uint8)
    mask[:, 0::4] = 1
    mask[:, 1::4] = 1
    r, c = g["sparse.row"], g["sparse.col"]
    g0 = c - c % 4
    mask[r, g0:g0 + 4] = [1, 0, 1, 0]
    tmap = np.array([[0, 1]], np.uint8)
    blob = oracle.pack("bf16", W, tmap, mask)
    u64 = lambda o: int.from_bytes(blob[o:o + 8].tobytes(), "little")
    u32 = lambda o: int.from_bytes(blob[o:o + 4].tobytes(), "little")
    u16 = lambda o: int.from_bytes(blob[o:o + 2].tobytes(), "little")
    assert blob.size == g["header.total_bytes"]
    assert u32(0) == 0x48435450 and u32(4) == g["header.version"] and u32(8) == 1
    assert (u32(12), u32(16), u32(20), u32(24), u32(28), u32(32)) == (128, 128, N, K, 1, 2)
    assert u32(36) == g["header.n_sparse"]
    assert u64(40) == 256 and u64(48) == g["header.data_offset"] and u64(64) == g["header.total_bytes"]
    assert u64(56) == g["header.total_bytes"] - g["header.data_offset"]
    assert u64(256) == g["table.0.offset"] and u32(264) == g["table.0.kind"]
    assert u64(272) == g["table.1.offset"] and u32(280) == g["table.1.kind"]
    assert u16(g["dense.byte_offset"]) == g["dense.bits"]
    assert u16(g["dense2.byte_offset"]) == g["dense2.bits"]
    assert u16(g["sparse.byte_offset"]) == g["sparse.bits"]
    assert blob[g["sparse.meta_byte_offset"]] == g["sparse.meta_byte_value"]
    assert u32(268) == g["table.0.stride"] and u32(284) == g["table.1.stride"]
    # every other metadata nibble of the sparse tile is code 4 (keeps 0 and 1)
    meta = np.concatenate([blob[g["table.1.offset"] + b * g["table.1.stride"] + 2048:
                                g["table.1.offset"] + b * g["table.1.stride"] + 2304] for b in range(8)])
    nib = np.stack([meta & 15, meta >> 4], -1).ravel()
    assert (nib == 4).sum() == nib.size - 1 and (nib == 8).sum() == 1


def test_packed_size_closed_form():
    for frac in (0.0, 0.3, 1.0):
        p = _problem(384, 640, "exact", frac, seed=12)
        T = p.tile_map.size
        ns = int(p.tile_map.sum())
        expect = -(-(256 + 16 * T) // 256) * 256 + 32768 * (T - ns) + 18432 * ns
        assert oracle.packed_bytes(p.N, p.K, p.tile_map) == expect
        assert oracle.pack("bf16", p.w, p.tile_map, p.mask).size == expect


def _unpack(blob, N, K):
    """Independent reader of the format (written from the format definition)."""
    NT, KT = N // 128, K // 128
    W = np.zeros((N, K), np.uint16)
    codes = []
    u64 = lambda o: int.from_bytes(blob[o:o + 8].tobytes(), "little")
    u32 = lambda o: int.from_bytes(blob[o:o + 4].tobytes(), "little")
    for i in range(NT):
        for j in range(KT):
            e = 256 + 16 * (i * KT + j)
            off, kind, stride = u64(e), u32(e + 8), u32(e + 12)
            for band in range(8):
                piece = blob[off + band * stride:off + band * stride + (4096 if kind == 0 else 2304)]
                if kind == 0:
                    # blocks (q, e) of 1 KB, lane l's 16 bytes at 16*l: element 2*g + u
                    ch = piece.view(np.uint16).reshape(2, 2, 64, 8)
                    for q in range(2):
                        for half in range(2):
                            for l in range(64):
                                r = i * 128 + band * 16 + l % 16
                                for g in range(4):
                                    for u in range(2):
                                        c = j * 128 + 64 * q + 16 * (l // 16) + 4 * g + 2 * half + u
                                        W[r, c] = ch[q, half, l, 2 * g + u]
                elif kind == 2:
                    # 4:8: block q holds lane l's four kept values of its groups u = 0, 1
                    # (columns 64q + 16(l/16) + 8u ..); byte 2q + u of the lane's mask
                    # word: positions kept in that group
                    vals = piece[:2048].view(np.uint16).reshape(2, 64, 8)
                    masks = piece[2048:2304].reshape(64, 4)
                    for l in range(64):
                        r = i * 128 + band * 16 + l % 16
                        for q in range(2):
                            for u in range(2):
                                m = int(masks[l, 2 * q + u])
                                codes.append(m)
                                kept = [pp for pp in range(8) if (m >> pp) & 1]
                                for s_, pp in enumerate(kept[:4]):
                                    W[r, j * 128 + 64 * q + 16 * (l // 16) + 8 * u + pp] = vals[q, l, 4 * u + s_]
                else:
                    vals = piece[:2048].view(np.uint16).reshape(2, 64, 8)
                    meta = piece[2048:2304].view(np.uint32)
                    for q in range(2):
                        for l in range(64):
                            r = i * 128 + band * 16 + l % 16
                            for p in range(4):
                                g = 16 * q + 4 * (l // 16) + p
                                code = (int(meta[l]) >> (16 * q + 4 * p)) & 15
                                codes.append(code)
                                i0, i1 = code & 3, code >> 2
                                W[r, j * 128 + 4 * g + i0] = vals[q, l, 2 * p]
                                W[r, j * 128 + 4 * g + i1] = vals[q, l, 2 * p + 1]
    return W, np.array(codes)


@pytest.mark.parametrize("mask_kind", ["top2", "uniform"])
def test_pack_round_trip_and_legal_codes(mask_kind):
    """unpack(pack(W)) == W o E bit-exactly; every code is one of the six
    patterns i0 | i1 << 2 with i0 < i1: {4, 8, 12, 9, 13, 14}."""
    p = _problem(256, 384, "bernoulli", 0.5, seed=13, mask=mask_kind)
    blob = oracle.pack("bf16", p.w, p.tile_map, p.mask)
    W2, codes = _unpack(blob, p.N, p.K)
    E = oracle.effective_mask(p.N, p.K, p.tile_map, p.mask)
    assert np.array_equal(W2, np.where(E != 0, p.w, 0).astype(np.uint16))
    assert set(np.unique(codes)) <= {4, 8, 12, 9, 13, 14}
    if mask_kind == "uniform":
        assert set(np.unique(codes)) == {4, 8, 12, 9, 13, 14}


def test_pack_keeps_negative_zero_bits():
    N = K = 128
    W = np.full((N, K), 0x8000, np.uint16)  # -0.0 everywhere
    mask = np.zeros((N, K), np.uint8)
    mask[:, 1::4] = 1
    mask[:, 3::4] = 1
    blob = oracle.pack("bf16", W, np.ones((1, 1), np.uint8), mask)
    # one sparse tile: 8 band pieces of 2304 bytes (2048 of values, 256 of codes) from byte 512
    pieces = blob[512:512 + 8 * 2304].reshape(8, 2304)
    assert np.all(pieces[:, :2048].copy().view(np.uint16) == 0x8000)
    assert np.all(pieces[:, 2048:] == (13 | (13 << 4)))  # code (1,3) = 1 | 3 << 2 = 13


# ------------------------------------------------------- format 4: 64 x 64 execution tiles
def test_pack_q64_hand_worked_example():
    g = _golden("pack_q64_example.txt")
    N, K = 128, 256
    W = np.full((N, K), 0x3F80, np.uint16)
    for x in "abcdef":
        W[g[x + ".row"], g[x + ".col"]] = g[x + ".bits"]
    mask = np.zeros((N, K), np.uint8)
    mask[:, 0::4] = 1
    mask[:, 1::4] = 1
    for x, keep in (("b", [1, 0, 0, 1]), ("c", [0, 1, 1, 0]), ("e", [0, 0, 1, 1])):
        r, c = g[x + ".row"], g[x + ".col"]
        mask[r, c - c % 4:c - c % 4 + 4] = keep
    qmap = np.array([[0, 1, 1, 1], [1, 0, 0, 0]], np.uint8)
    blob = oracle.pack_q64("bf16", W, qmap, mask)
    u64 = lambda o: int.from_bytes(blob[o:o + 8].tobytes(), "little")
    u32 = lambda o: int.from_bytes(blob[o:o + 4].tobytes(), "little")
    u16 = lambda o: int.from_bytes(blob[o:o + 2].tobytes(), "little")
    assert blob.size == g["header.total_bytes"] == oracle.packed_bytes_q64(N, K, qmap)
    assert u32(0) == 0x48435450 and u32(4) == g["header.version"] and u32(8) == 1
    assert u32(12) == u32(16) == g["header.tile"]
    assert (u32(20), u32(24), u32(28), u32(32)) == (N, K, g["header.nt_n"], g["header.nt_k"])
    assert u32(36) == g["header.n_sparse"] and u32(72) == 0
    assert u64(40) == 256 and u64(48) == g["header.data_offset"] and u64(64) == g["header.total_bytes"]
    assert u64(56) == g["header.total_bytes"] - g["header.data_offset"]
    for t in range(4):
        e = 256 + 16 * t
        assert (u64(e), u32(e + 8), u32(e + 12)) == (g[f"table.{t}.offset"], g[f"table.{t}.kind"],
                                                     g[f"table.{t}.stride"])
    for x in "abcdef":
        assert u16(g[x + ".byte_offset"]) == g[x + ".bits"], x
    for x in "bce":
        assert blob[g[x + ".code_byte_offset"]] == g[x + ".code_byte_value"], x
    for x in "bc":
        assert blob[g[x + ".zero_code_byte_offset"]] == 0, x


def _unpack_q64(blob, N, K):
    """Independent reader of format 4 (written from its definition): W o E
    and the codes of every 2:4 group."""
    R, KC = N // 64, K // 128
    W = np.zeros((N, K), np.uint16)
    codes = []
    u64 = lambda o: int.from_bytes(blob[o:o + 8].tobytes(), "little")
    u32 = lambda o: int.from_bytes(blob[o:o + 4].tobytes(), "little")
    for r in range(R):
        for j in range(KC):
            e = 256 + 16 * (r * KC + j)
            off, kb, stride = u64(e), u32(e + 8), u32(e + 12)
            starts = [0, 1024 if kb & 1 else 2048]
            code_at = starts[1] + (1024 if kb & 2 else 2048)
            for band in range(4):
                base = off + band * stride
                for q in range(2):
                    part = base + starts[q]
                    for l in range(64):
                        row = 64 * r + 16 * band + l % 16
                        h = l // 16
                        if (kb >> q) & 1:
                            word = u32(base + code_at + 4 * l)
                            vals = blob[part + 16 * l:part + 16 * l + 16].view(np.uint16)
                            for p in range(4):
                                G = 16 * q + 4 * h + p
                                code = (word >> (16 * q + 4 * p)) & 15
                                codes.append(code)
                                W[row, 128 * j + 4 * G + (code & 3)] = vals[2 * p]
                                W[row, 128 * j + 4 * G + (code >> 2)] = vals[2 * p + 1]
                        else:
                            if kb:  # a dense slice leaves its code bits zero
                                assert (u32(base + code_at + 4 * l) >> (16 * q)) & 0xFFFF == 0
                            for half in range(2):
                                vals = blob[part + 1024 * half + 16 * l:part + 1024 * half + 16 * l + 16].view(np.uint16)
                                for gg in range(4):
                                    for u in range(2):
                                        W[row, 128 * j + 64 * q + 16 * h + 4 * gg + 2 * half + u] = vals[2 * gg + u]
    return W, np.array(codes)


def _quad_problem(N, K, frac, seed, mask="uniform"):
    rng = np.random.default_rng(seed)
    qmap = (rng.random((N // 64, K // 64)) < frac).astype(np.uint8)
    w = rng.integers(0, 1 << 16, (N, K), dtype=np.uint16)
    # a random pair of the four positions in every group
    pick = rng.integers(0, 6, (N, K // 4))
    pairs = np.array([[0, 1], [0, 2], [0, 3], [1, 2], [1, 3], [2, 3]])
    mk = np.zeros((N, K // 4, 4), np.uint8)
    sel = pairs[pick]
    np.put_along_axis(mk, sel, 1, axis=2)
    if mask == "top2":
        mk[:] = 0
        mk[:, :, :2] = 1
    return qmap, w, mk.reshape(N, K)


@pytest.mark.parametrize("frac", [0.0, 0.4, 1.0])
def test_pack_q64_round_trip_and_legal_codes(frac):
    """unpack(pack(W)) == W o E for E from the 64 x 64 quadrant map,
    bit-exactly; the codes are the six 2:4 patterns."""
    N, K = 256, 384
    qmap, w, mk = _quad_problem(N, K, frac, seed=41)
    blob = oracle.pack_q64("bf16", w, qmap, mk)
    W2, codes = _unpack_q64(blob, N, K)
    E = oracle.effective_mask(N, K, qmap, mk, tile_n=64, tile_k=64)
    assert np.array_equal(W2, np.where(E != 0, w, 0).astype(np.uint16))
    if frac > 0:
        assert set(np.unique(codes)) == {4, 8, 12, 9, 13, 14}


def test_pack_q64_size_closed_form():
    """total = data offset + 8192 per dense quadrant + 4096 per 2:4 quadrant
    + 1024 per cell (pair of quadrants) holding any 2:4 quadrant."""
    N, K = 384, 640
    for frac in (0.0, 0.3, 1.0):
        qmap, w, mk = _quad_problem(N, K, frac, seed=42)
        ns = int(qmap.sum())
        nq = qmap.size
        cells = qmap.reshape(N // 64, K // 128, 2).max(axis=2)
        E = (N // 64) * (K // 128)
        expect = -(-(256 + 16 * E) // 256) * 256 + 8192 * (nq - ns) + 4096 * ns + 1024 * int(cells.sum())
        assert oracle.packed_bytes_q64(N, K, qmap) == expect
        assert oracle.pack_q64("f16", w, qmap, mk).size == expect


def test_pack_q64_tile_constant_map_has_the_128_tile_data_bytes():
    """A quadrant map constant on every 128 x 128 tile stores the same data
    bytes as the 128 x 128 format (pieces of both-dense and both-2:4 cells
    are the 128 x 128 format's pieces, in the same order)."""
    N, K = 256, 512
    rng = np.random.default_rng(43)
    tmap = (rng.random((N // 128, K // 128)) < 0.5).astype(np.uint8)
    qmap = np.kron(tmap, np.ones((2, 2), np.uint8))
    _, w, mk = _quad_problem(N, K, 0.5, seed=44)
    b3 = oracle.pack("bf16", w, tmap, mk)
    b4 = oracle.pack_q64("bf16", w, qmap, mk)
    d3 = int.from_bytes(b3[48:56].tobytes(), "little")
    d4 = int.from_bytes(b4[48:56].tobytes(), "little")
    assert np.array_equal(b3[d3:], b4[d4:])


def test_pack_q64_rejects_bad_input():
    N, K = 128, 256
    qmap, w, mk = _quad_problem(N, K, 1.0, seed=45)
    bad = qmap.copy()
    bad[0, 0] = 2  # 4:8 is not a quadrant kind
    with pytest.raises(oracle.OracleError) as ei:
        oracle.pack_q64("bf16", w, bad, mk)
    assert ei.value.code == 1
    mk2 = mk.copy()
    mk2[3, 64:68] = [1, 1, 1, 0]  # three kept in a 2:4 quadrant
    with pytest.raises(oracle.OracleError) as ei:
        oracle.pack_q64("bf16", w, qmap, mk2)
    assert ei.value.code == 3
    with pytest.raises(oracle.OracleError):
        oracle.pack_q64("bf16", w[:, :192], qmap[:, :3], mk[:, :192])  # K not a multiple of 128


def test_gemm_q64_brute_force_tiny():
    """The product with a 64 x 64 tile map, against sums written out over
    the kept weights (fp64, exact for these small integers)."""
    N, K, M = 128, 128, 3
    rng = np.random.default_rng(46)
    qmap = np.array([[1, 0], [0, 1]], np.uint8)
    _, _, mk = _quad_problem(N, K, 0.5, seed=47)
    wv = rng.integers(-4, 5, (N, K)).astype(np.float32)
    xv = rng.integers(-4, 5, (M, K)).astype(np.float32)
    w = (wv.view(np.uint32) >> 16).astype(np.uint16)
    x = (xv.view(np.uint32) >> 16).astype(np.uint16)
    Y = oracle.gemm_f64("bf16", x, w, qmap, mk, tile_n=64, tile_k=64)
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                sparse = qmap[n // 64, k // 64] == 1
                if not sparse or mk[n, k]:
                    s += float(xv[m, k]) * float(wv[n, k])
            assert Y[m, n] == s


# ------------------------------------------------------------------ gated MLP product (SiLU)
def test_silu_closed_forms():
    """SiLU(x) = x / (1 + e^-x): zero at zero; SiLU(ln 3) = (3/4) ln 3
    exactly in the reals; its odd part is x / 2, i.e. SiLU(x) - SiLU(-x) = x
    (a wrong sign in the exponent or a dropped factor breaks this); it
    tends to x for large x and to 0 for very negative x."""
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    for x in np.linspace(-30.0, 30.0, 121):
        assert oracle.silu(x) - oracle.silu(-x) == pytest.approx(x, rel=1e-13, abs=1e-13)
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(oracle.silu(-40.0)) < 1e-15
    # sigmoid(1) = e / (1 + e)
    assert oracle.silu(1.0) == pytest.approx(math.e / (1.0 + math.e), rel=1e-15)


def test_swiglu_brute_force_tiny():
    """8 x 8 gate and up weights with 4 x 4 tiles, different tile maps and
    2:4 patterns for the two, integer X and W: H = SiLU(yg) * yu with yg, yu
    summed by hand over the kept positions and SiLU from math.exp."""
    rng = np.random.default_rng(31)
    M, F, K = 5, 8, 8
    Xi = rng.integers(-3, 4, (M, K))
    Gi = rng.integers(-3, 4, (F, K))
    Ui = rng.integers(-3, 4, (F, K))
    maps = [np.array([[1, 0], [0, 1]], np.uint8), np.array([[0, 1], [1, 1]], np.uint8)]
    pats = [rng.integers(0, 6, (F, K // 4)) for _ in range(2)]
    masks = []
    for pt in pats:
        mk = np.zeros((F, K), np.uint8)
        for n in range(F):
            for g in range(K // 4):
                for d in inputs.PATTERNS[pt[n, g]]:
                    mk[n, 4 * g + d] = 1
        masks.append(mk)
    H = oracle.swiglu_f64("bf16", _int_bits(Xi, "bf16"), _int_bits(Gi, "bf16"), _int_bits(Ui, "bf16"), maps[0],
                          maps[1], masks[0], masks[1], tile_n=4, tile_k=4)

    def y(Wi, tmap, mk, m, n):
        return sum(Xi[m, k] * Wi[n, k] for k in range(K) if (not tmap[n // 4, k // 4]) or mk[n, k])

    for m in range(M):
        for n in range(F):
            g, u = y(Gi, maps[0], masks[0], m, n), y(Ui, maps[1], masks[1], m, n)
            ref = g / (1.0 + math.exp(-g)) * u
            assert H[m, n] == pytest.approx(ref, rel=1e-13, abs=1e-13), (m, n)


def test_swiglu_identity_x_is_silu_of_gate_weights_times_up_weights():
    """X = identity rows: H^T = SiLU(Wg o Eg) * (Wu o Eu) elementwise, with
    SiLU evaluated by numpy; swapping the roles of gate and up changes it."""
    pg = _problem(256, 256, "bernoulli", 0.5, seed=12)
    pu = _problem(256, 256, "bernoulli", 0.5, seed=13)
    X = inputs.to_bits(np.eye(256), "bf16")
    H = oracle.swiglu_f64("bf16", X, pg.w, pu.w, pg.tile_map, pu.tile_map, pg.mask, pu.mask)
    G = inputs.bits_to_f32(pg.w, "bf16").astype(np.float64) * oracle.effective_mask(256, 256, pg.tile_map, pg.mask)
    U = inputs.bits_to_f32(pu.w, "bf16").astype(np.float64) * oracle.effective_mask(256, 256, pu.tile_map, pu.mask)
    ref = G / (1.0 + np.exp(-G)) * U
    np.testing.assert_allclose(H.T, ref, rtol=1e-14, atol=1e-18)
    Hs = oracle.swiglu_f64("bf16", X, pu.w, pg.w, pu.tile_map, pg.tile_map, pu.mask, pg.mask)
    assert not np.allclose(Hs, H)


def test_interleave_gate_up_rows():
    """Blocks of rows alternate gate, up, gate, up, ... and nothing else moves."""
    g = np.arange(6 * 3).reshape(6, 3)
    u = 100 + np.arange(6 * 3).reshape(6, 3)
    out = oracle.interleave_gate_up(g, u, 2)
    assert out.shape == (12, 3)
    for i in range(3):
        assert np.array_equal(out[4 * i:4 * i + 2], g[2 * i:2 * i + 2])
        assert np.array_equal(out[4 * i + 2:4 * i + 4], u[2 * i:2 * i + 2])
    tm = oracle.interleave_gate_up(np.array([[1, 0]], np.uint8), np.array([[0, 1]], np.uint8), 1)
    assert np.array_equal(tm, np.array([[1, 0], [0, 1]], np.uint8))


# ---------------------------------------------------------------- hybrid-mask sampler (Gumbel-Softmax forward)
# gist.science explainer, section 2 "Methodology: PATCH", "Learnable
# Distributions": tile selection (dense vs 2:4) and pattern selection (one of
# six) are learnable distributions sampled with Gumbel-Softmax.
def test_gumbel_transform_is_the_gumbel_inverse_cdf():
    """g(u) = -ln(-ln u) is the standard Gumbel quantile function: it matches
    scipy.stats.gumbel_r.ppf (library routine) and inverts the textbook CDF
    F(g) = exp(-exp(-g)); g(1/e) = 0 and g(exp(-exp(-2))) = 2."""
    from scipy import stats

    us = np.concatenate([np.linspace(1e-6, 1 - 1e-6, 97), [2.0 ** -24, 0.5, 1 - 2.0 ** -24]])
    got = np.array([oracle.gumbel(u) for u in us])
    np.testing.assert_allclose(got, stats.gumbel_r.ppf(us), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.exp(-np.exp(-got)), us, rtol=1e-12)
    assert abs(oracle.gumbel(math.exp(-1.0))) < 1e-15
    assert abs(oracle.gumbel(math.exp(-math.exp(-2.0))) - 2.0) < 1e-14


@pytest.mark.parametrize("tau", [0.1, 0.5, 1.0, 2.0])
def test_gumbel_softmax_is_softmax_of_perturbed_logits(tau):
    """The soft sample equals scipy.special.softmax((l + g) / tau) with g the
    library's Gumbel quantiles of the same uniforms (library routines), and
    with u = 1/e (g = 0 up to float32 rounding of u) it is softmax(l / tau)."""
    from scipy import special, stats

    rng = np.random.default_rng(5)
    for n in (2, 6):
        l = rng.standard_normal(n).astype(np.float32)
        u = inputs.gen_uniform_open(rng, n)
        y, best = oracle.gumbel_softmax(l, u, tau)
        g = stats.gumbel_r.ppf(u.astype(np.float64))
        np.testing.assert_allclose(y, special.softmax((l.astype(np.float64) + g) / tau), rtol=1e-12, atol=1e-15)
        assert best == int(np.argmax(l.astype(np.float64) + g))
        y0, _ = oracle.gumbel_softmax(l, np.full(n, math.exp(-1.0), np.float32), tau)
        np.testing.assert_allclose(y0, special.softmax(l.astype(np.float64) / tau), rtol=2e-6, atol=1e-9)


def test_gumbel_max_frequencies_follow_softmax():
    """Gumbel-max trick: the hard sample argmax(l + g) is distributed as
    softmax(l).  Over ~303k groups with one set of six pattern logits and
    ~76k tiles of 4 x 4 with one pair of tile logits, each class frequency is
    within 5 binomial standard deviations of softmax(l) -- a wrong sign or
    form of the Gumbel transform moves them by far more."""
    from scipy import special

    N, K, tn, tk = 128, 9472, 4, 4
    G = K // 4
    rng = np.random.default_rng(7)
    lp = np.array([0.3, -1.0, 2.0, 0.5, 0.0, -0.2], dtype=np.float32)
    lt = np.array([0.7, -0.4], dtype=np.float32)
    pl = np.broadcast_to(lp, (N, G, 6))
    tl = np.broadcast_to(lt, (N // tn, K // tk, 2))
    tmap, mask, _ = oracle.sample_mask(tl, inputs.gen_uniform_open(rng, tl.shape), pl,
                                       inputs.gen_uniform_open(rng, pl.shape), 1.0, tn, tk, soft=False)
    groups = mask.reshape(N, G, 4)
    counts = np.zeros(6)
    for p, (a, b) in enumerate(oracle.PATTERN_PAIRS):
        counts[p] = np.count_nonzero(groups[:, :, a] & groups[:, :, b])
    assert counts.sum() == N * G
    for freq, prob, n in ((counts / (N * G), special.softmax(lp.astype(np.float64)), N * G),
                          (np.bincount(tmap.ravel(), minlength=2) / tmap.size,
                           special.softmax(lt.astype(np.float64)), tmap.size)):
        sd = np.sqrt(prob * (1 - prob) / n)
        assert np.all(np.abs(freq - prob) < 5 * sd), (freq, prob)


def test_soft_mask_invariants_and_hard_mask_validity():
    """Soft mask: values in [0, 1]; in a group the four values sum to
    4 y_dense + 2 y_sparse = 2 + 2 y_dense, so the sum is the same in every
    group of a tile; no value is below y_dense.  Hard outputs: every group keeps
    exactly two positions, so the sampled map and mask pass the pack's
    validation and have sparsity 0.5 x (fraction of 2:4 tiles)."""
    N, K = 256, 384
    s = inputs.make_sampler_inputs(N, K, 3)
    tmap, mask, soft = oracle.sample_mask(s.tile_logits, s.tile_u, s.pat_logits, s.pat_u, 0.7)
    assert soft.min() >= 0.0 and soft.max() <= 1.0 + 1e-15
    sums = soft.reshape(N, K // 4, 4).sum(axis=2)
    for i in range(N // 128):
        for j in range(K // 128):
            blk = sums[128 * i:128 * (i + 1), 32 * j:32 * (j + 1)]
            y_dense = blk.mean() / 2 - 1
            np.testing.assert_allclose(blk, blk.mean(), rtol=0, atol=1e-12)
            assert soft[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)].min() >= y_dense - 1e-12
    assert np.all(mask.reshape(N, K // 4, 4).sum(axis=2) == 2)
    oracle.validate(N, K, tmap, mask)
    E = oracle.effective_mask(N, K, tmap, mask)
    assert (E == 0).sum() * tmap.size * 2 == N * K * int(tmap.sum())


@pytest.mark.parametrize("p", range(6))
def test_degenerate_distributions_give_the_pure_options(p):
    """A tile whose dense logit dominates has soft mask 1 and map byte 0; one
    whose sparse logit and pattern-p logit dominate has map byte 1 and soft
    mask = hard mask = the indicator of pattern p's pair (lexicographic order
    of the six pairs)."""
    N, K = 128, 256
    rng = np.random.default_rng(11 + p)
    tl = np.zeros((1, 2, 2), np.float32)
    tl[0, 0] = (60.0, 0.0)
    tl[0, 1] = (0.0, 60.0)
    pl = np.zeros((N, K // 4, 6), np.float32)
    pl[:, :, p] = 60.0
    tmap, mask, soft = oracle.sample_mask(tl, inputs.gen_uniform_open(rng, tl.shape), pl,
                                          inputs.gen_uniform_open(rng, pl.shape), 1.0)
    assert tmap.tolist() == [[0, 1]]
    pair = np.zeros(4)
    pair[list(oracle.PATTERN_PAIRS[p])] = 1
    assert oracle.PATTERN_PAIRS[p] == tuple(int(v) for v in inputs.PATTERNS[p])
    np.testing.assert_allclose(soft[:, :128], 1.0, atol=1e-12)
    np.testing.assert_allclose(soft[:, 128:], np.tile(pair, (N, 32)), atol=1e-12)
    assert np.array_equal(mask, np.tile(pair, (N, K // 4)).astype(np.uint8))


def test_temperature_limits():
    """tau -> 0: the soft sample tends to the one-hot hard sample; tau -> inf:
    to the uniform distribution."""
    rng = np.random.default_rng(13)
    for n in (2, 6):
        for _ in range(20):
            l = rng.standard_normal(n).astype(np.float32)
            u = inputs.gen_uniform_open(rng, n)
            y, best = oracle.gumbel_softmax(l, u, 1e-4)
            scores = np.sort(l.astype(np.float64) + np.array([oracle.gumbel(v) for v in u]))
            if scores[-1] - scores[-2] > 0.01:
                assert y[best] > 1 - 1e-12
            y, _ = oracle.gumbel_softmax(l, u, 1e7)
            np.testing.assert_allclose(y, 1.0 / n, atol=1e-5)


# ---------------------------------------------------------------- mask tiles finer than execution tiles
# gist.science explainer, section 4 "Ablation Studies", "Tile Size": the mask
# can be learnt on tiles as fine as 4 x 4 while the hardware executes
# 128 x 128 tiles.
@pytest.mark.parametrize("en,ek", [(8, 8), (8, 4), (4, 8)])
def test_exec_map_brute_force(en, ek):
    """8 x 8 weight, 4 x 4 fine tiles, every one of the 16 fine maps: an
    execution tile is 2:4 exactly when all fine tiles inside it are."""
    for bits in range(16):
        fm = np.array([(bits >> i) & 1 for i in range(4)], dtype=np.uint8).reshape(2, 2)
        got = oracle.exec_map(8, 8, fm, 4, 4, en, ek)
        for i in range(8 // en):
            for j in range(8 // ek):
                sub = [fm[a, b] for a in range(2) for b in range(2)
                       if i * en <= 4 * a < (i + 1) * en and j * ek <= 4 * b < (j + 1) * ek]
                assert got[i, j] == int(all(sub)), (bits, i, j)


def test_exec_map_identity_and_monotone():
    """Fine tiles of the execution size map to themselves; coarser execution
    tiles never hold more 2:4 tiles' worth of area than the fine map."""
    rng = np.random.default_rng(3)
    fm = inputs.gen_fine_map(rng, 384, 512, 128, 128, 0.3, 0.5)
    assert np.array_equal(oracle.exec_map(384, 512, fm, 128, 128), fm)
    for b1, b2 in ((4, 4), (32, 16), (64, 128)):
        fm = inputs.gen_fine_map(rng, 384, 512, b1, b2, 0.3, 0.7)
        em = oracle.exec_map(384, 512, fm, b1, b2)
        assert em.sum() * 128 * 128 <= fm.sum() * b1 * b2


def test_apply_fine_mask_bits():
    """Kept weights keep their bits (-0 included); pruned ones become +0;
    dense fine tiles are untouched."""
    p = inputs.make_fine("bf16", 256, 256, 16, 32, 4)
    p.w[0, :8] = 0x8000  # -0
    p.tile_map[0, 0] = 1
    out = oracle.apply_fine_mask(p.w, p.tile_map, p.mask, 16, 32)
    E = oracle.effective_mask(256, 256, p.tile_map, p.mask, 16, 32)
    assert np.array_equal(out[E == 1], p.w[E == 1])
    assert np.all(out[E == 0] == 0)
    dense = np.repeat(np.repeat(p.tile_map == 0, 16, axis=0), 32, axis=1)
    assert np.array_equal(out[dense], p.w[dense])


@pytest.mark.parametrize("b1,b2", [(4, 4), (16, 16), (32, 64), (128, 128)])
def test_fine_policy_preserves_the_product(b1, b2):
    """Executing on 128 x 128 tiles with the policy's map and the masked
    weight gives exactly the fine-tiled product X (W o E_fine)^T (binary64,
    same terms in the same order)."""
    N, K, M = 256, 384, 9
    p = inputs.make_fine("f16", N, K, b1, b2, 5)
    X = inputs.make_custom_x("f16", M, K, 6)
    em = oracle.exec_map(N, K, p.tile_map, b1, b2)
    W2 = oracle.apply_fine_mask(p.w, p.tile_map, p.mask, b1, b2)
    fine = oracle.gemm_f64("f16", X, p.w, p.tile_map, p.mask, tile_n=b1, tile_k=b2)
    execd = oracle.gemm_f64("f16", X, W2, em, p.mask)
    assert np.array_equal(fine, execd)
    assert 0 < em.sum() < em.size  # both execution kinds occur
    if (b1, b2) != (128, 128):
        # some dense execution tiles hold pruned (2:4) fine tiles
        assert (p.tile_map.sum() * b1 * b2) > em.sum() * 128 * 128



# ---------------------------------------------------------------- 4:8 tiles (another N:M pattern)
# gist.science explainer, section 5 "Significance", "Future Direction": the
# framework is pattern-agnostic and extends to other N:M patterns, e.g. 4:8.
def test_pack_48_hand_worked_example():
    g = _golden("pack_48_example.txt")
    N = K = 128
    W = np.full((N, K), 0x3F80, np.uint16)
    W[g["value.row"], g["value.col"]] = g["value.bits"]
    mask = np.zeros((N, K), np.uint8)
    for p in range(4):
        mask[:, p::8] = 1
    mask[37, 72:80] = [0, 1, 0, 0, 1, 1, 0, 1]
    blob = oracle.pack("bf16", W, np.array([[2]], np.uint8), mask)
    u64 = lambda o: int.from_bytes(blob[o:o + 8].tobytes(), "little")
    u32 = lambda o: int.from_bytes(blob[o:o + 4].tobytes(), "little")
    u16 = lambda o: int.from_bytes(blob[o:o + 2].tobytes(), "little")
    assert blob.size == g["header.total_bytes"] and u64(64) == g["header.total_bytes"]
    assert u32(36) == g["header.n_sparse"] and u32(72) == g["header.n_48"]
    assert (u64(256), u32(264), u32(268)) == (g["table.0.offset"], g["table.0.kind"], g["table.0.stride"])
    assert u16(g["value.byte_offset"]) == g["value.bits"]
    assert u16(g["value0.byte_offset"]) == g["value0.bits"]
    assert blob[g["mask.byte_offset"]] == g["mask.value"]
    assert blob[g["mask0.byte_offset"]] == g["mask0.value"]


@pytest.mark.parametrize("mask_kind", ["top", "uniform"])
def test_pack_mixed_kinds_round_trip(mask_kind):
    """Dense, 2:4 and 4:8 tiles in one blob: unpack(pack(W)) == W o E
    bit-exactly; every 4:8 mask byte keeps exactly four positions; sizes as
    the closed form (a 4:8 tile takes as many bytes as a 2:4 one)."""
    p = inputs.make_mixed("bf16", 384, 640, 14, 0.35, 0.35, mask_kind)
    assert set(np.unique(p.tile_map)) == {0, 1, 2}
    blob = oracle.pack("bf16", p.w, p.tile_map, p.mask)
    T, ns = p.tile_map.size, int((p.tile_map != 0).sum())
    assert blob.size == -(-(256 + 16 * T) // 256) * 256 + 32768 * (T - ns) + 18432 * ns
    W2, _ = _unpack(blob, p.N, p.K)
    E = oracle.effective_mask(p.N, p.K, p.tile_map, p.mask)
    assert np.array_equal(W2, np.where(E != 0, p.w, 0).astype(np.uint16))
    tiles48 = np.repeat(np.repeat(p.tile_map == 2, 128, 0), 128, 1)
    assert np.all(p.mask[tiles48].reshape(-1, 8).sum(axis=1) == 4)
    # sparsity: half of every 2:4 and 4:8 tile
    assert (E == 0).sum() * 2 == ns * 128 * 128


def test_validate_48_groups():
    """A 4:8 tile's group keeping 3 or 5 of 8 is an error; map bytes other
    than 0, 1, 2 are rejected; a 4:8 group need not be 2:4 within it."""
    N = K = 128
    W = np.zeros((N, K), np.uint16)
    mask = np.zeros((N, K), np.uint8)
    mask[:, 0:4] = 1  # positions 0..3 of the first group: 4 of 8, not 2 of 4 in each half
    for p in range(4):
        mask[:, p::8] = 1
    assert oracle.validate(N, K, np.array([[2]], np.uint8), mask) is None
    assert oracle.validate(N, K, np.array([[1]], np.uint8), mask) == (0, 0)  # as 2:4: 4 of 4 kept
    for bad in (3, 5):
        m = mask.copy()
        m[9, 16:24] = 0
        m[9, 16:16 + bad] = 1
        assert oracle.validate(N, K, np.array([[2]], np.uint8), m) == (9, 2)
    with pytest.raises(oracle.OracleError) as e:
        oracle.validate(N, K, np.array([[3]], np.uint8), mask)
    assert e.value.code == 1


def test_gemm_48_brute_force_tiny():
    """16 x 16 weight with 8 x 8 tiles of all kinds, small integers: the GEMM
    equals a second formulation that sums only the kept positions of each
    group (exact in binary64)."""
    rng = np.random.default_rng(21)
    N = K = 16
    M = 5
    for tmap in (np.array([[2, 0], [1, 2]], np.uint8), np.array([[2, 2], [2, 2]], np.uint8)):
        Wv = rng.integers(-3, 4, (N, K)).astype(np.float64)
        Xv = rng.integers(-3, 4, (M, K)).astype(np.float64)
        W, X = inputs.to_bits(Wv, "f16"), inputs.to_bits(Xv, "f16")
        mask = np.zeros((N, K), np.uint8)
        for n in range(N):
            for g in range(K // 8):
                mask[n, 8 * g + rng.permutation(8)[:4]] = 1
            for g in range(K // 4):
                blk = mask[n, 4 * g:4 * g + 4]
                if tmap[n // 8, (4 * g) // 8] == 1:
                    blk[:] = 0
                    blk[rng.permutation(4)[:2]] = 1
        Y = oracle.gemm_f64("f16", X, W, tmap, mask, tile_n=8, tile_k=8)
        ref = np.zeros((M, N))
        for m in range(M):
            for n in range(N):
                for k in range(K):
                    kind = tmap[n // 8, k // 8]
                    if kind == 0 or mask[n, k]:
                        ref[m, n] += Xv[m, k] * Wv[n, k]
        assert np.array_equal(Y, ref)
