"""Seeded synthetic inputs for the hybrid tile-sparse GEMM.

This module only draws data: activations X, weights W, tile maps and 2:4
masks.  It holds none of the method's arithmetic (no masking, no packing, no
products) and imports neither the oracle nor the HIP binding, so both sides
of every parity test can take their inputs from here.

Shapes and distributions stand in for LLaMA-2-7B / 13B linear layers (the
pages measure on LLaMA-2 7B, gist.science explainer, section 4
"Experimental Results"); no weights or datasets are used.

* X ~ N(0, 1) and W ~ N(0, 0.02) are drawn in float64 with numpy's PCG64,
  rounded to float32, then to the 16-bit type with round-to-nearest-even
  (numpy for binary16, torch's CPU cast for bfloat16).
* Tile maps (a byte per 128 x 128 tile, nonzero = 2:4 sparse):
  ``bernoulli`` -- each tile sparse with probability s;
  ``exact``     -- exactly round_half_even(s * T) sparse tiles chosen
                   uniformly without replacement;
  ``rowcluster``-- the first half of the row blocks dense, the rest sparse.
* Masks (a byte per weight, nonzero = keep), drawn for every group of four
  consecutive weights along K, also inside dense tiles (where the method
  ignores them):
  ``top2``    -- keep the two largest |w| of the stored 16-bit values, ties
                 broken toward the lower column;
  ``uniform`` -- one of the six 2:4 patterns uniformly at random, patterns
                 numbered in lexicographic order (0,1) (0,2) (0,3) (1,2)
                 (1,3) (2,3).
* Every stream is seeded from ``numpy.random.SeedSequence(seed,
  spawn_key=(config, matrix, s_index, role))``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Sequence, Tuple

import numpy as np

TILE = 128

ROLE_X, ROLE_W, ROLE_MAP, ROLE_MASK = 0, 1, 2, 3

# the six 2:4 patterns, lexicographic
PATTERNS = np.array([(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)], dtype=np.int64)


def rng_for(seed: int, config: int, matrix: int, s_index: int, role: int) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(config, matrix, s_index, role))
    return np.random.Generator(np.random.PCG64(ss))


def to_bits(a64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> float32 -> 16-bit (RNE); returns the uint16 bit patterns."""
    a32 = np.asarray(a64, dtype=np.float32)
    if dtype == "f16":
        return a32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(np.ascontiguousarray(a32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"unknown dtype {dtype}")


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit patterns -> float32 (exact widening)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(f"unknown dtype {dtype}")


def gen_x(rng: np.random.Generator, M: int, K: int, dtype: str) -> np.ndarray:
    return to_bits(rng.standard_normal((M, K)), dtype)


def gen_w(rng: np.random.Generator, N: int, K: int, dtype: str, std: float = 0.02) -> np.ndarray:
    return to_bits(rng.standard_normal((N, K)) * std, dtype)


def round_half_even(x: float) -> int:
    return int(np.round(x))  # numpy rounds halves to even


def gen_tile_map(rng: np.random.Generator, NT: int, KT: int, kind: str, s: float) -> np.ndarray:
    T = NT * KT
    if kind == "bernoulli":
        return (rng.random(T) < s).astype(np.uint8).reshape(NT, KT)
    if kind == "exact":
        n_sparse = round_half_even(s * T)
        m = np.zeros(T, dtype=np.uint8)
        m[rng.permutation(T)[:n_sparse]] = 1
        return m.reshape(NT, KT)
    if kind == "rowcluster":
        m = np.zeros((NT, KT), dtype=np.uint8)
        m[NT // 2:, :] = 1
        return m
    if kind == "dense":
        return np.zeros((NT, KT), dtype=np.uint8)
    if kind == "sparse":
        return np.ones((NT, KT), dtype=np.uint8)
    raise ValueError(f"unknown tile-map kind {kind}")


def gen_mask_top2(w_bits: np.ndarray, dtype: str) -> np.ndarray:
    """Keep the two largest |w| of each group of four along K (stored values),
    ties toward the lower column."""
    N, K = w_bits.shape
    a = np.abs(bits_to_f32(w_bits, dtype)).reshape(N, K // 4, 4)
    order = np.argsort(-a, axis=-1, kind="stable")  # stable: equal keys keep column order
    keep = order[..., :2]
    mask = np.zeros((N, K // 4, 4), dtype=np.uint8)
    np.put_along_axis(mask, keep, 1, axis=-1)
    return mask.reshape(N, K)


def gen_mask_uniform(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    pat = rng.integers(0, 6, size=(N, K // 4))
    mask = np.zeros((N, K // 4, 4), dtype=np.uint8)
    pos = PATTERNS[pat]  # (N, K/4, 2)
    np.put_along_axis(mask, pos, 1, axis=-1)
    return mask.reshape(N, K)


@dataclasses.dataclass(frozen=True)
class Matrix:
    name: str
    N: int
    K: int


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    dtype: str
    matrices: Tuple[Matrix, ...]
    Ms: Tuple[int, ...]
    map_kind: str
    fractions: Tuple[float, ...]
    mask_kind: str


LLAMA7B = (
    Matrix("q_proj", 4096, 4096),
    Matrix("k_proj", 4096, 4096),
    Matrix("v_proj", 4096, 4096),
    Matrix("o_proj", 4096, 4096),
    Matrix("gate_proj", 11008, 4096),
    Matrix("up_proj", 11008, 4096),
    Matrix("down_proj", 4096, 11008),
)

CONFIGS: Dict[str, Config] = {
    "tiny": Config(0, "tiny", "f16", (Matrix("w", 256, 256),), (16,), "bernoulli", (0.5,), "top2"),
    "decode": Config(1, "decode", "bf16", (Matrix("q_proj", 4096, 4096),), (1, 4, 16), "exact", (0.5,), "top2"),
    "prefill_mlp": Config(
        2, "prefill_mlp", "bf16", (Matrix("gate_up_proj", 11008, 4096), Matrix("down_proj", 4096, 11008)), (2048,),
        "exact", (0.8,), "top2"),
    "sweep": Config(3, "sweep", "bf16", LLAMA7B, (1, 16, 128, 2048), "exact", (0.0, 0.25, 0.5, 0.75, 1.0), "top2"),
    "imbalanced_13b": Config(
        4, "imbalanced_13b", "bf16", (Matrix("attn_5120", 5120, 5120), Matrix("mlp_13824", 13824, 5120)), (4096,),
        "rowcluster", (0.5,), "uniform"),
}


@dataclasses.dataclass
class Problem:
    """One weight matrix with its tile map and mask, plus activations."""
    dtype: str
    N: int
    K: int
    w: np.ndarray          # uint16 (N, K)
    tile_map: np.ndarray   # uint8 (NT, KT)
    mask: np.ndarray       # uint8 (N, K)
    seeds: dict


def make_weights(cfg: Config, matrix_index: int, s_index: int, seed: int = 0,
                 map_kind: str | None = None, fraction: float | None = None, reuse: Problem | None = None) -> Problem:
    """reuse: a Problem made by this function for the same config, matrix and
    seed; its weights and mask (which do not depend on s_index) are taken
    as they are instead of being drawn again."""
    mat = cfg.matrices[matrix_index]
    N, K = mat.N, mat.K
    frac = cfg.fractions[s_index] if fraction is None else fraction
    kind = cfg.map_kind if map_kind is None else map_kind
    tmap = gen_tile_map(rng_for(seed, cfg.cid, matrix_index, s_index, ROLE_MAP), N // TILE, K // TILE, kind, frac)
    if reuse is not None:
        sd = reuse.seeds
        if (sd.get("config"), sd.get("matrix"), sd.get("seed")) != (cfg.cid, matrix_index, seed):
            raise ValueError("reuse must come from the same config, matrix and seed")
        w, mask = reuse.w, reuse.mask
    else:
        w = gen_w(rng_for(seed, cfg.cid, matrix_index, 0, ROLE_W), N, K, cfg.dtype)
        if cfg.mask_kind == "top2":
            mask = gen_mask_top2(w, cfg.dtype)
        else:
            mask = gen_mask_uniform(rng_for(seed, cfg.cid, matrix_index, 0, ROLE_MASK), N, K)
    return Problem(cfg.dtype, N, K, w, tmap, mask,
                   dict(seed=seed, config=cfg.cid, matrix=matrix_index, s_index=s_index, map_kind=kind,
                        fraction=frac))


def make_x(cfg: Config, M: int, K: int, seed: int = 0, matrix_index: int = 0) -> np.ndarray:
    return gen_x(rng_for(seed, cfg.cid, matrix_index, M, ROLE_X), M, K, cfg.dtype)


def make_custom(dtype: str, N: int, K: int, seed: int, map_kind: str, fraction: float, mask_kind: str,
                key: int = 99) -> Problem:
    """Inputs for shapes outside the named configs (edge cases in tests)."""
    w = gen_w(rng_for(seed, key, N, K, ROLE_W), N, K, dtype)
    tmap = gen_tile_map(rng_for(seed, key, N, K, ROLE_MAP), N // TILE, K // TILE, map_kind, fraction)
    if mask_kind == "top2":
        mask = gen_mask_top2(w, dtype)
    else:
        mask = gen_mask_uniform(rng_for(seed, key, N, K, ROLE_MASK), N, K)
    return Problem(dtype, N, K, w, tmap, mask, dict(seed=seed, key=key, map_kind=map_kind, fraction=fraction))


def make_custom_x(dtype: str, M: int, K: int, seed: int, key: int = 99) -> np.ndarray:
    return gen_x(rng_for(seed, key, M, K, ROLE_X), M, K, dtype)


# ---------------------------------------------------------------------------- sampler inputs
ROLE_SAMPLER = 7


def gen_uniform_open(rng: np.random.Generator, shape) -> np.ndarray:
    """float32 uniforms in the open interval (0, 1): k / 2^24, k in [1, 2^24)
    (every value exactly representable, never 0 or 1)."""
    return (rng.integers(1, 1 << 24, size=shape, dtype=np.int64).astype(np.float64) / float(1 << 24)).astype(
        np.float32)


@dataclasses.dataclass
class SamplerInputs:
    """Logits and uniforms of the forward hybrid-mask sampler for an N x K
    weight: tile logits / uniforms [N/tn, K/tk, 2] (class 0 dense, 1 sparse),
    pattern logits / uniforms [N, K/4, 6]; float32."""
    tile_logits: np.ndarray
    tile_u: np.ndarray
    pat_logits: np.ndarray
    pat_u: np.ndarray


def make_sampler_inputs(N: int, K: int, seed: int, tile_n: int = 128, tile_k: int = 128, sparse_bias: float = 0.0,
                        pattern_scale: float = 1.0) -> SamplerInputs:
    """Synthetic learnable distributions: logits ~ N(0, 1) (the sparse class
    shifted by sparse_bias; pattern logits scaled by pattern_scale), and the
    sampler's uniforms."""
    rng = rng_for(seed, 40, N, K, ROLE_SAMPLER)
    NT, KT, G = N // tile_n, K // tile_k, K // 4
    tl = rng.standard_normal((NT, KT, 2))
    tl[:, :, 1] += sparse_bias
    pl = pattern_scale * rng.standard_normal((N, G, 6))
    return SamplerInputs(tl.astype(np.float32), gen_uniform_open(rng, (NT, KT, 2)), pl.astype(np.float32),
                         gen_uniform_open(rng, (N, G, 6)))


# ---------------------------------------------------------------------------- fine mask tiles
ROLE_FINE = 8


def gen_fine_map(rng: np.random.Generator, N: int, K: int, b1: int, b2: int, s_exec: float,
                 p_sub: float) -> np.ndarray:
    """Fine tile map (N/b1 x K/b2) of mask tiles b1 x b2: each 128 x 128
    execution tile is, with probability s_exec, 2:4 in every fine tile, else
    each of its fine tiles is 2:4 with probability p_sub."""
    NT, KT = N // TILE, K // TILE
    fn, fk = TILE // b1, TILE // b2
    whole = rng.random((NT, KT)) < s_exec
    sub = rng.random((NT, fn, KT, fk)) < p_sub
    sub |= whole[:, None, :, None]
    return sub.reshape(N // b1, K // b2).astype(np.uint8)


def make_fine(dtype: str, N: int, K: int, b1: int, b2: int, seed: int, s_exec: float = 0.4,
              p_sub: float = 0.6) -> Problem:
    """Weights with a fine tile map (tile_map holds the N/b1 x K/b2 fine map)
    and a mask with one of the six patterns in every group (read only inside
    2:4 fine tiles)."""
    rng = rng_for(seed, 41, N, K, ROLE_FINE)
    w = gen_w(rng, N, K, dtype)
    fmap = gen_fine_map(rng, N, K, b1, b2, s_exec, p_sub)
    return Problem(dtype, N, K, w, fmap, gen_mask_uniform(rng, N, K), {"seed": seed, "b1": b1, "b2": b2})


# ---------------------------------------------------------------------------- 4:8 tiles
ROLE_48 = 9
KIND_DENSE, KIND_24, KIND_48 = 0, 1, 2


def gen_mask_top4of8(w_bits: np.ndarray, dtype: str) -> np.ndarray:
    """Keep the four largest |w| of each group of eight along K (stored
    values), ties toward the lower column."""
    N, K = w_bits.shape
    a = np.abs(bits_to_f32(w_bits, dtype)).reshape(N, K // 8, 8)
    order = np.argsort(-a, axis=-1, kind="stable")
    mask = np.zeros((N, K // 8, 8), dtype=np.uint8)
    np.put_along_axis(mask, order[..., :4], 1, axis=-1)
    return mask.reshape(N, K)


def gen_mask_uniform48(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """One of the 70 patterns of four kept in eight per group, uniformly."""
    keys = rng.random((N, K // 8, 8))
    order = np.argsort(keys, axis=-1)
    mask = np.zeros((N, K // 8, 8), dtype=np.uint8)
    np.put_along_axis(mask, order[..., :4], 1, axis=-1)
    return mask.reshape(N, K)


def make_mixed(dtype: str, N: int, K: int, seed: int, frac24: float, frac48: float, mask_kind: str = "top") -> Problem:
    """Tiles of all three kinds: each 128 x 128 tile 2:4 with probability
    frac24, 4:8 with probability frac48, else dense; the mask keeps the top-2
    of 4 (2:4 tiles) / top-4 of 8 (4:8 tiles) by |w|, or (mask_kind
    "uniform") a uniformly drawn pattern."""
    rng = rng_for(seed, 42, N, K, ROLE_48)
    w = gen_w(rng, N, K, dtype)
    NT, KT = N // TILE, K // TILE
    u = rng.random((NT, KT))
    tmap = np.where(u < frac24, KIND_24, np.where(u < frac24 + frac48, KIND_48, KIND_DENSE)).astype(np.uint8)
    if mask_kind == "top":
        m24, m48 = gen_mask_top2(w, dtype), gen_mask_top4of8(w, dtype)
    else:
        m24, m48 = gen_mask_uniform(rng, N, K), gen_mask_uniform48(rng, N, K)
    sel48 = np.repeat(np.repeat(tmap == KIND_48, TILE, axis=0), TILE, axis=1)
    mask = np.where(sel48, m48, m24).astype(np.uint8)
    return Problem(dtype, N, K, w, tmap, mask, {"seed": seed, "frac24": frac24, "frac48": frac48})
