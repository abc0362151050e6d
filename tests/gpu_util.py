"""Helpers shared by the GPU tests: moving generated bit patterns to the
device and comparing a GPU result with the oracle.

The tolerance is the one fixed for this path: relative Frobenius error
<= 2e-3 and max |error| <= 1e-2 * max |Y_ref| against the fp64 oracle for a
16-bit output.  Rounding a result to bfloat16 (8 significant bits) with
round-to-nearest-even alone costs about 1.7e-3 relative Frobenius error on
Gaussian-like outputs; fp32 accumulation adds ~1e-6 at K <= 16384, so the
2e-3 bar leaves about 20% for the kernel.  A float32 output is held to 1e-5.
"""
import numpy as np
import torch

REL_TOL = 2e-3
MAX_TOL = 1e-2
REL_TOL_F32 = 1e-5
MAX_TOL_F32 = 1e-5

TORCH = {"bf16": torch.bfloat16, "f16": torch.float16}


def dev_bits(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH[dtype])
    return t.to(device)


def dev_u8(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def host_f64(y: torch.Tensor) -> np.ndarray:
    return y.detach().float().cpu().numpy().astype(np.float64)


def errors(y: np.ndarray, ref: np.ndarray):
    err = y - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    mref = np.abs(ref).max()
    mx = np.abs(err).max() / mref if mref > 0 else np.abs(err).max()
    return float(rel), float(mx)


def assert_close(y_gpu: torch.Tensor, ref: np.ndarray, f32: bool = False, what: str = ""):
    y = host_f64(y_gpu)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), what
    rel, mx = errors(y, ref)
    rt, mt = (REL_TOL_F32, MAX_TOL_F32) if f32 else (REL_TOL, MAX_TOL)
    assert rel <= rt and mx <= mt, f"{what}: rel-Frobenius {rel:.3e} (tol {rt}), max {mx:.3e} (tol {mt})"
    return rel, mx
