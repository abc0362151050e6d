"""Python binding of libpatch.so (C ABI in include/patch.h).

Argument marshalling only: every step of the hybrid GEMM runs in the HIP
kernels behind the C ABI.  torch provides device memory and the current HIP
stream; nothing here computes on the CPU, and there is no fallback -- if the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpatch.so")

PATCH_F16, PATCH_BF16, PATCH_F32 = 0, 1, 2
VARIANTS = {"auto": 0, "decode": 1, "prefill": 2, "prefill_w64": 3, "prefill_w128": 4, "prefill_w192": 5,
            "prefill_w256": 6, "prefill_w128_lds": 7, "prefill_w192_lds": 8, "prefill_w256_lds": 9,
            "prefill_w64_lds": 10, "prefill_big": 11, "prefill_big_w128": 12, "prefill_big_w192": 13,
            "prefill_big_w256": 14, "prefill_big8_w128": 15, "prefill_big8_w256": 16}
STATUS = {0: "PATCH_OK", 1: "PATCH_ERR_INVALID_ARG", 2: "PATCH_ERR_SHAPE", 3: "PATCH_ERR_MASK",
          4: "PATCH_ERR_BUFFER_TOO_SMALL", 5: "PATCH_ERR_UNSUPPORTED", 6: "PATCH_ERR_HIP"}

_TORCH_DT = {torch.float16: PATCH_F16, torch.bfloat16: PATCH_BF16, torch.float32: PATCH_F32}
_DT_TORCH = {PATCH_F16: torch.float16, PATCH_BF16: torch.bfloat16, PATCH_F32: torch.float32}


class PatchError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class Desc(ctypes.Structure):
    _fields_ = [("version", ctypes.c_uint32), ("dtype", ctypes.c_uint32), ("tile_n", ctypes.c_uint32),
                ("tile_k", ctypes.c_uint32), ("N", ctypes.c_uint32), ("K", ctypes.c_uint32),
                ("nt_n", ctypes.c_uint32), ("nt_k", ctypes.c_uint32), ("n_sparse", ctypes.c_uint32),
                ("n_48", ctypes.c_uint32), ("table_offset", ctypes.c_uint64), ("data_offset", ctypes.c_uint64),
                ("total_bytes", ctypes.c_uint64)]


EXPORTS = ("patch_abi_version", "patch_packed_bytes", "patch_pack", "patch_packed_bytes_q64", "patch_pack_q64",
           "patch_desc_from_header",
           "patch_gemm_workspace_bytes", "patch_dense_gemm_workspace_bytes", "patch_gemm", "patch_gemm_ex",
           "patch_dense_gemm", "patch_dense_gemm_ex", "patch_packed_bytes_gate_up", "patch_pack_gate_up",
           "patch_gemm_swiglu_workspace_bytes", "patch_gemm_swiglu", "patch_dense_gemm_swiglu_workspace_bytes",
           "patch_dense_gemm_swiglu", "patch_packed_bytes_concat", "patch_pack_concat", "patch_sample_mask",
           "patch_exec_tile_map", "patch_apply_fine_mask", "patch_probe_stream_read", "patch_probe_matrix_rate", "patch_probe_copy_rate", "patch_probe_copy_bytes",
           "patch_debug_tail_wait",
           "patch_probe_matrix_flops", "patch_noalloc_scratch_bytes", "patch_gemm_noalloc", "patch_status_string",
           "patch_last_error")

_lib = None


def load():
    """Load libpatch.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_gemm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, U64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int32
    DP = ctypes.POINTER(Desc)
    lib.patch_abi_version.argtypes = []
    lib.patch_abi_version.restype = I32
    lib.patch_packed_bytes.argtypes = [ctypes.c_int, I64, I64, P]
    lib.patch_packed_bytes.restype = U64
    lib.patch_pack.argtypes = [ctypes.c_int, I64, I64, P, P, P, P, U64, DP, P]
    lib.patch_pack.restype = ctypes.c_int
    lib.patch_packed_bytes_q64.argtypes = [ctypes.c_int, I64, I64, P]
    lib.patch_packed_bytes_q64.restype = U64
    lib.patch_pack_q64.argtypes = [ctypes.c_int, I64, I64, P, P, P, P, U64, DP, P]
    lib.patch_pack_q64.restype = ctypes.c_int
    lib.patch_desc_from_header.argtypes = [P, U64, DP]
    lib.patch_desc_from_header.restype = ctypes.c_int
    lib.patch_gemm_workspace_bytes.argtypes = [DP, I64]
    lib.patch_gemm_workspace_bytes.restype = U64
    lib.patch_dense_gemm_workspace_bytes.argtypes = [I64, I64, I64]
    lib.patch_dense_gemm_workspace_bytes.restype = U64
    lib.patch_gemm.argtypes = [DP, P, P, I64, P, ctypes.c_int, P, U64, P]
    lib.patch_gemm.restype = ctypes.c_int
    lib.patch_gemm_ex.argtypes = [DP, P, P, I64, P, ctypes.c_int, P, U64, I32, P]
    lib.patch_gemm_ex.restype = ctypes.c_int
    lib.patch_dense_gemm.argtypes = [ctypes.c_int, I64, I64, I64, P, P, P, ctypes.c_int, P, U64, P]
    lib.patch_dense_gemm.restype = ctypes.c_int
    lib.patch_dense_gemm_ex.argtypes = [ctypes.c_int, I64, I64, I64, P, P, P, ctypes.c_int, P, U64, I32, P]
    lib.patch_dense_gemm_ex.restype = ctypes.c_int
    lib.patch_packed_bytes_gate_up.argtypes = [ctypes.c_int, I64, I64, P, P]
    lib.patch_packed_bytes_gate_up.restype = U64
    lib.patch_pack_gate_up.argtypes = [ctypes.c_int, I64, I64, P, P, P, P, P, P, P, U64, DP, P]
    lib.patch_pack_gate_up.restype = ctypes.c_int
    lib.patch_gemm_swiglu_workspace_bytes.argtypes = [DP, I64]
    lib.patch_gemm_swiglu_workspace_bytes.restype = U64
    lib.patch_gemm_swiglu.argtypes = [DP, P, P, I64, P, ctypes.c_int, P, U64, I32, P]
    lib.patch_gemm_swiglu.restype = ctypes.c_int
    lib.patch_dense_gemm_swiglu_workspace_bytes.argtypes = [I64, I64, I64]
    lib.patch_dense_gemm_swiglu_workspace_bytes.restype = U64
    lib.patch_dense_gemm_swiglu.argtypes = [ctypes.c_int, I64, I64, I64, P, P, P, P, ctypes.c_int, P, U64, I32, P]
    lib.patch_dense_gemm_swiglu.restype = ctypes.c_int
    lib.patch_packed_bytes_concat.argtypes = [ctypes.c_int, I32, P, I64, P]
    lib.patch_packed_bytes_concat.restype = U64
    lib.patch_pack_concat.argtypes = [ctypes.c_int, I32, P, I64, P, P, P, P, U64, DP, P]
    lib.patch_pack_concat.restype = ctypes.c_int
    lib.patch_sample_mask.argtypes = [I64, I64, P, P, P, P, ctypes.c_float, P, P, P, P]
    lib.patch_sample_mask.restype = ctypes.c_int
    lib.patch_exec_tile_map.argtypes = [I64, I64, I64, I64, P, P, ctypes.POINTER(I64)]
    lib.patch_exec_tile_map.restype = ctypes.c_int
    lib.patch_apply_fine_mask.argtypes = [ctypes.c_int, I64, I64, I64, I64, P, P, P, P, P]
    lib.patch_apply_fine_mask.restype = ctypes.c_int
    lib.patch_probe_stream_read.argtypes = [P, U64, P, U64, P]
    lib.patch_probe_stream_read.restype = ctypes.c_int
    lib.patch_probe_matrix_rate.argtypes = [I32, I32, I32, P, P]
    lib.patch_probe_matrix_rate.restype = ctypes.c_int
    lib.patch_probe_matrix_flops.argtypes = [I32, I32, I32]
    lib.patch_probe_matrix_flops.restype = U64
    lib.patch_probe_copy_rate.argtypes = [P, U64, U64, I32, I32, P, U64, P]
    lib.patch_probe_copy_rate.restype = ctypes.c_int
    lib.patch_probe_copy_bytes.argtypes = [I32, I32]
    lib.patch_probe_copy_bytes.restype = U64
    lib.patch_debug_tail_wait.argtypes = [I32]
    lib.patch_debug_tail_wait.restype = None
    lib.patch_noalloc_scratch_bytes.argtypes = []
    lib.patch_noalloc_scratch_bytes.restype = U64
    lib.patch_gemm_noalloc.argtypes = [DP, P, P, I64, P, ctypes.c_int, P]
    lib.patch_gemm_noalloc.restype = ctypes.c_int
    lib.patch_status_string.argtypes = [ctypes.c_int]
    lib.patch_status_string.restype = ctypes.c_char_p
    lib.patch_last_error.argtypes = []
    lib.patch_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise PatchError(rc, load().patch_last_error().decode())


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device_index: Optional[int] = None) -> int:
    """The current HIP stream of the device, as an integer handle."""
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device() if device_index is None else device_index)
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dt(dtype: torch.dtype) -> int:
    if dtype not in _TORCH_DT:
        raise TypeError(f"unsupported dtype {dtype}")
    return _TORCH_DT[dtype]


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_dev(t: torch.Tensor, name: str, dtype=None, shape=None, on_device: bool = True):
    """A contiguous (device) tensor of the given dtype and shape: the C ABI
    takes raw pointers and cannot check any of this itself.  Type, dtype,
    shape and layout are checked before the device, so every one of these
    errors can be raised without a GPU."""
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}, not {t.dtype}")
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if on_device:
        _need(t.is_cuda, f"{name} must be a device tensor")


def _check_out(out: Optional[torch.Tensor], shape, dtype):
    if out is not None:
        _check_dev(out, "out", dtype, shape, on_device=False)


def _same_device(X: torch.Tensor, *others):
    """Every tensor on X's device (after the shape checks)."""
    _need(X.is_cuda, "X must be a device tensor")
    for name, t in others:
        if t is not None:
            _need(t.is_cuda and t.device == X.device, f"{name} must be on the same device as X")


def _host_map(tile_map) -> np.ndarray:
    if isinstance(tile_map, torch.Tensor):
        tile_map = tile_map.detach().cpu().numpy()
    return np.ascontiguousarray(tile_map, dtype=np.uint8)


@dataclasses.dataclass
class PackedWeight:
    blob: torch.Tensor  # uint8, device
    desc: Desc

    @property
    def N(self) -> int:
        return self.desc.N

    @property
    def K(self) -> int:
        return self.desc.K

    @property
    def dtype(self) -> torch.dtype:
        return _DT_TORCH[self.desc.dtype]

    @property
    def n_sparse(self) -> int:
        """Compressed (2:4 and 4:8) tiles."""
        return self.desc.n_sparse

    @property
    def n_48(self) -> int:
        """4:8 tiles among the compressed ones."""
        return self.desc.n_48

    @property
    def nbytes(self) -> int:
        return self.desc.total_bytes


def packed_bytes(dtype: torch.dtype, N: int, K: int, tile_map) -> int:
    tm = _host_map(tile_map)
    return int(load().patch_packed_bytes(_dt(dtype), N, K, tm.ctypes.data_as(ctypes.c_void_p)))


def pack(W: torch.Tensor, tile_map, mask: torch.Tensor, out: Optional[torch.Tensor] = None) -> PackedWeight:
    """Pack W (N x K, f16/bf16, device), a host tile map (0 dense, 1 2:4,
    2 4:8) and a device byte mask (nonzero = keep) into a blob (patch_pack)."""
    lib = load()
    _need(isinstance(W, torch.Tensor) and W.dim() == 2, "W must be a 2-D tensor (N x K)")
    _need(W.dtype in (torch.float16, torch.bfloat16), "W must be float16 or bfloat16")
    N, K = W.shape
    _check_dev(W, "W", on_device=False)
    _check_dev(mask, "mask", torch.uint8, (N, K), on_device=False)
    tm = _host_map(tile_map)
    _need(tm.shape == (N // 128, K // 128) or N % 128 or K % 128, f"tile map must have shape {(N // 128, K // 128)}")
    if out is not None:
        _check_dev(out, "out", torch.uint8, on_device=False)
    _need(W.is_cuda and mask.is_cuda and (out is None or out.is_cuda), "W, mask and out must be device tensors")
    nbytes = packed_bytes(W.dtype, N, K, tm)
    if nbytes == 0:
        # let the library name what is wrong (it checks before the buffer size)
        probe = torch.empty(16, dtype=torch.uint8, device=W.device)
        _check(lib.patch_pack(_dt(W.dtype), N, K, _ptr(W), tm.ctypes.data_as(ctypes.c_void_p), _ptr(mask),
                              _ptr(probe), 0, ctypes.byref(Desc()), _stream()))
        raise PatchError(2, f"invalid arguments for pack: {tuple(W.shape)} {W.dtype}")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    desc = Desc()
    _check(lib.patch_pack(_dt(W.dtype), N, K, _ptr(W), tm.ctypes.data_as(ctypes.c_void_p), _ptr(mask), _ptr(out),
                          out.numel(), ctypes.byref(desc), _stream()))
    return PackedWeight(out, desc)


def packed_bytes_q64(dtype: torch.dtype, N: int, K: int, quad_map) -> int:
    """Blob size for 64 x 64 execution tiles (format 4) and a (N/64, K/64)
    quadrant map (0 dense, 1 2:4); 0 for invalid arguments."""
    qm = _host_map(quad_map)
    if qm.shape != (N // 64, K // 64):
        return 0
    return int(load().patch_packed_bytes_q64(_dt(dtype), N, K, qm.ctypes.data_as(ctypes.c_void_p)))


def pack_q64(W: torch.Tensor, quad_map, mask: torch.Tensor, out: Optional[torch.Tensor] = None) -> PackedWeight:
    """Pack W (N x K, f16/bf16, device), a host quadrant map ((N/64) x (K/64):
    0 dense, 1 2:4) and a device byte mask into a blob of 64 x 64 execution
    tiles (patch_pack_q64)."""
    lib = load()
    _need(isinstance(W, torch.Tensor) and W.dim() == 2, "W must be a 2-D tensor (N x K)")
    _need(W.dtype in (torch.float16, torch.bfloat16), "W must be float16 or bfloat16")
    N, K = W.shape
    _check_dev(W, "W", on_device=False)
    _check_dev(mask, "mask", torch.uint8, (N, K), on_device=False)
    qm = _host_map(quad_map)
    _need(qm.shape == (N // 64, K // 64) or N % 128 or K % 128, f"quadrant map must have shape {(N // 64, K // 64)}")
    if out is not None:
        _check_dev(out, "out", torch.uint8, on_device=False)
    _need(W.is_cuda and mask.is_cuda and (out is None or out.is_cuda), "W, mask and out must be device tensors")
    nbytes = packed_bytes_q64(W.dtype, N, K, qm)
    if nbytes == 0:
        probe = torch.empty(16, dtype=torch.uint8, device=W.device)
        _check(lib.patch_pack_q64(_dt(W.dtype), N, K, _ptr(W), qm.ctypes.data_as(ctypes.c_void_p), _ptr(mask),
                                  _ptr(probe), 0, ctypes.byref(Desc()), _stream()))
        raise PatchError(2, f"invalid arguments for pack_q64: {tuple(W.shape)} {W.dtype}")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    desc = Desc()
    _check(lib.patch_pack_q64(_dt(W.dtype), N, K, _ptr(W), qm.ctypes.data_as(ctypes.c_void_p), _ptr(mask),
                              _ptr(out), out.numel(), ctypes.byref(desc), _stream()))
    return PackedWeight(out, desc)


def desc_from_header(header: bytes) -> Desc:
    buf = (ctypes.c_uint8 * len(header)).from_buffer_copy(header)
    d = Desc()
    _check(load().patch_desc_from_header(ctypes.cast(buf, ctypes.c_void_p), len(header), ctypes.byref(d)))
    return d


_WS_BYTES = {}


def _ws_bytes(kind: str, M: int, N: int, K: int, dev: int, query) -> int:
    """The library's workspace query, remembered per shape (it is a pure
    function of the shape on a given device)."""
    key = (kind, M, N, K, dev)
    nb = _WS_BYTES.get(key)
    if nb is None:
        nb = int(query())
        if len(_WS_BYTES) > 4096:
            _WS_BYTES.clear()
        _WS_BYTES[key] = nb
    return nb


def _check_x(X: torch.Tensor, dtype: torch.dtype, K: int):
    _need(isinstance(X, torch.Tensor) and X.dim() == 2, "X must be a 2-D tensor (M x K)")
    _need(X.shape[1] == K, f"X must have K = {K} columns, not {X.shape[1]}")
    _check_dev(X, "X", dtype, on_device=False)


def _check_out_dtype(od: torch.dtype, xd: torch.dtype):
    _need(od in (xd, torch.float32), f"out_dtype must be {xd} or torch.float32, not {od}")


def _workspace(nbytes: int, workspace, device):
    """workspace="auto": a fresh buffer of the size the library asks for
    (from torch's caching allocator) on every call; None: no workspace; a
    tensor: used as given.  Callers that run the same shapes repeatedly keep
    one buffer per call site (sized by patch_gemm_workspace_bytes) and pass
    it: with the per-call allocation a step of two tail-split GEMMs measured
    up to 3% slower."""
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace must be 'auto', None or a tensor, not {workspace!r}")
        return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes > 0 else None
    if workspace is not None:
        _check_dev(workspace, "workspace")
        _need(workspace.device == device, "workspace must be on the same device as X")
    return workspace


def gemm(X: torch.Tensor, packed: PackedWeight, out_dtype: Optional[torch.dtype] = None, variant: str = "auto",
         out: Optional[torch.Tensor] = None, workspace="auto") -> torch.Tensor:
    """Y = X (W o E)^T from a packed blob (patch_gemm_ex)."""
    lib = _lib or load()
    _check_x(X, packed.dtype, packed.K)
    _check_dev(packed.blob, "packed blob", torch.uint8, on_device=False)
    _need(packed.blob.numel() >= packed.nbytes, "packed blob is smaller than its descriptor's total_bytes")
    M = X.shape[0]
    od = out_dtype or X.dtype
    _check_out_dtype(od, X.dtype)
    _check_out(out, (M, packed.N), od)
    _same_device(X, ("packed blob", packed.blob), ("out", out))
    dev = X.get_device()
    if out is None:
        out = torch.empty((M, packed.N), dtype=od, device=X.device)
    ws, nb = None, 0
    if workspace is not None:
        nb = _ws_bytes("packed", M, packed.N, packed.K, dev,
                       lambda: lib.patch_gemm_workspace_bytes(ctypes.byref(packed.desc), M))
        ws = _workspace(nb, workspace, X.device)
        nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.patch_gemm_ex(ctypes.byref(packed.desc), packed.blob.data_ptr(), X.data_ptr(), M, out.data_ptr(),
                             _dt(od), None if ws is None else ws.data_ptr(), nb, VARIANTS[variant],
                             _stream(dev)))
    return out


def gemm_noalloc(X: torch.Tensor, packed: PackedWeight, out: torch.Tensor,
                 out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Y = X (W o E)^T into a caller-supplied `out` with the library's own
    device scratch (patch_gemm_noalloc): nothing is allocated, by the
    library or here."""
    lib = _lib or load()
    _check_x(X, packed.dtype, packed.K)
    _check_dev(packed.blob, "packed blob", torch.uint8, on_device=False)
    _need(packed.blob.numel() >= packed.nbytes, "packed blob is smaller than its descriptor's total_bytes")
    od = out_dtype or out.dtype
    _check_out_dtype(od, X.dtype)
    _check_out(out, (X.shape[0], packed.N), od)
    _same_device(X, ("packed blob", packed.blob), ("out", out))
    _check(lib.patch_gemm_noalloc(ctypes.byref(packed.desc), packed.blob.data_ptr(), X.data_ptr(), X.shape[0],
                                  out.data_ptr(), _dt(od), _stream(X.get_device())))
    return out


def dense_gemm(X: torch.Tensor, W: torch.Tensor, out_dtype: Optional[torch.dtype] = None, variant: str = "auto",
               out: Optional[torch.Tensor] = None, workspace="auto") -> torch.Tensor:
    """Same-shape dense baseline Y = X W^T from row-major W (patch_dense_gemm_ex)."""
    lib = _lib or load()
    _need(W.dim() == 2, "W must be 2-D (N x K)")
    _check_x(X, W.dtype, W.shape[1])
    _check_dev(W, "W", X.dtype, on_device=False)
    M, K = X.shape
    N = W.shape[0]
    od = out_dtype or X.dtype
    _check_out_dtype(od, X.dtype)
    _check_out(out, (M, N), od)
    _same_device(X, ("W", W), ("out", out))
    dev = X.get_device()
    if out is None:
        out = torch.empty((M, N), dtype=od, device=X.device)
    ws, nb = None, 0
    if workspace is not None:
        nb = _ws_bytes("dense", M, N, K, dev, lambda: lib.patch_dense_gemm_workspace_bytes(M, N, K))
        ws = _workspace(nb, workspace, X.device)
        nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.patch_dense_gemm_ex(_dt(X.dtype), M, N, K, X.data_ptr(), W.data_ptr(), out.data_ptr(), _dt(od),
                                   None if ws is None else ws.data_ptr(), nb, VARIANTS[variant], _stream(dev)))
    return out


def pack_gate_up(Wg: torch.Tensor, Wu: torch.Tensor, map_g, map_u, mask_g: torch.Tensor, mask_u: torch.Tensor,
                 out: Optional[torch.Tensor] = None) -> PackedWeight:
    """Pack gate and up weights (F x K each, device) into one blob of their
    row-block interleave (patch_pack_gate_up)."""
    lib = load()
    F, K = Wg.shape
    if tuple(Wu.shape) != (F, K) or Wu.dtype != Wg.dtype:
        raise ValueError("gate and up weights must have the same shape and dtype")
    tg, tu = _host_map(map_g), _host_map(map_u)
    nbytes = int(lib.patch_packed_bytes_gate_up(_dt(Wg.dtype), F, K, tg.ctypes.data_as(ctypes.c_void_p),
                                                tu.ctypes.data_as(ctypes.c_void_p)))
    if nbytes == 0:
        raise PatchError(2, f"invalid shape/dtype for pack_gate_up: {tuple(Wg.shape)} {Wg.dtype}")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=Wg.device)
    desc = Desc()
    _check(lib.patch_pack_gate_up(_dt(Wg.dtype), F, K, _ptr(Wg), _ptr(Wu), tg.ctypes.data_as(ctypes.c_void_p),
                                  tu.ctypes.data_as(ctypes.c_void_p), _ptr(mask_g), _ptr(mask_u), _ptr(out),
                                  out.numel(), ctypes.byref(desc), _stream()))
    return PackedWeight(out, desc)


def gemm_swiglu(X: torch.Tensor, packed: PackedWeight, out_dtype: Optional[torch.dtype] = None,
                variant: str = "auto", out: Optional[torch.Tensor] = None, workspace="auto") -> torch.Tensor:
    """H = SiLU(X Wg^T) * (X Wu^T) from a gate/up blob (patch_gemm_swiglu)."""
    lib = _lib or load()
    _check_x(X, packed.dtype, packed.K)
    _check_dev(packed.blob, "packed blob", torch.uint8, on_device=False)
    _need(packed.blob.numel() >= packed.nbytes, "packed blob is smaller than its descriptor's total_bytes")
    M = X.shape[0]
    F = packed.N // 2
    od = out_dtype or X.dtype
    _check_out_dtype(od, X.dtype)
    _check_out(out, (M, F), od)
    _same_device(X, ("packed blob", packed.blob), ("out", out))
    dev = X.get_device()
    if out is None:
        out = torch.empty((M, F), dtype=od, device=X.device)
    ws, nb = None, 0
    if workspace is not None:
        nb = _ws_bytes("swiglu", M, packed.N, packed.K, dev,
                       lambda: lib.patch_gemm_swiglu_workspace_bytes(ctypes.byref(packed.desc), M))
        ws = _workspace(nb, workspace, X.device)
        nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.patch_gemm_swiglu(ctypes.byref(packed.desc), packed.blob.data_ptr(), X.data_ptr(), M, out.data_ptr(),
                                 _dt(od), None if ws is None else ws.data_ptr(), nb, VARIANTS[variant], _stream(dev)))
    return out


def dense_gemm_swiglu(X: torch.Tensor, Wg: torch.Tensor, Wu: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
                      variant: str = "auto", out: Optional[torch.Tensor] = None, workspace="auto") -> torch.Tensor:
    """Same-shape dense baseline of gemm_swiglu from row-major Wg, Wu (patch_dense_gemm_swiglu)."""
    lib = _lib or load()
    _need(Wg.dim() == 2, "Wg must be 2-D (F x K)")
    _check_x(X, Wg.dtype, Wg.shape[1])
    _check_dev(Wg, "Wg", X.dtype, on_device=False)
    _check_dev(Wu, "Wu", X.dtype, tuple(Wg.shape), on_device=False)
    M, K = X.shape
    F = Wg.shape[0]
    od = out_dtype or X.dtype
    _check_out_dtype(od, X.dtype)
    _check_out(out, (M, F), od)
    _same_device(X, ("Wg", Wg), ("Wu", Wu), ("out", out))
    dev = X.get_device()
    if out is None:
        out = torch.empty((M, F), dtype=od, device=X.device)
    ws, nb = None, 0
    if workspace is not None:
        nb = _ws_bytes("dense_swiglu", M, F, K, dev, lambda: lib.patch_dense_gemm_swiglu_workspace_bytes(M, F, K))
        ws = _workspace(nb, workspace, X.device)
        nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.patch_dense_gemm_swiglu(_dt(X.dtype), M, F, K, X.data_ptr(), Wg.data_ptr(), Wu.data_ptr(),
                                       out.data_ptr(), _dt(od), None if ws is None else ws.data_ptr(), nb,
                                       VARIANTS[variant], _stream(dev)))
    return out


def pack_concat(Ws, tile_maps, masks, out: Optional[torch.Tensor] = None) -> PackedWeight:
    """Pack the row-concatenation of several weights with the same K (device
    tensors, host tile maps, device masks) into one blob (patch_pack_concat):
    one GEMM on it returns the projections side by side."""
    lib = load()
    n = len(Ws)
    if not (len(tile_maps) == len(masks) == n) or n < 1:
        raise ValueError("one tile map and one mask per weight")
    K = Ws[0].shape[1]
    if any(W.dtype != Ws[0].dtype or W.shape[1] != K for W in Ws):
        raise ValueError("the weights must share dtype and K")
    Ns = (ctypes.c_int64 * n)(*[int(W.shape[0]) for W in Ws])
    maps = [_host_map(t) for t in tile_maps]
    mp = (ctypes.c_void_p * n)(*[m.ctypes.data for m in maps])
    wp = (ctypes.c_void_p * n)(*[W.data_ptr() for W in Ws])
    kp = (ctypes.c_void_p * n)(*[m.data_ptr() for m in masks])
    nbytes = int(lib.patch_packed_bytes_concat(_dt(Ws[0].dtype), n, Ns, K, mp))
    if nbytes == 0:
        raise PatchError(2, "invalid shapes for pack_concat")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=Ws[0].device)
    desc = Desc()
    _check(lib.patch_pack_concat(_dt(Ws[0].dtype), n, Ns, K, wp, mp, kp, _ptr(out), out.numel(), ctypes.byref(desc),
                                 _stream()))
    return PackedWeight(out, desc)


def sample_mask(tile_logits: torch.Tensor, tile_u: torch.Tensor, pat_logits: torch.Tensor, pat_u: torch.Tensor,
                tau: float, soft: bool = True, out=None):
    """Forward hybrid-mask sampler (patch_sample_mask) on device float32
    tensors: tile_logits, tile_u [N/128, K/128, 2]; pat_logits, pat_u
    [N, K/4, 6].  Returns (tile_map uint8 [N/128, K/128], mask uint8 [N, K],
    soft float32 [N, K] or None); out = (tile_map, mask, soft) reuses
    buffers."""
    lib = load()
    N, G = int(pat_logits.shape[0]), int(pat_logits.shape[1])
    K = 4 * G
    for t, shape in ((tile_logits, (N // 128, K // 128, 2)), (tile_u, (N // 128, K // 128, 2)),
                     (pat_logits, (N, G, 6)), (pat_u, (N, G, 6))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"expected a contiguous float32 device tensor of shape {shape}")
    dev = pat_logits.device
    if out is None:
        out = (torch.empty((N // 128, K // 128), dtype=torch.uint8, device=dev),
               torch.empty((N, K), dtype=torch.uint8, device=dev),
               torch.empty((N, K), dtype=torch.float32, device=dev) if soft else None)
    tmap, mask, sf = out
    _check(lib.patch_sample_mask(N, K, _ptr(tile_logits), _ptr(tile_u), _ptr(pat_logits), _ptr(pat_u), float(tau),
                                 _ptr(tmap), _ptr(mask), _ptr(sf) if soft else ctypes.c_void_p(0),
                                 _stream(dev.index)))
    return tmap, mask, (sf if soft else None)


def exec_tile_map(N: int, K: int, fine_map, b1: int, b2: int) -> np.ndarray:
    """128 x 128 execution tile map from a fine tile map of b1 x b2 tiles
    (patch_exec_tile_map): 1 where every fine tile is 2:4."""
    fm = _host_map(fine_map)
    if fm.shape != (N // b1, K // b2):
        raise ValueError(f"fine map must be {(N // b1, K // b2)}")
    out = np.zeros((N // 128, K // 128), dtype=np.uint8)
    n = ctypes.c_int64(0)
    _check(load().patch_exec_tile_map(N, K, b1, b2, fm.ctypes.data, out.ctypes.data, ctypes.byref(n)))
    return out


def apply_fine_mask(W: torch.Tensor, fine_map: torch.Tensor, mask: torch.Tensor, b1: int, b2: int,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W o E_fine on the device (patch_apply_fine_mask): fine_map uint8
    [N/b1, K/b2] and mask uint8 [N, K] device tensors."""
    N, K = W.shape
    if out is None:
        out = torch.empty_like(W)
    _check(load().patch_apply_fine_mask(_dt(W.dtype), N, K, b1, b2, _ptr(W), _ptr(fine_map), _ptr(mask), _ptr(out),
                                        _stream(W.device.index)))
    return out


def pack_fine(W: torch.Tensor, fine_map, mask: torch.Tensor, b1: int, b2: int) -> PackedWeight:
    """Pack a layer whose mask was learnt on b1 x b2 tiles: execution map by
    the all-2:4 policy, dense execution tiles from W o E_fine."""
    N, K = W.shape
    fm_host = _host_map(fine_map)
    emap = exec_tile_map(N, K, fm_host, b1, b2)
    Wm = apply_fine_mask(W, torch.from_numpy(fm_host).to(W.device), mask, b1, b2)
    return pack(Wm, emap, mask)


def probe_stream_read(src: torch.Tensor, sink: torch.Tensor) -> None:
    """Read every byte of src once (patch_probe_stream_read); time it around
    the call.  sink: a device scratch tensor (its bytes bound the grid)."""
    _check_dev(src, "src")
    _check_dev(sink, "sink")
    nb = src.numel() * src.element_size()
    _check(load().patch_probe_stream_read(_ptr(src), nb - nb % 16, _ptr(sink), sink.numel() * sink.element_size(),
                                          _stream(src.device.index)))


def probe_matrix_rate(kind: int, iters: int, workgroups: int, sink: torch.Tensor) -> int:
    """Launch the matrix-instruction rate probe (patch_probe_matrix_rate);
    returns the flops it executes (dense-equivalent for the sparse kinds)."""
    _check_dev(sink, "sink")
    _need(sink.numel() * sink.element_size() >= 4 * workgroups, "sink needs 4 bytes a workgroup")
    lib = load()
    _check(lib.patch_probe_matrix_rate(kind, iters, workgroups, _ptr(sink), _stream(sink.device.index)))
    return int(lib.patch_probe_matrix_flops(kind, iters, workgroups))


def debug_tail_wait(polls: int) -> None:
    """For tests of the tail split's bounded wait (patch_debug_tail_wait):
    polls > 0 makes the first K range of every left-over block wait for a
    flag value no range stores, give up after that many polls and mark its
    block's outputs NaN; polls <= 0 restores normal launches."""
    (_lib or load()).patch_debug_tail_wait(int(polls))


def probe_copy_rate(src: torch.Tensor, window_bytes: int, iters: int, workgroups: int, sink: torch.Tensor) -> int:
    """Launch the global -> LDS copy-rate probe (patch_probe_copy_rate) over
    src (its size a multiple of window_bytes); returns the bytes it copies."""
    _check_dev(src, "src")
    _check_dev(sink, "sink")
    lib = load()
    _check(lib.patch_probe_copy_rate(_ptr(src), src.numel() * src.element_size(), window_bytes, iters, workgroups,
                                     _ptr(sink), sink.numel() * sink.element_size(), _stream(src.device.index)))
    return int(lib.patch_probe_copy_bytes(iters, workgroups))
