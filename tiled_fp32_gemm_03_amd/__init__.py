"""Python binding of the gfx950 fp32 matrix-multiply library ``libgemm_f32.so``.

Argument marshalling only: every step of C = A x B runs in the library's HIP
kernels.  If the library is missing the import fails loudly; there is no
CPU or PyTorch fallback.

Raw C-ABI mirrors (same names and argument order as ``include/gemm_f32.h``):
  gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, variant, stream)
  gemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, variant, config, stream)
  gemm_f32_tile(variant, config, M, N, K) -> dict
  gemm_f32_num_configs(variant), gemm_f32_status_string(rc), gemm_f32_version()
  gemm_f32_probe_stream(kind, n, x, y, z, stream)      (include/gemm_f32_probes.h)
  gemm_f32_probe_mfma(workgroups, iters, out, stream), gemm_f32_probe_mfma_flops(...)
  gemm_f32_probe_mfma16(shape, workgroups, iters, out, stream), gemm_f32_probe_mfma16_flops(...)
  gemm_f32_probe_valu(workgroups, iters, out, stream), gemm_f32_probe_valu_flops(...)
  gemm_f32_probe_lds(workgroups, iters, out, stream), gemm_f32_probe_lds_bytes(...)
  gemm_f32_probe_fused(mode, workgroups, trips, out, out_bytes, clocks, stream),
  gemm_f32_probe_fused_flops(mode, ...), gemm_f32_probe_fused_bytes(mode, ...)
  gemm_f32_device_props(device) -> dict
  gemm_f32_splitk(M, N, K, A, lda, B, ldb, C, ldc, config, splits, workspace,
                  workspace_bytes, stream), gemm_f32_splitk_plan(M, N, K, config, splits)
  gemm_f32_splitk_noalloc(M, N, K, A, lda, B, ldb, C, ldc, config, splits, stream)
  gemm_mixed(M, N, K, A, lda, B, ldb, C, ldc, format, config, stream)
  gemm_mixed_tile(config, M, N, K) -> dict, gemm_mixed_num_configs()
                                                        (include/gemm_mixed.h)
Pointers are device addresses (ints); ``stream`` is a hipStream_t as int
(0 = null stream).  A non-zero status raises ``GemmError``.

Tensor conveniences: ``matmul(A, B, out=None, variant="prod", config=-1)``
takes float32 CUDA tensors whose last stride is 1 and passes ``stride(0)`` as
the leading dimension, on torch's current stream.  ``matmul_mixed(A, B,
out=None, config=-1)`` does the same for bfloat16 or float16 tensors (fp32
result); ``format`` names the 16-bit format when A and B hold raw codes
(int16 / uint16).  ``matmul_splitk(A, B, out=None, config=-1, splits=0,
workspace=None)`` runs the split-K form; it allocates the workspace as a torch
tensor when none is given.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "GemmError", "VARIANTS", "config_name", "PROBE_COPY", "PROBE_FILL", "PROBE_VADD",
    "gemm_f32", "gemm_f32_ex", "gemm_f32_tile", "gemm_f32_num_configs",
    "gemm_f32_status_string", "gemm_f32_version", "gemm_f32_last_error", "gemm_f32_probe_stream",
    "gemm_f32_probe_mfma", "gemm_f32_probe_mfma_flops", "gemm_f32_probe_mfma16",
    "gemm_f32_probe_mfma16_flops", "gemm_f32_probe_valu",
    "gemm_f32_probe_valu_flops", "gemm_f32_probe_lds", "gemm_f32_probe_lds_bytes",
    "gemm_f32_probe_fused", "gemm_f32_probe_fused_flops", "gemm_f32_probe_fused_bytes",
    "FUSED_BOTH", "FUSED_MFMA", "FUSED_STORE",
    "gemm_f32_device_props", "matmul",
    "gemm_f32_splitk", "gemm_f32_splitk_plan", "matmul_splitk", "gemm_f32_splitk_noalloc",
    "NOALLOC_SCRATCH_BYTES",
    "gemm_mixed", "gemm_mixed_tile", "gemm_mixed_num_configs", "matmul_mixed", "MIXED_FORMATS",
    "mixed_config_name",
    "library_path",
    "exported_symbols",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgemm_f32.so")

# One HIP runtime per process: PyTorch ships its own libamdhip64 (same
# soname).  Loading torch first makes this library bind to that copy instead
# of pulling in a second runtime from /opt/rocm, which could not launch on
# memory that torch's runtime allocated.
import torch  # noqa: E402,F401

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is not built; run __graft_entry__.build() or "
        "python tiled_fp32_gemm_03_amd/build_lib.py (needs ROCm hipcc)")

_lib = ctypes.CDLL(_LIB_PATH)

_i = ctypes.c_int
_ll = ctypes.c_longlong
_p = ctypes.c_void_p
_ip = ctypes.POINTER(ctypes.c_int)

_SIGS = {
    "gemm_f32": ([_i, _i, _i, _p, _i, _p, _i, _p, _i, _i, _p], _i),
    "gemm_f32_ex": ([_i, _i, _i, _p, _i, _p, _i, _p, _i, _i, _i, _p], _i),
    "gemm_f32_num_configs": ([_i], _i),
    "gemm_f32_tile": ([_i, _i, _i, _i, _i, _ip, _ip, _ip, _ip, _ip], _i),
    "gemm_f32_status_string": ([_i], ctypes.c_char_p),
    "gemm_f32_version": ([], ctypes.c_char_p),
    "gemm_f32_last_error": ([], ctypes.c_char_p),
    "gemm_f32_probe_stream": ([_i, _ll, _p, _p, _p, _p], _i),
    "gemm_f32_probe_mfma": ([_i, _i, _p, _p], _i),
    "gemm_f32_probe_mfma_flops": ([_i, _i], _ll),
    "gemm_f32_probe_mfma16": ([_i, _i, _i, _p, _p], _i),
    "gemm_f32_probe_mfma16_flops": ([_i, _i, _i], _ll),
    "gemm_f32_probe_valu": ([_i, _i, _p, _p], _i),
    "gemm_f32_probe_valu_flops": ([_i, _i], _ll),
    "gemm_f32_probe_lds": ([_i, _i, _p, _p], _i),
    "gemm_f32_splitk": ([_i, _i, _i, _p, _i, _p, _i, _p, _i, _i, _i, _p, _ll, _p], _i),
    "gemm_f32_splitk_plan": ([_i, _i, _i, _i, _i, _ip, _ip, _ip, ctypes.POINTER(_ll)], _i),
    "gemm_f32_splitk_noalloc": ([_i, _i, _i, _p, _i, _p, _i, _p, _i, _i, _i, _p], _i),
    "gemm_mixed": ([_i, _i, _i, _p, _i, _p, _i, _p, _i, _i, _i, _p], _i),
    "gemm_mixed_num_configs": ([], _i),
    "gemm_mixed_tile": ([_i, _i, _i, _i, _ip, _ip, _ip, _ip, _ip], _i),
    "gemm_f32_probe_lds_bytes": ([_i, _i], _ll),
    "gemm_f32_device_props": ([_i, _ip, _ip, _ip, _ip, _ip], _i),
    "gemm_f32_probe_fused": ([_i, _i, _i, _p, _ll, _p, _p], _i),
    "gemm_f32_probe_fused_flops": ([_i, _i, _i], _ll),
    "gemm_f32_probe_fused_bytes": ([_i, _i, _i], _ll),
}
for _name, (_args, _ret) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _ret

# Variant ids of include/gemm_f32.h.
VARIANTS = {"naive": 0, "tiled": 1, "prod": 2, "tiled32": 3, "tiled4": 4, "tiled32_pad": 5,
            "valu": 6}
PROBE_COPY, PROBE_FILL, PROBE_VADD = 0, 1, 2
FUSED_BOTH, FUSED_MFMA, FUSED_STORE = 0, 1, 2
# GEMM_F32_NOALLOC_SCRATCH_BYTES of include/gemm_f32.h: the fixed split-K
# scratch of gemm_f32_splitk_noalloc on each GPU.
NOALLOC_SCRATCH_BYTES = 64 << 20
# Input formats of include/gemm_mixed.h.
MIXED_FORMATS = {"bf16": 0, "f16": 1}


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = gemm_f32_last_error() if status == 5 else ""
        super().__init__(f"{where}: status {status} ({gemm_f32_status_string(status)})"
                         + (f": {detail}" if detail else ""))


def library_path() -> str:
    return _LIB_PATH


def exported_symbols() -> tuple[str, ...]:
    return tuple(_SIGS)


def _variant(v) -> int:
    if isinstance(v, str):
        try:
            return VARIANTS[v]
        except KeyError:
            raise ValueError(f"unknown variant {v!r}; one of {sorted(VARIANTS)}") from None
    return int(v)


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise GemmError(rc, where)


def gemm_f32_status_string(status: int) -> str:
    return _lib.gemm_f32_status_string(int(status)).decode()


def gemm_f32_last_error() -> str:
    return _lib.gemm_f32_last_error().decode()


def gemm_f32_version() -> str:
    return _lib.gemm_f32_version().decode()


def gemm_f32_num_configs(variant) -> int:
    return int(_lib.gemm_f32_num_configs(_variant(variant)))


def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, variant, stream=0) -> None:
    rc = _lib.gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, _variant(variant), stream or None)
    _check(rc, "gemm_f32")


def gemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, variant, config, stream=0) -> None:
    rc = _lib.gemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, _variant(variant), int(config),
                          stream or None)
    _check(rc, "gemm_f32_ex")


def gemm_f32_tile(variant, config, M, N, K) -> dict:
    vals = [ctypes.c_int(0) for _ in range(5)]
    rc = _lib.gemm_f32_tile(_variant(variant), int(config), M, N, K,
                            *[ctypes.byref(v) for v in vals])
    _check(rc, "gemm_f32_tile")
    bm, bn, bk, nt, chosen = (v.value for v in vals)
    return {"BM": bm, "BN": bn, "BK": bk, "threads": nt, "config": chosen}


def gemm_f32_probe_stream(kind, n, x, y, z, stream=0) -> None:
    _check(_lib.gemm_f32_probe_stream(int(kind), int(n), x or None, y or None, z or None,
                                      stream or None), "gemm_f32_probe_stream")


def gemm_f32_probe_mfma(workgroups, iters, out, stream=0) -> None:
    _check(_lib.gemm_f32_probe_mfma(int(workgroups), int(iters), out or None, stream or None),
           "gemm_f32_probe_mfma")


def gemm_f32_probe_mfma_flops(workgroups, iters) -> int:
    return int(_lib.gemm_f32_probe_mfma_flops(int(workgroups), int(iters)))


def gemm_f32_probe_mfma16(shape, workgroups, iters, out, stream=0) -> None:
    _check(_lib.gemm_f32_probe_mfma16(int(shape), int(workgroups), int(iters), out or None,
                                      stream or None), "gemm_f32_probe_mfma16")


def gemm_f32_probe_mfma16_flops(shape, workgroups, iters) -> int:
    return int(_lib.gemm_f32_probe_mfma16_flops(int(shape), int(workgroups), int(iters)))


def gemm_f32_probe_valu(workgroups, iters, out, stream=0) -> None:
    _check(_lib.gemm_f32_probe_valu(int(workgroups), int(iters), out or None, stream or None),
           "gemm_f32_probe_valu")


def gemm_f32_probe_valu_flops(workgroups, iters) -> int:
    return int(_lib.gemm_f32_probe_valu_flops(int(workgroups), int(iters)))


def gemm_f32_probe_lds(workgroups, iters, out, stream=0) -> None:
    _check(_lib.gemm_f32_probe_lds(int(workgroups), int(iters), out or None, stream or None),
           "gemm_f32_probe_lds")


def gemm_f32_probe_lds_bytes(workgroups, iters) -> int:
    return int(_lib.gemm_f32_probe_lds_bytes(int(workgroups), int(iters)))


def gemm_f32_probe_fused(mode, workgroups, trips, out, out_bytes, clocks=0, stream=0) -> None:
    _check(_lib.gemm_f32_probe_fused(int(mode), int(workgroups), int(trips), out or None,
                                     int(out_bytes), clocks or None, stream or None),
           "gemm_f32_probe_fused")


def gemm_f32_probe_fused_flops(mode, workgroups, trips) -> int:
    return int(_lib.gemm_f32_probe_fused_flops(int(mode), int(workgroups), int(trips)))


def gemm_f32_probe_fused_bytes(mode, workgroups, trips) -> int:
    return int(_lib.gemm_f32_probe_fused_bytes(int(mode), int(workgroups), int(trips)))


def gemm_f32_device_props(device: int = 0) -> dict:
    vals = [ctypes.c_int(0) for _ in range(5)]
    _check(_lib.gemm_f32_device_props(int(device), *[ctypes.byref(v) for v in vals]),
           "gemm_f32_device_props")
    cus, clk, lds, wave, l2 = (v.value for v in vals)
    return {"cus": cus, "clock_mhz": clk / 1000.0, "lds_bytes_per_cu": lds, "wave_size": wave,
            "l2_bytes": l2}


def gemm_f32_splitk_plan(M, N, K, config=-1, splits=0) -> dict:
    ints = [ctypes.c_int(0) for _ in range(3)]
    ws = ctypes.c_longlong(0)
    rc = _lib.gemm_f32_splitk_plan(M, N, K, int(config), int(splits),
                                   *[ctypes.byref(v) for v in ints], ctypes.byref(ws))
    _check(rc, "gemm_f32_splitk_plan")
    cfg, used, kc = (v.value for v in ints)
    return {"config": cfg, "splits": used, "kc": kc, "workspace_bytes": ws.value}


def gemm_f32_splitk(M, N, K, A, lda, B, ldb, C, ldc, config, splits, workspace,
                    workspace_bytes, stream=0) -> None:
    rc = _lib.gemm_f32_splitk(M, N, K, A or None, lda, B or None, ldb, C or None, ldc,
                              int(config), int(splits), workspace or None, int(workspace_bytes),
                              stream or None)
    _check(rc, "gemm_f32_splitk")


def gemm_f32_splitk_noalloc(M, N, K, A, lda, B, ldb, C, ldc, config=-1, splits=0,
                            stream=0) -> None:
    rc = _lib.gemm_f32_splitk_noalloc(M, N, K, A or None, lda, B or None, ldb, C or None, ldc,
                                      int(config), int(splits), stream or None)
    _check(rc, "gemm_f32_splitk_noalloc")


def _format(fmt) -> int:
    if isinstance(fmt, str):
        try:
            return MIXED_FORMATS[fmt]
        except KeyError:
            raise ValueError(f"unknown 16-bit format {fmt!r}; one of {sorted(MIXED_FORMATS)}") from None
    return int(fmt)


def gemm_mixed(M, N, K, A, lda, B, ldb, C, ldc, format, config=-1, stream=0) -> None:
    rc = _lib.gemm_mixed(M, N, K, A or None, lda, B or None, ldb, C or None, ldc,
                         _format(format), int(config), stream or None)
    _check(rc, "gemm_mixed")


def gemm_mixed_num_configs() -> int:
    return int(_lib.gemm_mixed_num_configs())


def gemm_mixed_tile(config, M, N, K) -> dict:
    vals = [ctypes.c_int(0) for _ in range(5)]
    rc = _lib.gemm_mixed_tile(int(config), M, N, K, *[ctypes.byref(v) for v in vals])
    _check(rc, "gemm_mixed_tile")
    bm, bn, bk, nt, chosen = (v.value for v in vals)
    return {"BM": bm, "BN": bn, "BK": bk, "threads": nt, "config": chosen}


def config_name(variant, config: int = -1, M: int = 1, N: int = 1, K: int = 1) -> str:
    """Readable name of a launch-table entry, e.g. "prod#0:128x128x32/256t"."""
    t = gemm_f32_tile(variant, config, M, N, K)
    v = _variant(variant)
    vname = next(k for k, val in VARIANTS.items() if val == v)
    return f"{vname}#{t['config']}:{t['BM']}x{t['BN']}x{t['BK']}/{t['threads']}t"


def mixed_config_name(fmt, config: int = -1, M: int = 1, N: int = 1, K: int = 1) -> str:
    """Readable name of a gemm_mixed entry, e.g. "bf16#0:256x256x64/512t"."""
    t = gemm_mixed_tile(config, M, N, K)
    f = next(k for k, val in MIXED_FORMATS.items() if val == _format(fmt))
    return f"{f}#{t['config']}:{t['BM']}x{t['BN']}x{t['BK']}/{t['threads']}t"


def _ld(t) -> int:
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("the last dimension must be contiguous (stride 1)")
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError("rows overlap (row stride smaller than the row length)")
    return max(1, t.stride(0) if t.shape[0] > 1 else t.shape[1])


def matmul(A, B, out=None, variant="prod", config: int = -1, stream=None):
    """C = A x B on the GPU for float32 tensors (row-major views with unit last stride)."""
    import torch

    for name, t in (("A", A), ("B", B)):
        if t.dtype != torch.float32 or not t.is_cuda:
            raise TypeError(f"{name} must be a float32 CUDA tensor")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {tuple(A.shape)} x {tuple(B.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M, N) or not out.is_cuda:
        raise TypeError("out must be a float32 CUDA tensor of shape (M, N)")
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    lda = max(_ld(A), max(1, K))
    ldb = max(_ld(B), max(1, N))
    ldc = max(_ld(out), max(1, N))
    gemm_f32_ex(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(), ldc,
                variant, config, stream)
    return out


def matmul_mixed(A, B, out=None, config: int = -1, stream=None, format=None):
    """C = A x B on the GPU for bfloat16 or float16 tensors, fp32 result.

    A and B must share one 16-bit dtype (or be int16 / uint16 codes with
    ``format`` given) and have unit last stride.
    """
    import torch

    kinds = {torch.bfloat16: "bf16", torch.float16: "f16"}
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    if A.dtype in kinds:
        fmt = kinds[A.dtype] if format is None else format
        if format is not None and _format(format) != MIXED_FORMATS[kinds[A.dtype]]:
            raise TypeError(f"format {format!r} does not match dtype {A.dtype}")
    elif A.dtype in (torch.int16, torch.uint16) and format is not None:
        fmt = format
    else:
        raise TypeError("A and B must be bfloat16 / float16 tensors (or 16-bit codes with format=)")
    if not (A.is_cuda and B.is_cuda):
        raise TypeError("A and B must be CUDA tensors")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {tuple(A.shape)} x {tuple(B.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M, N) or not out.is_cuda:
        raise TypeError("out must be a float32 CUDA tensor of shape (M, N)")
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    lda = max(_ld(A), max(1, K))
    ldb = max(_ld(B), max(1, N))
    ldc = max(_ld(out), max(1, N))
    gemm_mixed(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(), ldc, fmt,
               config, stream)
    return out


def matmul_splitk(A, B, out=None, config: int = -1, splits: int = 0, workspace=None, stream=None):
    """C = A x B through the split-K plan, for float32 CUDA tensors.

    ``workspace`` is a CUDA tensor of at least the plan's workspace bytes; when
    None, one is allocated with torch for this call.
    """
    import torch

    for name, t in (("A", A), ("B", B)):
        if t.dtype != torch.float32 or not t.is_cuda:
            raise TypeError(f"{name} must be a float32 CUDA tensor")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {tuple(A.shape)} x {tuple(B.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M, N) or not out.is_cuda:
        raise TypeError("out must be a float32 CUDA tensor of shape (M, N)")
    plan = gemm_f32_splitk_plan(M, N, K, config, splits)
    if workspace is None and plan["workspace_bytes"] > 0:
        workspace = torch.empty(plan["workspace_bytes"] // 4, dtype=torch.float32, device=A.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    lda = max(_ld(A), max(1, K))
    ldb = max(_ld(B), max(1, N))
    ldc = max(_ld(out), max(1, N))
    gemm_f32_splitk(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(), ldc, config,
                    splits, ws_ptr, ws_bytes, stream)
    return out
