"""ctypes binding of libtdgemm.so (the C ABI in include/tdgemm.h).

Argument marshalling only: every step of the product runs in the library's
HIP kernels.  Tensors give device pointers, shapes and row strides; the
stream is torch's current stream on the operands' device.  There is no CPU
fallback -- a missing library or device raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtdgemm.so")

TDG_OK = 0
TDG_ERR_INVALID_ARG = -1
TDG_ERR_UNSUPPORTED = -2
TDG_ERR_LAUNCH = -3
TDG_ERR_NO_DEVICE = -4
TDG_ERR_SCRATCH = -5
TDG_NOALLOC_SCRATCH_BYTES = 32 << 20

TDG_DTYPE_F16F32 = 0
TDG_DTYPE_I8I32 = 1
TDG_DTYPE_F32F32 = 2

TDG_VARIANT_AUTO = 0
TDG_VARIANT_SINGLE = 1
TDG_VARIANT_REG_PREFETCH = 2
TDG_VARIANT_DIRECT_LDS = 3
TDG_DEBUG_POISON_LDS = 1
TDG_DEBUG_NO_K_ROTATION = 2

VARIANT_NAMES = {0: "auto", 1: "single", 2: "reg_prefetch", 3: "direct_lds"}

TDG_TRANSPOSE_AUTO = 0
TDG_TRANSPOSE_NAIVE = 1
TDG_TRANSPOSE_LDS = 2
TDG_TRANSPOSE_LDS_PADDED = 3
TDG_TRANSPOSE_LDS_SWIZZLED = 4
TDG_TRANSPOSE_VEC = 5

TRANSPOSE_NAMES = {1: "naive", 2: "lds", 3: "lds_padded", 4: "lds_swizzled", 5: "vec"}

# Every symbol include/tdgemm.h declares.
EXPORTED = (
    "gemm_f16f32", "gemm_i8i32", "gemm_f16f32_pipelined", "gemm_i8i32_pipelined",
    "gemm_f16f32_ex", "gemm_i8i32_ex", "gemm_f32f32", "gemm_f32f32_pipelined", "gemm_f32f32_ex",
    "tdg_plan", "tdg_plan_operands", "tdg_tile_figures", "tdg_config_count",
    "tdg_config_at", "tdg_status_string", "tdg_set_debug_flags", "tdg_copy_f32", "tdg_transpose_f32",
    "tdg_mfma_probe", "tdg_mfma_probe_ops", "tdg_mfma_probe_sink_floats", "tdg_lds_probe",
    "tdg_lds_probe_bytes",
    "gemm_f16f32_splitk", "gemm_i8i32_splitk", "gemm_f32f32_splitk", "tdg_splitk_plan",
    "tdg_config_resources", "gemm_splitk_noalloc", "tdg_predict_us",
)


class TdgKernelResources(ctypes.Structure):
    _fields_ = [("vgprs", ctypes.c_int), ("spill_bytes", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("threads", ctypes.c_int), ("wg_per_cu", ctypes.c_int)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class TdgConfig(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int), ("bn", ctypes.c_int), ("bk", ctypes.c_int),
                ("waves", ctypes.c_int), ("lds_stages", ctypes.c_int), ("variant", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class TdgPlanInfo(ctypes.Structure):
    _fields_ = [("ratio", ctypes.c_double), ("band", ctypes.c_int), ("lds_bytes", ctypes.c_size_t),
                ("wg_per_cu", ctypes.c_int), ("num_tiles", ctypes.c_int64),
                ("grid", ctypes.c_int64), ("est_regs", ctypes.c_int), ("guarded", ctypes.c_int),
                ("need_bytes_per_clk", ctypes.c_double), ("mfma_per_load", ctypes.c_double),
                ("pipelined", ctypes.c_int), ("k_rotated", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class TdgError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: %s (status %d)" % (what, status_string(status), status))
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libtdgemm.so (built by tiled_dense_gemm_loop_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch ships its own HIP runtime under the same soname
    # (libamdhip64.so.7).  Loading torch first makes this library bind to
    # that one runtime, so device pointers and torch's hipStream_t handles
    # mean the same thing on both sides; loading the library first would put
    # a second HIP runtime into the process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError("libtdgemm.so is not built (%s); run __graft_entry__.build() or "
                          "python tiled_dense_gemm_loop_amd/build.py" % path)
    lib = ctypes.CDLL(path)
    i64, vp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    gemm_args = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    for name in ("gemm_f16f32", "gemm_i8i32", "gemm_f16f32_pipelined", "gemm_i8i32_pipelined",
                 "gemm_f32f32", "gemm_f32f32_pipelined"):
        fn = getattr(lib, name)
        fn.argtypes = gemm_args
        fn.restype = c_int
    for name in ("gemm_f16f32_ex", "gemm_i8i32_ex", "gemm_f32f32_ex"):
        fn = getattr(lib, name)
        fn.argtypes = gemm_args + [ctypes.POINTER(TdgConfig)]
        fn.restype = c_int
    lib.tdg_plan.argtypes = [c_int, i64, i64, i64, ctypes.POINTER(TdgConfig),
                             ctypes.POINTER(TdgPlanInfo)]
    lib.tdg_plan.restype = c_int
    lib.tdg_plan_operands.argtypes = [c_int, i64, i64, i64, ctypes.c_void_p, i64, ctypes.c_void_p, i64,
                                      ctypes.POINTER(TdgConfig), ctypes.POINTER(TdgPlanInfo)]
    lib.tdg_plan_operands.restype = c_int
    lib.tdg_tile_figures.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, i64, i64,
                                     i64, ctypes.POINTER(TdgPlanInfo)]
    lib.tdg_tile_figures.restype = c_int
    lib.tdg_config_count.argtypes = [c_int]
    lib.tdg_config_count.restype = c_int
    lib.tdg_config_at.argtypes = [c_int, c_int, ctypes.POINTER(TdgConfig)]
    lib.tdg_config_at.restype = c_int
    lib.tdg_config_resources.argtypes = [c_int, c_int, ctypes.POINTER(TdgKernelResources)]
    lib.tdg_config_resources.restype = c_int
    lib.tdg_status_string.argtypes = [c_int]
    lib.tdg_status_string.restype = ctypes.c_char_p
    lib.tdg_set_debug_flags.argtypes = [c_int]
    lib.tdg_set_debug_flags.restype = c_int
    for name in ("gemm_f16f32_splitk", "gemm_i8i32_splitk", "gemm_f32f32_splitk"):
        fn = getattr(lib, name)
        fn.argtypes = gemm_args[:9] + [c_int, vp, ctypes.c_size_t, vp]
        fn.restype = c_int
    lib.tdg_predict_us.argtypes = [c_int, c_int, c_int, c_int, c_int, i64, i64, i64,
                                   ctypes.POINTER(ctypes.c_double)]
    lib.tdg_predict_us.restype = c_int
    lib.gemm_splitk_noalloc.argtypes = [c_int] + gemm_args[:9] + [c_int, vp]
    lib.gemm_splitk_noalloc.restype = c_int
    lib.tdg_splitk_plan.argtypes = [c_int, i64, i64, i64, ctypes.POINTER(c_int),
                                    ctypes.POINTER(ctypes.c_size_t)]
    lib.tdg_splitk_plan.restype = c_int
    lib.tdg_copy_f32.argtypes = [i64, i64, vp, i64, vp, i64, vp]
    lib.tdg_copy_f32.restype = c_int
    lib.tdg_transpose_f32.argtypes = [c_int, i64, i64, vp, i64, vp, i64, vp]
    lib.tdg_transpose_f32.restype = c_int
    lib.tdg_mfma_probe.argtypes = [c_int, i64, vp, vp]
    lib.tdg_mfma_probe.restype = c_int
    lib.tdg_mfma_probe_ops.argtypes = [c_int, i64]
    lib.tdg_mfma_probe_ops.restype = i64
    lib.tdg_mfma_probe_sink_floats.argtypes = []
    lib.tdg_mfma_probe_sink_floats.restype = i64
    lib.tdg_lds_probe.argtypes = [c_int, i64, vp, vp]
    lib.tdg_lds_probe.restype = c_int
    lib.tdg_lds_probe_bytes.argtypes = [c_int, i64]
    lib.tdg_lds_probe_bytes.restype = i64
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().tdg_status_string(status).decode()


# ------------------------------------------------------------------ raw calls

_FNS = {}


def _fn(name: str):
    """The library's entry point `name` (looked up once)."""
    f = _FNS.get(name)
    if f is None:
        f = _FNS[name] = getattr(load_library(), name)
    return f


def call_raw(name: str, M, N, K, a_ptr, lda, b_ptr, ldb, c_ptr, ldc, stream=0, cfg=None) -> int:
    """Call a GEMM entry point with raw device pointers; returns the status."""
    fn = getattr(load_library(), name)
    args = [M, N, K, a_ptr, lda, b_ptr, ldb, c_ptr, ldc, stream]
    if name.endswith("_ex"):
        args.append(ctypes.byref(cfg) if cfg is not None else None)
    return fn(*args)


# -------------------------------------------------------------- torch tensors

def _torch():
    import torch
    return torch


_raw_stream_fn = None


def _stream_handle(device_index: int) -> int:
    """The hipStream_t of torch's current stream on a device.  torch's raw
    query returns the handle directly (~0.1 us); the public
    torch.cuda.current_stream(...).cuda_stream builds a Stream object first
    (~2.7 us per call, most of a small GEMM's host cost), so it is only the
    fallback."""
    global _raw_stream_fn
    torch = _torch()
    if _raw_stream_fn is None:
        fn = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _raw_stream_fn = fn if fn is not None else (
            lambda dev: torch.cuda.current_stream(dev).cuda_stream)
    return _raw_stream_fn(device_index)


def _matrix(t, dtypes, what):
    shape = t.shape
    if len(shape) != 2:
        raise ValueError("%s must be 2-D, got shape %s" % (what, tuple(shape)))
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s; expected one of %s" % (what, t.dtype, dtypes))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % what)
    rows, cols = shape
    if rows == 0 or cols == 0:
        return rows, cols, t.data_ptr(), max(cols, 1)
    st = t.stride()
    if cols > 1 and st[1] != 1:
        raise ValueError("%s: elements within a row must be contiguous" % what)
    ld = st[0] if rows > 1 else cols
    return rows, cols, t.data_ptr(), max(ld, 1)


def _gemm(name, A, B, C, cfg, f16, splitk=None):
    """f16: True (binary16 in), False (int8 in) or "f32" (binary32 in)."""
    torch = _torch()
    if f16 == "f32":
        in_types = (torch.float32,)
    else:
        in_types = (torch.float16, torch.int16) if f16 else (torch.int8,)
    M, K, pa, lda = _matrix(A, in_types, "A")
    K2, N, pb, ldb = _matrix(B, in_types, "B")
    if K != K2:
        raise ValueError("inner dimensions differ: A is %dx%d, B is %dx%d" % (M, K, K2, N))
    if A.device != B.device:
        raise ValueError("A and B are on different devices")
    out_type = torch.float32 if f16 else torch.int32  # "f32" is truthy
    if C is None:
        C = torch.empty((M, N), dtype=out_type, device=A.device)
    Mc, Nc, pc, ldc = _matrix(C, (out_type,), "C")
    if (Mc, Nc) != (M, N):
        raise ValueError("C has shape %s, expected %s" % ((Mc, Nc), (M, N)))
    if C.device != A.device:
        raise ValueError("C is on %s, A and B on %s" % (C.device, A.device))
    fn = _fn(name)
    tail = (ctypes.byref(cfg) if cfg is not None else None,) if name.endswith("_ex") else ()
    mid = ()
    if splitk is not None:  # (parts, workspace tensor or None)
        parts, ws = splitk
        parts = int(parts)
        if parts < 0:
            raise ValueError("parts must be >= 0 (0: the planner's choice), got %d" % parts)
        if ws is None:
            if parts == 0:  # the planner's choice, planned here to size the workspace
                parts, need = tdg_splitk_plan(
                    {"gemm_f16f32_splitk": TDG_DTYPE_F16F32, "gemm_i8i32_splitk": TDG_DTYPE_I8I32,
                     "gemm_f32f32_splitk": TDG_DTYPE_F32F32}[name], M, N, K)
            else:
                need = parts * M * N * 4 if parts > 1 else 0
            # parts == 1 runs the plain product, which needs no workspace
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=A.device) if parts > 1 else None
        elif not ws.is_cuda or ws.device != A.device or not ws.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on %s" % A.device)
        mid = (parts, ws.data_ptr() if ws is not None else None,
               ws.numel() * ws.element_size() if ws is not None else 0)
    dev = A.device.index
    cur = torch.cuda.current_device()
    if dev is None or dev == cur:
        rc = fn(M, N, K, pa, lda, pb, ldb, pc, ldc, *mid, _stream_handle(cur), *tail)
    else:
        with torch.cuda.device(A.device):
            rc = fn(M, N, K, pa, lda, pb, ldb, pc, ldc, *mid, _stream_handle(dev), *tail)
    if rc != TDG_OK:
        raise TdgError(rc, name)
    return C


def _cfg(cfg):
    if cfg is None or isinstance(cfg, TdgConfig):
        return cfg
    c = TdgConfig()
    for k, v in dict(cfg).items():
        setattr(c, k, int(v))
    return c


def gemm_f16f32(A, B, C=None):
    """Sequential single-buffer baseline: C (float32) = A . B (float16)."""
    return _gemm("gemm_f16f32", A, B, C, None, True)


def gemm_i8i32(A, B, C=None):
    """Sequential single-buffer baseline: C (int32) = A . B (int8)."""
    return _gemm("gemm_i8i32", A, B, C, None, False)


def gemm_f16f32_pipelined(A, B, C=None):
    """Software-pipelined double-buffered K loop, FP16 -> FP32."""
    return _gemm("gemm_f16f32_pipelined", A, B, C, None, True)


def gemm_i8i32_pipelined(A, B, C=None):
    """Software-pipelined double-buffered K loop, INT8 -> INT32."""
    return _gemm("gemm_i8i32_pipelined", A, B, C, None, False)


def gemm_f16f32_ex(A, B, C=None, cfg=None):
    """Explicit configuration (dict or TdgConfig; zero fields are planned)."""
    return _gemm("gemm_f16f32_ex", A, B, C, _cfg(cfg), True)


def gemm_i8i32_ex(A, B, C=None, cfg=None):
    return _gemm("gemm_i8i32_ex", A, B, C, _cfg(cfg), False)


def gemm_f32f32(A, B, C=None):
    """Sequential single-buffer baseline: C (float32) = A . B (float32)."""
    return _gemm("gemm_f32f32", A, B, C, None, "f32")


def gemm_f32f32_pipelined(A, B, C=None):
    """Software-pipelined double-buffered K loop, FP32 -> FP32."""
    return _gemm("gemm_f32f32_pipelined", A, B, C, None, "f32")


def gemm_f32f32_ex(A, B, C=None, cfg=None):
    return _gemm("gemm_f32f32_ex", A, B, C, _cfg(cfg), "f32")


def tdg_plan(dtype: int, M: int, N: int, K: int, cfg=None):
    """(config dict, plan-info dict) the planner picks for this shape."""
    c = _cfg(cfg) or TdgConfig()
    info = TdgPlanInfo()
    rc = load_library().tdg_plan(dtype, M, N, K, ctypes.byref(c), ctypes.byref(info))
    if rc != TDG_OK:
        raise TdgError(rc, "tdg_plan")
    return c.as_dict(), info.as_dict()


def tdg_plan_operands(dtype: int, M: int, N: int, K: int, a_addr: int, lda: int, b_addr: int, ldb: int,
                      cfg=None):
    """(config dict, plan-info dict) a call on operands at these addresses
    and leading dimensions would run; the addresses are only compared."""
    c = _cfg(cfg) or TdgConfig()
    info = TdgPlanInfo()
    rc = load_library().tdg_plan_operands(dtype, M, N, K, ctypes.c_void_p(a_addr), lda,
                                          ctypes.c_void_p(b_addr), ldb, ctypes.byref(c), ctypes.byref(info))
    if rc != TDG_OK:
        raise TdgError(rc, "tdg_plan_operands")
    return c.as_dict(), info.as_dict()


def tdg_tile_figures(dtype: int, bm: int, bn: int, bk: int, waves: int = 4, stages: int = 1,
                     variant: int = TDG_VARIANT_SINGLE, M: int = 0, N: int = 0, K: int = 0) -> dict:
    """The planner's arithmetic (ratio, band, LDS bytes, WG/CU, ...) for any tile."""
    info = TdgPlanInfo()
    rc = load_library().tdg_tile_figures(dtype, bm, bn, bk, waves, stages, variant, M, N, K,
                                         ctypes.byref(info))
    if rc != TDG_OK:
        raise TdgError(rc, "tdg_tile_figures")
    return info.as_dict()


def tdg_predict_us(dtype: int, bm: int, bn: int, waves: int, stages: int, M: int, N: int,
                   K: int) -> float:
    """The planner's predicted kernel time (us) of one measured configuration
    for an M x N x K product."""
    us = ctypes.c_double()
    rc = load_library().tdg_predict_us(dtype, bm, bn, waves, stages, M, N, K, ctypes.byref(us))
    if rc != TDG_OK:
        raise TdgError(rc, "tdg_predict_us")
    return us.value


def tdg_splitk_plan(dtype: int, M: int, N: int, K: int):
    """(parts, workspace bytes) the split-K entry points choose for this product."""
    parts, ws = ctypes.c_int(), ctypes.c_size_t()
    rc = load_library().tdg_splitk_plan(dtype, M, N, K, ctypes.byref(parts), ctypes.byref(ws))
    if rc != TDG_OK:
        raise TdgError(rc, "tdg_splitk_plan")
    return parts.value, ws.value


def gemm_f16f32_splitk(A, B, C=None, parts: int = 0, workspace=None):
    """C (float32) = A . B (float16) with K split over `parts` (0: planner's
    choice); the workspace is allocated here when not given."""
    return _gemm("gemm_f16f32_splitk", A, B, C, None, True, splitk=(parts, workspace))


def gemm_i8i32_splitk(A, B, C=None, parts: int = 0, workspace=None):
    """C (int32) = A . B (int8) with K split over `parts`; exact."""
    return _gemm("gemm_i8i32_splitk", A, B, C, None, False, splitk=(parts, workspace))


def gemm_f32f32_splitk(A, B, C=None, parts: int = 0, workspace=None):
    """C (float32) = A . B (float32) with K split over `parts`."""
    return _gemm("gemm_f32f32_splitk", A, B, C, None, "f32", splitk=(parts, workspace))


def gemm_splitk_noalloc(A, B, C=None, parts: int = 0):
    """C = A . B with K split over `parts` (0: the planner's count among those
    that fit), the partial products kept in the library's built-in scratch
    array: the library allocates nothing (C is allocated here when not
    given).  The dtype follows A and B: float16 -> float32 C, int8 -> int32,
    float32 -> float32.  Calls that overlap in time on one GPU race on the
    array; calls on one stream do not."""
    torch = _torch()
    dt = {torch.float16: TDG_DTYPE_F16F32, torch.int16: TDG_DTYPE_F16F32,
          torch.int8: TDG_DTYPE_I8I32, torch.float32: TDG_DTYPE_F32F32}.get(A.dtype)
    if dt is None:
        raise TypeError("A has dtype %s; expected float16, int8 or float32" % A.dtype)
    in_types = {TDG_DTYPE_F16F32: (torch.float16, torch.int16), TDG_DTYPE_I8I32: (torch.int8,),
                TDG_DTYPE_F32F32: (torch.float32,)}[dt]
    M, K, pa, lda = _matrix(A, in_types, "A")
    K2, N, pb, ldb = _matrix(B, in_types, "B")
    if K != K2:
        raise ValueError("inner dimensions differ: A is %dx%d, B is %dx%d" % (M, K, K2, N))
    if A.device != B.device:
        raise ValueError("A and B are on different devices")
    out_type = torch.int32 if dt == TDG_DTYPE_I8I32 else torch.float32
    if C is None:
        C = torch.empty((M, N), dtype=out_type, device=A.device)
    Mc, Nc, pc, ldc = _matrix(C, (out_type,), "C")
    if (Mc, Nc) != (M, N):
        raise ValueError("C has shape %s, expected %s" % ((Mc, Nc), (M, N)))
    if C.device != A.device:
        raise ValueError("C is on %s, A and B on %s" % (C.device, A.device))
    with torch.cuda.device(A.device):
        rc = _fn("gemm_splitk_noalloc")(dt, M, N, K, pa, lda, pb, ldb, pc, ldc, int(parts),
                                         _stream_handle(A.device.index))
    if rc != TDG_OK:
        raise TdgError(rc, "gemm_splitk_noalloc")
    return C


def tdg_set_debug_flags(flags: int) -> int:
    """Sets the process-wide TDG_DEBUG_* bits; returns the previous ones."""
    rc = load_library().tdg_set_debug_flags(flags)
    if rc < 0:
        raise TdgError(rc, "tdg_set_debug_flags")
    return rc


def tdg_config_count(dtype: int) -> int:
    return load_library().tdg_config_count(dtype)


def tdg_config_at(dtype: int, index: int) -> dict:
    c = TdgConfig()
    rc = load_library().tdg_config_at(dtype, index, ctypes.byref(c))
    if rc != TDG_OK:
        raise TdgError(rc, "tdg_config_at")
    return c.as_dict()


def tdg_config_resources(dtype: int, index: int) -> dict:
    """Registers, spill bytes, LDS bytes, threads and runtime workgroups per
    CU of the index-th built configuration's kernel (needs the GPU)."""
    r = TdgKernelResources()
    rc = load_library().tdg_config_resources(dtype, index, ctypes.byref(r))
    if rc != TDG_OK:
        raise TdgError(rc, "tdg_config_resources")
    return r.as_dict()


def tdg_status_string(status: int) -> str:
    return status_string(status)


# ------------------------------------------------------ copy / transpose ladder

def _move(x, out, transpose, method):
    torch = _torch()
    rows, cols, px, ldi = _matrix(x, (torch.float32,), "in")
    shape = (cols, rows) if transpose else (rows, cols)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    orow, ocol, po, ldo = _matrix(out, (torch.float32,), "out")
    if (orow, ocol) != shape:
        raise ValueError("out has shape %s, expected %s" % ((orow, ocol), shape))
    if out.device != x.device:
        raise ValueError("out is on %s, in on %s" % (out.device, x.device))
    lib = load_library()
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        if transpose:
            rc = lib.tdg_transpose_f32(int(method), rows, cols, px, ldi, po, ldo, stream)
        else:
            rc = lib.tdg_copy_f32(rows, cols, px, ldi, po, ldo, stream)
    if rc != TDG_OK:
        raise TdgError(rc, "tdg_transpose_f32" if transpose else "tdg_copy_f32")
    return out


def tdg_copy_f32(x, out=None):
    """out[i][j] = x[i][j] (float32, device tensors; rows may be strided)."""
    return _move(x, out, False, 0)


def tdg_transpose_f32(x, out=None, method=TDG_TRANSPOSE_AUTO):
    """out[j][i] = x[i][j] with one of the ladder's methods."""
    return _move(x, out, True, method)


# ------------------------------------------------------ measured compute ceiling

def tdg_mfma_probe_ops(dtype: int, iters: int) -> int:
    """Operations one tdg_mfma_probe launch performs."""
    return load_library().tdg_mfma_probe_ops(dtype, iters)


def tdg_mfma_probe_sink_floats() -> int:
    return load_library().tdg_mfma_probe_sink_floats()


LDS_PROBE_MODES = {"b128": 0, "b64_tr_b16": 1, "b64": 2}


def tdg_lds_probe_bytes(mode: int, iters: int) -> int:
    """Bytes one workgroup of tdg_lds_probe reads."""
    return load_library().tdg_lds_probe_bytes(mode, iters)


def tdg_lds_probe(mode: int, iters: int = 4096, out=None) -> float:
    """Run the LDS read-rate kernel on the current stream and wait for it;
    returns the mean bytes per shader clock per compute unit."""
    torch = _torch()
    if out is None:
        out = torch.zeros(512, dtype=torch.int32, device="cuda")
    if out.dtype != torch.int32 or out.numel() < 512 or not out.is_cuda:
        raise ValueError("out must be a device int32 tensor of at least 512 elements")
    lib = load_library()
    with torch.cuda.device(out.device):
        stream = torch.cuda.current_stream(out.device).cuda_stream
        rc = lib.tdg_lds_probe(mode, iters, out.data_ptr(), stream)
    if rc != TDG_OK:
        raise TdgError(rc, "tdg_lds_probe")
    torch.cuda.synchronize(out.device)
    cycles = out[:256].cpu().long() & 0xFFFFFFFF
    return tdg_lds_probe_bytes(mode, iters) / float(cycles.double().mean())


def tdg_mfma_probe(dtype: int, iters: int, sink=None):
    """Launch the MFMA-only kernel on the current stream; returns the sink
    tensor (allocated when not given)."""
    torch = _torch()
    n = tdg_mfma_probe_sink_floats()
    if sink is None:
        sink = torch.empty(n, dtype=torch.float32, device="cuda")
    if sink.dtype != torch.float32 or sink.numel() < n or not sink.is_cuda:
        raise ValueError("sink must be a device float32 tensor of at least %d elements" % n)
    lib = load_library()
    with torch.cuda.device(sink.device):
        stream = torch.cuda.current_stream(sink.device).cuda_stream
        rc = lib.tdg_mfma_probe(dtype, iters, sink.data_ptr(), stream)
    if rc != TDG_OK:
        raise TdgError(rc, "tdg_mfma_probe")
    return sink
