"""MI355X (gfx950) software-pipelined tiled dense GEMM.

C = A . B with FP16 inputs / FP32 accumulation and INT8 inputs / INT32
accumulation, plus the copy / transpose ladder on HBM, computed by
hand-written HIP kernels behind the C ABI of include/tdgemm.h.  This package is the thin Python binding of that library
(argument marshalling only) plus its build script.
"""
from ._binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    TDG_DTYPE_F16F32,
    TDG_DTYPE_I8I32,
    TDG_ERR_INVALID_ARG,
    TDG_ERR_LAUNCH,
    TDG_ERR_NO_DEVICE,
    TDG_ERR_UNSUPPORTED,
    TDG_OK,
    TDG_TRANSPOSE_AUTO,
    TDG_TRANSPOSE_LDS,
    TDG_TRANSPOSE_LDS_PADDED,
    TDG_TRANSPOSE_LDS_SWIZZLED,
    TDG_TRANSPOSE_NAIVE,
    TDG_TRANSPOSE_VEC,
    TRANSPOSE_NAMES,
    TDG_VARIANT_AUTO,
    TDG_VARIANT_DIRECT_LDS,
    TDG_VARIANT_REG_PREFETCH,
    TDG_VARIANT_SINGLE,
    VARIANT_NAMES,
    TdgConfig,
    TdgError,
    TdgPlanInfo,
    call_raw,
    gemm_f16f32,
    gemm_f16f32_ex,
    gemm_f16f32_pipelined,
    gemm_i8i32,
    gemm_i8i32_ex,
    gemm_i8i32_pipelined,
    load_library,
    tdg_config_at,
    tdg_config_count,
    tdg_copy_f32,
    tdg_plan,
    tdg_status_string,
    tdg_tile_figures,
    tdg_transpose_f32,
)
