"""gemm_splitk_noalloc: split K with the partial products in the library's
built-in scratch array, for callers that cannot allocate device memory.

On the GPU its output must equal the gemm_*_splitk entry point's (same part
count, so the same kernels and summation order: bit for bit) and the oracle
(INT8 exactly, FP16 / FP32 within 1e-4 * sum |a b|), on two calls in a row,
the second smaller, so that it runs over what the first left in the array.
On the CPU: argument checks and the scratch limit, before any HIP call.
"""
import ctypes

import numpy as np
import pytest

import synthetic_inputs as si
import tiled_dense_gemm_loop_amd as tdg
from conftest import no_device_only
from gpu_util import F16, F32, I8, check_f16, check_f32, check_i8, to_device

CODE = {F16: 0, I8: 1, F32: 2}
SPLITK = {F16: "gemm_f16f32_splitk", I8: "gemm_i8i32_splitk", F32: "gemm_f32f32_splitk"}


def _operands(dtype, M, N, K, seed):
    if dtype == I8:
        return si.i8_uniform(M, K, seed), si.i8_uniform(K, N, seed + 1)
    if dtype == F32:
        return si.f32_normal(M, K, seed), si.f32_normal(K, N, seed + 1)
    return si.f16_normal(M, K, seed), si.f16_normal(K, N, seed + 1)


def _check(dtype, C, A, B):
    {I8: check_i8, F16: check_f16, F32: check_f32}[dtype](C, A, B)


# --- CPU: validation and the scratch limit -----------------------------------------------

def _raw(dtype, M, N, K, lda, ldb, ldc, parts, A=1 << 40, B=1 << 44, C=1 << 46):
    lib = tdg.load_library()
    return lib.gemm_splitk_noalloc(dtype, M, N, K, A, lda, B, ldb, C, ldc, parts, None)


def test_noalloc_rejects_bad_arguments_before_the_device():
    assert _raw(7, 64, 64, 64, 64, 64, 64, 2) == tdg.TDG_ERR_INVALID_ARG     # unknown dtype
    assert _raw(0, 64, 64, 64, 64, 64, 64, -1) == tdg.TDG_ERR_INVALID_ARG    # negative parts
    assert _raw(0, 64, 64, 64, 32, 64, 64, 2) == tdg.TDG_ERR_INVALID_ARG     # lda < K
    assert _raw(1, 64, 64, 64, 64, 64, 64, 2, C=0) == tdg.TDG_ERR_INVALID_ARG  # NULL C
    assert _raw(0, 0, 64, 64, 64, 64, 64, 2) == tdg.TDG_OK                   # empty: nothing to do


def test_noalloc_refuses_partials_beyond_its_scratch():
    """parts * M * N * 4 bytes beyond the array: TDG_ERR_SCRATCH, before any
    HIP call (made-up addresses are never used)."""
    cap = tdg.TDG_NOALLOC_SCRATCH_BYTES
    M = N = 1024
    fit = cap // (M * N * 4)                     # 8 parts of 1024 x 1024 fit 32 MiB
    assert fit >= 2
    for dtype in (0, 1, 2):
        assert _raw(dtype, M, N, 8192, 8192, N, N, fit + 1) == tdg.TDG_ERR_SCRATCH
        assert _raw(dtype, M, N, 8192, 8192, N, N, 1 << 20) == tdg.TDG_ERR_SCRATCH
    assert "scratch" in tdg.tdg_status_string(tdg.TDG_ERR_SCRATCH)


@no_device_only
def test_noalloc_within_the_limit_reaches_the_device_check():
    """A count that fits, and the planner's count (limited to those that
    fit) on a product whose unlimited choice would not, get as far as the
    device check (TDG_ERR_NO_DEVICE on a host without a GPU)."""
    cap = tdg.TDG_NOALLOC_SCRATCH_BYTES
    M = N = 1024
    for dtype in (0, 1, 2):
        assert _raw(dtype, M, N, 8192, 8192, N, N, cap // (M * N * 4)) == tdg.TDG_ERR_NO_DEVICE
        assert _raw(dtype, M, N, 1 << 20, 1 << 20, N, N, 0) == tdg.TDG_ERR_NO_DEVICE
    # without the limit the planner would split this product into partials
    # larger than the array
    parts, need = tdg.tdg_splitk_plan(0, M, N, 1 << 20)
    assert parts > 1 and need > cap


# --- GPU: the same results as the split-K entry point with a workspace --------------------

@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tdg.load_library()
    return tdg


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_noalloc_equals_splitk_on_two_calls(lib, dtype):
    """Two calls in a row, the second smaller (it runs over the first call's
    partials left in the array): each equals gemm_*_splitk with the same part
    count bit for bit and the oracle within the bar.  Then the planner's
    count (parts = 0) on a few-tile, long-K product and a smaller one."""
    import torch
    splitk = getattr(lib, SPLITK[dtype])
    cases = [(512, 384, 8192, 6), (130, 70, 3000, 3),      # explicit counts, second smaller
             (256, 256, 32768, 0), (64, 64, 4096, 0)]      # the planner's, second smaller
    for i, (M, N, K, parts) in enumerate(cases):
        print("noalloc case", dtype, M, N, K, parts, flush=True)
        A, B = _operands(dtype, M, N, K, seed=500 + 10 * i)
        dA, dB = to_device(A), to_device(B)
        got = lib.gemm_splitk_noalloc(dA, dB, parts=parts)
        want = splitk(dA, dB, parts=parts)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (M, N, K, parts)
        _check(dtype, got, A, B)


@pytest.mark.gpu
def test_noalloc_through_raw_pointers_into_a_strided_output(lib):
    """The C entry point called with raw device pointers (what a caller with
    no allocator of its own does), into a view of a wider C whose padding
    must stay untouched."""
    import torch
    M, N, K, P = 200, 136, 5000, 5
    A, B = _operands(F16, M, N, K, seed=610)
    dA, dB = to_device(A), to_device(B)
    big = torch.full((M, N + 9), -3.0, dtype=torch.float32, device="cuda")
    C = big[:, 4:4 + N]
    rc = lib.load_library().gemm_splitk_noalloc(
        lib.TDG_DTYPE_F16F32, M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, C.data_ptr(), N + 9, P,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == lib.TDG_OK
    torch.cuda.synchronize()
    check_f16(C, A, B)
    assert torch.equal(C, lib.gemm_f16f32_splitk(dA, dB, parts=P))
    assert torch.all(big[:, :4] == -3.0) and torch.all(big[:, 4 + N:] == -3.0)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [F16, I8, F32])
def test_noalloc_under_graph_capture(lib, dtype):
    """The callers it is for: the allocation-free split K captured in a HIP
    graph (C allocated before the capture, the first call made outside it),
    then replayed three times with new operand values copied in between,
    the program's own eager work and synchronisations between the replays.
    Every replay equals the eager split-K call with a workspace bit for bit
    and matches the oracle."""
    import torch
    splitk = getattr(lib, SPLITK[dtype])
    M, N, K, P = 256, 192, 8192, 4
    A, B = _operands(dtype, M, N, K, seed=700)
    dA, dB = to_device(A), to_device(B)
    out_t = torch.int32 if dtype == I8 else torch.float32
    C = torch.empty((M, N), dtype=out_t, device="cuda")
    lib.gemm_splitk_noalloc(dA, dB, C, parts=P)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.gemm_splitk_noalloc(dA, dB, C, parts=P)
    for rep in range(3):
        print("noalloc graph replay", dtype, rep, flush=True)
        A, B = _operands(dtype, M, N, K, seed=710 + 10 * rep)
        dA.copy_(to_device(A))
        dB.copy_(to_device(B))
        C.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check(dtype, C, A, B)
        want = splitk(dA, dB, parts=P)
        torch.cuda.synchronize()
        assert torch.equal(C, want), rep
