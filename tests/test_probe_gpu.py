"""The measured-ceiling probe runs and reports the work it does."""
import pytest

pytestmark = pytest.mark.gpu


def test_mfma_probe_runs_and_counts():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tiled_dense_gemm_loop_amd as t
    t.load_library()
    for code in (t.TDG_DTYPE_F16F32, t.TDG_DTYPE_I8I32, t.TDG_DTYPE_F32F32):
        sink = t.tdg_mfma_probe(code, 8)
        torch.cuda.synchronize()
        assert torch.isfinite(sink).all()
        k = {t.TDG_DTYPE_F16F32: 16, t.TDG_DTYPE_I8I32: 32, t.TDG_DTYPE_F32F32: 2}[code]
        assert t.tdg_mfma_probe_ops(code, 8) == 2 * 32 * 32 * k * 8 * 8 * 2048
    with pytest.raises(t.TdgError):
        t.tdg_mfma_probe(t.TDG_DTYPE_F16F32, 6)   # not a multiple of 4
