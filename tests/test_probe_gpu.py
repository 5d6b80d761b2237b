"""The measured-ceiling probes (MFMA-only, LDS read rate) run and report the
work they do; the runtime's view of every built kernel matches the
planner's LDS arithmetic."""
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


def test_lds_probe_rates():
    """The LDS read-rate probe runs in every mode and counts its bytes; the
    rates it measures are what the micro-kernel's schedule assumes: 16-byte
    reads move at least 1.5 times the bytes per clock of the 8-byte
    (transposing or plain) reads, and no mode exceeds the 256 bytes per
    clock that 64 banks of 4 bytes deliver."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tiled_dense_gemm_loop_amd as t
    t.load_library()
    rates = {}
    for name, mode in t.LDS_PROBE_MODES.items():
        assert t.tdg_lds_probe_bytes(mode, 100) == 100 * 8 * 512 * (16 if mode == 0 else 8)
        rates[name] = t.tdg_lds_probe(mode, 2048)
        assert 0 < rates[name] <= 256 * 1.02, rates
    assert rates["b128"] >= 1.5 * rates["b64_tr_b16"], rates
    assert rates["b128"] >= 1.5 * rates["b64"], rates
    with pytest.raises(t.TdgError):
        t.tdg_lds_probe(3, 10)


def test_config_resources_match_the_lds_budget():
    """Every built configuration: the runtime's static LDS equals the
    planner's lds_stages x (BM*BK + BK*BN) x sizeof(T); the workgroup holds
    waves x 64 threads; no kernel spills registers; the runtime's
    workgroups per CU never exceed what 160 KiB of LDS allows."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tiled_dense_gemm_loop_amd as t
    t.load_library()
    for code in (t.TDG_DTYPE_F16F32, t.TDG_DTYPE_I8I32, t.TDG_DTYPE_F32F32):
        for i in range(t.tdg_config_count(code)):
            c = t.tdg_config_at(code, i)
            r = t.tdg_config_resources(code, i)
            fig = t.tdg_tile_figures(code, c["bm"], c["bn"], c["bk"], c["waves"], c["lds_stages"],
                                     c["variant"])
            assert r["lds_bytes"] == fig["lds_bytes"], (code, c, r)
            assert r["threads"] == 64 * c["waves"], (code, c, r)
            assert r["spill_bytes"] == 0, (code, c, r)
            assert 0 < r["vgprs"] <= 512, (code, c, r)
            assert 1 <= r["wg_per_cu"] <= max(1, 160 * 1024 // r["lds_bytes"]), (code, c, r)
    with pytest.raises(t.TdgError):
        t.tdg_config_resources(t.TDG_DTYPE_F16F32, t.tdg_config_count(t.TDG_DTYPE_F16F32))
