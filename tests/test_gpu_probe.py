"""The two diagnostic probes (measured MFMA and HBM-read ceilings) run through
the C ABI and report plausible figures.  They are not part of the attention
path; the benchmark uses them as same-run denominators."""

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def test_mfma_probe_reports_clock_and_rate():
    import attention_sconv_amd as ink
    groups, iters = 512, 2000
    out = torch.zeros(3 * groups, dtype=torch.float32, device="cuda")
    ink.inkattn_probe_mfma_bf16(groups, iters, out)            # first launch: clocks ramp
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    ink.inkattn_probe_mfma_bf16(groups, iters, out)
    e1.record()
    torch.cuda.synchronize()
    r = out.view(groups, 3).cpu()
    assert torch.isfinite(r[:, 0]).all()
    mhz = (r[:, 1] / r[:, 2] * 100.0).median().item()
    assert 500.0 < mhz < 3000.0, mhz
    flop = groups * iters * ink.PROBE_MFMA_WAVES * ink.PROBE_MFMA_CHAINS * 32768
    tflops = flop / (e0.elapsed_time(e1) * 1e-3) / 1e12
    assert 200.0 < tflops < 2600.0, tflops


def test_stream_read_probe_runs_and_keeps_data():
    import attention_sconv_amd as ink
    buf = torch.arange(1 << 22, dtype=torch.int32, device="cuda")     # 16 MiB
    ref = buf.clone()
    out = torch.zeros(ink.PROBE_READ_GROUPS, dtype=torch.float32, device="cuda")
    for _ in range(2):
        ink.inkattn_probe_stream_read(buf, out)
    # a ragged tail: a length that is not a multiple of the grid's stride
    ink.inkattn_probe_stream_read(buf[: (1 << 22) - 4 * 1000], out)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)
