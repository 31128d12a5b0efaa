"""The MFMA-only probe behind bench.py's measured peaks: it runs, writes
finite sinks, and reports a sustained rate between a third of the published
dense peak and that peak (plus 5 % for timing)."""
import pytest
import torch

import attention_fa_fwd_04_amd as fa

pytestmark = pytest.mark.gpu

SPEC = {0: 2516.6, 1: 5033.2, 2: 5033.2}      # TFLOP/s (TOP/s) at 2.4 GHz, dense


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_mfma_probe(kind):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    rate = fa.mfma_peak(kind, ms_target=20.0, warmup_ms=60.0)
    print(f"probe kind {kind}: {rate:.1f} T/s = {rate / SPEC[kind]:.3f} of the published peak", flush=True)
    assert SPEC[kind] / 3 < rate < SPEC[kind] * 1.05
    out = torch.full((4 * 8,), float("nan"), device="cuda")
    assert fa.fa_mfma_probe(kind, 8, 10, out.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


def test_mfma_probe_errors():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    out = torch.empty(64, device="cuda")
    assert fa.fa_mfma_probe(0, 8, 10, None, None) == fa.FA_ERR_NULL
    assert fa.fa_mfma_probe(0, 0, 10, out.data_ptr(), None) == fa.FA_ERR_SHAPE
    assert fa.fa_mfma_probe(5, 8, 10, out.data_ptr(), None) == fa.FA_ERR_ARG
