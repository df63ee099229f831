"""GPU: the achievable-peak probe runs every MFMA it claims. With every
operand element equal to 1/16 (exact in bf16 and e4m3fn), each thread's sum
of accumulator elements has a closed form (mla_probe_mfma_expected), which a
dropped or repeated MFMA would miss."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_decode_04_amd as m
    m.probe_library()   # raises if the probe library is missing
    return m


@pytest.mark.parametrize("shape", [0, 1, 2], ids=["16x16x32_bf16", "32x32x16_bf16", "16x16x128_fp8"])
@pytest.mark.parametrize("wgs,iters", [(8, 16), (300, 37)])
def test_probe_results_are_exact(mla, shape, wgs, iters):
    out = torch.full((wgs * mla.PROBE_THREADS,), float("nan"), dtype=torch.float32, device="cuda:0")
    mla.mla_probe_mfma(shape, wgs, iters, 0.0625, out)
    torch.cuda.synchronize()
    want = mla.probe_library().mla_probe_mfma_expected(shape, iters, 0.0625)
    assert want > 0
    assert torch.all(out == want), f"shape {shape}: {out.min().item()}..{out.max().item()} != {want}"
