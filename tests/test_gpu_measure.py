"""GPU check of the measurement aid fa_mfma_ceiling (libfa16measure.so, marked
gpu): it runs through its C ABI, writes one finite value per thread, and
repeats exactly."""
import pytest

from parity_util import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_mfma_ceiling_runs_and_repeats():
    from fp16_attention_amd import measure
    say("fa_mfma_ceiling iters 64")
    a = torch.full((measure.MFMA_CEILING_OUT,), float("nan"), dtype=torch.float32, device="cuda")
    b = torch.full_like(a, float("nan"))
    measure.mfma_ceiling(a, 64)
    measure.mfma_ceiling(b, 64)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all()
    assert (a != 0).any()
    assert torch.equal(a, b)
