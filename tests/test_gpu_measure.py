"""GPU check of the measurement aid fa_mfma_ceiling (marked gpu): it runs
through the C ABI, writes one finite value per thread, and repeats exactly."""
import pytest

from parity_util import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_mfma_ceiling_runs_and_repeats(lib):
    say("fa_mfma_ceiling iters 64")
    a = torch.full((lib.MFMA_CEILING_OUT,), float("nan"), dtype=torch.float32, device="cuda")
    b = torch.full_like(a, float("nan"))
    lib.mfma_ceiling(a, 64)
    lib.mfma_ceiling(b, 64)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all()
    assert (a != 0).any()
    assert torch.equal(a, b)
