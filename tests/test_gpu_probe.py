"""The streaming copy probe (a measurement helper, not part of the method): an
exact byte copy through the C ABI, including sizes that leave a ragged last
workgroup."""
import numpy as np
import pytest

from hc_testutil import have_gpu, note

pytestmark = pytest.mark.gpu

if have_gpu():
    import torch
    import stream_residual_mixing_amd as hc


@pytest.mark.parametrize("nbytes", [16, 16 * 1023, 16 * 1024 + 48, 1 << 22])
def test_copy_probe_is_an_exact_copy(nbytes):
    note(f"hc_copy_probe {nbytes} bytes")
    rng = np.random.default_rng(nbytes)
    src = torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).cuda()
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    hc.hc_copy_probe(src, dst[:nbytes])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dst[:nbytes].cpu().numpy(), src.cpu().numpy())
    assert int(dst[nbytes:].abs().sum()) == 0  # nothing written past the end
