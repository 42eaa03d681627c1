"""The measurement probes: the copy probe copies bit for bit (whole buffers and a tail shorter
than a workgroup's span), and the MFMA probe runs to completion with finite outputs."""
import pytest
import torch

import streaming_kv_cache_write_amd as skv  # noqa: E402  (a missing library fails collection)
pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("nbytes", [16, 8192, 8192 + 48, 1 << 24])
def test_probe_copy_is_exact(nbytes):
    g = torch.Generator(device=DEV).manual_seed(nbytes)
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device=DEV, generator=g)
    dst = torch.zeros_like(src)
    assert skv.probe_copy(dst, src) == 2 * nbytes
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_probe_mfma_runs():
    out = torch.full((8 * 256,), float("nan"), dtype=torch.float32, device=DEV)
    assert skv.probe_mfma_bf16(out, 8, 10) == 8 * 16 * 10 * 32768
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
