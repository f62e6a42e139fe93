"""The streaming copy kernel (the benchmark's reference rate): bit-exact on
sizes below, at and across its 32 KiB units, and on a buffer with more units
than the grid has workgroups; the bytes past the copied range stay
untouched."""

import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("nbytes", [16, 24 * 1024, 32 * 1024, 32 * 1024 + 16, (10 << 20) + 48,
                                    (80 << 20) + 16])
def test_stream_copy_bit_exact(nbytes):
    import paged_recurrent_state_amd as gdn
    gdn.load()
    g = torch.Generator(device=DEV).manual_seed(nbytes % 1000)
    n = nbytes // 4
    src = torch.randint(-2**31, 2**31 - 1, (n + 64,), dtype=torch.int32, device=DEV, generator=g)
    dst = torch.full((n + 64,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    gdn.stream_copy(dst[:n], src[:n])
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src[:n])
    assert bool((dst[n:] == 0x5A5A5A5A).all())
