"""GPU: the library's plain 16-byte copy (the attainable-bandwidth reference
of the measurements) moves every byte exactly, for sizes below, at and past
one workgroup's 1024 vectors, and leaves the bytes after the range alone."""
import pytest
import torch

import memory_bound_row_amd as mb
from gpu_helpers import case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("vectors", [1, 255, 1023, 1024, 1025, 3 * 4096 + 7, 1 << 22])
def test_copy_exact(vectors):
    case(f"hbm_copy {vectors} x 16 B")
    g = torch.Generator(device="cuda").manual_seed(vectors)
    src = torch.randint(-2**31, 2**31 - 1, (vectors * 4 + 4,), dtype=torch.int32,
                        device="cuda", generator=g)
    dst = torch.full_like(src, 0x5A5A5A5A)
    mb.hbm_copy(src[:vectors * 4], dst[:vectors * 4])
    torch.cuda.synchronize()
    assert torch.equal(dst[:vectors * 4], src[:vectors * 4])
    assert (dst[vectors * 4:] == 0x5A5A5A5A).all()


def test_copy_rejects_misaligned():
    case("hbm_copy misaligned")
    src = torch.zeros(64, dtype=torch.int32, device="cuda")
    dst = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):
        mb.hbm_copy(src[1:5], dst[:4])
    with pytest.raises(RuntimeError):
        mb.hbm_copy(src[:3], dst[:3])
