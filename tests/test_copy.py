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


@pytest.mark.parametrize("nsrc", [1, 2, 3])
@pytest.mark.parametrize("ndst", [0, 1, 2])
@pytest.mark.parametrize("vectors", [1, 257, 3 * 4096 + 5])
def test_stream_exact(nsrc, ndst, vectors):
    # destination 0 = xor of the sources, destination 1 = their sum (uint32
    # lanes, wrapping); bytes after the range are left alone
    case(f"hbm_stream {nsrc}R{ndst}W {vectors} x 16 B")
    g = torch.Generator(device="cuda").manual_seed(nsrc * 10 + ndst)
    n = vectors * 4
    srcs = [torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, device="cuda",
                          generator=g) for _ in range(nsrc)]
    dsts = [torch.full((n + 4,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
            for _ in range(ndst)]
    mb.hbm_stream(srcs, [d[:n] for d in dsts])
    torch.cuda.synchronize()
    x = srcs[0].clone()
    s = srcs[0].to(torch.int64)
    for t in srcs[1:]:
        x ^= t
        s = s + t.to(torch.int64)
    s = ((s + 2**31) % 2**32 - 2**31).to(torch.int32)
    for k, d in enumerate(dsts):
        assert torch.equal(d[:n], x if k == 0 else s)
        assert (d[n:] == 0x5A5A5A5A).all()


def test_stream_rejects_bad_arguments():
    case("hbm_stream argument checks")
    a = torch.zeros(64, dtype=torch.int32, device="cuda")
    b = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):
        mb.hbm_stream([a[:16]], [a[8:24]])          # destination over its source
    with pytest.raises(RuntimeError):
        mb.hbm_stream([a[:16]], [b[:16], b[8:24]])  # destinations overlap
    with pytest.raises(RuntimeError):
        mb.hbm_stream([a[1:5]], [b[:4]])            # misaligned source
    with pytest.raises(RuntimeError):
        mb.hbm_stream([a[:4]] * 4, [b[:4]])         # four sources
