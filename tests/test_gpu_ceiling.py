"""The bandwidth-ceiling kernels (include/qstate_ceiling.h) move exactly the
bytes they are asked to: a copy reproduces its source, an in-place
read-modify-write xors every 32-bit word with the pattern, for sizes from one
16-byte vector to several tiles with a ragged tail, with and without the
non-temporal hint, and leaves the bytes past the end untouched."""

import ctypes

import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a gfx950 GPU")]

SIZES = [16, 4096 + 16, (1 << 20) + 48, 64 << 20]


@pytest.mark.parametrize("nt", [0, 1])
@pytest.mark.parametrize("nbytes", SIZES)
def test_copy_and_rmw(nbytes, nt):
    import torch

    from bit_recurrent_state_amd._lib import check, lib
    L = lib()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    g = torch.Generator(device="cpu").manual_seed(nbytes + nt)
    guard = 4096
    src = torch.randint(0, 256, (nbytes + guard,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.randint(0, 256, (nbytes + guard,), dtype=torch.uint8, generator=g).cuda()
    dst_before = dst.clone()
    check("qstate_ceiling_copy", L.qstate_ceiling_copy(ctypes.c_void_p(src.data_ptr()),
                                                       ctypes.c_void_p(dst.data_ptr()),
                                                       nbytes, nt, sp))
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert torch.equal(dst[nbytes:], dst_before[nbytes:])

    pattern = 0x9E3779B9
    buf = src.clone()
    check("qstate_ceiling_rmw", L.qstate_ceiling_rmw(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                                     pattern, nt, sp))
    torch.cuda.synchronize()
    words = buf[:nbytes].view(torch.int32).cpu()
    want = src[:nbytes].view(torch.int32).cpu() ^ torch.tensor(pattern, dtype=torch.int64).to(torch.int32)
    assert torch.equal(words, want)
    assert torch.equal(buf[nbytes:], src[nbytes:])
