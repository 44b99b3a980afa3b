"""The measurement-only page-read probe (m3s_probe_page_reads) reads exactly the bytes it is
meant to: the XOR of the folded words its workgroups leave in the sink equals the XOR, on the
host, of every word of the listed pages (page modes) or of the first pages of both planes
(stream mode). A probe that skipped or repeated part of a page, or read outside it, would
disagree."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _xor_all(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(a.ravel())) if a.size else 0


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("num_sink", [1, 7, 64])
def test_probe_reads_every_listed_byte_once(gpu, mode, num_sink):
    P = 300
    g = torch.Generator().manual_seed(21 + mode)
    pay = torch.randint(0, 256, (P, 128, 64), generator=g, dtype=torch.uint8)
    scl = torch.randint(0, 256, (P, 128, 8), generator=g, dtype=torch.uint8)
    pages = torch.randperm(P, generator=g)[:211].to(torch.int32)
    sink = torch.zeros(num_sink, dtype=torch.int32, device=DEV)
    gpu.m3s_probe_page_reads(pay.to(DEV), scl.to(DEV), pages.to(DEV), mode, sink)
    torch.cuda.synchronize()
    got = _xor_all(sink.cpu().numpy().view(np.uint32))
    if mode == 2:  # the first pages.numel() pages of both planes, front to back
        n = pages.numel()
        want = _xor_all(pay[:n].numpy().view(np.uint32)) ^ _xor_all(scl[:n].numpy().view(np.uint32))
    else:
        sel = pages.long()
        want = _xor_all(pay[sel].numpy().view(np.uint32))
        s = scl[sel].numpy()
        want ^= _xor_all(s.view(np.uint16).astype(np.uint32)) if mode == 0 else _xor_all(s.view(np.uint32))
    assert got == want, (hex(got), hex(want))
