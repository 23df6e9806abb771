"""The page-read ceiling probe bench.py runs beside the step (libdsa_probe.so):
its argument checks (host only) and, on the GPU, that it really reads every
page of its list -- its per-lane checksum is the XOR of the first dword of the
lane's 16-byte slot over the wave's run of pages, computed here on the host."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "sparse_attention_fp8_amd", "libdsa_probe.so")
PAGE = 64 * 132
HIP_ERROR_INVALID_VALUE = 1


def probe():
    # torch first, so the library binds to the HIP runtime torch already loaded
    import torch  # noqa: F401
    lib = ctypes.CDLL(PROBE)
    lib.dsa_probe_page_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.dsa_probe_page_read.restype = ctypes.c_int
    return lib


def test_probe_rejects_bad_arguments_before_launching():
    lib = probe()
    fake = ctypes.c_void_p(0x10000)     # never dereferenced: every call fails validation
    assert lib.dsa_probe_page_read(None, PAGE, fake, 1, fake, 1, None) == HIP_ERROR_INVALID_VALUE
    assert lib.dsa_probe_page_read(fake, PAGE, None, 1, fake, 1, None) == HIP_ERROR_INVALID_VALUE
    assert lib.dsa_probe_page_read(fake, PAGE, fake, 1, None, 1, None) == HIP_ERROR_INVALID_VALUE
    assert lib.dsa_probe_page_read(fake, PAGE - 1, fake, 1, fake, 1, None) == HIP_ERROR_INVALID_VALUE
    assert lib.dsa_probe_page_read(fake, PAGE, fake, -1, fake, 1, None) == HIP_ERROR_INVALID_VALUE
    assert lib.dsa_probe_page_read(fake, PAGE, fake, 1, fake, 0, None) == HIP_ERROR_INVALID_VALUE


@pytest.mark.gpu
@pytest.mark.parametrize("total,grid,stride", [(1, 1, PAGE), (37, 2, PAGE), (700, 3, PAGE + 256), (5000, 4, PAGE)])
def test_probe_reads_every_listed_page(total, grid, stride):
    import torch
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(total)
    npool = 97
    pool = rng.integers(0, 256, size=npool * stride, dtype=np.uint8)
    ids = rng.integers(0, npool, size=total, dtype=np.int32)
    out = torch.zeros(grid * 512, dtype=torch.int32, device=dev)
    pool_d = torch.from_numpy(pool).to(dev)
    ids_d = torch.from_numpy(ids).to(dev)
    rc = probe().dsa_probe_page_read(ctypes.c_void_p(pool_d.data_ptr()), stride, ctypes.c_void_p(ids_d.data_ptr()),
                                     total, ctypes.c_void_p(out.data_ptr()), grid,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32).reshape(grid * 8, 64)
    words = pool.reshape(npool, stride)[:, :64 * 16].reshape(npool, 64, 16)[:, :, :4].copy().view(np.uint32)[:, :, 0]
    nw = grid * 8
    for w in range(nw):
        p0, p1 = total * w // nw, total * (w + 1) // nw
        want = np.zeros(64, np.uint32)
        for p in range(p0, p1):
            want ^= words[ids[p]]
        assert np.array_equal(got[w], want), f"wave {w}: pages {p0}..{p1}"
