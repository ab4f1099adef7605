"""ltc_compress_noalloc (workspace in the library's own device array) against
ltc_compress (caller's workspace), both called through the C ABI: three
calls in a row on one stream, each smaller than the one before, so every
call after the first runs on the array as the previous call left it.  Blobs
and sizes must be identical byte for byte, and equal to the oracle's."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import banner

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ltc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import lossless_tensor_compression_amd as m
    m.lib()
    return m


def _inputs():
    rng = np.random.default_rng(77)
    # 1. BF16, 48 MiB (384 chunks of 128 KiB: about 53 MB of workspace),
    #    mostly N(0, sigma) with a few random-byte and constant chunks
    n = 24 << 20
    x = (rng.standard_normal(n) * np.repeat(rng.uniform(0.005, 0.05, n >> 16), 1 << 16)).astype(np.float32)
    bf = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8).copy()
    for c in (3, 100, 250):
        bf[c * 131072:(c + 1) * 131072] = rng.integers(0, 256, 131072, dtype=np.uint8)
    bf[7 * 131072:8 * 131072] = 0
    # 2. FP32, about 3 MB with a ragged last chunk, 64 KiB chunks
    f = (rng.standard_normal((3 << 20) // 4 + 3) * 0.02).astype(np.float32).view(np.uint8)
    # 3. U8, 100,003 bytes, 8 KiB chunks
    u = np.concatenate([rng.integers(0, 5, 60000), rng.integers(0, 256, 40003)]).astype(np.uint8)
    return [(bf, 1, 131072), (f, 3, 65536), (u, 0, 8192)]


def test_noalloc_equals_compress_on_three_calls_in_a_row(ltc):
    L = ltc.lib()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    cases = _inputs()
    # every device buffer exists before the first call
    bufs = []
    for data, dtype, chunk in cases:
        src = torch.from_numpy(data).cuda()
        cap = ltc.compress_bound(data.size, dtype, chunk)
        ws_n = ltc.workspace_size([data.size], dtype, chunk)
        assert ws_n <= ltc.NOALLOC_SCRATCH_BYTES
        bufs.append(dict(src=src, cap=cap, ws=torch.empty(ws_n, dtype=torch.uint8, device="cuda"),
                         a=torch.full((cap,), 0xA5, dtype=torch.uint8, device="cuda"),
                         b=torch.full((cap,), 0x5A, dtype=torch.uint8, device="cuda"),
                         na=torch.zeros(1, dtype=torch.int64, device="cuda"),
                         nb=torch.zeros(1, dtype=torch.int64, device="cuda")))
    torch.cuda.synchronize()
    for (data, dtype, chunk), bu in zip(cases, bufs):
        banner(f"noalloc: dtype {dtype}, {data.size} bytes, chunk {chunk}")
        src = ctypes.c_void_p(bu["src"].data_ptr())
        rc = L.ltc_compress(src, data.size, dtype, chunk, 0.95, ctypes.c_void_p(bu["a"].data_ptr()), bu["cap"],
                            ctypes.c_void_p(bu["na"].data_ptr()), ctypes.c_void_p(bu["ws"].data_ptr()),
                            bu["ws"].numel(), sp)
        assert rc == 0
        rc = L.ltc_compress_noalloc(src, data.size, dtype, chunk, 0.95, ctypes.c_void_p(bu["b"].data_ptr()),
                                    bu["cap"], ctypes.c_void_p(bu["nb"].data_ptr()), sp)
        assert rc == 0
        torch.cuda.synchronize()
        na, nb = int(bu["na"].item()), int(bu["nb"].item())
        assert na == nb
        got = bu["b"][:nb].cpu().numpy()
        assert np.array_equal(got, bu["a"][:na].cpu().numpy())
        want = oracle.compress(data, dtype, chunk, 0.95, nthreads=8)
        assert np.array_equal(got, want)
    # the third call left the array as its own input needed; a repeat of the
    # first (largest) call over it still gives the same blob
    data, dtype, chunk = cases[0]
    bu = bufs[0]
    bu["b"].fill_(0x33)
    rc = L.ltc_compress_noalloc(ctypes.c_void_p(bu["src"].data_ptr()), data.size, dtype, chunk, 0.95,
                                ctypes.c_void_p(bu["b"].data_ptr()), bu["cap"],
                                ctypes.c_void_p(bu["nb"].data_ptr()), sp)
    assert rc == 0
    torch.cuda.synchronize()
    nb = int(bu["nb"].item())
    assert torch.equal(bu["b"][:nb], bu["a"][:nb])


def test_noalloc_refuses_too_large_input(ltc):
    L = ltc.lib()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    fake = ctypes.c_void_p(1 << 20)
    # refused on the host, nothing launched
    assert L.ltc_compress_noalloc(fake, 1 << 30, 1, 131072, 0.95, fake, 1 << 31, fake, sp) == -7
