"""Every compress and decompress entry point of include/ltc.h called directly
through the C ABI on the GPU (the Python helpers route through the batch
forms): single-tensor calls, the batch calls without the general flags, the
profiling variants with their events, checksummed and delta calls, and the
host-blob decode.  Each result must equal the oracle's blob, checksums or
bytes."""
import ctypes
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, to_gpu

pytestmark = pytest.mark.gpu
VP = ctypes.c_void_p


@pytest.fixture(scope="module")
def ltc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import lossless_tensor_compression_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def hip():
    path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line)
    L = ctypes.CDLL(path)
    L.hipEventCreate.argtypes = [ctypes.POINTER(VP)]
    return L


def _events(hip, n):
    out = []
    for _ in range(n):
        e = VP()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        out.append(e.value)
    return (VP * n)(*out)


def _stream():
    return VP(torch.cuda.current_stream().cuda_stream)


def _ws(ltc, nbytes):
    n = ctypes.c_uint64()
    assert ltc.lib().ltc_compress_workspace_size(nbytes, 1, 131072, ctypes.byref(n)) == 0
    return torch.empty(max(n.value, 256), dtype=torch.uint8, device="cuda")


def _input():
    x = workloads.c1()[:300_000]
    return x, to_gpu(x, 1), x.nbytes


def _read_blob(blob, size_t):
    n = int(size_t.item())
    return blob[:n].cpu().numpy()


def test_single_and_batch_compress(ltc, hip):
    L = ltc.lib()
    x, t, nb = _input()
    want = oracle.compress(x, 1)
    cap = ltc.compress_bound(nb, 1)
    ws = _ws(ltc, nb)
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    blob = torch.empty(cap, dtype=torch.uint8, device="cuda")
    banner("ltc_compress")
    assert L.ltc_compress(VP(t.data_ptr()), nb, 1, 131072, 0.95, VP(blob.data_ptr()), cap, VP(size.data_ptr()),
                          VP(ws.data_ptr()), ws.numel(), _stream()) == 0
    assert np.array_equal(_read_blob(blob, size), want)
    banner("ltc_compress_batch and its profiling form")
    for prof in (False, True):
        blob.zero_()
        args = [1, (VP * 1)(t.data_ptr()), (ctypes.c_uint64 * 1)(nb), 1, 131072, 0.95, (VP * 1)(blob.data_ptr()),
                (ctypes.c_uint64 * 1)(cap), VP(size.data_ptr()), VP(ws.data_ptr()), ws.numel(), _stream()]
        rc = L.ltc_compress_batch_prof(*args, _events(hip, 5)) if prof else L.ltc_compress_batch(*args)
        assert rc == 0
        assert np.array_equal(_read_blob(blob, size), want)


def test_checksummed_compress(ltc, hip):
    L = ltc.lib()
    x, t, nb = _input()
    want = oracle.compress(x, 1)
    want_crc = [zlib.crc32(want[i:i + 16384].tobytes()) for i in range(0, want.size, 16384)]
    cap = ltc.compress_bound(nb, 1)
    ccap = (cap + 16383) // 16384
    ws = _ws(ltc, nb)
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    blob = torch.empty(cap, dtype=torch.uint8, device="cuda")
    crc = torch.zeros(ccap, dtype=torch.int32, device="cuda")
    banner("ltc_compress_with_crc32")
    assert L.ltc_compress_with_crc32(VP(t.data_ptr()), nb, 1, 131072, 0.95, VP(blob.data_ptr()), cap,
                                     VP(size.data_ptr()), 16384, VP(crc.data_ptr()), ccap, VP(ws.data_ptr()),
                                     ws.numel(), _stream()) == 0
    assert np.array_equal(_read_blob(blob, size), want)
    assert crc[:len(want_crc)].cpu().numpy().view(np.uint32).tolist() == want_crc
    banner("ltc_compress_batch_with_crc32 and its profiling form")
    for prof in (False, True):
        blob.zero_()
        crc.zero_()
        args = [1, (VP * 1)(t.data_ptr()), (ctypes.c_uint64 * 1)(nb), 1, 131072, 0.95, (VP * 1)(blob.data_ptr()),
                (ctypes.c_uint64 * 1)(cap), VP(size.data_ptr()), 16384, (VP * 1)(crc.data_ptr()),
                (ctypes.c_uint64 * 1)(ccap), VP(ws.data_ptr()), ws.numel(), _stream()]
        rc = (L.ltc_compress_batch_with_crc32_prof(*args, _events(hip, 6)) if prof
              else L.ltc_compress_batch_with_crc32(*args))
        assert rc == 0
        assert np.array_equal(_read_blob(blob, size), want)
        assert crc[:len(want_crc)].cpu().numpy().view(np.uint32).tolist() == want_crc


def test_decode_entry_points(ltc, hip):
    L = ltc.lib()
    x, t, nb = _input()
    want = oracle.compress(x, 1)
    hdr = bytes(want[:64])
    dblob = torch.from_numpy(want.copy()).cuda()
    dst = torch.empty(nb, dtype=torch.uint8, device="cuda")
    status = torch.full((1,), -99, dtype=torch.int32, device="cuda")
    banner("ltc_decompress")
    assert L.ltc_decompress(hdr, VP(dblob.data_ptr()), want.size, VP(dst.data_ptr()), nb, VP(status.data_ptr()),
                            _stream()) == 0
    assert int(status.item()) == 0 and np.array_equal(dst.cpu().numpy(), x.view(np.uint8))
    banner("ltc_decompress_batch_prof")
    dst.zero_()
    hdrs = (VP * 1)(ctypes.cast(ctypes.c_char_p(hdr), VP))
    assert L.ltc_decompress_batch_prof(1, hdrs, (VP * 1)(dblob.data_ptr()), (ctypes.c_uint64 * 1)(want.size),
                                       (VP * 1)(dst.data_ptr()), (ctypes.c_uint64 * 1)(nb), VP(status.data_ptr()),
                                       _stream(), _events(hip, 3)) == 0
    assert int(status.item()) == 0 and np.array_equal(dst.cpu().numpy(), x.view(np.uint8))
    banner("ltc_decompress_from_host")
    dst.zero_()
    hb = torch.empty(want.size, dtype=torch.uint8, pin_memory=True)
    hb.numpy()[:] = want
    stage = torch.empty(want.size, dtype=torch.uint8, device="cuda")
    assert L.ltc_decompress_from_host(VP(hb.data_ptr()), want.size, VP(dst.data_ptr()), nb, VP(status.data_ptr()),
                                      VP(stage.data_ptr()), stage.numel(), _stream()) == 0
    assert int(status.item()) == 0 and np.array_equal(dst.cpu().numpy(), x.view(np.uint8))


def test_delta_entry_points(ltc):
    L = ltc.lib()
    x, tb, nb = _input()
    y = x.copy()
    y[::37] ^= 3
    ty = to_gpu(y, 1)
    for flags, shared in ((0, False), (ltc.FLAG_SHARED_TABLES, True)):
        want = oracle.compress_delta(y, x, 1, shared_tables=shared)
        cap = ltc.compress_bound(nb, 1, shared_tables=shared)
        ws = _ws(ltc, nb)
        size = torch.zeros(1, dtype=torch.int64, device="cuda")
        blob = torch.empty(cap, dtype=torch.uint8, device="cuda")
        banner(f"ltc_compress_delta flags={flags}")
        assert L.ltc_compress_delta(VP(ty.data_ptr()), VP(tb.data_ptr()), nb, 1, 131072, 0.95, flags,
                                    VP(blob.data_ptr()), cap, VP(size.data_ptr()), VP(ws.data_ptr()), ws.numel(),
                                    _stream()) == 0
        got = _read_blob(blob, size)
        assert np.array_equal(got, want)
        hdr = bytes(want[:64])
        need = ltc.delta_workspace_size([hdr])
        dws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        dst = torch.empty(nb, dtype=torch.uint8, device="cuda")
        status = torch.full((1,), -99, dtype=torch.int32, device="cuda")
        banner(f"ltc_decompress_delta flags={flags}")
        assert L.ltc_decompress_delta(hdr, VP(blob.data_ptr()), want.size, VP(tb.data_ptr()), VP(dst.data_ptr()), nb,
                                      VP(status.data_ptr()), VP(dws.data_ptr()), dws.numel(), _stream()) == 0
        assert int(status.item()) == 0 and np.array_equal(dst.cpu().numpy(), y.view(np.uint8))
