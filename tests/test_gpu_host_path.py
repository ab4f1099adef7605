"""GPU parity of the host-blob path (cuZipNN 0.1.0, "API": decompress_tensor
takes a blob in CPU memory and decodes on the GPU; compress_tensor returns a
CPU blob).  Blobs written by the oracle are placed in pinned host memory,
copied in chunk groups by the library and decoded as they arrive; the output
must equal the original bytes, and the device status must match the
oracle's verdict on corrupted blobs.  Inputs span one and many copy groups,
groups that split a batch between tensors, empty and one-element tensors,
and pageable host memory.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, to_gpu, to_np_bytes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ltc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import lossless_tensor_compression_amd as m
    m.lib()
    return m


def _host(blob_np, pin=True):
    t = torch.empty(blob_np.size, dtype=torch.uint8, pin_memory=pin)
    t.numpy()[:] = blob_np
    return t


def _check_host_decode(ltc, src, dtype, chunk=131072, pin=True, label=""):
    src = np.ascontiguousarray(src).reshape(-1).view(np.uint8)
    blob = oracle.compress(src, dtype, chunk)
    banner(f"host decode {label} dtype={dtype} bytes={src.size} blob={blob.size} pinned={pin}")
    out = ltc.decompress_from_host(_host(blob, pin))
    assert out.is_cuda
    assert np.array_equal(to_np_bytes(out), src)


def test_c1_one_group(ltc):
    _check_host_decode(ltc, workloads.c1(), 1, label="C1")


def test_c2_many_groups(ltc):
    # a ~50 MB blob: three copy groups, each decoded as it lands
    _check_host_decode(ltc, workloads.c2(), 3, label="C2")


def test_fp16_and_pageable(ltc):
    _, h = workloads.c4()
    _check_host_decode(ltc, h.reshape(-1)[: 12 << 20], 2, label="C4 fp16 slice")
    _check_host_decode(ltc, h.reshape(-1)[: 3 << 20], 2, pin=False, label="C4 fp16 pageable")


@pytest.mark.parametrize("dtype,nelem,chunk", [(0, 0, 4096), (0, 1, 4096), (1, 5003, 8), (3, 70001, 131072),
                                               (2, 63, 24), (1, 12 << 20, 4096)])
def test_small_and_ragged(ltc, dtype, nelem, chunk):
    rng = np.random.default_rng(nelem + dtype)
    x = rng.standard_normal(nelem) * 0.02
    if dtype == 0:
        arr = np.clip(np.rint(x * 2000) + 128, 0, 255).astype(np.uint8)
    elif dtype == 1:
        arr = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    else:
        arr = x.astype(np.float16 if dtype == 2 else np.float32)
    _check_host_decode(ltc, arr, dtype, chunk, label=f"n={nelem}")


def test_batch_groups_split_tensors(ltc):
    """A batch whose copy groups start and end inside different tensors."""
    rng = np.random.default_rng(12)
    sizes = (9_000_001, 0, 1, 7_500_000, 17, 12_000_000, 1_000)  # ~90 MB of blobs: 5 groups
    arrs = [(rng.standard_normal(n) * rng.choice([0.02, 1.0, 1e-3])).astype(np.float32) for n in sizes]
    blobs = [oracle.compress(a, 3, 65536) for a in arrs]
    banner(f"host batch: {len(arrs)} blobs, {sum(b.size for b in blobs)} bytes")
    outs = ltc.decompress_batch_from_host([_host(b) for b in blobs])
    for a, o in zip(arrs, outs):
        assert np.array_equal(to_np_bytes(o), a.view(np.uint8))
    # the same blobs decoded from device memory give the same tensors
    dev = ltc.decompress_batch([torch.from_numpy(b).cuda() for b in blobs])
    for o, d in zip(outs, dev):
        assert torch.equal(o.view(torch.uint8), d.view(torch.uint8))


def test_corrupt_blobs_match_oracle_verdicts(ltc):
    x = workloads.c2().reshape(-1)[: 6 << 20]
    blob = oracle.compress(x, 3, 131072)
    k = int.from_bytes(blob[20:24].tobytes(), "little")
    e = 4
    base = 64 + 16 * k * e
    rng = np.random.default_rng(2)
    cases = []
    b = blob.copy(); b[64 + 16 * 5] ^= 0x10; cases.append(("offset breaks chain", b))
    b = blob.copy(); b[64 + 16 * 9 + 8] ^= 1; cases.append(("size breaks chain", b))
    for i in range(6):
        b = blob.copy()
        pos = int(rng.integers(base, b.size))
        b[pos] ^= 1 << int(rng.integers(0, 8))
        cases.append((f"payload flip {pos}", b))
    for name, cb in cases:
        banner(f"host corruption {name}")
        want_rc, want = oracle.decompress(cb)
        outs = ltc.decompress_batch_from_host([_host(cb)], check=False)
        # status is read back inside the call; redo the device path to compare
        dev_status = torch.full((1,), -99, dtype=torch.int32, device="cuda")
        hb = _host(cb)
        info = ltc.blob_info(bytes(cb[:64]))
        dst = torch.empty(info["nbytes"], dtype=torch.uint8, device="cuda")
        stage = torch.empty(cb.size, dtype=torch.uint8, device="cuda")
        ltc.decompress_from_host_raw([hb.data_ptr()], [cb.size], [dst.data_ptr()], [dst.numel()],
                                     dev_status.data_ptr(), [stage.data_ptr()], [stage.numel()])
        st = int(dev_status.item())
        assert st == want_rc, (name, st, want_rc)
        if st == 0:
            assert np.array_equal(dst.cpu().numpy(), want)
            assert np.array_equal(to_np_bytes(outs[0]), want)


def test_argument_errors(ltc):
    blob = oracle.compress(workloads.c1()[:1000], 1, 131072)
    hb = _host(blob)
    dst = torch.empty(2000, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    stage = torch.empty(blob.size, dtype=torch.uint8, device="cuda")
    with pytest.raises(ltc.LTCError) as e:  # staging buffer too small
        ltc.decompress_from_host_raw([hb.data_ptr()], [blob.size], [dst.data_ptr()], [2000],
                                     status.data_ptr(), [stage.data_ptr()], [blob.size - 16])
    assert e.value.code == -6
    with pytest.raises(ltc.LTCError) as e:  # size disagrees with the header
        ltc.decompress_from_host_raw([hb.data_ptr()], [blob.size - 16], [dst.data_ptr()], [2000],
                                     status.data_ptr(), [stage.data_ptr()], [blob.size])
    assert e.value.code == -5
    with pytest.raises(ltc.LTCError) as e:  # destination too small
        ltc.decompress_from_host_raw([hb.data_ptr()], [blob.size], [dst.data_ptr()], [1999],
                                     status.data_ptr(), [stage.data_ptr()], [blob.size])
    assert e.value.code == -6


def test_compress_to_host_round_trip(ltc):
    x = workloads.c1()
    t = to_gpu(x, 1)
    hb = ltc.compress_to_host(t)
    assert not hb.is_cuda and hb.is_pinned()
    assert np.array_equal(hb.numpy(), oracle.compress(x, 1, 131072))
    out = ltc.decompress_from_host(hb)
    assert torch.equal(out.view(torch.int16), t.view(torch.int16))
