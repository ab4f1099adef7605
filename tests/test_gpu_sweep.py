"""GPU parity over a seeded random sweep of the options together: dtype,
chunk size, threshold, format v1 / v2, directory order / top-last, plain or
XOR deltas, checksums of several chunk sizes, batches of one to five tensors
of ragged and empty sizes, and contents from smooth weights to random bytes,
constants, sparse changes and special values.  Every case compares the blobs
and checksums with the oracle's byte for byte and decodes them back (the
deltas against their bases).  A few cases are large enough for the pipelined
groups and for the encoder placing the top streams' payloads (4096 chunks or
more).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import banner, to_gpu, to_np_bytes

pytestmark = pytest.mark.gpu

NCASES = 1200


@pytest.fixture(scope="module")
def ltc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import lossless_tensor_compression_amd as m
    m.lib()
    return m


def _content(rng, dtype, n, kind=None):
    """n elements of one of the content kinds, as a numpy array of the dtype's width."""
    e = oracle.ELEM_BYTES[dtype]
    kind = kind or rng.choice(["normal", "normal", "random", "const", "special", "narrow"])
    if dtype == 0:
        if kind == "random":
            return rng.integers(0, 256, n, dtype=np.uint8)
        if kind == "const":
            return np.full(n, rng.integers(0, 256), dtype=np.uint8)
        return rng.integers(0, int(rng.choice([2, 6, 40])), n).astype(np.uint8)
    if kind == "random":
        return rng.integers(0, 1 << (8 * e), n, dtype=np.uint64).astype({2: np.uint16, 4: np.uint32}[e])
    if kind == "const":
        v = rng.integers(0, 1 << (8 * e))
        return np.full(n, v, dtype={2: np.uint16, 4: np.uint32}[e])
    sigma = 0.02 if kind == "weights" else float(rng.choice([1e-4, 0.02, 1.0, 300.0]))
    x = rng.standard_normal(n) * sigma
    if kind == "narrow":
        x = np.round(x * 4) / 4
    if kind == "special" and n:
        idx = rng.integers(0, n, max(1, n // 50))
        x[idx] = rng.choice([np.inf, -np.inf, np.nan, 0.0, -0.0, 1e-40, 6e4], idx.size)
    if dtype == 1:
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == 2:
        with np.errstate(over="ignore"):
            return x.astype(np.float16).view(np.uint16)
    return x.astype(np.float32).view(np.uint32)


def _case(seed):
    rng = np.random.default_rng(9000 + seed)
    dtype = int(rng.integers(0, 4))
    e = oracle.ELEM_BYTES[dtype]
    big = seed % 12 == 5  # 4096 chunks or more
    chunk = int(rng.choice([2048, 4096]) if big else rng.choice([8, 24, 1000, 4096, 8192, 65536, 131072]))
    count = int(rng.integers(1, 6))
    if big:
        total = 4200 * chunk // e
        cuts = np.sort(rng.integers(0, total, count - 1))
        sizes = np.diff(np.concatenate([[0], cuts, [total]])).tolist()
    else:
        sizes = [int(rng.choice([0, 1, 7, rng.integers(1, 300000 // e)])) for _ in range(count)]
    # the large cases are weights (their top streams coded), mostly top-last
    # and plain, so that the encoder places payloads across tensor borders
    arrs = [_content(rng, dtype, n, "weights" if big else None) for n in sizes]
    opts = dict(thr=0.95 if big else float(rng.choice([0.5, 0.88, 0.95, 1.0])),
                shared=bool(rng.random() < 0.3), top_last=bool(rng.random() < (0.8 if big else 0.5)),
                delta=not big and bool(rng.random() < 0.25), crc=int(rng.choice([0, 0, 1000, 16384])))
    bases = None
    if opts["delta"]:
        bases = []
        for a in arrs:
            b = a.copy()
            if b.size:
                idx = rng.integers(0, b.size, max(1, b.size // 20))
                b[idx] ^= rng.integers(1, 8, idx.size).astype(b.dtype)
            bases.append(b)
    return dtype, chunk, arrs, bases, opts


@pytest.mark.parametrize("seed", range(NCASES))
def test_random_case(ltc, seed):
    dtype, chunk, arrs, bases, o = _case(seed)
    nbytes = [a.nbytes for a in arrs]
    banner(f"sweep seed={seed} dtype={dtype} chunk={chunk} sizes={nbytes} {o}")
    ts = [to_gpu(a, dtype) for a in arrs]
    bs = [to_gpu(b, dtype) for b in bases] if bases is not None else None
    flags = (ltc.FLAG_SHARED_TABLES if o["shared"] else 0) | (ltc.FLAG_TOP_LAST if o["top_last"] else 0)
    caps = [ltc.compress_bound(n, dtype, chunk, o["shared"]) for n in nbytes]
    ws_n = ltc.workspace_size(nbytes, dtype, chunk)
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device="cuda")
    blobs = [torch.empty(c, dtype=torch.uint8, device="cuda") for c in caps]
    sizes = torch.zeros(len(ts), dtype=torch.int64, device="cuda")
    k = o["crc"]
    ccap = [(c + k - 1) // k for c in caps] if k else None
    crcs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in ccap] if k else None
    ltc.compress_ex_raw([t.data_ptr() for t in ts], nbytes, dtype, chunk, o["thr"], flags,
                        [b.data_ptr() for b in blobs], caps, sizes.data_ptr(), ws.data_ptr(), ws.numel(),
                        k, [c.data_ptr() for c in crcs] if k else None, ccap,
                        base_ptrs=[b.data_ptr() for b in bs] if bs is not None else None)
    torch.cuda.synchronize()
    got = [b[:s] for b, s in zip(blobs, sizes.cpu().tolist())]
    for i, a in enumerate(arrs):
        if bases is None:
            want = oracle.compress(a, dtype, chunk, o["thr"], shared_tables=o["shared"], top_last=o["top_last"])
        else:
            want = oracle.compress_delta(a, bases[i], dtype, chunk, o["thr"], shared_tables=o["shared"],
                                         top_last=o["top_last"])
        g = to_np_bytes(got[i])
        assert g.size == want.size and np.array_equal(g, want), (seed, i, g.size, want.size)
        if k:
            c = crcs[i][:(want.size + k - 1) // k].cpu().numpy().view(np.uint32)
            assert np.array_equal(c, oracle.crc32_chunks(want, k)), (seed, i)
    outs = ltc.decompress_batch(got) if bases is None else ltc.decompress_batch_delta(got, bs)
    for a, out in zip(arrs, outs):
        assert np.array_equal(to_np_bytes(out), np.ascontiguousarray(a).reshape(-1).view(np.uint8)), seed
