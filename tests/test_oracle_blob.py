"""Pins for the oracle's blob format: hand-assembled golden blobs, brute force
over tiny inputs, round trips on awkward shapes and special values, and the
structural error checks."""
import itertools
import json
import os
import struct

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "blobs.json")
CASES = json.load(open(GOLDEN))["cases"]


def _golden_bytes(case):
    if "hex" in case:
        return bytes.fromhex(case["hex"].replace(" ", ""))
    fl = case["fields"]
    e = {0: 1, 1: 2, 2: 2, 3: 4}[case["dtype"]]
    hdr = b"LTCB" + struct.pack("<HBBQIIHBBIQQ", 1, case["dtype"], e, fl["N"],
                                case["chunk_bytes"], fl["K"], 64, 12, 0, 0,
                                fl["blob_nbytes"], fl["payload_base"]) + bytes(16)
    en = fl["entry"]
    dire = struct.pack("<QIBBH", en["offset"], en["size"], en["mode"], en["cval"], 0)
    p = fl["payload"]
    states = [p["states"].get(str(l), p["states"]["default"]) for l in range(64)]
    pl = struct.pack("<IBB", p["W"], p["sym_lo"], p["sym_hi"]) + bytes(10)
    pl += struct.pack("<64I", *states) + struct.pack(f"<{len(p['f'])}H", *p["f"])
    pl += bytes(p["WO"] - len(pl)) + struct.pack(f"<{len(p['words'])}H", *p["words"])
    return hdr + dire + pl


def _golden_input(case):
    if "input_hex" in case:
        return np.frombuffer(bytes.fromhex(case["input_hex"]), dtype=np.uint8).copy()
    x = np.zeros(case["input"]["n"], dtype=np.uint8)
    x[case["input"]["ones_at"]] = 1
    return x


@pytest.mark.parametrize("case", CASES, ids=lambda c: c["name"])
def test_golden_blobs(case):
    src = _golden_input(case)
    blob = oracle.compress(src, case["dtype"], case["chunk_bytes"], case["threshold"])
    assert blob.tobytes() == _golden_bytes(case), case["derivation"]
    rc, out = oracle.decompress(blob)
    assert rc == 0 and out.tobytes() == src.tobytes()


def test_brute_force_u8_tiny():
    """Every U8 tensor of length 0..4 over {0, 1, 255}, chunk 8."""
    for n in range(5):
        for vals in itertools.product([0, 1, 255], repeat=n):
            src = np.array(vals, dtype=np.uint8)
            blob = oracle.compress(src, 0, 8)
            assert blob.size == oracle.compress_bound(n, 0, 8) or blob.size <= oracle.compress_bound(n, 0, 8)
            rc, out = oracle.decompress(blob)
            assert rc == 0 and np.array_equal(out, src)
            # one stream per chunk: CONST iff all equal, else RAW (tiny)
            if n:
                mode = blob[64 + 12]
                assert mode == (2 if len(set(vals)) == 1 else 0)


BF16_PATTERNS = [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x807F,
                 0x3F80, 0xBF80, 0x0080, 0x7F7F, 0xFF7F, 0x3C23, 0xBC23, 0x4049]


def test_brute_force_bf16_one_and_two_elements():
    """All 1- and 2-element BF16 tensors over 16 patterns (zeros, infinities,
    NaNs, subnormals, extremes, ordinary values)."""
    for n in (1, 2):
        for vals in itertools.product(BF16_PATTERNS, repeat=n):
            src = np.array(vals, dtype=np.uint16)
            blob = oracle.compress(src, 1, 8)
            rc, out = oracle.decompress(blob)
            assert rc == 0 and out.tobytes() == src.tobytes()


@pytest.mark.parametrize("dtype,chunk", [(0, 8), (0, 24), (1, 8), (1, 16), (1, 1000),
                                         (2, 4096), (3, 8), (3, 136), (3, 131072)])
def test_round_trip_ragged(dtype, chunk):
    rng = np.random.default_rng(chunk + dtype)
    e = oracle.ELEM_BYTES[dtype]
    for nelem in (0, 1, 63, 64, 65, 127, 129, 1000, 5003):
        vals = (rng.standard_normal(nelem) * 0.02)
        if dtype == 0:
            src = rng.integers(0, 4, nelem).astype(np.uint8)
        elif dtype == 1:
            src = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
        elif dtype == 2:
            src = vals.astype(np.float16)
        else:
            src = vals.astype(np.float32)
        blob = oracle.compress(src, dtype, chunk)
        assert blob.size <= oracle.compress_bound(nelem * e, dtype, chunk)
        assert blob.size % 16 == 0
        rc, out = oracle.decompress(blob)
        assert rc == 0 and out.tobytes() == np.ascontiguousarray(src).tobytes()
        # determinism and re-compression of the decoded bytes
        assert np.array_equal(oracle.compress(out, dtype, chunk), blob)


def test_special_values_fp32_and_fp16():
    specials32 = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 3.4e38,
                           1.17e-38, 1.0], dtype=np.float32)
    rng = np.random.default_rng(1)
    src = np.tile(specials32, 500)[rng.permutation(5000)]
    for dtype, arr in ((3, src), (2, src.astype(np.float16))):
        blob = oracle.compress(arr, dtype, 4096)
        rc, out = oracle.decompress(blob)
        assert rc == 0 and out.tobytes() == arr.tobytes()


def test_threshold_extremes():
    rng = np.random.default_rng(2)
    src = rng.integers(0, 3, 20000).astype(np.uint8)   # ~1.58 bits/symbol
    coded = oracle.compress(src, 0, 8192, 0.95)
    assert (coded[64 + 12::16][:3] == 1).all()
    tiny = oracle.compress(src, 0, 8192, 1e-6)       # nothing can be that small
    assert (tiny[64 + 12:64 + 16 * 3:16] == 0).all()
    for blob in (coded, tiny):
        rc, out = oracle.decompress(blob)
        assert rc == 0 and np.array_equal(out, src)


def test_argument_errors():
    src = np.zeros(10, dtype=np.uint8)
    for bad in (dict(chunk_bytes=7), dict(chunk_bytes=12), dict(chunk_bytes=(1 << 24) + 8),
                dict(threshold=0.0), dict(threshold=1.5), dict(threshold=float("nan"))):
        with pytest.raises(ValueError):
            oracle.compress(src, 0, **bad)
    with pytest.raises(ValueError):
        oracle.compress(np.zeros(3, dtype=np.uint8), 1)  # 3 bytes is not whole BF16
    with pytest.raises(ValueError):
        oracle.compress(src, 9)


def _sample_blob():
    x = (np.random.default_rng(8).standard_normal(30000) * 0.02).astype(np.float32)
    return oracle.compress(torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy(), 1, 8192)


def test_corruption_is_detected():
    blob = _sample_blob()
    assert oracle.decompress(blob)[0] == 0
    b = blob.copy(); b[0] ^= 1
    assert oracle.decompress(b)[0] == oracle.ERR_BAD_MAGIC
    b = blob.copy(); b[4] = 3                 # no such version
    assert oracle.decompress(b)[0] == oracle.ERR_BAD_VERSION
    b = blob.copy(); b[4] = 2                 # v2 needs the shared-table flag and records
    assert oracle.decompress(b)[0] == oracle.ERR_CORRUPT
    b = blob.copy(); b[6] = 9
    assert oracle.decompress(b)[0] == oracle.ERR_UNSUPPORTED_DTYPE
    assert oracle.decompress(blob[:-16])[0] == oracle.ERR_CORRUPT
    assert oracle.decompress(blob[:40])[0] == oracle.ERR_CORRUPT
    b = blob.copy(); b[64 + 12] = 7           # bad mode
    assert oracle.decompress(b)[0] == oracle.ERR_CORRUPT
    b = blob.copy(); b[64 + 8] ^= 1           # size breaks the offset chain
    assert oracle.decompress(b)[0] == oracle.ERR_CORRUPT
    # a RANS payload field: find the first RANS entry and break its state
    modes = blob[64 + 12:64 + 16 * 8:16]
    i = int(np.nonzero(modes == 1)[0][0])
    off = int.from_bytes(blob[64 + 16 * i:64 + 16 * i + 8].tobytes(), "little")
    b = blob.copy(); b[off + 16 + 3] = 0; b[off + 16 + 2] = 0   # state < 65536
    assert oracle.decompress(b)[0] == oracle.ERR_CORRUPT
    b = blob.copy(); b[off + 272] ^= 1        # frequency sum != 4096
    assert oracle.decompress(b)[0] == oracle.ERR_CORRUPT
    b = blob.copy(); b[off] ^= 1              # word count disagrees with the size
    assert oracle.decompress(b)[0] == oracle.ERR_CORRUPT


def test_random_bit_flips_never_crash():
    blob = _sample_blob()
    rng = np.random.default_rng(0)
    outcomes = set()
    for _ in range(300):
        b = blob.copy()
        pos = int(rng.integers(0, b.size))
        b[pos] ^= 1 << int(rng.integers(0, 8))
        outcomes.add(oracle.decompress(b)[0])
    assert outcomes <= {0, oracle.ERR_CORRUPT, oracle.ERR_BAD_MAGIC, oracle.ERR_BAD_VERSION,
                        oracle.ERR_UNSUPPORTED_DTYPE}
