"""Config-level pins for the oracle on the synthetic stand-ins for the pages'
workloads: round trips, the per-byte-group pattern of ZipNN's Table II
("NOTE-241: ZipNN", Key results: exponent group ~33%, sign/mantissa groups
~100%, clean FP32 low bytes 0.0%), the exponent-histogram shape of its Fig. 2,
order-0 invariance under shuffling (its parameter-shuffle experiment) and the
entropy margin of every coded stream."""
import math

import numpy as np
import pytest

import oracle
import workloads


def parse(blob):
    e = int(blob[7])
    k = int.from_bytes(blob[20:24].tobytes(), "little")
    d = blob[64:64 + 16 * k * e].reshape(-1, 16)
    offs = d[:, :8].copy().view(np.uint64).ravel()
    sizes = d[:, 8:12].copy().view(np.uint32).ravel()
    return e, k, offs, sizes, d[:, 12].copy(), d[:, 13].copy()


def per_group_percent(blob, n_per_stream):
    e, k, offs, sizes, modes, _ = parse(blob)
    return [100.0 * sizes[g::e].sum() / (n_per_stream * k) for g in range(e)], modes.reshape(k, e)


def entropy_bits(sym):
    h = np.bincount(sym, minlength=256).astype(np.float64)
    q = h[h > 0] / h.sum()
    return float(-(q * np.log2(q)).sum())


def test_c1_bf16():
    x = workloads.c1()
    blob = oracle.compress(x, 1)
    rc, out = oracle.decompress(blob)
    assert rc == 0 and out.tobytes() == x.tobytes()
    pct, modes = per_group_percent(blob, 65536)
    assert (modes[:, 0] == 0).all() and (modes[:, 1] == 1).all()  # mantissa RAW, exponent RANS
    assert pct[0] == 100.0
    assert 30.0 < pct[1] < 35.0                                    # Table II: 32.5-34.8
    assert 0.64 < blob.size / x.nbytes < 0.68                      # ~ 1/2*33 + 1/2*100


def test_c1_exponent_shape():
    """Synthetic analogue of Fig. 2: few exponent values, top 12 ~ all mass."""
    x = workloads.c1()
    e = oracle.chunk_stream(x, 1, 2 * x.size, 0, 1)
    h = np.sort(np.bincount(e, minlength=256))[::-1]
    assert 15 <= (h > 0).sum() <= 40
    assert h[:12].sum() / h.sum() >= 0.998
    assert 2.0 < entropy_bits(e) < 3.0                             # within the ~1.6-2.6 bracket +


def test_c2_fp32_groups():
    x = workloads.c2()
    blob = oracle.compress(x, 3)
    rc, out = oracle.decompress(blob)
    assert rc == 0 and out.tobytes() == x.tobytes()
    pct, modes = per_group_percent(blob, 32768)
    assert (modes[:, :3] == 0).all() and (modes[:, 3] == 1).all()
    assert pct[:3] == [100.0, 100.0, 100.0] and 30.0 < pct[3] < 35.0
    assert 0.81 < blob.size / x.nbytes < 0.85                      # ~ 1/4*33 + 3/4*100


def test_c4_clean_fp32_and_fp16():
    clean, h = workloads.c4()
    blob = oracle.compress(clean, 3)
    rc, out = oracle.decompress(blob)
    assert rc == 0 and out.tobytes() == clean.tobytes()
    pct, modes = per_group_percent(blob, 32768)
    # T5-base pattern of Table II: the two low fraction bytes cost nothing
    assert (modes[:, 0] == 2).all() and (modes[:, 1] == 2).all()
    assert pct[0] == 0.0 and pct[1] == 0.0
    assert (modes[:, 2] == 0).all() and (modes[:, 3] == 1).all()
    assert blob.size / clean.nbytes < 0.36
    blob16 = oracle.compress(h, 2)
    rc, out = oracle.decompress(blob16)
    assert rc == 0 and out.tobytes() == h.tobytes()
    pct16, modes16 = per_group_percent(blob16, 65536)
    assert (modes16[:, 0] == 0).all() and (modes16[:, 1] == 1).all()
    assert 66.0 < pct16[1] < 72.0                                  # Table II FP16: 68.8-69.6


def test_shuffle_invariance_order0():
    """Permuting the elements of a chunk leaves histogram, table and symbol
    range unchanged and moves the coded size by < 1%."""
    x = workloads.c1()[:65536]
    perm = np.random.default_rng(0).permutation(x.size)
    a = oracle.chunk_stream(x, 1, 131072, 0, 1)
    b = oracle.chunk_stream(x[perm], 1, 131072, 0, 1)
    ha, hb = oracle.histogram(a), oracle.histogram(b)
    assert np.array_equal(ha, hb)
    assert np.array_equal(oracle.normalize(ha), oracle.normalize(hb))
    ma, _, sa, _ = oracle.encode_chunk(x, 1, 131072, 0.95, 0)
    mb, _, sb, _ = oracle.encode_chunk(x[perm], 1, 131072, 0.95, 0)
    assert ma.tolist() == mb.tolist()
    assert abs(int(sa[1]) - int(sb[1])) < 0.01 * sa[1]


@pytest.mark.parametrize("which", ["c1", "c2"])
def test_entropy_margin_every_coded_stream(which):
    x = workloads.c1() if which == "c1" else workloads.c2()
    dtype = 1 if which == "c1" else 3
    blob = oracle.compress(x, dtype)
    e, k, offs, sizes, modes, _ = parse(blob)
    for i in np.nonzero(modes == 1)[0][:64]:
        c, s = divmod(int(i), e)
        sym = oracle.chunk_stream(x, dtype, 131072, c, s)
        H = entropy_bits(sym)
        lo, hi = int(blob[offs[i] + 4]), int(blob[offs[i] + 5])
        wo = (272 + 2 * (hi - lo + 1) + 15) // 16 * 16
        payload_bits = 8 * (int(sizes[i]) - wo)
        assert payload_bits <= 1.01 * sym.size * H + 1024
        assert payload_bits >= sym.size * H - 0.1862 * sym.size - 1024


def test_offsets_follow_cursor_rule():
    x = workloads.c1()
    blob = oracle.compress(x, 1)
    e, k, offs, sizes, modes, _ = parse(blob)
    cur = 64 + 16 * k * e
    for o, s in zip(offs.tolist(), sizes.tolist()):
        assert o == cur
        cur = (o + s + 15) // 16 * 16
    assert cur == blob.size == int.from_bytes(blob[32:40].tobytes(), "little")
