"""HIP graph capture of a compress-with-CRC + decompress step through the C
ABI.  The library allocates nothing, never synchronises and clears what must
start at zero with kernels, so its calls can be captured; a graph built from
them is replayed several times, with eager work and synchronisations between
the replays, and every replay must give the eager call's blobs, checksums and
decoded bytes.  Cases: a small single tensor (top-last), a pipelined
directory-order batch on the caller's stream only and on two streams (the
library's internal stream joins the capture), and a top-last call whose
encoder places the coded payloads.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import banner, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ltc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import lossless_tensor_compression_amd as m
    m.lib()
    return m


def _weights(rng, n, dtype):
    x = (rng.standard_normal(n) * 0.02).astype(np.float32)
    if dtype == 1:
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x.view(np.uint32)


CASES = {
    "small top-last": (1, [1 << 20], 131072, "top-last"),
    "pipelined directory order, caller stream": (3, [1100003, 5, 3100000], 4096, "caller"),
    "pipelined directory order, two streams": (3, [1100003, 5, 3100000], 4096, "directory"),
    "placed top-last": (1, [4200 * 2048 + 7], 4096, "top-last"),
}


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_match_eager(ltc, case):
    dtype, sizes, chunk, mode = CASES[case]
    rng = np.random.default_rng(len(case))
    arrs = [_weights(rng, n, dtype) for n in sizes]
    nbytes = [a.nbytes for a in arrs]
    flags = {"top-last": ltc.FLAG_TOP_LAST, "caller": ltc.FLAG_CALLER_STREAM_ONLY, "directory": 0}[mode]
    ts = [to_gpu(a, dtype) for a in arrs]
    caps = [ltc.compress_bound(n, dtype, chunk) for n in nbytes]
    ws_n = ltc.workspace_size(nbytes, dtype, chunk)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    blobs = [torch.empty(c, dtype=torch.uint8, device="cuda") for c in caps]
    sizes_d = torch.zeros(len(ts), dtype=torch.int64, device="cuda")
    k = 16384
    ccap = [(c + k - 1) // k for c in caps]
    crcs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in ccap]
    outs = [torch.empty(n, dtype=torch.uint8, device="cuda") for n in nbytes]
    status = torch.zeros(len(ts), dtype=torch.int32, device="cuda")
    banner(f"graph {case}: chunks={sum((n + chunk - 1) // chunk for n in nbytes)} flags={flags}")

    def compress():
        ltc.compress_ex_raw([t.data_ptr() for t in ts], nbytes, dtype, chunk, 0.95, flags,
                            [b.data_ptr() for b in blobs], caps, sizes_d.data_ptr(), ws.data_ptr(), ws_n,
                            k, [c.data_ptr() for c in crcs], ccap)

    # eager reference; the decode arguments (headers, blob sizes) come from it
    compress()
    torch.cuda.synchronize()
    bsz = sizes_d.cpu().tolist()
    want = [b[:s].clone() for b, s in zip(blobs, bsz)]
    want_crc = [c[:(s + k - 1) // k].clone() for c, s in zip(crcs, bsz)]
    headers = [bytes(b[:64].cpu().numpy().tobytes()) for b in want]
    for i, a in enumerate(arrs):  # the eager call itself against the oracle
        w = oracle.compress(a, dtype, chunk, 0.95, top_last=mode == "top-last")
        assert np.array_equal(want[i].cpu().numpy(), w), i

    def decompress():
        ltc.decompress_raw(headers, [b.data_ptr() for b in blobs], bsz, [o.data_ptr() for o in outs],
                           nbytes, status.data_ptr())

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            compress()
            decompress()
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between replays: scribble over every output
        for b in blobs:
            b.fill_(0xA5)
        for c in crcs:
            c.fill_(-1)
        for o in outs:
            o.zero_()
        status.fill_(-99)
        sizes_d.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert sizes_d.cpu().tolist() == bsz, rep
        assert status.cpu().tolist() == [0] * len(ts), rep
        for i in range(len(ts)):
            assert torch.equal(blobs[i][:bsz[i]], want[i]), (rep, i)
            assert torch.equal(crcs[i][:(bsz[i] + k - 1) // k], want_crc[i]), (rep, i)
            assert np.array_equal(outs[i].cpu().numpy(), np.ascontiguousarray(arrs[i]).view(np.uint8)), (rep, i)
