#!/usr/bin/env python3
"""Benchmark of the gfx950 lossless tensor codec on one GPU.

A step is one pass of the whole hot path over the workload, inputs resident
in HBM: batch compress (histogram, normalise, rANS encode, scan, pack),
batch decompress (validate, decode, inverse regroup and reorder), and the
CRC-32 of every blob in 16 KiB chunks.  Prints one JSON line.

--crc fused (default): the step is compress_with_crc32 (the pack kernel
checksums the payload as it writes it) then decompress.  --crc beside: plain
compress, then the CRC kernel over the blobs on a second stream beside the
decompression.

compress/decompress/CRC throughputs come from HIP events around each call
repeated back to back; per-kernel times (kernel_ms, roofline) come from a
separate pass that launches the kernels one by one on one stream.  With
--isolated the timed steps run that way too (the mode the committed
rocprofv3 kernel summary is taken in).

Default workload: 28 BF16 tensors shaped like four Llama-3-8B-style layers
(1.74 GB), generated on the GPU from a fixed seed (see workloads.py).
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decompress GB/s (orig bytes, HBM-resident) + compress GB/s + ratio, BF16"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD public specification
# 32-bit integer VALU peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (a wave64
# VALU instruction occupies a 16-lane SIMD for 4 cycles)
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# integer operations one rANS encode step needs (table read, renormalisation
# test, word emit, shift, quotient, remainder (multiply + subtract), scale by
# M, two adds)
ENC_OPS_PER_SYMBOL = 10
CHUNK = 131072
THRESHOLD = 0.95
CRC_CHUNK = 16384


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads of the multi-threaded baseline (0: the host's CPU share)")
    ap.add_argument("--configs", default="c1,c2,c4,c5",
                    help="other workloads also measured and reported under 'configs' (comma list of "
                         "c1, c2, c4, c5; empty for none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a device-to-device copy of 1 GiB (HBM counter calibration)")
    ap.add_argument("--isolated", action="store_true",
                    help="run every step kernel by kernel on one stream (for per-kernel profiles)")
    ap.add_argument("--crc", default="fused", choices=["fused", "beside"],
                    help="CRC-32 of the blobs in the compress call (compress_with_crc32), or by its "
                         "own kernel after a plain compress")
    ap.add_argument("--layout", default="top-last", choices=["top-last", "directory"],
                    help="payload order: top streams after all others (LTC_FLAG_TOP_LAST, the "
                         "compressor then writes RAW streams straight into the blob) or directory "
                         "order; the other one's compress times are reported beside")
    ap.add_argument("--no-other-layout", action="store_true",
                    help="skip timing the other payload order (profiling runs: only the measured "
                         "layout's kernels then appear)")
    ap.add_argument("--tables", default="own", choices=["own", "shared"],
                    help="blob format: v1 (a frequency table per coded stream) or v2 (one per "
                         "stream index, shared by all chunks of a tensor)")
    ap.add_argument("--delta", action="store_true",
                    help="also time XOR-delta compress and decompress of the C3D checkpoint pair "
                         "(C3 and a slightly trained copy); reported beside value, never as value")
    ap.add_argument("--host-path", action="store_true",
                    help="also time decoding from pinned host blobs (copies over the host link "
                         "overlapped with decoding) against plain host-to-device copies of the "
                         "original bytes; reported beside value, never as value")
    return ap.parse_args()


class Hip:
    """hipEvent_t helpers on the HIP runtime torch already loaded."""

    def __init__(self):
        path = None
        for line in open("/proc/self/maps"):
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
        self.L = ctypes.CDLL(path or "libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]

    def events(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.L.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def record(self, ev, stream):
        self.L.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))

    def wait(self, stream, ev):
        if self.L.hipStreamWaitEvent(ctypes.c_void_p(stream), ctypes.c_void_p(ev), 0) != 0:
            raise RuntimeError("hipStreamWaitEvent failed")

    def ms(self, a, b):
        v = ctypes.c_float()
        if self.L.hipEventElapsedTime(ctypes.byref(v), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(v.value)


def make_workload(name, torch, workloads):
    dev = "cuda"
    if name == "c3":
        ts = workloads.c3_gpu(dev)
        desc = {"workload": "C3: 28 BF16 tensors of a 4-layer Llama-3-8B-like stack, "
                            "N(0, sigma), sigma log-uniform [0.005, 0.05]",
                "tensors": len(ts), "dtype": "bf16"}
    elif name == "c5":
        buf = workloads.c5_gpu(dev)
        ts = [buf.view(torch.bfloat16)]
        desc = {"workload": "C5: 8 GiB BF16 stream of 64 tensors 8192x8192, every 8th random bytes",
                "tensors": 1, "dtype": "bf16"}
    elif name == "c1":
        ts = [torch.from_numpy(workloads.c1().view("int16")).cuda().view(torch.bfloat16)]
        desc = {"workload": "C1: BF16 2**20 elements N(0, 0.02)", "tensors": 1, "dtype": "bf16"}
    elif name == "c2":
        ts = [torch.from_numpy(workloads.c2()).cuda()]
        desc = {"workload": "C2: FP32 4096x4096 N(0, 0.02)", "tensors": 1, "dtype": "fp32"}
    else:
        clean, h = workloads.c4()
        ts = [torch.from_numpy(clean).cuda()]
        desc = {"workload": "C4 (clean FP32 part): bf16-rounded values widened to FP32, 2048x8192",
                "tensors": 1, "dtype": "fp32"}
    return ts, desc


def copy_calibration(torch):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.time()
    for _ in range(20):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.time() - t0) / 20
    print(json.dumps({"copy_bytes": n, "copy_read_plus_write_gbs": 2 * n / dt / 1e9}), flush=True)


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the summary is missing, was taken on another workload, or the
    kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("bench_workload") != workload:
        return None
    # the kernel's source file and the headers it includes, hashed together
    srcs = [os.path.join(ROOT, f) for f in rec.get("sources", [])]
    if not srcs or not all(os.path.exists(f) for f in srcs):
        return None
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    if h.hexdigest() != rec.get("sources_sha256"):
        return None
    return rec.get("hbm_bytes_per_launch")


def host_path(ts, blobs, bsz, outs, nbytes, N, B, hip, sptr, torch):
    """Blobs in pinned host memory decoded onto the GPU (ltc_decompress_batch_from_host:
    chunk-group copies overlapped with decoding), against host-to-device copies
    of the original bytes from pinned memory (what loading them uncompressed
    costs on this link)."""
    import lossless_tensor_compression_amd as ltc
    count = len(ts)
    hblobs = [torch.empty(s, dtype=torch.uint8, pin_memory=True) for s in bsz]
    for hb, b, s in zip(hblobs, blobs, bsz):
        hb.copy_(b[:s])
    hraw = [torch.empty(n, dtype=torch.uint8, pin_memory=True) for n in nbytes]
    for h, t in zip(hraw, ts):
        h.copy_(t.contiguous().view(-1).view(torch.uint8))
    stages = [torch.empty(s, dtype=torch.uint8, device="cuda") for s in bsz]
    status = torch.zeros(count, dtype=torch.int32, device="cuda")
    ev = hip.events(2)

    def load():
        ltc.decompress_from_host_raw([h.data_ptr() for h in hblobs], bsz, [o.data_ptr() for o in outs],
                                     nbytes, status.data_ptr(), [st.data_ptr() for st in stages], bsz)

    def raw():
        for o, h in zip(outs, hraw):
            o.copy_(h, non_blocking=True)

    res = {}
    for name, fn in (("load", load), ("raw", raw)):
        fn()
        torch.cuda.synchronize()
        reps = 5
        hip.record(ev[0], sptr)
        for _ in range(reps):
            fn()
        hip.record(ev[1], sptr)
        torch.cuda.synchronize()
        res[name] = hip.ms(ev[0], ev[1]) / reps
    load()
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0] * count, "host-path decode status"
    for t, o in zip(ts, outs):
        assert torch.equal(t.contiguous().view(-1).view(torch.uint8), o), "host-path round trip"
    return {"load_ms": round(res["load"], 3), "load_gbs": round(N / (res["load"] * 1e-3) / 1e9, 2),
            "blob_link_gbs": round(B / (res["load"] * 1e-3) / 1e9, 2),
            "raw_h2d_ms": round(res["raw"], 3), "raw_h2d_gbs": round(N / (res["raw"] * 1e-3) / 1e9, 2),
            "speedup_vs_raw_copy": round(res["raw"] / res["load"], 3),
            "note": "PCIe-inclusive; original bytes per second"}


def delta_bench(args, hip, sptr, torch):
    """C3D: the later checkpoint of a pair coded as its XOR with the base
    (ltc_compress_batch_ex with bases, ltc_decompress_delta_batch), against the
    same tensors compressed on their own.  Algorithmic bytes: compress reads
    source and base and writes the blob (2N + B); decompress reads blob and
    base and writes the output (2N + B)."""
    import lossless_tensor_compression_amd as ltc
    import workloads
    fine, base = workloads.c3_delta_gpu("cuda")
    count = len(fine)
    nbytes = [t.numel() * 2 for t in fine]
    N = sum(nbytes)
    caps = [ltc.compress_bound(n, 1, CHUNK) for n in nbytes]
    blobs = [torch.empty(c, dtype=torch.uint8, device="cuda") for c in caps]
    ws_n = ltc.workspace_size(nbytes, 1, CHUNK)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    sizes = torch.zeros(count, dtype=torch.int64, device="cuda")
    src_ptrs = [t.data_ptr() for t in fine]
    base_ptrs = [t.data_ptr() for t in base]
    blob_ptrs = [b.data_ptr() for b in blobs]

    def comp():
        ltc.compress_ex_raw(src_ptrs, nbytes, 1, CHUNK, THRESHOLD, 0, blob_ptrs, caps, sizes.data_ptr(),
                            ws.data_ptr(), ws_n, base_ptrs=base_ptrs)

    comp()
    bsz = sizes.cpu().tolist()
    B = sum(bsz)
    headers = [bytes(b[:64].cpu().numpy().tobytes()) for b in blobs]
    dws_n = ltc.delta_workspace_size(headers)
    dws = torch.empty(max(dws_n, 256), dtype=torch.uint8, device="cuda")
    outs = [torch.empty(n, dtype=torch.uint8, device="cuda") for n in nbytes]
    status = torch.zeros(count, dtype=torch.int32, device="cuda")

    def dec():
        ltc.decompress_delta_raw(headers, blob_ptrs, bsz, base_ptrs, [o.data_ptr() for o in outs], nbytes,
                                 status.data_ptr(), dws.data_ptr(), dws_n)

    for _ in range(max(1, args.warmup)):
        comp()
        dec()
    torch.cuda.synchronize()
    assert sizes.cpu().tolist() == bsz and status.cpu().tolist() == [0] * count, "delta status"
    for t, o in zip(fine, outs):
        assert torch.equal(t.view(-1).view(torch.uint8), o), "delta round trip"
    ev = hip.events(2)
    reps = max(3, min(args.steps, 10))
    res = {}
    for name, fn in (("compress", comp), ("decompress", dec)):
        hip.record(ev[0], sptr)
        for _ in range(reps):
            fn()
        hip.record(ev[1], sptr)
        torch.cuda.synchronize()
        res[name] = hip.ms(ev[0], ev[1]) / reps
    modes = {"raw": 0, "rans": 0, "const": 0, "zrun": 0}
    for b, s in zip(blobs, bsz):
        for m in ltc.blob_stats(b[:s])["modes"]:
            for kk in modes:
                modes[kk] += m[kk]
    alone = sum(b.numel() for b in ltc.compress_batch(fine))
    algo = 2 * N + B
    return {"workload": "C3D: C3 and a copy moved by sigma*lr*N(0,1), lr log-uniform [5e-4, 5e-3], "
                        "tensor 0 unchanged", "orig_bytes": N, "blob_bytes": B,
            "ratio": round(B / N, 5), "standalone_ratio": round(alone / N, 5),
            "compress_ms": round(res["compress"], 4), "decompress_ms": round(res["decompress"], 4),
            "compress_gbs": round(N / (res["compress"] * 1e-3) / 1e9, 2),
            "decompress_gbs": round(N / (res["decompress"] * 1e-3) / 1e9, 2),
            "compress_roofline_frac": round(algo / (res["compress"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "decompress_roofline_frac": round(algo / (res["decompress"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "stream_modes": modes}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, ts, torch):
    """The oracle (plain scalar C, OpenMP over chunks) on the host cores:
    compress + decompress + CRC-32 of the blob, on a bounded sample of the
    workload, best of 3 runs, once on one thread and once on the host's CPU
    share.  The share is the CPUs this process may run on, capped by
    OMP_NUM_THREADS when set (a machine that shares its cores among its GPUs
    sets it to one GPU's share)."""
    import numpy as np

    import oracle
    affinity = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    share = min(affinity, int(omp)) if omp.isdigit() and int(omp) > 0 else affinity
    threads = args.cpu_threads or share
    code = {torch.bfloat16: 1, torch.float16: 2, torch.float32: 3, torch.uint8: 0}[ts[0].dtype]

    def sample(cap):  # whole tensors from the start of the workload, at most cap bytes
        out, taken = [], 0
        for t in ts:
            b = t.contiguous().view(-1).view(torch.uint8)
            if taken and taken + b.numel() > cap:
                break
            take = min(b.numel(), cap)
            out.append(b[:take].cpu().numpy())
            taken += take
            if taken >= cap:
                break
        return out

    def best_of_3(parts, nthreads):
        best = None
        for _ in range(3):
            t0 = time.time()
            for s in parts:
                blob = oracle.compress(s, code, CHUNK, THRESHOLD, nthreads=nthreads)
                rc, out = oracle.decompress(blob, nthreads=nthreads)
                assert rc == 0 and np.array_equal(out, s)
                oracle.crc32_chunks(blob, CRC_CHUNK)
            dt = time.time() - t0
            best = dt if best is None else min(best, dt)
        return best

    many = sample(1664 << 20)
    one = sample(32 << 20)
    n_many = sum(s.size for s in many)
    n_one = sum(s.size for s in one)
    t_many = best_of_3(many, threads)
    t_one = best_of_3(one, 1)
    return {"value": round(n_many / t_many / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n_many / 2**20:.0f} MiB of the workload: compress + decompress + CRC-32, "
                      f"OpenMP over chunks on {threads} threads, best of 3 ({t_many:.2f} s)",
            "single_thread": {"value": round(n_one / t_one / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"first {n_one / 2**20:.0f} MiB of the workload, best of 3 "
                                        f"({t_one:.2f} s)"},
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "affinity_cpus": affinity,
            "omp_num_threads": omp or None,
            "speedup_threads_vs_one": round(t_one / n_one * n_many / t_many, 2)}


def digests(torch, tensors, sizes=None):
    """SHA-256 of each tensor's bytes (the first sizes[i] bytes when given)."""
    out = []
    for i, t in enumerate(tensors):
        b = t.contiguous().view(-1).view(torch.uint8)
        if sizes is not None:
            b = b[:sizes[i]]
        out.append(hashlib.sha256(b.cpu().numpy().tobytes()).hexdigest())
    return out


def config_figures(name, ts, hip, sptr, torch, reps, flags, hashes=True):
    """Compress, compress_with_crc32, decompress and the CRC-32 kernel over
    one workload's tensors (batch calls, inputs in HBM), each call repeated
    back to back between two events; the exact round trip and the device
    status are checked first.  Roofline fractions count N + B per call."""
    import lossless_tensor_compression_amd as ltc
    code = ltc.DTYPE_CODE[ts[0].dtype]
    count = len(ts)
    nbytes = [t.numel() * t.element_size() for t in ts]
    N = sum(nbytes)
    caps = [ltc.compress_bound(n, code, CHUNK) for n in nbytes]
    blobs = [torch.empty(c, dtype=torch.uint8, device="cuda") for c in caps]
    ws_n = ltc.workspace_size(nbytes, code, CHUNK)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    sizes = torch.zeros(count, dtype=torch.int64, device="cuda")
    outs = [torch.empty(n, dtype=torch.uint8, device="cuda") for n in nbytes]
    status = torch.zeros(count, dtype=torch.int32, device="cuda")
    src_ptrs = [t.data_ptr() for t in ts]
    blob_ptrs = [b.data_ptr() for b in blobs]
    out_ptrs = [o.data_ptr() for o in outs]
    fcap = [(c + CRC_CHUNK - 1) // CRC_CHUNK for c in caps]
    fcrcs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in fcap]

    # every call's arguments are marshalled once (ltc.Prepared), so a small
    # workload's figures are the GPU's, not the Python caller's
    comp = ltc.compress_ex_raw(src_ptrs, nbytes, code, CHUNK, THRESHOLD, flags, blob_ptrs, caps,
                               sizes.data_ptr(), ws.data_ptr(), ws_n, prepare=True)
    comp_crc = ltc.compress_ex_raw(src_ptrs, nbytes, code, CHUNK, THRESHOLD, flags, blob_ptrs, caps,
                                   sizes.data_ptr(), ws.data_ptr(), ws_n, CRC_CHUNK,
                                   [c.data_ptr() for c in fcrcs], fcap, prepare=True)

    comp()
    bsz = sizes.cpu().tolist()
    headers = [bytes(b[:64].cpu().numpy().tobytes()) for b in blobs]
    B = sum(bsz)
    ncrc = [(s + CRC_CHUNK - 1) // CRC_CHUNK for s in bsz]
    crcs = [torch.empty(max(n, 1), dtype=torch.int32, device="cuda") for n in ncrc]

    dec = ltc.decompress_raw(headers, blob_ptrs, bsz, out_ptrs, nbytes, status.data_ptr(), prepare=True)
    crc = ltc.crc32_raw(blob_ptrs, bsz, CRC_CHUNK, [c.data_ptr() for c in crcs], prepare=True)

    for fn in (comp_crc, dec, crc):
        fn()
    torch.cuda.synchronize()
    assert sizes.cpu().tolist() == bsz, f"{name}: blob sizes changed"
    assert status.cpu().tolist() == [0] * count, f"{name}: decode status"
    for t, o in zip(ts, outs):
        assert torch.equal(t.contiguous().view(-1).view(torch.uint8), o), f"{name}: round trip"
    for a, b, n in zip(crcs, fcrcs, ncrc):
        assert torch.equal(a[:n], b[:n]), f"{name}: CRC-32 paths differ"
    ev = hip.events(2)

    def timed(fn):
        fn()
        hip.record(ev[0], sptr)
        for _ in range(reps):
            fn()
        hip.record(ev[1], sptr)
        torch.cuda.synchronize()
        return hip.ms(ev[0], ev[1]) / reps

    t_c, t_cc, t_d, t_x = timed(comp), timed(comp_crc), timed(dec), timed(crc)
    nck = sum(ncrc)

    def gbs(nb, ms):
        return round(nb / (ms * 1e-3) / 1e9, 2)

    def frac(nb, ms):
        return round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)

    sha = ({"inputs": digests(torch, ts), "blobs": digests(torch, blobs, bsz)} if hashes else
           "not taken (8 GiB; the full-size GPU test compares the whole blob with the oracle's)")
    return {"orig_bytes": N, "blob_bytes": B, "ratio": round(B / N, 5), "tensors": count, "sha256": sha,
            "dtype": {1: "bf16", 2: "fp16", 3: "fp32", 0: "u8"}[code],
            "compress_ms": round(t_c, 4), "decompress_ms": round(t_d, 4),
            "compress_with_crc32_ms": round(t_cc, 4), "crc32_ms": round(t_x, 4),
            "compress_gbs": gbs(N, t_c), "decompress_gbs": gbs(N, t_d),
            "compress_with_crc32_gbs": gbs(N, t_cc), "crc32_blob_gbs": gbs(B, t_x),
            "compress_roofline_frac": frac(N + B, t_c), "decompress_roofline_frac": frac(N + B, t_d),
            "crc32_roofline_frac": frac(B + 4 * nck, t_x)}


def other_configs(which, hip, sptr, torch, reps, flags):
    """The figures of the other workloads, one after another (each freed
    before the next is generated): C1, C2, the two parts of C4 and their
    combination, and C5 (8 GiB)."""
    import numpy as np

    import workloads
    res = {}
    for name in which:
        if name == "c1":
            ts = [torch.from_numpy(workloads.c1().view(np.int16)).cuda().view(torch.bfloat16)]
            res["C1"] = config_figures(name, ts, hip, sptr, torch, reps, flags)
        elif name == "c2":
            ts = [torch.from_numpy(workloads.c2()).cuda()]
            res["C2"] = config_figures(name, ts, hip, sptr, torch, reps, flags)
        elif name == "c4":
            clean, h = workloads.c4()
            a = config_figures("c4a", [torch.from_numpy(clean).cuda()], hip, sptr, torch, reps, flags)
            b = config_figures("c4b", [torch.from_numpy(h).cuda()], hip, sptr, torch, reps, flags)
            res["C4a"], res["C4b"] = a, b
            n, bb = a["orig_bytes"] + b["orig_bytes"], a["blob_bytes"] + b["blob_bytes"]
            tc, td = a["compress_ms"] + b["compress_ms"], a["decompress_ms"] + b["decompress_ms"]
            res["C4"] = {"orig_bytes": n, "blob_bytes": bb, "ratio": round(bb / n, 5),
                         "compress_gbs": round(n / (tc * 1e-3) / 1e9, 2),
                         "decompress_gbs": round(n / (td * 1e-3) / 1e9, 2),
                         "compress_roofline_frac": round((n + bb) / (tc * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "decompress_roofline_frac": round((n + bb) / (td * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "note": "C4a then C4b, one call each"}
        elif name == "c5":
            buf = workloads.c5_gpu("cuda")
            res["C5"] = config_figures(name, [buf.view(torch.bfloat16)], hip, sptr, torch, reps, flags,
                                       hashes=False)
            del buf
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch

    import lossless_tensor_compression_amd as ltc
    import workloads

    ltc.lib()
    if args.copy_calibration:
        copy_calibration(torch)
        return
    torch.cuda.set_device(0)
    ts, desc = make_workload(args.workload, torch, workloads)
    code = ltc.DTYPE_CODE[ts[0].dtype]
    count = len(ts)
    nbytes = [t.numel() * t.element_size() for t in ts]
    N = sum(nbytes)
    shared = args.tables == "shared"
    layout_flag = ltc.FLAG_TOP_LAST if args.layout == "top-last" else 0
    flags = (ltc.FLAG_SHARED_TABLES if shared else 0) | layout_flag
    caps = [ltc.compress_bound(n, code, CHUNK, shared) for n in nbytes]
    blobs = [torch.empty(c, dtype=torch.uint8, device="cuda") for c in caps]
    ws_n = ltc.workspace_size(nbytes, code, CHUNK)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    sizes = torch.zeros(count, dtype=torch.int64, device="cuda")
    outs = [torch.empty(n, dtype=torch.uint8, device="cuda") for n in nbytes]
    status = torch.zeros(count, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    src_ptrs = [t.data_ptr() for t in ts]
    blob_ptrs = [b.data_ptr() for b in blobs]
    out_ptrs = [o.data_ptr() for o in outs]

    hip = Hip()
    ev_c = hip.events(5)
    ev_d = hip.events(3)
    ev_x = hip.events(2)

    # Every call's arguments are marshalled once per (call, events, stream)
    # and the prepared call is repeated (ltc.Prepared): the timed loops then
    # pay only the foreign call on the host.
    prepared = {}

    def once(key, make):
        if key not in prepared:
            prepared[key] = make()
        return prepared[key]

    # first pass: sizes and headers (host copies) for the decode and CRC launches
    def compress_plain(events=None):
        once(("c", id(events)), lambda: ltc.compress_ex_raw(
            src_ptrs, nbytes, code, CHUNK, THRESHOLD, flags, blob_ptrs, caps, sizes.data_ptr(),
            ws.data_ptr(), ws_n, events=events, prepare=True))()

    compress_plain(ev_c if args.isolated else None)
    bsz = sizes.cpu().tolist()
    headers = [bytes(b[:64].cpu().numpy().tobytes()) for b in blobs]
    B = sum(bsz)
    ncrc = [(s + CRC_CHUNK - 1) // CRC_CHUNK for s in bsz]
    crcs = torch.empty(sum(ncrc), dtype=torch.int32, device="cuda")
    crc_ptrs = [crcs.data_ptr() + 4 * sum(ncrc[:i]) for i in range(count)]
    # compress_with_crc32 writes into capacity for the bound
    fcap = [(c + CRC_CHUNK - 1) // CRC_CHUNK for c in caps]
    fcrcs = torch.empty(sum(fcap), dtype=torch.int32, device="cuda")
    fcrc_ptrs = [fcrcs.data_ptr() + 4 * sum(fcap[:i]) for i in range(count)]
    ev_f = hip.events(6)
    fused = args.crc == "fused"

    def compress_crc(events=None):
        if events is None and args.isolated:
            events = ev_f  # kernel by kernel
        once(("cc", id(events)), lambda: ltc.compress_ex_raw(
            src_ptrs, nbytes, code, CHUNK, THRESHOLD, flags, blob_ptrs, caps, sizes.data_ptr(),
            ws.data_ptr(), ws_n, CRC_CHUNK, fcrc_ptrs, fcap, events=events, prepare=True))()

    def decompress(events=None):
        once(("d", id(events)), lambda: ltc.decompress_raw(
            headers, blob_ptrs, bsz, out_ptrs, nbytes, status.data_ptr(), events=events, prepare=True))()

    def crc32(stream=None):
        once(("x", id(stream)), lambda: ltc.crc32_raw(blob_ptrs, bsz, CRC_CHUNK, crc_ptrs, stream=stream,
                                                      prepare=True))()

    ev_p = hip.events(2)
    side = torch.cuda.Stream()  # default priority
    ev_fork, ev_join = hip.events(2)

    def step(prof, plain=False):
        """One pass of the hot path.  Fused CRC (unless plain):
        compress_with_crc32 then decompress.  Otherwise compress, decompress
        and the CRC kernel: with prof one after another on one stream, kernel
        by kernel with events between the kernels, else the CRC-32 of the
        blobs runs on a second stream beside the decompression, which does not
        depend on it.  A plain compress call over many chunks runs its chunk
        groups on two streams (library-internal) unless prof."""
        if fused and not plain:
            compress_crc(ev_f if prof else None)
            decompress(ev_d if prof else None)
            return
        compress_plain(ev_c if prof else None)
        if not prof:
            hip.record(ev_fork, sptr)
            hip.wait(side.cuda_stream, ev_fork)
            crc32(side)
            hip.record(ev_join, side.cuda_stream)
        decompress(ev_d if prof else None)
        if prof:
            hip.record(ev_x[0], sptr)
            crc32()
            hip.record(ev_x[1], sptr)
        else:
            hip.wait(sptr, ev_join)

    for _ in range(max(1, args.warmup)):
        step(args.isolated)
    torch.cuda.synchronize()
    # correctness of what is timed: sizes stable, status OK, exact round trip
    assert sizes.cpu().tolist() == bsz, "blob sizes changed between steps"
    assert status.cpu().tolist() == [0] * count, f"decode status {status.cpu().tolist()}"
    for t, o in zip(ts, outs):
        assert torch.equal(t.contiguous().view(-1).view(torch.uint8), o), "round trip mismatch"
    # both checksum paths agree on the blobs
    compress_crc()
    ltc.crc32_raw(blob_ptrs, bsz, CRC_CHUNK, crc_ptrs)
    torch.cuda.synchronize()
    for i in range(count):
        a = crcs[sum(ncrc[:i]):sum(ncrc[:i + 1])]
        b = fcrcs[sum(fcap[:i]):sum(fcap[:i]) + ncrc[i]]
        assert torch.equal(a, b), f"CRC-32 of blob {i} differs between the two paths"

    # timed region: K whole steps bracketed by synchronisation
    torch.cuda.synchronize()
    t_wall = time.time()
    start_ev = hip.events(2)
    hip.record(start_ev[0], sptr)
    for _ in range(args.steps):
        step(args.isolated)
    hip.record(start_ev[1], sptr)
    torch.cuda.synchronize()
    wall = time.time() - t_wall
    ms_step = hip.ms(start_ev[0], start_ev[1]) / args.steps

    # phase times: each call repeated back to back between two events, as
    # the timed steps run (so the host's enqueue time stays hidden)
    reps = max(3, min(args.steps, 10))

    def timed(fn):
        fn()  # untimed first call: a first use creates the library's internal streams
        torch.cuda.synchronize()
        hip.record(ev_p[0], sptr)
        for _ in range(reps):
            fn()
        hip.record(ev_p[1], sptr)
        torch.cuda.synchronize()
        return hip.ms(ev_p[0], ev_p[1]) / reps

    t_comp = timed(lambda: compress_plain(ev_c if args.isolated else None))
    t_dec = timed(lambda: decompress(ev_d if args.isolated else None))
    t_crc = timed(lambda: crc32())
    # compress_with_crc32 alone (the fused path's first call)
    t_fused = timed(lambda: compress_crc())

    # per-kernel durations (same work, events between the kernels; in the
    # top-last layout k_hist's interval also holds the lower streams' k_encode
    # and scan, C3 about 0.015 ms, so that k_encode's is the top streams'
    # coding alone)
    k = {"k_hist": 0.0, "k_encode": 0.0, "k_scan": 0.0, "k_pack": 0.0, "k_decode": 0.0,
         "k_decode_multi": 0.0, "k_crc32": 0.0}
    for _ in range(reps):
        step(True, plain=True)
        torch.cuda.synchronize()
        k["k_hist"] += hip.ms(ev_c[0], ev_c[1])
        k["k_encode"] += hip.ms(ev_c[1], ev_c[2])
        k["k_scan"] += hip.ms(ev_c[2], ev_c[3])
        k["k_pack"] += hip.ms(ev_c[3], ev_c[4])
        k["k_decode"] += hip.ms(ev_d[0], ev_d[1])
        k["k_decode_multi"] += hip.ms(ev_d[1], ev_d[2])
        k["k_crc32"] += hip.ms(ev_x[0], ev_x[1])
    k = {n: v / reps for n, v in k.items()}
    # compress_with_crc32, kernel by kernel: directory order checksums the
    # blob in k_pack (k_pack_crc) and chains the 1 KiB frame remainders
    # (k_crc_frames); the top-last layout packs plainly and k_crc32 reads the
    # finished blobs back
    kp, kc = ("k_pack_then_crc32", "k_crc32_blob") if layout_flag else ("k_pack_crc", "k_crc_frames")
    kf = {kp: 0.0, kc: 0.0}
    for _ in range(reps):
        compress_crc(ev_f)
        torch.cuda.synchronize()
        kf[kp] += hip.ms(ev_f[3], ev_f[4]) / reps
        kf[kc] += hip.ms(ev_f[4], ev_f[5]) / reps

    # the other payload order, same inputs and buffers (its blobs have the
    # same sizes); then the measured layout's blobs are written again
    other = None
    if not args.no_other_layout:
        oflags = flags ^ ltc.FLAG_TOP_LAST
        t_ocomp = timed(ltc.compress_ex_raw(src_ptrs, nbytes, code, CHUNK, THRESHOLD, oflags, blob_ptrs,
                                            caps, sizes.data_ptr(), ws.data_ptr(), ws_n, prepare=True))
        t_ofused = timed(ltc.compress_ex_raw(src_ptrs, nbytes, code, CHUNK, THRESHOLD, oflags, blob_ptrs,
                                             caps, sizes.data_ptr(), ws.data_ptr(), ws_n, CRC_CHUNK,
                                             fcrc_ptrs, fcap, prepare=True))
        compress_plain()
        torch.cuda.synchronize()
        assert sizes.cpu().tolist() == bsz
        other = {"layout": "directory" if layout_flag else "top-last",
                 "compress_ms": round(t_ocomp, 4), "compress_with_crc32_ms": round(t_ofused, 4),
                 "compress_roofline_frac": round((N + B) / (t_ocomp * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    # algorithmic bytes per launch (what the method must move):
    #   k_decode reads the blob and writes the original bytes: B + N
    #   k_hist reads the input once: N;  k_crc32 reads the blobs: B
    #   k_encode reads the elements of the streams it codes; k_pack writes
    #   the blob and reads the input for RAW streams: B + N (in the top-last
    #   layout k_encode writes the RAW streams it staged, so this overstates
    #   k_pack's share; it only matters if k_pack were the dominant kernel)
    #   k_encode reads the input; in a top-last call of 4096 chunks or more
    #   (the library places the coded payloads there) it also writes the
    #   blob's payloads, the RAW lower streams and the coded top streams:
    #   N + B, the compress path's bytes; otherwise it writes only the
    #   workspace, and integer issue bounds it (below)
    total_chunks = sum((n + CHUNK - 1) // CHUNK for n in nbytes)
    placed = bool(layout_flag) and total_chunks >= 4096
    algo = {"k_decode": B + N, "k_hist": N, "k_pack": B + N, "k_crc32": B,
            "k_encode": N + B if placed else N, "k_scan": 0, "k_decode_multi": 0}
    dom = max((n for n in k if algo[n]), key=lambda n: k[n])
    traffic = traffic_from_profiles(dom, args.workload)
    coded = 0
    if dom == "k_encode":
        # the operations of every symbol the encoder codes (streams that end
        # in RANS mode; every chunk of the bench workloads is full, so a
        # stream holds CHUNK / E symbols)
        e = ts[0].element_size()
        for b, s in zip(blobs, bsz):
            st = ltc.blob_stats(b[:s])
            coded += sum(m["rans"] for m in st["modes"]) * (CHUNK // e)
    if dom == "k_encode" and not placed:
        achieved = coded * ENC_OPS_PER_SYMBOL / (k[dom] * 1e-3) / 1e12
        roof = {"bound": "alu", "kernel": dom, "achieved": round(achieved, 3),
                "peak": round(ALU_PEAK_TOPS, 2), "unit": "Top/s",
                "frac": round(achieved / ALU_PEAK_TOPS, 4), "traffic": traffic,
                "coded_symbols": coded, "ops_per_symbol": ENC_OPS_PER_SYMBOL}
    else:
        achieved = algo[dom] / (k[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
        if dom == "k_encode":  # the integer-issue view beside it
            ops = coded * ENC_OPS_PER_SYMBOL / (k[dom] * 1e-3) / 1e12
            roof["alu"] = {"achieved": round(ops, 3), "peak": round(ALU_PEAK_TOPS, 2), "unit": "Top/s",
                           "frac": round(ops / ALU_PEAK_TOPS, 4), "coded_symbols": coded,
                           "ops_per_symbol": ENC_OPS_PER_SYMBOL}

    value = N / (ms_step * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {**desc, "global_batch": count, "orig_bytes": N, "blob_bytes": B,
                   "chunk_bytes": CHUNK, "passthrough_threshold": THRESHOLD,
                   "crc_chunk_bytes": CRC_CHUNK, "parallelism": "single GPU",
                   "crc": ("in the compress call (compress_with_crc32): " +
                           ("k_crc32 reads the finished blobs" if layout_flag else "accumulated while packing"))
                          if fused else "own kernel beside decompress",
                   "format": "v2, one table per stream index" if shared else "v1, a table per coded stream",
                   "layout": "top streams last (LTC_FLAG_TOP_LAST)" if layout_flag else "directory order",
                   "launch": "kernel by kernel, one stream" if args.isolated
                             else "one stream, the encoder placing the top streams' payloads" if placed
                             else "compress in 2 chunk groups on 2 streams" if total_chunks >= 4096
                             else "one stream"},
        "decompress_gbs": round(N / (t_dec * 1e-3) / 1e9, 2),
        "compress_gbs": round(N / (t_comp * 1e-3) / 1e9, 2),
        "crc32_blob_gbs": round(B / (t_crc * 1e-3) / 1e9, 2),
        "ratio": round(B / N, 5),
        "decompress_roofline_frac": round((N + B) / (t_dec * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "compress_roofline_frac": round((N + B) / (t_comp * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "compress_with_crc32_gbs": round(N / (t_fused * 1e-3) / 1e9, 2),
        "phase_ms": {"compress": round(t_comp, 4), "decompress": round(t_dec, 4),
                     "crc32": round(t_crc, 4), "compress_with_crc32": round(t_fused, 4)},
        "kernel_ms": {**{n: round(v, 4) for n, v in k.items()},
                      **{n: round(v, 4) for n, v in kf.items()}},
        "roofline": roof,
        "other_layout": other,
        "wall_s_timed": round(wall, 3),
    }
    rec["sha256"] = {"inputs": digests(torch, ts), "blobs": digests(torch, blobs, bsz)}
    if args.host_path:
        rec["host_path"] = host_path(ts, blobs, bsz, outs, nbytes, N, B, hip, sptr, torch)
    if args.delta:
        rec["delta"] = delta_bench(args, hip, sptr, torch)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args, ts, torch)
    which = [w for w in args.configs.split(",") if w and w != args.workload]
    if which:
        del ts, blobs, ws, outs
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        rec["configs"] = other_configs(which, hip, sptr, torch, reps, flags)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
