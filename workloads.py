"""Seeded synthetic inputs for the codec's tests and benchmark.

This module only draws random numbers and converts them to the target dtype;
it holds none of the codec's arithmetic, and both the oracle's tests and the
GPU path consume what it returns.

The pages measure on trained Hugging Face checkpoints (Llama 3.1, Granite,
OLMo, ...: "NOTE-241: ZipNN", Table II and Table III), which are not available
here.  Seeded normal tensors with per-tensor scales stand in for them:
  C1  BF16 1-D, 2**20 elements: numpy PCG64 seed 0, N(0,1) float64 * 0.02,
      rounded to float32 then to bfloat16 (round-to-nearest-even both times).
  C2  FP32 4096x4096: numpy seed 1, float64 * 0.02 -> float32.
  C3  28 BF16 tensors shaped like one Llama-3-8B-style layer stack, 4 layers x
      (q 4096x4096, k 1024x4096, v 1024x4096, o 4096x4096, gate 14336x4096,
      up 14336x4096, down 4096x14336); per tensor a scale sigma drawn
      log-uniform in [0.005, 0.05] from numpy seed 2, values from torch's
      Philox generator on the GPU (seed 2), float32 * sigma -> bfloat16.
  C4  "clean" mix: FP32 2048x8192 = bfloat16(N(0,0.02)) widened back to
      float32 (two low mantissa bytes zero), numpy seed 3; plus FP16
      8192x8192 N(0,0.02), numpy seed 4.
  C5  64 BF16 tensors 8192x8192 concatenated into one 8 GiB buffer; sigma
      log-uniform in [1e-3, 1e-1] from numpy seed 5, values from torch Philox
      on the GPU (seed 5); tensors with index % 8 == 7 are uniform random
      bytes instead (incompressible).
  C3D a checkpoint pair over C3 for XOR deltas ("NOTE-241: ZipNN", Deltas:
      every parameter moves a little each epoch, the exponent least): the
      base is C3; the later checkpoint is bfloat16(float32(base) + sigma *
      lr * N(0,1)) per tensor, lr log-uniform in [5e-4, 5e-3] from numpy
      seed 6, the noise from torch Philox on the GPU (seed 6); tensor 0
      (a frozen layer) is left unchanged.
The numpy recipes are reproducible on any host; the torch-on-GPU recipes are
reproducible for a given torch build and device type, and every consumer
records the SHA-256 of what it used.
"""
import hashlib

import numpy as np

DTYPE_CODE = {"u8": 0, "bf16": 1, "fp16": 2, "fp32": 3}

C3_SHAPES = []
for _layer in range(4):
    for _name, _shape in (("q", (4096, 4096)), ("k", (1024, 4096)), ("v", (1024, 4096)),
                          ("o", (4096, 4096)), ("gate", (14336, 4096)),
                          ("up", (14336, 4096)), ("down", (4096, 14336))):
        C3_SHAPES.append((f"layers.{_layer}.{_name}", _shape))


def sha256(buf) -> str:
    if hasattr(buf, "numpy"):
        buf = buf.detach().cpu().contiguous().view(-1).view(_torch().uint8).numpy()
    return hashlib.sha256(np.ascontiguousarray(buf).view(np.uint8).tobytes()).hexdigest()


def _torch():
    import torch
    return torch


def _to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    torch = _torch()
    x32 = x64.astype(np.float32)
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def c1() -> np.ndarray:
    """BF16 bit patterns (np.uint16), 2**20 elements."""
    x = np.random.default_rng(0).standard_normal(1 << 20) * 0.02
    return _to_bf16_bits(x)


def c2() -> np.ndarray:
    """FP32 4096x4096."""
    return (np.random.default_rng(1).standard_normal((4096, 4096)) * 0.02).astype(np.float32)


def c4() -> tuple:
    """(clean FP32 2048x8192, FP16 8192x8192)."""
    x = np.random.default_rng(3).standard_normal((2048, 8192)) * 0.02
    bits = _to_bf16_bits(x).astype(np.uint32) << 16
    clean = bits.view(np.float32).reshape(2048, 8192)
    h = (np.random.default_rng(4).standard_normal((8192, 8192)) * 0.02).astype(np.float16)
    return clean, h


def c3_sigmas() -> list:
    rng = np.random.default_rng(2)
    return [float(np.exp(rng.uniform(np.log(0.005), np.log(0.05)))) for _ in C3_SHAPES]


def c3_gpu(device="cuda", count=None) -> list:
    """The 28 C3 tensors (or the first `count`) as bfloat16 tensors on `device`."""
    torch = _torch()
    g = torch.Generator(device=device).manual_seed(2)
    out = []
    for (name, shape), sigma in zip(C3_SHAPES[:count] if count else C3_SHAPES, c3_sigmas()):
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        out.append(t.mul_(sigma).to(torch.bfloat16))
        del t
    return out


def c3_delta_lrs() -> list:
    rng = np.random.default_rng(6)
    return [float(np.exp(rng.uniform(np.log(5e-4), np.log(5e-3)))) for _ in C3_SHAPES]


def c3_delta_gpu(device="cuda", count=None) -> tuple:
    """(later checkpoint, base) lists of the C3D pair, bfloat16 on `device`."""
    torch = _torch()
    base = c3_gpu(device, count)
    g = torch.Generator(device=device).manual_seed(6)
    fine = []
    for i, (b, sigma, lr) in enumerate(zip(base, c3_sigmas(), c3_delta_lrs())):
        if i == 0:
            fine.append(b.clone())
            continue
        t = torch.randn(b.shape, generator=g, device=device, dtype=torch.float32)
        fine.append(t.mul_(sigma * lr).add_(b.float()).to(torch.bfloat16))
        del t
    return fine, base


def c5_sigmas() -> list:
    rng = np.random.default_rng(5)
    return [float(np.exp(rng.uniform(np.log(1e-3), np.log(1e-1)))) for _ in range(64)]


def c5_gpu(device="cuda", ntensors=64) -> "object":
    """One uint8 buffer holding `ntensors` 8192x8192 BF16 tensors back to back."""
    torch = _torch()
    per = 8192 * 8192
    buf = torch.empty(ntensors * per * 2, dtype=torch.uint8, device=device)
    g = torch.Generator(device=device).manual_seed(5)
    sig = c5_sigmas()
    for i in range(ntensors):
        view = buf[i * per * 2:(i + 1) * per * 2]
        if i % 8 == 7:
            view.copy_(torch.randint(0, 256, (per * 2,), generator=g, device=device,
                                     dtype=torch.uint8))
        else:
            t = torch.randn(per, generator=g, device=device, dtype=torch.float32)
            view.view(torch.bfloat16).copy_(t.mul_(sig[i]).to(torch.bfloat16))
            del t
    return buf
