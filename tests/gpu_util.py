"""Helpers shared by the GPU tests: move numpy bytes to the GPU as a typed
tensor and back.  No codec arithmetic lives here."""
import numpy as np
import torch

TORCH_DTYPE = {0: torch.uint8, 1: torch.bfloat16, 2: torch.float16, 3: torch.float32}


def to_gpu(arr, dtype_code):
    b = np.ascontiguousarray(arr).reshape(-1).view(np.uint8)
    if b.size == 0:
        return torch.empty(0, dtype=TORCH_DTYPE[dtype_code], device="cuda")
    return torch.from_numpy(b.copy()).cuda().view(TORCH_DTYPE[dtype_code])


def to_np_bytes(t):
    return t.contiguous().view(-1).view(torch.uint8).cpu().numpy()


def banner(msg):
    print(f"[gpu] {msg}", flush=True)


def stream_modes(blob):
    """Directory modes of a blob (public format): array [K, E] of mode bytes."""
    b = np.asarray(blob, dtype=np.uint8)
    e = int(b[7])
    k = int(b[20:24].view(np.uint32)[0])
    return b[64:64 + 16 * k * e].reshape(k, e, 16)[:, :, 12].copy()


def rans_streams(blob):
    """Number of RANS (mode 1) streams in a blob's directory."""
    b = np.asarray(blob, dtype=np.uint8)
    return int((stream_modes(b) == 1).sum()) if b.size > 64 else 0
