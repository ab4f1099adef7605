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
