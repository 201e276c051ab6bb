"""Small helpers for the GPU tests: moving seeded numpy inputs (fp32 values
or bf16 bit patterns) to the device and GPU outputs back as fp64."""
import sys

import numpy as np
import torch

DEV = "cuda"


def announce(*args):
    """Name the case before a GPU step, flushed, so a fault names its case."""
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def dev_i64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(DEV)


def bits(t):
    """Raw bit patterns of a GPU tensor (for bitwise comparisons)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.cpu().numpy().view(np.uint32)
    return t.cpu().numpy()


def f64(t):
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        b = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def sync():
    torch.cuda.synchronize()
