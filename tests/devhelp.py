"""numpy <-> torch device helpers for the GPU tests (bit patterns are moved unchanged)."""
import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def words(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(dev())


def f16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(dev())


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()
