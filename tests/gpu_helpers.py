"""Shared helpers of the GPU parity tests: load the HIP binding (never a fallback), move
tensors between device and host, and print the case before each GPU step."""
import sys

import numpy as np
import torch


def gq():
    """The HIP binding; fails loudly if libgq.so is missing."""
    from allreduce_compatible_gradient_amd import gq as mod
    return mod


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def first_diff(a: np.ndarray, b: np.ndarray) -> str:
    a = np.asarray(a)
    b = np.asarray(b)
    if a.shape != b.shape:
        return "shape %s vs %s" % (a.shape, b.shape)
    bad = np.flatnonzero(a.reshape(-1) != b.reshape(-1))
    if bad.size == 0:
        return "equal"
    i = bad[0]
    return "%d mismatches, first at %d: %r vs %r" % (bad.size, i, a.reshape(-1)[i], b.reshape(-1)[i])
