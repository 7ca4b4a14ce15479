"""Seeded synthetic workloads: shapes, segment tables and gradient generators.

This module holds no arithmetic of the quantisation method.  It only draws random numbers and
lays out shapes, so that the HIP path and the CPU oracle can be fed the very same inputs.

Workloads (each a :class:`Workload`):

``flat-1M-f32-K4-uniform31``
    d = 2^20 fp32 per worker, K = 4, entries N(0, 1); uniform grid s = 31, int8 codes,
    int32 sums, fp32 mean.
``resnet50-161t-f32-K8-exp7``
    the 161 parameter tensors of ResNet-50 (25,557,032 fp32), K = 8, each tensor Laplace(0, b)
    with b = 10^U(-4, -1) drawn per tensor and shared by the workers; exponential grid with
    levels {0, 2^-6 .. 2^0} (E = 7), 4-bit sign+index codes, int16 sums, fp32 mean.
    Segments = tensors.
``gpt2s-148t-bf16-K16-uniform7``
    the 148 parameter tensors of GPT-2 small (124,439,808, tied head), bf16, K = 16,
    1e-3 * Student-t(3); 9 buckets of at most 25 MiB in reverse registration order; uniform
    s = 7, 4-bit codes, int16 sums, bf16 mean.  Segments = buckets.
``flat-1.3G-f32-K8-uniform127``
    one flat bucket of 1.3e9 fp32 per worker, K = 8, 1e-3 * N(0, 1) with 1% of the entries
    multiplied by 100; uniform s = 127, int8 codes, int16 sums, fp32 mean; fused pass.
``lq-4096x4096`` / ``lq-4096x11008``
    LQ-SGD: fp32 gradient matrices, noise of standard deviation 1e-3 plus a rank-8 signal
    U V^T with U, V entries N(0, 1e-3/sqrt(8)) (so both parts carry the same expected
    energy); ranks {1, 4, 7}; alpha = 10, b = 8; Q_0 ~ N(0, 1); E_0 = 0.

Large workloads are drawn on the GPU with torch's counter-based generator in fixed chunks of
2^26 elements, each chunk seeded from (workload, worker, chunk), so any chunk can be redrawn
alone; small ones are drawn on the CPU the same way.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional, Sequence

import numpy as np
import torch

UNIFORM, EXP = 0, 1
CHUNK = 1 << 26
BASE_SEED = 20261203


# ----------------------------------------------------------------------------- shapes
def resnet50_param_shapes() -> List[int]:
    """Element counts of ResNet-50's parameters in registration order (161 tensors)."""
    sizes = [64 * 3 * 7 * 7, 64, 64]
    inplanes = 64
    for planes, blocks in ((64, 3), (128, 4), (256, 6), (512, 3)):
        for b in range(blocks):
            width, out = planes, planes * 4
            sizes += [width * inplanes, width, width]            # 1x1 conv + bn
            sizes += [width * width * 9, width, width]           # 3x3 conv + bn
            sizes += [out * width, out, out]                     # 1x1 conv + bn
            if b == 0:
                sizes += [out * inplanes, out, out]              # downsample conv + bn
            inplanes = out
    sizes += [1000 * 2048, 1000]                                 # fc
    return sizes


def gpt2_small_param_shapes() -> List[int]:
    """Element counts of GPT-2 small's parameters in registration order (148, tied head)."""
    d, ff, vocab, ctx = 768, 3072, 50257, 1024
    sizes = [vocab * d, ctx * d]
    for _ in range(12):
        sizes += [d, d, d * 3 * d, 3 * d, d * d, d, d, d, d * ff, ff, ff * d, d]
    sizes += [d, d]
    return sizes


def ddp_buckets(sizes: Sequence[int], cap_elems: int) -> List[int]:
    """Bucket sizes: whole tensors in reverse registration order, a bucket closed before it
    would exceed the cap; a tensor larger than the cap forms a bucket of its own."""
    buckets, cur = [], 0
    for s in reversed(list(sizes)):
        if cur and cur + s > cap_elems:
            buckets.append(cur)
            cur = 0
        cur += s
        if cur > cap_elems:
            buckets.append(cur)
            cur = 0
    if cur:
        buckets.append(cur)
    return buckets


def offsets_from_sizes(sizes: Sequence[int]) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(sizes, np.int64))]).astype(np.int64)


# ----------------------------------------------------------------------------- workloads
@dataclasses.dataclass
class Workload:
    name: str
    K: int
    n: int
    dtype: str            # "f32" or "bf16"
    grid: int             # UNIFORM or EXP
    levels: int           # s (uniform) or E (exponential)
    bits: int             # code width: 4 or 8
    acc_bits: int         # 16 or 32
    out_dtype: str        # "f32" or "bf16"
    offsets: np.ndarray   # int64, nseg + 1 entries
    dist: str             # "normal", "laplace-per-tensor", "t3", "normal-outliers"
    fused: bool = False
    tensor_sizes: Optional[List[int]] = None

    @property
    def nseg(self) -> int:
        return int(self.offsets.size - 1)

    def grad_bytes(self) -> int:
        return self.K * self.n * (2 if self.dtype == "bf16" else 4)


def _flat(n):
    return offsets_from_sizes([n])


def get(name: str, n: Optional[int] = None) -> Workload:
    """Named workload.  ``n`` shrinks a flat workload (same distribution) for oracle-sized
    parity cases."""
    if name == "flat-1M-f32-K4-uniform31":
        d = n or (1 << 20)
        return Workload(name, 4, d, "f32", UNIFORM, 31, 8, 32, "f32", _flat(d), "normal")
    if name == "resnet50-161t-f32-K8-exp7":
        sizes = resnet50_param_shapes()
        return Workload(name, 8, int(sum(sizes)), "f32", EXP, 7, 4, 16, "f32",
                        offsets_from_sizes(sizes), "laplace-per-tensor", tensor_sizes=sizes)
    if name == "gpt2s-148t-bf16-K16-uniform7":
        sizes = gpt2_small_param_shapes()
        # tensors are laid out bucket by bucket (reverse registration order)
        buckets = ddp_buckets(sizes, (25 << 20) // 2)
        return Workload(name, 16, int(sum(sizes)), "bf16", UNIFORM, 7, 4, 16, "bf16",
                        offsets_from_sizes(buckets), "t3", tensor_sizes=sizes[::-1])
    if name == "flat-1.3G-f32-K8-uniform127":
        d = n or 1_300_000_000
        return Workload(name, 8, d, "f32", UNIFORM, 127, 8, 16, "f32", _flat(d),
                        "normal-outliers", fused=True)
    raise KeyError(name)


def reduced(name: str) -> Workload:
    """Oracle-sized variant of a workload: same distribution, segment structure and codec,
    a few million elements per worker, a ragged end where the layout allows one."""
    if name == "flat-1M-f32-K4-uniform31":
        return get(name)
    if name == "resnet50-161t-f32-K8-exp7":
        full = get(name)
        sizes = full.tensor_sizes[:60]
        w = dataclasses.replace(full, name=name + "-first60", n=int(sum(sizes)),
                                offsets=offsets_from_sizes(sizes), tensor_sizes=sizes)
        return w
    if name == "gpt2s-148t-bf16-K16-uniform7":
        full = get(name)
        tensors, total = [], 0
        for s in full.tensor_sizes:          # reverse registration order
            tensors.append(s)
            total += s
            if total >= 3_000_000:
                break
        buckets = ddp_buckets(tensors[::-1], 1 << 19)
        return dataclasses.replace(full, name=name + "-tail3M", n=int(total),
                                   offsets=offsets_from_sizes(buckets), tensor_sizes=tensors)
    if name == "flat-1.3G-f32-K8-uniform127":
        return get(name, n=(1 << 22) + 13)
    raise KeyError(name)


GLOBAL_QSGD_WORKLOADS = ("flat-1M-f32-K4-uniform31", "resnet50-161t-f32-K8-exp7",
                         "gpt2s-148t-bf16-K16-uniform7", "flat-1.3G-f32-K8-uniform127")
LQ_SHAPES = ((4096, 4096), (4096, 11008))
LQ_RANKS = (1, 4, 7)
LQ_ALPHA = 10.0
LQ_BITS = 8
LQ_WORKERS = 8      # workers of the K-worker step (the flat Global-QSGD workload's count)


# ----------------------------------------------------------------------------- drawing
def _seed(*parts) -> int:
    h = hashlib.sha256(repr((BASE_SEED,) + tuple(parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _draw_chunk(dist: str, cnt: int, g: torch.Generator, device, scale: float = 1.0):
    if dist == "normal":
        return torch.randn(cnt, generator=g, device=device, dtype=torch.float32)
    if dist == "normal-outliers":
        z = torch.randn(cnt, generator=g, device=device, dtype=torch.float32)
        u = torch.rand(cnt, generator=g, device=device, dtype=torch.float32)
        z.mul_(1e-3)
        z[u < 0.01] *= 100.0
        return z
    if dist == "laplace":
        u = torch.rand(cnt, generator=g, device=device, dtype=torch.float64) - 0.5
        x = -scale * torch.sign(u) * torch.log1p(-2.0 * u.abs())
        return x.to(torch.float32)
    if dist == "t3":
        z = torch.randn(cnt, generator=g, device=device, dtype=torch.float64)
        c = torch.randn(3, cnt, generator=g, device=device, dtype=torch.float64)
        chi2 = (c * c).sum(0)
        return (1e-3 * z / torch.sqrt(chi2 / 3.0)).to(torch.float32)
    raise KeyError(dist)


def laplace_scales(w: Workload) -> np.ndarray:
    """Per-tensor Laplace scale b = 10^U(-4, -1), shared by all workers."""
    rng = np.random.default_rng(_seed(w.name, "laplace-b"))
    return 10.0 ** rng.uniform(-4.0, -1.0, size=len(w.tensor_sizes))


def gradient(w: Workload, worker: int, device="cpu") -> torch.Tensor:
    """Worker ``worker``'s flat gradient (torch tensor on ``device``; bf16 workloads return
    torch.bfloat16)."""
    out = torch.empty(w.n, dtype=torch.float32, device=device)
    if w.dist == "laplace-per-tensor":
        b = laplace_scales(w)
        pos = 0
        for t, size in enumerate(w.tensor_sizes):
            g = _gen(device, w.name, worker, "tensor", t)
            out[pos:pos + size] = _draw_chunk("laplace", size, g, device, float(b[t]))
            pos += size
    else:
        for c0 in range(0, w.n, CHUNK):
            cnt = min(CHUNK, w.n - c0)
            g = _gen(device, w.name, w.n, worker, "chunk", c0 // CHUNK)
            out[c0:c0 + cnt] = _draw_chunk(w.dist, cnt, g, device)
    if w.dtype == "bf16":
        return out.to(torch.bfloat16)
    return out


def gradients(w: Workload, device="cpu") -> List[torch.Tensor]:
    return [gradient(w, k, device) for k in range(w.K)]


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host copy; bf16 becomes its uint16 bit pattern."""
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def lq_problem(n: int, m: int, r: int, step: int, device="cpu"):
    """(G_step, Q_0) for the LQ-SGD workload: G = noise(std 1e-3) + U V^T (rank 8)."""
    g = _gen(device, "lq", n, m, "signal")
    sig = (1e-3 / np.sqrt(8.0)) ** 0.5
    U = torch.randn(n, 8, generator=g, device=device, dtype=torch.float64) * sig
    V = torch.randn(m, 8, generator=g, device=device, dtype=torch.float64) * sig
    gs = _gen(device, "lq", n, m, "noise", step)
    G = (torch.randn(n, m, generator=gs, device=device, dtype=torch.float64) * 1e-3
         + U @ V.T).to(torch.float32)
    gq = _gen(device, "lq", n, m, r, "q0")
    Q0 = torch.randn(m, r, generator=gq, device=device, dtype=torch.float32)
    return G.contiguous(), Q0.contiguous()


def lq_worker_problem(n: int, m: int, r: int, step: int, worker: int, device="cpu"):
    """(G, Q_0) of one worker of the K-worker LQ-SGD workload: the shared rank-8 signal of
    lq_problem plus the worker's own noise (std 1e-3); every worker starts from the same Q_0."""
    g = _gen(device, "lq", n, m, "signal")
    sig = (1e-3 / np.sqrt(8.0)) ** 0.5
    U = torch.randn(n, 8, generator=g, device=device, dtype=torch.float64) * sig
    V = torch.randn(m, 8, generator=g, device=device, dtype=torch.float64) * sig
    gs = _gen(device, "lq", n, m, "noise", step, "worker", worker)
    G = (torch.randn(n, m, generator=gs, device=device, dtype=torch.float64) * 1e-3
         + U @ V.T).to(torch.float32)
    gq = _gen(device, "lq", n, m, r, "q0")
    Q0 = torch.randn(m, r, generator=gq, device=device, dtype=torch.float32)
    return G.contiguous(), Q0.contiguous()
