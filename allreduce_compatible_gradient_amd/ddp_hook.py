"""Global-QSGD as a PyTorch DDP communication hook (one process per GPU, RCCL).

The pages measure allreduce-compatible quantisation against the methods built into the deep
learning frameworks ("Unbiased Single-scale and Multi-scale Quantizers for Distributed
Optimization", abstract); DDP's communication hooks are where such a method plugs into
PyTorch.  Per gradient bucket the hook runs the Global-QSGD exchange ("Global-QSGD:
Allreduce-Compatible Quantization ...", abstract: global norm scaling, codes summed by
Allreduce):

  1. the bucket's local L2 norm (gq_global_norm, one worker: squares in fp64);
  2. an all-reduce MAX of that norm over the ranks, so that every rank scales by the same
     S = fp32(max_k |x_k|) -- the shared scale of the K-buffer path;
  3. the rank's quantisation as a summable wire payload (gq_quantize_wire, worker = rank);
  4. an all-reduce SUM of the payload as int32 words (RCCL adds 32-bit words; the lanes are
     sized so that no lane carries into the next, and two's-complement int32 addition wraps
     exactly as the unsigned sum the payload is defined on);
  5. the decode of the mean into the bucket (gq_dequantize_wire, world = ranks).

The norm, the quantisation and the decode run in libgq's kernels, the exchange in the
collectives.  Between the two all-reduces the hook does the one-element bookkeeping of the
scale with torch ops on the device: a NaN norm becomes +inf before the MAX (so that it wins,
as an infinite one does), a non-finite maximum becomes 0, and the fp64 maximum is rounded
once to fp32.  A rank whose bucket norm is not finite therefore makes every rank use scale 0
for the bucket (all-zero codes, a zero mean), as a non-finite segment does in gq_global_norm.
"""
import dataclasses
from typing import List, Optional

import torch
import torch.distributed as dist

from allreduce_compatible_gradient_amd import gq


@dataclasses.dataclass
class GlobalQSGDState:
    """Hook state.  grid/levels: the shared level grid (gq.UNIFORM with s levels, or gq.EXP
    with E levels); seed: the run's base seed, from which every (step, bucket) draws a seed of
    its own; record: if a list, each call appends (iteration, seed, bucket input copy, bucket
    output) for inspection."""
    process_group: Optional[dist.ProcessGroup] = None
    grid: int = gq.UNIFORM
    levels: int = 127
    seed: int = 0
    iteration: int = 0
    record: Optional[List] = None


def bucket_seed(state: GlobalQSGDState, bucket_index: int) -> int:
    """The stochastic-rounding seed of one bucket in one step: the same on every rank (the
    ranks differ by their worker key), different for every (step, bucket), so that buckets,
    whose element counters all start at 0, never reuse a stream."""
    return ((state.seed * 0x100000001B3 + state.iteration) * 0x10001 + bucket_index) % (1 << 64)


def global_qsgd_hook(state: GlobalQSGDState,
                     bucket: dist.GradBucket) -> torch.futures.Future[torch.Tensor]:
    pg = state.process_group if state.process_group is not None else dist.group.WORLD
    world = dist.get_world_size(pg)
    rank = dist.get_rank(pg)
    buf = bucket.buffer()
    if buf.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("Global-QSGD hook: bucket dtype %s (float32 or bfloat16)" % buf.dtype)
    if gq.wire_lane_bytes(state.grid, state.levels, world) == 0:
        raise ValueError("no wire lane holds %d ranks at grid %d, levels %d"
                         % (world, state.grid, state.levels))
    n = buf.numel()
    seed = bucket_seed(state, bucket.index())
    if state.record is not None:
        inp = buf.detach().clone()
    norm = torch.empty(1, dtype=torch.float64, device=buf.device)
    scale = torch.empty(1, dtype=torch.float32, device=buf.device)
    gq.global_norm([buf], scale_out=scale, norms_out=norm)
    # a NaN norm must win the MAX like an infinite one (and an infinite one stay infinite)
    torch.nan_to_num_(norm, nan=float("inf"), posinf=float("inf"))
    dist.all_reduce(norm, op=dist.ReduceOp.MAX, group=pg)
    norm.masked_fill_(~torch.isfinite(norm), 0.0)
    scale.copy_(norm)  # fp64 -> fp32, round to nearest even: fp32(max_k |x_k|)
    payload = gq.quantize_wire(buf, scale, state.grid, state.levels, seed, rank, world)
    dist.all_reduce(payload.view(torch.int32), op=dist.ReduceOp.SUM, group=pg)
    gq.dequantize_wire(payload, n, scale, state.grid, state.levels, world,
                       out_dtype=gq.BF16 if buf.dtype == torch.bfloat16 else gq.F32, out=buf)
    if state.record is not None:
        state.record.append((state.iteration, seed, inp, buf.detach().clone()))
    if bucket.is_last():
        state.iteration += 1
    fut = torch.futures.Future()
    fut.set_result(buf)
    return fut
