"""The Global-QSGD DDP communication hook on one GPU (RCCL process group of one rank).

A small model's buckets go through the hook (global norm, all-reduce MAX of the norm, wire
quantiser, int32 all-reduce SUM of the payload, wire decode); each bucket's result must equal,
bit for bit, the oracle's whole path on the same bucket gradient with the same seed: the
shared scale of one worker, its quantisation and the decode of the summed codes.  The
gradients DDP leaves in the parameters are the hook's output.
"""
import os
import socket

import numpy as np
import pytest
import torch

from tests.gpu_helpers import first_diff, say

pytestmark = pytest.mark.gpu


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


@pytest.fixture(scope="module")
def process_group():
    import torch.distributed as dist
    if not dist.is_initialized():
        dist.init_process_group("nccl", init_method="tcp://127.0.0.1:%d" % _free_port(),
                                rank=0, world_size=1)
        yield dist.group.WORLD
        dist.destroy_process_group()
    else:
        yield dist.group.WORLD


def _model(dtype):
    torch.manual_seed(5)
    m = torch.nn.Sequential(torch.nn.Linear(96, 512), torch.nn.ReLU(),
                            torch.nn.Linear(512, 256), torch.nn.ReLU(),
                            torch.nn.Linear(256, 40)).to("cuda", dtype)
    return m


@pytest.mark.parametrize("grid,levels,dtype", [(0, 127, torch.float32), (1, 7, torch.float32),
                                               (0, 7, torch.bfloat16)])
def test_hook_buckets_equal_the_oracle(process_group, grid, levels, dtype):
    from torch.nn.parallel import DistributedDataParallel as DDP
    from allreduce_compatible_gradient_amd import ddp_hook
    from allreduce_compatible_gradient_amd import workloads as W
    from oracle import oracle as orc
    say("ddp hook", grid, levels, dtype)
    model = DDP(_model(dtype), device_ids=[0], bucket_cap_mb=0.25)
    state = ddp_hook.GlobalQSGDState(process_group=process_group, grid=grid, levels=levels,
                                     seed=11, record=[])
    model.register_comm_hook(state, ddp_hook.global_qsgd_hook)
    gen = torch.Generator(device="cuda").manual_seed(3)
    for step in range(2):
        x = torch.randn(64, 96, device="cuda", generator=gen).to(dtype)
        model(x).float().square().mean().backward()
    torch.cuda.synchronize()
    assert state.iteration == 2
    assert {it for it, _, _, _ in state.record} == {0, 1}
    seeds = [s for _, s, _, _ in state.record]
    assert len(set(seeds)) == len(seeds)     # a fresh stream per bucket and step
    out_dtype = orc.BF16 if dtype == torch.bfloat16 else orc.F32
    for _, seed, inp, out in state.record:
        xs = [W.to_numpy(inp)]
        ref = orc.allreduce_mean(xs, grid, levels, 8, 32, seed, 0, out_dtype=out_dtype)
        got = W.to_numpy(out)
        assert np.array_equal(got, ref["mean"]), first_diff(got, ref["mean"])
    # the last step's gradients are the hook's outputs of that step's buckets
    last = [r for r in state.record if r[0] == 1]
    flat = torch.cat([o.flatten() for _, _, _, o in last])
    grads = torch.cat([p.grad.flatten() for p in model.parameters()])
    assert sorted(flat.float().tolist()) == sorted(grads.float().tolist())


def test_hook_zero_scale_for_a_non_finite_bucket(process_group):
    """A NaN in a bucket makes the all-reduced norm non-finite: scale 0, an all-zero mean."""
    from torch.nn.parallel import DistributedDataParallel as DDP
    from allreduce_compatible_gradient_amd import ddp_hook
    say("ddp hook non-finite")
    model = DDP(_model(torch.float32), device_ids=[0], bucket_cap_mb=25)
    state = ddp_hook.GlobalQSGDState(process_group=process_group, record=[])
    model.register_comm_hook(state, ddp_hook.global_qsgd_hook)
    x = torch.randn(8, 96, device="cuda")
    x[0, 0] = float("nan")
    model(x).square().mean().backward()
    torch.cuda.synchronize()
    assert state.record
    for _, _, inp, out in state.record:
        assert not torch.isfinite(inp).all()
        assert not out.any()
