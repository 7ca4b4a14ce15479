"""Thin Python binding of libgq.so (the C ABI in include/gq.h).

Argument marshalling only: every step of the path runs in the library's HIP kernels.  PyTorch
supplies device memory and the current stream; outputs that the caller does not pass are
allocated with ``torch.empty`` on the inputs' device.  If libgq.so is missing this module
raises at import: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import threading
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgq.so")

OK, EINVAL, EOVERFLOW, EALIGN, ELAUNCH, ENONFINITE, ENOMEM = range(7)
F32, BF16 = 0, 1
UNIFORM, EXP = 0, 1
NORM_L2, NORM_MAX = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError("libgq.so is not built (%s); run `python -m "
                      "allreduce_compatible_gradient_amd.build`" % LIB_PATH)

_lib = C.CDLL(LIB_PATH)
_p, _i32, _i64, _u32, _u64, _d = (C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_uint64,
                                   C.c_double)
_SIGS = {
    "gq_create": (_i32, [C.POINTER(C.c_void_p)]),
    "gq_destroy": (None, [_p]),
    "gq_last_error": (C.c_char_p, [_p]),
    "gq_version": (C.c_char_p, []),
    "gq_read_status": (_i32, [_p, _p]),
    "gq_global_norm": (_i32, [_p, _p, _i32, _i32, _i64, _p, _i32, _p, _p, _p]),
    "gq_quantize_pack": (_i32, [_p, _p, _i32, _i64, _p, _i32, _p, _i32, _i32, _i32, _u64, _u32,
                                _u32, _p, _p]),
    "gq_accumulate_codes": (_i32, [_p, _p, _i32, _i64, _i32, _i32, _i32, _i32, _p, _p]),
    "gq_dequantize": (_i32, [_p, _p, _i32, _i64, _p, _i32, _p, _i32, _i32, _i32, _i32, _p, _p]),
    "gq_fused_mean": (_i32, [_p, _p, _i32, _i32, _i64, _p, _i32, _p, _i32, _i32, _i32, _u64, _u32,
                             _i32, _p, _p, _i32, _p, _p]),
    "gq_worker_scales": (_i32, [_p, _p, _i32, _i32, _i64, _p, _i32, _i32, _p, _p]),
    "gq_worker_mean": (_i32, [_p, _p, _i32, _i32, _i64, _p, _i32, _p, _i32, _i32, _u64, _u32,
                              _i32, _p, _p]),
    "gq_decode_workers": (_i32, [_p, _p, _i32, _i64, _p, _i32, _p, _i32, _i32, _i32, _i32, _p,
                                 _p]),
    "gq_logquant": (_i32, [_p, _p, _i64, _i32, _d, _i32, _p, _p, _p, _p]),
    "gq_wire_lane_bytes": (_i32, [_i32, _i32, _i32]),
    "gq_quantize_wire": (_i32, [_p, _p, _i32, _i64, _p, _i32, _p, _i32, _i32, _u64, _u32, _u32,
                                _i32, _p, _p]),
    "gq_dequantize_wire": (_i32, [_p, _p, _i64, _p, _i32, _p, _i32, _i32, _i32, _i32, _p, _p]),
    "gq_powersgd_logquant": (_i32, [_p, _p, _p, _p, _i64, _i64, _i32, _d, _i32, _i32, _p, _p,
                                    _p, _p, _p, _p, _p, _p]),
    "gq_lq_step_workers": (_i32, [_p, _p, _p, _p, _i32, _i64, _i64, _i32, _d, _i32, _i32, _p,
                                  _p, _p, _p, _p, _p, _p, _p]),
    "gq_trim": (_i32, [_p]),
    "gq_global_norm_noalloc": (_i32, [_p, _p, _i32, _i32, _i64, _p, _i32, _p, _p, _p]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class GQError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("gq error %d: %s" % (code, msg))
        self.code = code


class Context:
    """A gq_ctx on the current device.  Not thread-safe; one per stream."""

    def __init__(self):
        h = C.c_void_p()
        st = _lib.gq_create(C.byref(h))
        if st != OK:
            raise GQError(st, "gq_create failed")
        self.handle = h

    def close(self):
        if self.handle:
            _lib.gq_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def check(self, st: int):
        if st != OK:
            raise GQError(st, _lib.gq_last_error(self.handle).decode())


_tls = threading.local()


def context() -> Context:
    """The default context of this thread for the current device.  It is shared by every
    stream, which keeps the usual pattern working -- warm up eagerly, then capture the same
    calls into a graph on another stream without allocating during capture; work issued on
    two streams at the same time needs a Context for each (ctx=...), since a context's
    scratch must not be used by two streams at once."""
    dev = torch.cuda.current_device()
    ctxs = getattr(_tls, "ctxs", None)
    if ctxs is None:
        ctxs = _tls.ctxs = {}
    if dev not in ctxs:
        ctxs[dev] = Context()
    return ctxs[dev]


def version() -> str:
    return _lib.gq_version().decode()


# ----------------------------------------------------------------------------- marshalling
def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    return t.data_ptr()


def _elt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("gradients must be float32 or bfloat16, got %s" % t.dtype)


def _torch_dtype(code: int):
    return torch.float32 if code == F32 else torch.bfloat16


def _ptr_array(ptrs: Sequence[int]):
    return (C.c_void_p * len(ptrs))(*ptrs)


def _offsets(offsets, n):
    if offsets is None:
        return None, 1, None
    import numpy as np
    arr = np.ascontiguousarray(offsets, dtype=np.int64)
    return arr.ctypes.data_as(C.c_void_p), int(arr.size - 1), arr


def code_bytes(n: int, bits: int) -> int:
    return n if bits == 8 else (n + 1) // 2


# ----------------------------------------------------------------------------- Global-QSGD
def global_norm(grads: Sequence[torch.Tensor], offsets=None, scale_out=None, norms_out=None,
                ctx: Optional[Context] = None):
    """S_g = fp32(max_k ||x_k restricted to segment g||_2).  Returns (scale, norms)."""
    ctx = ctx or context()
    n = grads[0].numel()
    dt = _elt(grads[0])
    ptrs = [_dev(g, "grads[%d]" % k, grads[0].dtype) for k, g in enumerate(grads)]
    off, nseg, keep = _offsets(offsets, n)
    dev = grads[0].device
    if scale_out is None:
        scale_out = torch.empty(nseg, dtype=torch.float32, device=dev)
    ctx.check(_lib.gq_global_norm(ctx.handle, _ptr_array(ptrs), len(grads), dt, n, off, nseg,
                                  _dev(scale_out, "scale_out", torch.float32),
                                  None if norms_out is None else
                                  _dev(norms_out, "norms_out", torch.float64), _stream()))
    return scale_out, norms_out


def global_norm_noalloc(grads: Sequence[torch.Tensor], offsets, scale_out, norms_out=None,
                        ctx: Optional[Context] = None):
    """gq_global_norm_noalloc: global_norm with its temporaries in the library's fixed buffer;
    the caller passes scale_out (nseg fp32) and optionally norms_out (K*nseg fp64)."""
    ctx = ctx or context()
    n = grads[0].numel()
    dt = _elt(grads[0])
    ptrs = [_dev(g, "grads[%d]" % k, grads[0].dtype) for k, g in enumerate(grads)]
    off, nseg, keep = _offsets(offsets, n)
    ctx.check(_lib.gq_global_norm_noalloc(ctx.handle, _ptr_array(ptrs), len(grads), dt, n, off,
                                          nseg, _dev(scale_out, "scale_out", torch.float32),
                                          None if norms_out is None else
                                          _dev(norms_out, "norms_out", torch.float64),
                                          _stream()))
    return scale_out, norms_out


def quantize_pack(grad, scale, grid, levels, bits, seed, worker, index_base=0, offsets=None,
                  codes=None, ctx: Optional[Context] = None):
    ctx = ctx or context()
    n = grad.numel()
    off, nseg, keep = _offsets(offsets, n)
    if codes is None:
        codes = torch.empty(code_bytes(n, bits), dtype=torch.uint8, device=grad.device)
    ctx.check(_lib.gq_quantize_pack(ctx.handle, _dev(grad, "grad"), _elt(grad), n, off, nseg,
                                    _dev(scale, "scale", torch.float32), grid, levels, bits,
                                    seed, worker, index_base, _dev(codes, "codes", torch.uint8),
                                    _stream()))
    return codes


def accumulate_codes(codes: Sequence[torch.Tensor], n, grid, levels, bits, acc_bits, sums=None,
                     ctx: Optional[Context] = None):
    ctx = ctx or context()
    ptrs = [_dev(c, "codes[%d]" % k, torch.uint8) for k, c in enumerate(codes)]
    if sums is None:
        sums = torch.empty(n, dtype=torch.int16 if acc_bits == 16 else torch.int32,
                           device=codes[0].device)
    ctx.check(_lib.gq_accumulate_codes(ctx.handle, _ptr_array(ptrs), len(codes), n, grid, levels,
                                       bits, acc_bits, _dev(sums, "sums"), _stream()))
    return sums


def dequantize(sums, scale, grid, levels, K, out_dtype=F32, offsets=None, out=None,
               ctx: Optional[Context] = None):
    ctx = ctx or context()
    n = sums.numel()
    acc_bits = 16 if sums.dtype == torch.int16 else 32
    off, nseg, keep = _offsets(offsets, n)
    if out is None:
        out = torch.empty(n, dtype=_torch_dtype(out_dtype), device=sums.device)
    ctx.check(_lib.gq_dequantize(ctx.handle, _dev(sums, "sums", (torch.int16, torch.int32)),
                                 acc_bits, n, off, nseg, _dev(scale, "scale", torch.float32),
                                 grid, levels, K, out_dtype, _dev(out, "out"), _stream()))
    return out


def wire_lane_bytes(grid, levels, world) -> int:
    """Bytes per element of the summable wire payload for `world` workers (0: none fits)."""
    return int(_lib.gq_wire_lane_bytes(grid, levels, world))


def wire_bytes(n: int, grid, levels, world) -> int:
    return (n * wire_lane_bytes(grid, levels, world) + 3) // 4 * 4


def quantize_wire(grad, scale, grid, levels, seed, worker, world, index_base=0, offsets=None,
                  payload=None, ctx: Optional[Context] = None):
    """One worker's quantisation as a summable payload (uint8 tensor, a multiple of 4 bytes)."""
    ctx = ctx or context()
    n = grad.numel()
    off, nseg, keep = _offsets(offsets, n)
    if payload is None:
        payload = torch.empty(max(wire_bytes(n, grid, levels, world), 4), dtype=torch.uint8,
                              device=grad.device)
    ctx.check(_lib.gq_quantize_wire(ctx.handle, _dev(grad, "grad"), _elt(grad), n, off, nseg,
                                    _dev(scale, "scale", torch.float32), grid, levels, seed,
                                    worker, index_base, world,
                                    _dev(payload, "payload", torch.uint8), _stream()))
    return payload


def dequantize_wire(payload, n, scale, grid, levels, world, out_dtype=F32, offsets=None,
                    out=None, ctx: Optional[Context] = None):
    """The mean from the word-wise sum of `world` payloads."""
    ctx = ctx or context()
    off, nseg, keep = _offsets(offsets, n)
    if out is None:
        out = torch.empty(n, dtype=_torch_dtype(out_dtype), device=payload.device)
    ctx.check(_lib.gq_dequantize_wire(ctx.handle, _dev(payload, "payload", torch.uint8), n, off,
                                      nseg, _dev(scale, "scale", torch.float32), grid, levels,
                                      world, out_dtype, _dev(out, "out"), _stream()))
    return out


def fused_mean(grads, scale, grid, levels, bits, seed, acc_bits, out_dtype=F32, index_base=0,
               offsets=None, codes=None, sums=None, out=None, ctx: Optional[Context] = None):
    """Quantise every worker, sum the codes and decode the mean in one pass.  ``codes`` (list
    of K uint8 tensors) and ``sums`` are written only when given."""
    ctx = ctx or context()
    n = grads[0].numel()
    ptrs = [_dev(g, "grads[%d]" % k, grads[0].dtype) for k, g in enumerate(grads)]
    off, nseg, keep = _offsets(offsets, n)
    if out is None:
        out = torch.empty(n, dtype=_torch_dtype(out_dtype), device=grads[0].device)
    cptr = None
    if codes is not None:
        cptr = _ptr_array([_dev(c, "codes[%d]" % k, torch.uint8) for k, c in enumerate(codes)])
    ctx.check(_lib.gq_fused_mean(ctx.handle, _ptr_array(ptrs), len(grads), _elt(grads[0]), n, off,
                                 nseg, _dev(scale, "scale", torch.float32), grid, levels, bits,
                                 seed, index_base, acc_bits, cptr,
                                 None if sums is None else _dev(sums, "sums"), out_dtype,
                                 _dev(out, "out"), _stream()))
    return out


# ----------------------------------------------------------------------------- baselines
def worker_scales(grads, norm=NORM_L2, offsets=None, out=None, ctx: Optional[Context] = None):
    """Each worker's own scale per segment (K x nseg fp32): L2 norm, or largest magnitude for
    NORM_MAX (QSGD / QSGDinf)."""
    ctx = ctx or context()
    n = grads[0].numel()
    ptrs = [_dev(g, "grads[%d]" % k, grads[0].dtype) for k, g in enumerate(grads)]
    off, nseg, keep = _offsets(offsets, n)
    if out is None:
        out = torch.empty(len(grads), nseg, dtype=torch.float32, device=grads[0].device)
    ctx.check(_lib.gq_worker_scales(ctx.handle, _ptr_array(ptrs), len(grads), _elt(grads[0]), n,
                                    off, nseg, norm, _dev(out, "out", torch.float32), _stream()))
    return out


def worker_mean(grads, scales, grid, levels, seed, out_dtype=F32, index_base=0, offsets=None,
                out=None, ctx: Optional[Context] = None):
    """Mean of the workers' decoded values, each quantised and decoded with its own scale
    (scales: K x nseg fp32, e.g. from worker_scales)."""
    ctx = ctx or context()
    n = grads[0].numel()
    ptrs = [_dev(g, "grads[%d]" % k, grads[0].dtype) for k, g in enumerate(grads)]
    off, nseg, keep = _offsets(offsets, n)
    if scales.numel() != len(grads) * nseg:
        raise ValueError("scales must hold K * nseg values")
    if out is None:
        out = torch.empty(n, dtype=_torch_dtype(out_dtype), device=grads[0].device)
    ctx.check(_lib.gq_worker_mean(ctx.handle, _ptr_array(ptrs), len(grads), _elt(grads[0]), n,
                                  off, nseg, _dev(scales, "scales", torch.float32), grid, levels,
                                  seed, index_base, out_dtype, _dev(out, "out"), _stream()))
    return out


def decode_workers(codes, n, scales, grid, levels, bits, out_dtype=F32, offsets=None, out=None,
                   ctx: Optional[Context] = None):
    """Receiver's mean of K workers' packed codes (list of uint8 tensors), each decoded with
    its own scale (scales: K x nseg fp32)."""
    ctx = ctx or context()
    off, nseg, keep = _offsets(offsets, n)
    if scales.numel() != len(codes) * nseg:
        raise ValueError("scales must hold K * nseg values")
    if out is None:
        out = torch.empty(n, dtype=_torch_dtype(out_dtype), device=codes[0].device)
    cptr = _ptr_array([_dev(c, "codes[%d]" % k, torch.uint8) for k, c in enumerate(codes)])
    ctx.check(_lib.gq_decode_workers(ctx.handle, cptr, len(codes), n, off, nseg,
                                     _dev(scales, "scales", torch.float32), grid, levels, bits,
                                     out_dtype, _dev(out, "out"), _stream()))
    return out


def read_status(ctx: Optional[Context] = None) -> int:
    """Synchronises the current stream; returns ENONFINITE if a norm was not finite."""
    ctx = ctx or context()
    return _lib.gq_read_status(ctx.handle, _stream())


# ----------------------------------------------------------------------------- LQ-SGD
def logquant(F, alpha, bits, codes=None, colmax=None, F_hat=None, want_hat=True,
             ctx: Optional[Context] = None):
    ctx = ctx or context()
    rows, r = F.shape
    dev = F.device
    if codes is None:
        codes = torch.empty(rows, r, dtype=torch.int8, device=dev)
    if colmax is None:
        colmax = torch.empty(r, dtype=torch.float32, device=dev)
    if F_hat is None and want_hat:
        F_hat = torch.empty(rows, r, dtype=torch.float32, device=dev)
    ctx.check(_lib.gq_logquant(ctx.handle, _dev(F, "F", torch.float32), rows, r, alpha, bits,
                               _dev(codes, "codes", torch.int8),
                               _dev(colmax, "colmax", torch.float32),
                               None if F_hat is None else _dev(F_hat, "F_hat", torch.float32),
                               _stream()))
    return codes, colmax, F_hat


def powersgd_logquant(G, E, Q, alpha, bits, out=None, want_hat=True, want_pre=False,
                      bits_q=None, ctx: Optional[Context] = None):
    """One LQ-SGD compressor step; E and Q are updated in place.  ``bits`` is the code width of
    P, ``bits_q`` that of Q' (default: the same).  Returns a dict of outputs."""
    ctx = ctx or context()
    n, m = G.shape
    r = Q.shape[1]
    dev = G.device
    o = dict(out or {})
    o.setdefault("p_codes", torch.empty(n, r, dtype=torch.int8, device=dev))
    o.setdefault("p_colmax", torch.empty(r, dtype=torch.float32, device=dev))
    o.setdefault("q_codes", torch.empty(m, r, dtype=torch.int8, device=dev))
    o.setdefault("q_colmax", torch.empty(r, dtype=torch.float32, device=dev))
    if want_hat:
        o.setdefault("p_hat", torch.empty(n, r, dtype=torch.float32, device=dev))
    if want_pre:
        o.setdefault("p_pre", torch.empty(n, r, dtype=torch.float32, device=dev))
        o.setdefault("q_pre", torch.empty(m, r, dtype=torch.float32, device=dev))

    def opt(k):
        return None if o.get(k) is None else _dev(o[k], k, torch.float32)

    ctx.check(_lib.gq_powersgd_logquant(
        ctx.handle, _dev(G, "G", torch.float32), _dev(E, "E", torch.float32),
        _dev(Q, "Q", torch.float32), n, m, r, alpha, bits, bits if bits_q is None else bits_q,
        _dev(o["p_codes"], "p_codes", torch.int8), _dev(o["p_colmax"], "p_colmax", torch.float32),
        _dev(o["q_codes"], "q_codes", torch.int8), _dev(o["q_colmax"], "q_colmax", torch.float32),
        opt("p_hat"), opt("p_pre"), opt("q_pre"), _stream()))
    return o


def lq_step_workers(Gs, Es, Qs, alpha, bits, bits_q=None, out=None, want_pre=False,
                    ctx: Optional[Context] = None):
    """One LQ-SGD step of K workers (lists of n x m gradients, n x m errors and m x r warm
    starts; E's and Q's are updated in place).  Returns a dict with every worker's message
    stacked by worker (p_codes K x n x r, p_colmax K x r, q_codes K x m x r, q_colmax K x r)
    and G_hat (n x m), the mean of the decoded messages; with want_pre also every worker's
    factors before quantisation (p_pre K x n x r, q_pre K x m x r)."""
    ctx = ctx or context()
    K = len(Gs)
    if not (len(Es) == K and len(Qs) == K):
        raise ValueError("Gs, Es and Qs must have one entry per worker")
    n, m = Gs[0].shape
    r = Qs[0].shape[1]
    for k in range(K):
        if tuple(Gs[k].shape) != (n, m) or tuple(Es[k].shape) != (n, m):
            raise ValueError("worker %d: G and E must be %d x %d" % (k, n, m))
        if tuple(Qs[k].shape) != (m, r):
            raise ValueError("worker %d: Q must be %d x %d" % (k, m, r))
    dev = Gs[0].device
    o = dict(out or {})
    o.setdefault("p_codes", torch.empty(K, n, r, dtype=torch.int8, device=dev))
    o.setdefault("p_colmax", torch.empty(K, r, dtype=torch.float32, device=dev))
    o.setdefault("q_codes", torch.empty(K, m, r, dtype=torch.int8, device=dev))
    o.setdefault("q_colmax", torch.empty(K, r, dtype=torch.float32, device=dev))
    o.setdefault("G_hat", torch.empty(n, m, dtype=torch.float32, device=dev))
    if want_pre:
        o.setdefault("p_pre", torch.empty(K, n, r, dtype=torch.float32, device=dev))
        o.setdefault("q_pre", torch.empty(K, m, r, dtype=torch.float32, device=dev))

    def opt(k):
        return None if o.get(k) is None else _dev(o[k], k, torch.float32)

    gp = _ptr_array([_dev(G, "G[k]", torch.float32) for G in Gs])
    ep = _ptr_array([_dev(E, "E[k]", torch.float32) for E in Es])
    qp = _ptr_array([_dev(Q, "Q[k]", torch.float32) for Q in Qs])
    ctx.check(_lib.gq_lq_step_workers(
        ctx.handle, gp, ep, qp, K, n, m, r, alpha, bits, bits if bits_q is None else bits_q,
        _dev(o["p_codes"], "p_codes", torch.int8), _dev(o["p_colmax"], "p_colmax", torch.float32),
        _dev(o["q_codes"], "q_codes", torch.int8), _dev(o["q_colmax"], "q_colmax", torch.float32),
        _dev(o["G_hat"], "G_hat", torch.float32), opt("p_pre"), opt("q_pre"), _stream()))
    return o


def trim(ctx: Optional[Context] = None) -> None:
    """Wait for the device and free the buffers the context has retired (see gq_trim)."""
    ctx = ctx or context()
    ctx.check(_lib.gq_trim(ctx.handle))
