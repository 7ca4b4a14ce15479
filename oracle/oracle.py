"""ctypes binding of the plain C oracle (gq_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check at the repository root and the
``cpu_baseline`` leg of ``bench.py``.  The product package never imports this module, and this
module imports nothing from the product package.

Every function takes and returns numpy arrays; bf16 data travels as ``uint16`` bit patterns.
The library is compiled from ``gq_oracle.c`` by :func:`build` (gcc, ``-O2 -ffp-contract=off``,
no fast-math) and rebuilt automatically when the source is newer than the shared object.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gq_oracle.c")
HDR = os.path.join(HERE, "gq_oracle.h")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16 = 0, 1
UNIFORM, EXP = 0, 1
NORM_L2, NORM_MAX = 0, 1

_lib = None


def compile_library(src: str, out: str) -> str:
    """gcc -O2 -ffp-contract=off (no fast-math) of one oracle source into a shared object."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
                           "-fPIC", "-shared", "-Wall", "-Wextra", "-I", HERE, "-o", tmp, src,
                           "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc; returns its path."""
    stale = (not os.path.exists(LIB)) or any(
        os.path.getmtime(p) > os.path.getmtime(LIB) for p in (SRC, HDR))
    if force or stale:
        compile_library(SRC, LIB)
    return LIB


def lib():
    """The loaded oracle.  GQ_ORACLE_LIB names another build of it to load instead (the
    planted-mistake tests use this to run the pins against a deliberately wrong oracle)."""
    global _lib
    if _lib is None:
        path = os.environ.get("GQ_ORACLE_LIB")
        if not path:
            path = build()
        L = C.CDLL(path)
        p, i32, i64, u32, u64, d, f = (C.c_void_p, C.c_int32, C.c_int64, C.c_uint32,
                                       C.c_uint64, C.c_double, C.c_float)
        sig = {
            "orc_splitmix64_next": (u64, [C.POINTER(C.c_uint64)]),
            "orc_fmix32": (u32, [u32]),
            "orc_worker_key": (u32, [u64, u32]),
            "orc_uniform": (d, [u32, u32]),
            "orc_hash_fill": (None, [u32, u32, i64, p]),
            "orc_sumsq": (d, [p, i32, i64, d]),
            "orc_global_norm": (i32, [p, i32, i32, i64, p, i32, p, p]),
            "orc_norm_finish": (i32, [p, i32, i32, p, p]),
            "orc_quant_one": (i32, [i32, i32, f, f, u32, u32]),
            "orc_quantize": (None, [p, i32, i64, p, i32, p, i32, i32, u64, u32, u32, p]),
            "orc_quantize_list": (None, [p, p, p, i64, i32, i32, u32, p]),
            "orc_pack": (None, [p, i64, i32, i32, p]),
            "orc_unpack_one": (i32, [p, i64, i32, i32]),
            "orc_lin": (i64, [i32, i32]),
            "orc_accumulate": (i64, [p, i32, i64, i32, i32, i32, p]),
            "orc_decode_factor": (f, [i32, i32, i32, f]),
            "orc_wire_lane_bytes": (i32, [i32, i32, i32]),
            "orc_wire_encode": (None, [p, i64, i32, i32, i32, p]),
            "orc_wire_sum": (None, [p, i32, i64, p]),
            "orc_wire_decode": (None, [p, i64, i32, i32, i32, p]),
            "orc_f32_to_bf16": (C.c_uint16, [f]),
            "orc_dequantize": (None, [p, i32, i64, p, i32, p, i32, i32, i32, i32, p]),
            "orc_worker_scales": (i32, [p, i32, i32, i64, p, i32, i32, p]),
            "orc_worker_mean": (None, [p, i32, i32, i64, p, i32, p, i32, i32, u64, u32, i32, p]),
            "orc_decode_workers": (None, [p, i32, i64, p, i32, p, i32, i32, i32, i32, p]),
            "orc_logq_index": (i32, [f, d, i32]),
            "orc_logq_level": (f, [i32, d, i32]),
            "orc_logquant": (None, [p, i64, i32, d, i32, p, p, p]),
            "orc_mgs": (None, [p, i64, i32, i64]),
            "orc_mgs_rho": (d, [i64]),
            "orc_powersgd_logquant": (None, [p, p, p, i64, i64, i32, d, i32, i32, p, p, p, p, p,
                                             p, p]),
            "orc_lq_step_workers": (None, [p, p, p, i32, i64, i64, i32, d, i32, i32, p, p, p, p,
                                           p]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _ptrs(arrs):
    arr = (C.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    return arr


def _offsets(offsets, n):
    if offsets is None:
        offsets = [0, n]
    return _c(offsets, np.int64)


def _dtype_code(x):
    return BF16 if x.dtype == np.uint16 else F32


# ---------------------------------------------------------------- random numbers
def splitmix64_outputs(seed: int, count: int):
    st = C.c_uint64(seed)
    return [lib().orc_splitmix64_next(C.byref(st)) for _ in range(count)]


def fmix32(h: int) -> int:
    return lib().orc_fmix32(h & 0xFFFFFFFF)


def worker_key(seed: int, worker: int) -> int:
    return lib().orc_worker_key(seed, worker)


def uniform(key: int, counter: int) -> float:
    return lib().orc_uniform(key, counter)


def hash_fill(key: int, counter0: int, cnt: int):
    out = np.empty(cnt, np.uint32)
    lib().orc_hash_fill(key, counter0, cnt, _ptr(out))
    return out


# ---------------------------------------------------------------- global norm
def sumsq(x, acc: float = 0.0) -> float:
    x = np.ascontiguousarray(x)
    return lib().orc_sumsq(_ptr(x), _dtype_code(x), x.size, acc)


def global_norm(xs, offsets=None):
    """xs: list of K equal-length fp32 (or uint16-as-bf16) arrays.  Returns (S, norms, bad)."""
    xs = [np.ascontiguousarray(x) for x in xs]
    n = xs[0].size
    off = _offsets(offsets, n)
    nseg = off.size - 1
    S = np.zeros(nseg, np.float32)
    norms = np.zeros((len(xs), nseg), np.float64)
    bad = lib().orc_global_norm(_ptrs(xs), len(xs), _dtype_code(xs[0]), n, _ptr(off), nseg,
                                _ptr(S), _ptr(norms))
    return S, norms, bool(bad)


def norm_finish(sumsq):
    """(S, norms, bad) from a K x nseg array of per-worker, per-segment sums of squares (for
    data streamed through sumsq() chunk by chunk, in index order, which gives global_norm's
    arithmetic exactly)."""
    ss = _c(np.atleast_2d(sumsq), np.float64)
    K, nseg = ss.shape
    S = np.zeros(nseg, np.float32)
    norms = np.zeros((K, nseg), np.float64)
    bad = lib().orc_norm_finish(_ptr(ss), K, nseg, _ptr(S), _ptr(norms))
    return S, norms, bool(bad)


# ---------------------------------------------------------------- quantisation and codes
def quant_one(grid, levels, x, S, key, counter) -> int:
    return lib().orc_quant_one(grid, levels, float(np.float32(x)), float(np.float32(S)), key,
                               counter)


def quantize(x, scale, grid, levels, seed, worker, index_base=0, offsets=None):
    x = np.ascontiguousarray(x)
    off = _offsets(offsets, x.size)
    sc = _c(scale, np.float32)
    out = np.empty(x.size, np.int32)
    lib().orc_quantize(_ptr(x), _dtype_code(x), x.size, _ptr(off), off.size - 1, _ptr(sc),
                       grid, levels, seed, worker, index_base, _ptr(out))
    return out


def quantize_list(x, S, counters, grid, levels, key):
    x = _c(x, np.float32)
    S = _c(S, np.float32)
    cnt = _c(counters, np.uint32)
    out = np.empty(x.size, np.int32)
    lib().orc_quantize_list(_ptr(x), _ptr(S), _ptr(cnt), x.size, grid, levels, key, _ptr(out))
    return out


def pack(q, grid, bits):
    q = _c(q, np.int32)
    out = np.empty(q.size if bits == 8 else (q.size + 1) // 2, np.uint8)
    lib().orc_pack(_ptr(q), q.size, grid, bits, _ptr(out))
    return out


def unpack(codes, n, grid, bits):
    codes = _c(codes, np.uint8)
    return np.array([lib().orc_unpack_one(_ptr(codes), i, grid, bits) for i in range(n)],
                    np.int32)


def lin(grid, q) -> int:
    return lib().orc_lin(grid, q)


def accumulate(codes_list, n, grid, bits, acc_bits):
    codes_list = [_c(c, np.uint8) for c in codes_list]
    out = np.empty(n, np.int16 if acc_bits == 16 else np.int32)
    over = lib().orc_accumulate(_ptrs(codes_list), len(codes_list), n, grid, bits, acc_bits,
                                _ptr(out))
    return out, int(over)


def wire_lane_bytes(grid, levels, world) -> int:
    return lib().orc_wire_lane_bytes(grid, levels, world)


def wire_encode(q, grid, levels, world):
    """Summable payload (uint8 array, a multiple of 4 bytes) of signed levels q."""
    q = _c(q, np.int32)
    w = wire_lane_bytes(grid, levels, world)
    out = np.empty((q.size * w + 3) // 4 * 4, np.uint8)
    lib().orc_wire_encode(_ptr(q), q.size, grid, levels, world, _ptr(out))
    return out


def wire_sum(payloads):
    payloads = [_c(p, np.uint8) for p in payloads]
    out = np.empty(payloads[0].size, np.uint8)
    lib().orc_wire_sum(_ptrs(payloads), len(payloads), payloads[0].size, _ptr(out))
    return out


def wire_decode(payload, n, grid, levels, world):
    """Integer sums (int32) held by a summed payload."""
    payload = _c(payload, np.uint8)
    out = np.empty(n, np.int32)
    lib().orc_wire_decode(_ptr(payload), n, grid, levels, world, _ptr(out))
    return out


def decode_factor(grid, levels, K, S) -> float:
    return lib().orc_decode_factor(grid, levels, K, float(np.float32(S)))


def f32_to_bf16(v) -> int:
    return lib().orc_f32_to_bf16(float(np.float32(v)))


def dequantize(sums, scale, grid, levels, K, out_dtype=F32, offsets=None):
    sums = np.ascontiguousarray(sums)
    acc_bits = 16 if sums.dtype == np.int16 else 32
    off = _offsets(offsets, sums.size)
    sc = _c(scale, np.float32)
    out = np.empty(sums.size, np.uint16 if out_dtype == BF16 else np.float32)
    lib().orc_dequantize(_ptr(sums), acc_bits, sums.size, _ptr(off), off.size - 1, _ptr(sc),
                         grid, levels, K, out_dtype, _ptr(out))
    return out


def allreduce_mean(xs, grid, levels, bits, acc_bits, seed, index_base=0, offsets=None,
                   out_dtype=F32, scale=None):
    """The whole path, step by step: shared scale, per-worker quantise+pack, integer sum,
    decode.  Returns a dict with every intermediate."""
    n = np.asarray(xs[0]).size
    S, norms, bad = global_norm(xs, offsets)
    if scale is not None:
        S = _c(scale, np.float32)
    q = [quantize(x, S, grid, levels, seed, k, index_base, offsets) for k, x in enumerate(xs)]
    codes = [pack(qk, grid, bits) for qk in q]
    sums, over = accumulate(codes, n, grid, bits, acc_bits)
    mean = dequantize(sums, S, grid, levels, len(xs), out_dtype, offsets)
    return dict(scale=S, norms=norms, nonfinite=bad, levels=q, codes=codes, sums=sums,
                overflow=over, mean=mean)


# ---------------------------------------------------------------- per-worker-scale baselines
def worker_scales(xs, norm=NORM_L2, offsets=None):
    """K x nseg fp32 scales, each worker normalised on its own (L2 norm, or largest magnitude
    for NORM_MAX).  Returns (scales, bad)."""
    xs = [np.ascontiguousarray(x) for x in xs]
    n = xs[0].size
    off = _offsets(offsets, n)
    nseg = off.size - 1
    S = np.zeros((len(xs), nseg), np.float32)
    bad = lib().orc_worker_scales(_ptrs(xs), len(xs), _dtype_code(xs[0]), n, _ptr(off), nseg,
                                  norm, _ptr(S))
    return S, bool(bad)


def worker_mean(xs, scales, grid, levels, seed, index_base=0, offsets=None, out_dtype=F32):
    """Mean of the K workers' decoded values, each worker quantised and decoded with its own
    scale (scales: K x nseg)."""
    xs = [np.ascontiguousarray(x) for x in xs]
    n = xs[0].size
    off = _offsets(offsets, n)
    sc = _c(scales, np.float32)
    assert sc.size == len(xs) * (off.size - 1)
    out = np.empty(n, np.uint16 if out_dtype == BF16 else np.float32)
    lib().orc_worker_mean(_ptrs(xs), len(xs), _dtype_code(xs[0]), n, _ptr(off), off.size - 1,
                          _ptr(sc), grid, levels, seed, index_base, out_dtype, _ptr(out))
    return out


def decode_workers(codes_list, n, scales, grid, levels, bits, offsets=None, out_dtype=F32):
    """Receiver's mean from K workers' packed codes, each decoded with its own scale."""
    codes_list = [_c(c, np.uint8) for c in codes_list]
    off = _offsets(offsets, n)
    sc = _c(scales, np.float32)
    assert sc.size == len(codes_list) * (off.size - 1)
    out = np.empty(n, np.uint16 if out_dtype == BF16 else np.float32)
    lib().orc_decode_workers(_ptrs(codes_list), len(codes_list), n, _ptr(off), off.size - 1,
                             _ptr(sc), grid, levels, bits, out_dtype, _ptr(out))
    return out


# ---------------------------------------------------------------- LQ-SGD
def logq_index(y, alpha, L) -> int:
    return lib().orc_logq_index(float(np.float32(y)), alpha, L)


def logq_level(k, alpha, L) -> float:
    return lib().orc_logq_level(k, alpha, L)


def logquant(F, alpha, bits):
    F = _c(F, np.float32)
    rows, r = F.shape
    codes = np.empty((rows, r), np.int8)
    colmax = np.empty(r, np.float32)
    Fhat = np.empty((rows, r), np.float32)
    lib().orc_logquant(_ptr(F), rows, r, alpha, bits, _ptr(codes), _ptr(colmax), _ptr(Fhat))
    return codes, colmax, Fhat


def mgs(P, m):
    """Modified Gram-Schmidt of the oracle; m = the number of products summed in each entry
    of P (the inner dimension of P = M Q_prev), which sets the dependent-column cut."""
    P = np.array(P, dtype=np.float32, order="C", copy=True)
    lib().orc_mgs(_ptr(P), P.shape[0], P.shape[1], int(m))
    return P


def mgs_rho(m):
    """Relative rounding rho of an entry of P that sums m products: sqrt(m) 2^-24."""
    return lib().orc_mgs_rho(int(m))


def powersgd_logquant(G, E, Q, alpha, bits, bits_q=None):
    """One step (P coded with ``bits``, Q with ``bits_q``, default the same).  Returns a dict
    with the updated E and Q (new arrays) and all outputs."""
    G = _c(G, np.float32)
    E = np.array(E, dtype=np.float32, order="C", copy=True)
    Q = np.array(Q, dtype=np.float32, order="C", copy=True)
    n, m = G.shape
    r = Q.shape[1]
    pc = np.empty((n, r), np.int8)
    qc = np.empty((m, r), np.int8)
    pm = np.empty(r, np.float32)
    qm = np.empty(r, np.float32)
    ph = np.empty((n, r), np.float32)
    ppre = np.empty((n, r), np.float32)
    qpre = np.empty((m, r), np.float32)
    lib().orc_powersgd_logquant(_ptr(G), _ptr(E), _ptr(Q), n, m, r, alpha, bits,
                                bits if bits_q is None else bits_q, _ptr(pc),
                                _ptr(pm), _ptr(qc), _ptr(qm), _ptr(ph), _ptr(ppre), _ptr(qpre))
    return dict(E=E, Q=Q, p_codes=pc, p_colmax=pm, q_codes=qc, q_colmax=qm, p_hat=ph,
                P_pre=ppre, Q_pre=qpre)


def lq_step_workers(Gs, Es, Qs, alpha, bits, bits_q=None):
    """One step of K workers (lists of n x m gradients and errors, m x r warm starts).  Returns
    a dict with the updated E and Q lists (new arrays), the stacked messages and G_hat."""
    K = len(Gs)
    Gs = [_c(G, np.float32) for G in Gs]
    Es = [np.array(E, dtype=np.float32, order="C", copy=True) for E in Es]
    Qs = [np.array(Q, dtype=np.float32, order="C", copy=True) for Q in Qs]
    n, m = Gs[0].shape
    r = Qs[0].shape[1]
    pc = np.empty((K, n, r), np.int8)
    qc = np.empty((K, m, r), np.int8)
    pm = np.empty((K, r), np.float32)
    qm = np.empty((K, r), np.float32)
    gh = np.empty((n, m), np.float32)
    lib().orc_lq_step_workers(_ptrs(Gs), _ptrs(Es), _ptrs(Qs), K, n, m, r, alpha, bits,
                              bits if bits_q is None else bits_q, _ptr(pc), _ptr(pm), _ptr(qc),
                              _ptr(qm), _ptr(gh))
    return dict(E=Es, Q=Qs, p_codes=pc, p_colmax=pm, q_codes=qc, q_colmax=qm, G_hat=gh)
