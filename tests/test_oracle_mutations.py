"""Planted mistakes: the oracle's pins must catch a plausible error anywhere in it.

Each case below copies the oracle's C source, changes one line the way a plausible mistake
would (a wrong shift or constant, a dropped term, a flipped sign, a wrong index or bound, a
step left out), builds that copy, and runs the oracle pin suites (tests/test_oracle_*.py)
against it through GQ_ORACLE_LIB.  The run must fail.  A control run of the unchanged source
through the same route must pass.  CPU only; nothing here touches the product library.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gq_oracle.c")
PIN_SUITES = ["tests/test_oracle_rng.py", "tests/test_oracle_quant.py", "tests/test_oracle_lq.py",
              "tests/test_oracle_wire.py", "tests/test_oracle_baselines.py",
              "tests/test_oracle_lq_workers.py"]

# (name, text in gq_oracle.c, replacement)
MUTATIONS = [
    ("splitmix64 increment", "*state += 0x9E3779B97F4A7C15ULL;", "*state += 0x9E3779B97F4A7C17ULL;"),
    ("splitmix64 shift", "z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;",
     "z = (z ^ (z >> 26)) * 0x94D049BB133111EBULL;"),
    ("fmix32 shift", "    h ^= h >> 13;", "    h ^= h >> 12;"),
    ("fmix32 constant", "h *= 0xC2B2AE35U;", "h *= 0xC2B2AE37U;"),
    ("worker key is output k, not k+1", "for (j = 0; j <= worker; ++j)",
     "for (j = 0; j < worker; ++j)"),
    ("counter added to key, not xor-ed", "const float h = (float)orc_fmix32(counter ^ key);",
     "const float h = (float)orc_fmix32(counter + key);"),
    ("draw: hash not rounded to fp32", "const float h = (float)orc_fmix32(counter ^ key);",
     "const double h = (double)orc_fmix32(counter ^ key);"),
    ("draw: hash truncated to fp32", "const float h = (float)orc_fmix32(counter ^ key);",
     "const float h = (float)(orc_fmix32(counter ^ key) & ~((1u << (orc_fmix32(counter ^ key) >= (1u << 24) ? 8 : 0)) - 1u));"),
    ("norm: signed square", "acc += v * v;", "acc += v * fabs(v);"),
    ("norm: sum over workers, not max", "best = nrm;", "best += nrm;"),
    ("uniform: scale 1/S, not s/S", "inv = (float)s / S;", "inv = 1.0f / S;"),
    ("uniform: no clamp at s", "if (!(u < (float)s))", "if (u != u)"),
    ("uniform: round up on r <= p", "m = (int32_t)l + (r < p ? 1 : 0);",
     "m = (int32_t)l + (r <= p ? 1 : 0);"),
    ("uniform: nearest level, not floor", "l = floor((double)u);", "l = floor((double)u + 0.5);"),
    ("uniform: sign dropped", "return signbit(x) ? -m : m;", "return m;"),
    ("uniform: a NaN counted as positive", "return signbit(x) ? -m : m;",
     "return x < 0.0f ? -m : m;"),
    ("exponential: a NaN counted as positive", "return (signbit(x) && j > 0) ? -j : j;",
     "return (x < 0.0f && j > 0) ? -j : j;"),
    ("uniform: counter without index base", "scale[g], key, index_base + (uint32_t)i);",
     "scale[g], key, (uint32_t)i);"),
    ("exponential: probability over the upper level", "p = ((double)u - lo) / (hi - lo);",
     "p = ((double)u - lo) / hi;"),
    ("exponential: linear value 2^j", "int64_t v = j == 0 ? 0 : ((int64_t)1 << (j - 1));",
     "int64_t v = j == 0 ? 0 : ((int64_t)1 << j);"),
    ("exponential: sign bit one place low", "return (sign << (bits - 1)) | j;",
     "return (sign << (bits - 2)) | j;"),
    ("pack: nibble order swapped", "        if (i % 2 == 0)\n            out[i / 2]",
     "        if (i % 2 == 1)\n            out[i / 2]"),
    ("unpack: no sign extension", "return (int32_t)c - (int32_t)(1u << bits);",
     "return (int32_t)c;"),
    ("sum: negative overflow not counted", "if (acc > lim || acc < -lim - 1)",
     "if (acc > lim)"),
    ("decode: factor without K", "D = (double)levels * (double)K;", "D = (double)levels;"),
    ("decode: exponential factor 2^E", "D = (double)K * ldexp(1.0, levels - 1);",
     "D = (double)K * ldexp(1.0, levels);"),
    ("bf16: ties away from zero", "return (uint16_t)((lo & 1u) ? hi : lo);",
     "return (uint16_t)hi;"),
    ("bf16: truncation", "    if (dv - dl < dh - dv)\n        return (uint16_t)lo;",
     "    if (1)\n        return (uint16_t)lo;"),
    ("wire: lane offset dropped", "uint64_t lane = (uint64_t)(orc_lin(grid, q[i]) + o);",
     "uint64_t lane = (uint64_t)(orc_lin(grid, q[i]));"),
    ("wire: big-endian lanes", "payload[i * w + b] = (uint8_t)(lane >> (8 * b));",
     "payload[i * w + b] = (uint8_t)(lane >> (8 * (w - 1 - b)));"),
    ("wire: lanes twice as wide as needed", "if (top <= (int64_t)(((uint64_t)1 << (8 * w)) - 1))",
     "if (top <= (int64_t)(((uint64_t)1 << (8 * w - 1)) - 1))"),
    ("wire: decode without the world's offset", "sums[i] = (int32_t)((int64_t)lane - (int64_t)world * o);",
     "sums[i] = (int32_t)((int64_t)lane - o);"),
    ("log quantiser: natural log of alpha as the base", "/ log1p(alpha);", "/ log(alpha);"),
    ("log quantiser: rounding down", "double k = floor(z * (double)L + 0.5);",
     "double k = floor(z * (double)L);"),
    ("log decode: L+1 steps", "(double)k / (double)L) - 1.0) / alpha);",
     "(double)k / (double)(L + 1)) - 1.0) / alpha);"),
    ("log quantiser: column maximum starts at 1", "        float mx = 0.0f;\n        for (i = 0; i < rows; ++i) {\n            float a",
     "        float mx = 1.0f;\n        for (i = 0; i < rows; ++i) {\n            float a"),
    ("Gram-Schmidt: projection added", "V[i * r + c] -= d * V[i * r + j];",
     "V[i * r + c] += d * V[i * r + j];"),
    ("Gram-Schmidt: no normalisation", "V[i * r + c] = nrm > 0.0 ? V[i * r + c] / nrm : 0.0;",
     "V[i * r + c] = V[i * r + c];"),
    ("Gram-Schmidt: dependent columns kept", "        if (!(nrm > rho * bound))\n            nrm = 0.0;\n",
     "\n"),
    ("Gram-Schmidt: one fixed cut for every product length", "return sqrt((double)m) * 0x1p-24;",
     "return 0x1p-16;"),
    ("Gram-Schmidt: cut without the earlier columns' coefficients",
     "            bound += fabs(a[j]) * nrm0[j];\n", "\n"),
    ("Gram-Schmidt: coefficients from the wrong row of R", "t -= R[j][k] * a[k];",
     "t -= R[k][j] * a[k];"),
    ("power step: P not orthonormalised", "    orc_mgs(P, n, r, m);\n", "\n"),
    ("power step: no error fed back", "E[i] = G[i] + E[i];", "E[i] = G[i];"),
    ("power step: error of the wrong sign", "E[i * m + j] = (float)((double)E[i * m + j] - acc);",
     "E[i * m + j] = (float)((double)E[i * m + j] + acc);"),
    ("power step: Q from the transposed index", "Qacc[j * r + c] += (double)E[i * m + j] * (double)P[i * r + c];",
     "Qacc[j * r + c] += (double)E[i * m + j] * (double)P[i * r + (r - 1 - c)];"),
    ("power step: P coded with Q's width", "orc_logquant(P, n, r, alpha, bits_p,",
     "orc_logquant(P, n, r, alpha, bits_q,"),
    ("power step: Q not warm-started", "    memcpy(Q, Qh, (size_t)(m * r) * sizeof(float));\n", "\n"),
    ("worker scales: first nonzero magnitude, not the largest", "else if (a > v)",
     "else if (v == 0.0)"),
    ("worker scales: NaN ignored", "v = NAN; /* a NaN", "v = v; /* a NaN"),
    ("worker scales: L2 without the square root", "                v = sqrt(v);\n", "\n"),
    ("worker mean: worker 0's scale for every worker",
     "float S = scales[(int64_t)k * nseg + g];", "float S = scales[g];"),
    ("worker mean: factor without K", "float f = orc_decode_factor(grid, levels, K, S);",
     "float f = orc_decode_factor(grid, levels, 1, S);"),
    ("worker mean: worker 0's key for every worker",
     "keys[k] = orc_worker_key(seed, (uint32_t)k);", "keys[k] = orc_worker_key(seed, 0u);"),
    ("decode workers: worker 0's factor for every worker",
     "float f = orc_decode_factor(grid, levels, K, scales[(int64_t)k * nseg + g]);",
     "float f = orc_decode_factor(grid, levels, K, scales[g]);"),
    ("decode workers: worker 0's codes for every worker",
     "int32_t q = orc_unpack_one(codes[k], i, grid, bits);",
     "int32_t q = orc_unpack_one(codes[0], i, grid, bits);"),
    ("worker mean: last worker left out", "            for (k = 0; k < K; ++k) {\n                float S",
     "            for (k = 0; k + 1 < K; ++k) {\n                float S"),
    ("LQ workers: the sum of the messages, not their mean", "mean = acc / (double)K;",
     "mean = acc;"),
    ("LQ workers: last worker left out of the mean",
     "            for (w = 0; w < K; ++w) {\n                const float *pw",
     "            for (w = 0; w + 1 < K; ++w) {\n                const float *pw"),
    ("LQ workers: worker 0's Q factor in every product", "*qw = Qh + w * m * r;", "*qw = Qh;"),
    ("LQ workers: error against the sum, not the mean",
     "E[w][i * m + j] = (float)((double)E[w][i * m + j] - mean);",
     "E[w][i * m + j] = (float)((double)E[w][i * m + j] - acc);"),
    ("LQ workers: error against the rounded mean",
     "E[w][i * m + j] = (float)((double)E[w][i * m + j] - mean);",
     "E[w][i * m + j] = E[w][i * m + j] - G_hat[i * m + j];"),
    ("LQ workers: worker 0's warm start for every worker", "lq_compress(G[w], E[w], Q[w],",
     "lq_compress(G[w], E[w], Q[0],"),
    ("LQ workers: worker 0's gradient for every worker", "lq_compress(G[w], E[w], Q[w],",
     "lq_compress(G[0], E[w], Q[w],"),
]


def _build_variant(tmp, name, old, new):
    from oracle import oracle
    text = open(SRC).read()
    if old is not None:
        assert text.count(old) == 1, "planted mistake %r no longer matches the oracle" % name
        text = text.replace(old, new)
    d = os.path.join(tmp, "v%d" % abs(hash(name)))
    os.makedirs(d, exist_ok=True)
    shutil.copy(os.path.join(ROOT, "oracle", "gq_oracle.h"), d)
    src = os.path.join(d, "gq_oracle.c")
    open(src, "w").write(text)
    return oracle.compile_library(src, os.path.join(d, "liboracle_variant.so"))


def _run_pins(libpath):
    env = dict(os.environ, GQ_ORACLE_LIB=libpath, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"] + PIN_SUITES,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-3000:]


@pytest.fixture(scope="module")
def outcomes():
    tmp = tempfile.mkdtemp(prefix="gq_oracle_plant_")
    try:
        cases = [("control (unchanged source)", None, None)] + MUTATIONS
        libs = [_build_variant(tmp, *c) for c in cases]
        with ThreadPoolExecutor(max_workers=6) as ex:
            res = list(ex.map(_run_pins, libs))
        return {c[0]: r for c, r in zip(cases, res)}
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_control_passes(outcomes):
    rc, out = outcomes["control (unchanged source)"]
    assert rc == 0, out


@pytest.mark.parametrize("name", [m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(outcomes, name):
    rc, out = outcomes[name]
    # exit status 1: tests ran and at least one pin failed (not a collection or usage error)
    assert rc == 1, "pins did not catch %r (exit %d)\n%s" % (name, rc, out)
