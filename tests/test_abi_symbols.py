"""The C-ABI library loads and exports every function include/gq.h declares (CPU only: no
compute call is made without a GPU), and the oracle and the product share no code."""
import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gq.h")
PKG = os.path.join(ROOT, "allreduce_compatible_gradient_amd")
LIB = os.path.join(PKG, "libgq.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gq_[a-z_]+)\s*\(", text)))


def _ensure_built():
    if not os.path.exists(LIB):
        from allreduce_compatible_gradient_amd import build
        build.build()


def test_header_declares_the_path():
    names = _declared()
    for want in ("gq_global_norm", "gq_quantize_pack", "gq_accumulate_codes", "gq_dequantize",
                 "gq_fused_mean", "gq_logquant", "gq_powersgd_logquant", "gq_create",
                 "gq_destroy", "gq_last_error", "gq_read_status", "gq_version",
                 "gq_wire_lane_bytes", "gq_quantize_wire", "gq_dequantize_wire"):
        assert want in names


def test_library_exports_every_declared_symbol():
    _ensure_built()
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_exports_nothing_else():
    _ensure_built()
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = sorted({line.split()[-1] for line in out.splitlines()
                       if line.split()[1:2] == ["T"] and line.split()[-1].startswith("gq_")})
    assert exported == _declared()


def test_version_string_is_callable_without_gpu():
    _ensure_built()
    lib = ctypes.CDLL(LIB)
    lib.gq_version.restype = ctypes.c_char_p
    assert lib.gq_version().decode().startswith("gq ")


def test_oracle_and_product_share_no_code():
    csrc = os.path.join(PKG, "csrc")
    for f in os.listdir(csrc):
        txt = open(os.path.join(csrc, f)).read()
        assert "oracle" not in txt.lower(), f
    for f in ("gq_oracle.c", "gq_oracle.h", "oracle.py"):
        txt = open(os.path.join(ROOT, "oracle", f)).read()
        assert "allreduce_compatible_gradient_amd" not in txt and "gq.h" not in txt, f
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            txt = open(os.path.join(PKG, f)).read()
            assert "import oracle" not in txt and "from oracle" not in txt, f


def test_wire_lane_width_rule_matches_the_oracle():
    """gq_wire_lane_bytes is pure host code: callable without a GPU."""
    _ensure_built()
    from oracle import oracle
    lib = ctypes.CDLL(LIB)
    lib.gq_wire_lane_bytes.restype = ctypes.c_int32
    lib.gq_wire_lane_bytes.argtypes = [ctypes.c_int32] * 3
    for grid, top in ((0, 127), (1, 30)):
        for levels in range(1, top + 1):
            for world in (1, 2, 3, 8, 16, 64, 1000, 65536):
                assert lib.gq_wire_lane_bytes(grid, levels, world) == \
                    oracle.wire_lane_bytes(grid, levels, world), (grid, levels, world)
    assert lib.gq_wire_lane_bytes(0, 128, 1) == 0 and lib.gq_wire_lane_bytes(0, 7, 0) == 0


def test_header_is_plain_c99():
    """include/gq.h and a C program using it compile as C99 with gcc (no C++ or HIP types in
    the ABI), and the header alone also compiles with -pedantic."""
    import subprocess
    import tempfile
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    inc = os.path.join(ROOT, "include")
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only",
                           "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(rocm, "include"),
                           "-I" + inc, os.path.join(ROOT, "tests", "abi", "c_consumer.c")])
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "only_header.c")
        with open(src, "w") as f:
            f.write('#include "gq.h"\nint main(void) { return GQ_OK; }\n')
        subprocess.check_call(["gcc", "-std=c99", "-pedantic", "-Wall", "-Werror",
                               "-fsyntax-only", "-I" + inc, src])
