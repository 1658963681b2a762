"""The quantizers divide each block amax by 6 with a product and one fused
correction step (device.hpp, div6) instead of a division.  This CPU test checks
that identity against IEEE division for every binary32 from 2^-125 up to the
largest finite value (tests/native/div6_check.c, built here with gcc)."""
import ctypes
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def div6_lib(tmp_path_factory):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.fail("gcc is needed to build tests/native/div6_check.c")
    out = tmp_path_factory.mktemp("div6") / "libdiv6.so"
    subprocess.run([cc, "-O2", "-mfma", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                    os.path.join(HERE, "native", "div6_check.c"), "-o", str(out), "-lm"], check=True)
    lib = ctypes.CDLL(str(out))
    lib.div6_mismatches.restype = ctypes.c_uint64
    lib.div6_mismatches.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint32)]
    return lib


def test_div6_equals_division_for_every_binary32_above_2_pow_minus_125(div6_lib):
    first = ctypes.c_uint32()
    lo, hi = 0x01000000, 0x7F7FFFFF  # 2^-125 .. FLT_MAX
    bad = div6_lib.div6_mismatches(lo, hi, ctypes.byref(first))
    assert bad == 0, f"{bad} quotients differ; first at bits {first.value:#010x}"


def test_div6_check_sees_a_wrong_formula(div6_lib):
    """Below 2^-125 the quotient is subnormal and the identity fails (which is why
    the kernel divides there): the check must report those mismatches."""
    first = ctypes.c_uint32()
    bad = div6_lib.div6_mismatches(0x00000001, 0x00FFFFFF, ctypes.byref(first))
    assert bad > 0
