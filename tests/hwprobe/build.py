"""Build the test-only probe library libhwconv.so (tests/hwprobe/hw_converters.hip)
in-tree with the product's own compiler flags, so the device helpers it wraps
compile exactly as they do in the product."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from nvfp4_bit_microscaled_amd import build as product_build  # noqa: E402

SRC = os.path.join(HERE, "hw_converters.hip")
LIB = os.path.join(HERE, "libhwconv.so")


def build(verbose: bool = False) -> str:
    cmd = [product_build.HIPCC, *product_build.FLAGS, "-shared", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
