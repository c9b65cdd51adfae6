"""Build the GPU check kernels of the tests (not part of the library):
tests/gpu_checks/libcvt_check.so from cvt_bf16_check.hip, compiled with the
library's flags against its device header."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CVT_LIB = os.path.join(HERE, "libcvt_check.so")


def build(verbose: bool = False) -> str:
    from scaled_gemm_amd.build import FLAGS, HIPCC
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-shared", "-o", CVT_LIB + ".tmp",
           os.path.join(HERE, "cvt_bf16_check.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{r.stdout}")
    os.replace(CVT_LIB + ".tmp", CVT_LIB)
    return CVT_LIB


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    print(build(verbose="-v" in sys.argv))
