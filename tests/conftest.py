import ctypes
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a ``name value`` text fixture (``#`` starts a comment)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split(None, 1)
            out[key] = float(val) if "." in val else int(val)
    return out


def read_golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([int(x) for x in line.split()])
    return rows


# --------------------------------------------------------------------------
# The library's host code (tests/hostcheck): abi.cpp linked against a CPU
# simulator of the kernel launchers instead of the HIP kernels, so every call
# can run without a GPU. With GQAKV_HOSTCHECK_SANITIZE=1 in the environment
# (set by the sanitizer test, which also preloads the ASan runtime) it is
# built with AddressSanitizer and UndefinedBehaviorSanitizer.
# --------------------------------------------------------------------------

CSRC = os.path.join(ROOT, "gqa_attention_preallocated_amd", "csrc")
SANITIZE = os.environ.get("GQAKV_HOSTCHECK_SANITIZE") == "1"
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def build_hostcheck(out):
    """Compile abi.cpp + the launch simulator with g++ into `out` (host code only)."""
    flags = ["-O1", "-g"] + (SANITIZE_FLAGS if SANITIZE else [])
    cmd = ["g++", *flags, "-std=c++17", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "abi.cpp"), os.path.join(ROOT, "tests", "hostcheck", "launch_sim.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return ctypes.CDLL(str(out))


@pytest.fixture(scope="session")
def hostcheck_lib(tmp_path_factory):
    return build_hostcheck(tmp_path_factory.mktemp("hostcheck") / "libhostcheck.so")
