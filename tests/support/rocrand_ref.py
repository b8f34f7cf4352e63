"""Build and call the rocRAND-backed Philox4x32-10 reference (host code, g++)."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "philox_rocrand_ref.cpp")
ROCM_INC = "/opt/rocm/include"
_BIN = None


def _binary():
    global _BIN
    if _BIN is not None:
        return _BIN
    if not os.path.isfile(os.path.join(ROCM_INC, "rocrand", "rocrand_philox4x32_10.h")):
        pytest.skip("rocRAND headers not present: external Philox pin unavailable")
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler: external Philox pin unavailable")
    out = os.path.join(tempfile.mkdtemp(prefix="srat_philox_"), "philox_ref")
    subprocess.run([cxx, "-O1", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INC}", SRC, "-o", out],
                   check=True, capture_output=True)
    _BIN = out
    return out


def philox_words(cases):
    """cases: iterable of (seed, c0, c1, c2, c3) -> uint64 array [n, 4]."""
    lines = "".join(f"{s} {a} {b} {c} {d}\n" for s, a, b, c, d in cases)
    res = subprocess.run([_binary()], input=lines, capture_output=True, text=True, check=True)
    rows = [[int(x, 16) for x in ln.split()] for ln in res.stdout.strip().splitlines()]
    return np.array(rows, dtype=np.uint64)
