"""Pins the oracle's Philox4x32-10 to an independent implementation: rocRAND's header-only
engine (Salmon et al., SC'11 generator), compiled from its ROCm headers for the host CPU and
run there. Stochastic rounding draws its 16-bit fields from this generator ("Training LLMs with
MXFP4", abstract; "Stable FP4 Training via Transposition-Invariant Block Quantization", "The
fix, and its supporting cast")."""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "philox_kat", "rocrand_philox_words.cpp")


@pytest.fixture(scope="module")
def rocrand_words(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand"):
        pytest.skip("ROCm headers/hipcc not available: Philox third-party parity unpinned here")
    exe = str(tmp_path_factory.mktemp("kat") / "philox_words")
    subprocess.run([hipcc, "-O1", "-o", exe, SRC], check=True, capture_output=True)

    def run(pairs):
        inp = "".join(f"{s} {c}\n" for s, c in pairs)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [tuple(int(w) for w in line.split()) for line in out.strip().splitlines()]
    return run


def test_philox_matches_rocrand(orc, rocrand_words):
    rng = np.random.default_rng(123)
    pairs = [(0, 0), (1234, 0), (1234, 1), (2**64 - 1, 2**62 - 1), (1 << 32, 1 << 32)]
    pairs += [(int(rng.integers(0, 2**63)) * 2 + 1, int(rng.integers(0, 2**62))) for _ in range(300)]
    ref = rocrand_words(pairs)
    for (s, c), want in zip(pairs, ref):
        got = orc.philox4x32_10([c & 0xFFFFFFFF, c >> 32, 0, 0], [s & 0xFFFFFFFF, s >> 32])
        assert tuple(int(x) for x in got) == want, (s, c)
