"""Host checks of floating-point identities the HIP kernels rely on (no GPU)."""

import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.slow
@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_division_by_15_through_corrected_reciprocal():
    """The quantize kernel forms the group step (hi - lo) / 15 as a product
    with RN(1/15) plus one remainder correction instead of an IEEE division;
    every non-negative finite dividend must give the IEEE quotient."""
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "div15")
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", os.path.join(HERE, "div15_exhaustive.c"),
                        "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "mismatches: 0 of 2139095040" in out.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_exact_mean_quotient_is_correctly_rounded():
    """The activation statistic divides an exact 64-bit integer column sum by
    the row count M < 2^24.  The kernel's quotient routine (host build of the
    same header) must equal the correctly rounded quotient, which Python's
    integer true division gives, on random sums across the whole 64-bit
    range, sums just above 2^53, and exact halfway cases (ties to even)."""
    import random
    import struct
    csrc = os.path.join(os.path.dirname(HERE), "bit_weight_only_quantize_amd", "csrc")
    rng = random.Random(5)
    cases = []
    for _ in range(20000):
        bits = rng.randint(1, 64)
        cases.append((rng.getrandbits(bits) | 1 << (bits - 1), rng.randint(1, (1 << 24) - 1)))
    for _ in range(5000):
        cases.append(((1 << 53) + rng.getrandbits(20), rng.randint(1, (1 << 24) - 1)))
    for e in range(54, 64):
        for M in (1, 2, 4, 8, 1 << 20):
            # S / M exactly halfway between neighbouring doubles, both parities
            for k in (1, 2, 3):
                S = ((1 << 53) + k) * M * (1 << (e - 53)) + M * (1 << (e - 54))
                if S < 1 << 64:
                    cases.append((S, M))
    cases += [((1 << 64) - 1, 1), ((1 << 64) - 1, (1 << 24) - 1), (1 << 53, 3), ((1 << 53) - 1, 7)]
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "quot")
        subprocess.run(["g++", "-O2", "-std=c++17", "-I", csrc,
                        os.path.join(HERE, "quotient_check.cpp"), "-o", exe], check=True)
        out = subprocess.run([exe], input="".join(f"{S} {M}\n" for S, M in cases),
                             capture_output=True, text=True, timeout=120, check=True).stdout
    got = out.split()
    assert len(got) == len(cases)
    for (S, M), h in zip(cases, got):
        want = struct.unpack("<Q", struct.pack("<d", S / M))[0]
        assert int(h, 16) == want, (S, M)
