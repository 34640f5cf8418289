"""The library's host code (argument validation, kernel plans, workspace
layouts) under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU:
every source is compiled with the sanitizers on its host side only (device
code is unchanged), and tests/host_abi_check.cpp drives the C ABI's
validation and size functions without a GPU."""

import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.slow
@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_host_code_under_asan_and_ubsan():
    from bit_weight_only_quantize_amd import build as B
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    with tempfile.TemporaryDirectory(prefix="awq355_san_") as tmp:
        objs = []
        procs = []
        for src in B.SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [B.hipcc(), *B.common_flags(), *san, "-x", "hip", "-c",
                   os.path.join(B.CSRC, src), "-o", obj]
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                text=True)))
            objs.append(obj)
        for src, p in procs:
            out, _ = p.communicate(timeout=900)
            assert p.returncode == 0, f"{src}:\n{out}"
        lib = os.path.join(tmp, "libawq355_san.so")
        subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *san, *objs,
                        "-o", lib], check=True, capture_output=True, text=True)
        # the host code really is instrumented: the library calls both runtimes
        syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
        assert "__asan_" in syms and "__ubsan_handle" in syms
        exe = os.path.join(tmp, "host_abi_check")
        drv = os.path.join(tmp, "host_abi_check.o")
        subprocess.run([B.hipcc(), "-std=c++17", *san, "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(HERE, "host_abi_check.cpp"), "-o", drv],
                       check=True, capture_output=True, text=True)
        # the link line pulls in the sanitizer runtimes (host only)
        link_flags = ["-fno-gpu-sanitize", "-fsanitize=address", "-fsanitize=undefined"]
        link = subprocess.run([B.hipcc(), *link_flags, drv, lib, "-o", exe, f"-Wl,-rpath,{tmp}"],
                              capture_output=True, text=True)
        assert link.returncode == 0, link.stdout + link.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out
    assert "host ABI check ok" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
