"""CPU sanitizer runs: AddressSanitizer and UndefinedBehaviorSanitizer builds of the C
oracle and of the C-ABI host code (argument checks, plans, dispatch decisions).

* The host code (weight_only_quantized_qmm_amd/csrc/qmm_api.cpp) is compiled with g++ for
  the CPU alone, with the kernel launchers replaced by recording stubs
  (tests/sanitize/host_checks.cpp), and runs every entry point's checks and thousands of
  plans with leak detection on.
* The oracle (oracle/qmm_oracle.c) is compiled with gcc and the same sanitizers, and the
  oracle pins (tests/test_oracle_pins.py) run against that build in a child process with
  the sanitizer runtimes preloaded.
No GPU code is built or run here.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_only_quantized_qmm_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


needs_runtimes = pytest.mark.skipif(not (_runtime("libasan.so") and _runtime("libubsan.so")),
                                    reason="gcc's sanitizer runtimes are not installed")


@needs_runtimes
def test_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + INCLUDE,
                    "-I" + CSRC, os.path.join(CSRC, "qmm_api.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1"))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "host checks ok" in r.stdout
    # every small-M configuration the host picked is one the kernel source instantiates
    # (bits, mt, ns, gpw, at most MAXW waves, staged rows: 16*mt for QMM_CFG)
    import re
    src = open(os.path.join(CSRC, "qmm_w4a16_skinny.hip")).read()
    built = {tuple(int(x) for x in m) + (16 * int(m[1]),)
             for m in re.findall(r"QMM_CFG\((\d+), (\d+), (\d+), (\d+), (\d+)\)", src)}
    built |= {tuple(int(x) for x in m)
              for m in re.findall(r"QMM_CFGR\((\d+), (\d+), (\d+), (\d+), (\d+), (\d+)\)", src)}
    assert built
    maxw = {c[:4] + c[5:]: c[4] for c in built}
    picked = [tuple(int(x) for x in l.split()[2:]) for l in r.stdout.splitlines() if l.startswith("skinny config")]
    assert picked
    assert any(rows < 16 * mt for _, mt, _, _, _, rows in picked)  # decode's compact staging is exercised
    for bits, mt, ns, gpw, waves, rows in picked:
        key = (bits, mt, ns, gpw, rows)
        assert key in maxw, ("no kernel instantiation for", key)
        assert waves <= maxw[key], ("too many waves for", key, waves)


@needs_runtimes
def test_oracle_pins_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-pthread", *SAN,
                    os.path.join(ROOT, "oracle", "qmm_oracle.c"), "-o", lib, "-lm"], check=True)
    env = dict(os.environ, QMM_ORACLE_LIB=lib,
               LD_PRELOAD=" ".join([_runtime("libasan.so"), _runtime("libubsan.so")]),
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child really loads the sanitizer build
    r = subprocess.run([sys.executable, "-c", "import oracle; oracle.bf16_round(1.0); print(oracle._lib()._name)"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == lib, r.stdout + r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "failed" not in r.stdout
