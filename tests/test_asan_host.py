"""The C ABI's host code (planner, validation, queries) built with
AddressSanitizer and LeakSanitizer and driven by tests/asan_driver.cpp: plans
of the benchmark's shapes under several caps, hints, every query, and each
validation failure of the step calls (none of which reaches a GPU, so this
runs without one).  Only host code is instrumented: the kernels are built as
usual and never launched."""
import concurrent.futures as cf
import os
import subprocess

from matrix_aware_optimizer_muon_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


def test_host_code_under_address_sanitizer(tmp_path):
    hipcc = B._hipcc()
    flags = [f for f in B._flags() if f != "-O3"] + ["-O1", "-g"]
    objs = []
    jobs = []
    for src in B.SOURCES:
        obj = str(tmp_path / (src + ".o"))
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        asan = HOST_ASAN if src.endswith(".cpp") else []
        jobs.append([hipcc, *flags, *asan, *lang, "-c", os.path.join(B.CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(_run, jobs))
    lib = str(tmp_path / "libmuon_asan.so")
    _run([hipcc, f"--offload-arch={B.ARCH}", *HOST_ASAN, "-shared", "-fPIC", *objs, "-o", lib])
    drv = str(tmp_path / "asan_driver")
    _run([hipcc, f"--offload-arch={B.ARCH}", "-std=c++17", "-g", *HOST_ASAN, "-I", B.INCLUDE,
          os.path.join(HERE, "asan_driver.cpp"), f"-L{tmp_path}", "-lmuon_asan",
          f"-Wl,-rpath,{tmp_path}", "-o", drv])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([drv], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "LeakSanitizer" not in out, out
    assert r.returncode == 0 and "0 failures" in out, out
