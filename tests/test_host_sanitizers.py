"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): calibrate.cpp, rotation_file.cpp and the host sides of the .hip
sources (argument validation, launch set-up) are rebuilt with the sanitizers on
the host pass only (the device code is compiled as usual and never runs here),
linked with tests/host_checks.c, and driven through the C ABI:

  * every host-detectable argument error of every entry point;
  * calibration of a seeded workload (single and layer-batched calls), whose
    outputs must equal the regular library's bit for bit;
  * a rotation file written, read back and refused when damaged, whose bytes
    must equal the format's plain definition.

Any sanitizer report fails the run (-fno-sanitize-recover, abort on error)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import workloads as wl
from oracle import rotation_file_ref as rf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_int2_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

pytestmark = pytest.mark.skipif(not all(os.path.exists(x) for x in (CLANG, CLANGXX, HIPCC)),
                                reason="ROCm clang / hipcc missing")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-3000:] + r.stderr[-3000:]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    common = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer"]
    objs = []
    for src in ("calibrate.cpp", "rotation_file.cpp"):  # plain host C++
        obj = str(d / (src + ".o"))
        _run([CLANGXX, *common, *SAN, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", *inc, "-c",
              os.path.join(CSRC, src), "-o", obj], d)
        objs.append(obj)
    for src in ("append.hip", "decode.hip", "noalloc.hip", "runtime.hip"):  # sanitizers on the host pass only
        obj = str(d / (src + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", *common, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              *HOST_SAN, *inc, "-c", os.path.join(CSRC, src), "-o", obj], d)
        objs.append(obj)
    drv = str(d / "host_checks.o")
    _run([CLANG, "-std=c99", "-O1", "-g", "-Wall", "-Werror", *SAN, *inc, "-c",
          os.path.join(ROOT, "tests", "host_checks.c"), "-o", drv], d)
    exe = str(d / "host_checks")
    _run([CLANGXX, *SAN, drv, *objs, f"-L{ROCM}/lib", "-lamdhip64", "-lpthread", f"-Wl,-rpath,{ROCM}/lib", "-o",
          exe], d)
    return exe, d


def _exec(exe, *args, cwd):
    r = subprocess.run([exe, *args], cwd=cwd, capture_output=True, text=True, env=ENV, timeout=600)
    report = r.stdout + r.stderr
    assert "AddressSanitizer" not in report and "runtime error" not in report and "LeakSanitizer" not in report, report
    assert r.returncode == 0, report
    return report


def test_validation_paths_clean(driver):
    exe, d = driver
    _exec(exe, "validate", cwd=d)


def test_calibration_and_rotation_file_clean(driver):
    K = pytest.importorskip("kv_cache_int2_amd", reason="library not built")
    exe, d = driver
    s = wl.spec(1)
    q, k, v = wl.calibration_set(s)
    hkv, nq, nkv = q.shape[0], q.shape[1], k.shape[1]
    inp, out = d / "calib.in", d / "calib.out"
    with open(inp, "wb") as f:
        f.write(np.array([hkv, nq, nkv], np.int32).tobytes())
        f.write(np.ascontiguousarray(q, np.float32).tobytes())
        f.write(np.ascontiguousarray(k, np.float32).tobytes())
        f.write(np.ascontiguousarray(v, np.float32).tobytes())
    _exec(exe, "calibrate", str(inp), str(out), cwd=d)
    raw = out.read_bytes()
    rot = hkv * 128 * 128
    rk = np.frombuffer(raw, np.uint16, rot, 0).reshape(hkv, 128, 128)
    rv = np.frombuffer(raw, np.uint16, rot, 2 * rot).reshape(hkv, 128, 128)
    ek = np.frombuffer(raw, np.float64, hkv * 128, 4 * rot).reshape(hkv, 128)
    ev = np.frombuffer(raw, np.float64, hkv * 128, 4 * rot + 8 * hkv * 128).reshape(hkv, 128)
    assert raw[-1] == 1, "layer-batched calibration differs from the single call"
    rk0, rv0, ek0, ev0 = K.oscar_calibrate(K.make_shape(4 * hkv, hkv), q, k, v)
    assert np.array_equal(rk, rk0) and np.array_equal(rv, rv0)
    assert np.array_equal(ek, ek0) and np.array_equal(ev, ev0)
    path = d / "model.oscarrot"
    _exec(exe, "rotfile", str(out), str(path), str(hkv), cwd=d)
    want = rf.encode(np.stack([rk, rk]), np.stack([rv, rv]), 128, np.stack([ek, ek]), np.stack([ev, ev]))
    assert path.read_bytes() == want
