"""The library's argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

Every source of the library is compiled with the sanitizers on its host code
only (`-Xarch_host -fsanitize=...`; the gfx950 device code is built as usual),
and linked with `tests/native/abi_errors.cpp`, which calls every C-ABI entry
point with arguments one of its checks must reject and verifies the status and
the error text.  A rejected call touches neither the GPU nor any output, so the
program runs here without one.  The build is cached under `_build/sanitized`
and redone when a source changes (about a minute).
"""

import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_spatiotemporal_build_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "native", "abi_errors.cpp")
OUT = os.path.join(ROOT, "_build", "sanitized")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


def _sources():
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    hdrs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h"))
    return srcs, hdrs + [os.path.join(ROOT, "include", "bsa.h"), DRIVER]


def _digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(p.encode() + f.read())
    h.update(" ".join(FLAGS + SAN_HOST).encode())
    return h.hexdigest()[:16]


def _build():
    srcs, extra = _sources()
    exe = os.path.join(OUT, "abi_errors")
    stamp = os.path.join(OUT, "stamp")
    digest = _digest(srcs + extra)
    if os.path.exists(exe) and os.path.exists(stamp) and open(stamp).read() == digest:
        return exe
    os.makedirs(OUT, exist_ok=True)
    procs, objs = [], []
    for src in srcs:
        obj = os.path.join(OUT, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *FLAGS, *SAN_HOST, "-c", src, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p, src in zip(procs, srcs):
        out = p.communicate()[0].decode(errors="replace")
        assert p.returncode == 0, f"sanitized build of {src} failed:\n{out[-4000:]}"
    drv = os.path.join(OUT, "driver.o")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-c", DRIVER, "-o", drv], check=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN_HOST, "-o", exe, drv, *objs], check=True,
                   stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    with open(stamp, "w") as f:
        f.write(digest)
    return exe


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_every_rejected_call_is_clean_under_asan_and_ubsan():
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    last = [l for l in r.stdout.splitlines() if l.endswith("failures")]
    assert last and last[-1].split()[2] == "0", out[-4000:]
    assert int(last[-1].split()[0]) >= 70
