"""CPU-only sanitizer runs of the host code.

* The oracle (plain C) is rebuilt with gcc's AddressSanitizer and
  UndefinedBehaviorSanitizer, and every pin is run on that build.
* The HIP library is rebuilt with the same sanitizers on its host code only
  (device code is compiled as usual and never runs here), and the host-side
  ABI tests run on that build: every argument check of every entry point,
  with no GPU.

Each run happens in a child interpreter with the sanitizer runtime preloaded;
a report makes the child abort, so a non-zero exit fails the test.  The
instrumented library is cached under _build/ by a hash of its sources.
"""
import glob
import hashlib
import os
import shutil
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
RUNNER = os.path.join(HERE, "sanitized_run.py")
CACHE = os.path.join(ROOT, "_build", "sanitized")

SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    "OMP_NUM_THREADS": "2",
}


def _run(mode: str, lib: str, preload: str) -> None:
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    r = subprocess.run([sys.executable, RUNNER, mode, lib], env=env, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        pytest.fail(f"sanitized {mode} run exited {r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}")


def _gcc_runtime(name: str) -> str:
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else ""


def test_oracle_pins_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "libdlrm_oracle_san.so")
    oracle.compile_library(out=lib, extra_flags=["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                                                 "-fno-sanitize-recover=undefined"])
    _run("pins", lib, f"{asan} {ubsan}")


def _clang_asan_runtime(hipcc: str) -> str:
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))), "llvm")
    hits = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else ""


def _sanitized_library() -> str:
    from dlrm_embedding_interaction_amd import _build
    cc = _build.hipcc()
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(_build.CSRC, "*")) + [os.path.join(_build.INCLUDE, "dlrm_mi355x.h")]):
        with open(p, "rb") as f:
            h.update(f.read())
    out = os.path.join(CACHE, f"libdlrm_mi355x_san_{h.hexdigest()[:16]}.so")
    if os.path.exists(out):
        return out
    shutil.rmtree(CACHE, ignore_errors=True)
    os.makedirs(CACHE)
    # sanitizers on the host side only: each -fsanitize= right after -Xarch_host
    host_san = "-g -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer"
    objs = []
    procs = []
    for src in _build.SOURCES:
        obj = os.path.join(CACHE, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *_build.common_flags(), *host_san.split(), "-c", os.path.join(_build.CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    for src, p in procs:
        _, err = p.communicate()
        if p.returncode != 0:
            raise RuntimeError(f"sanitized build of {src} failed:\n{err}")
    r = subprocess.run([cc, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", *objs, "-o", out],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    return out


def test_host_abi_under_address_and_undefined_behaviour_sanitizers():
    from dlrm_embedding_interaction_amd import _build
    try:
        cc = _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    rt = _clang_asan_runtime(cc)
    if not rt:
        pytest.skip("clang AddressSanitizer runtime not found next to hipcc")
    _run("abi", _sanitized_library(), rt)
