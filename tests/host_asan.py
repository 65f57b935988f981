"""Host-only AddressSanitizer + UBSan build of libkvq (not a test module).

csrc/kvq_api.hip (the whole C ABI) is compiled for the host side only, with
-fsanitize=address,undefined on the host pass, and linked with stand-ins for
the kernel launchers (tests/host_asan_stubs.hip) into
_build/asan/libkvq_asan.so. That library runs the C ABI's validation, cache
layout and split-planning code exactly as the product build does; every
launch in it returns a HIP error, so only host-side paths can be exercised
(they are all the CPU tests call). test_host_asan.py runs the CPU ABI and
binding tests against it with the sanitizer runtime preloaded.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_paged_kv_store_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT, "libkvq_asan.so")
# -Xarch_host keeps the sanitizers on the host pass
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]
FLAGS = ["-x", "hip", "--cuda-host-only", "-O1", "-g", "-fPIC", "-std=c++17", "-fno-omit-frame-pointer",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str | None:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return p if os.path.exists(p) else None


def asan_runtime() -> str | None:
    """The clang ASan runtime the library links against (to be preloaded
    into the Python process, which is not itself instrumented)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc() or "")), "..", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(cand):
            for name in ("libclang_rt.asan.so", "libclang_rt.asan-x86_64.so"):
                r = subprocess.run([cand, f"-print-file-name={name}"], capture_output=True, text=True)
                p = r.stdout.strip()
                if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p):
                    return p
    return None


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")


def build() -> str:
    cc = hipcc()
    if cc is None:
        raise RuntimeError("hipcc not found")
    os.makedirs(OUT, exist_ok=True)
    # the C ABI's host code, and stand-ins for the kernel launchers (a
    # host-only build of the kernel sources would need their device code)
    srcs = [os.path.join(CSRC, "kvq_api.hip"), os.path.join(ROOT, "tests", "host_asan_stubs.hip")]
    objs = [os.path.join(OUT, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for f in [ex.submit(_run, [cc, *FLAGS, *SAN, "-c", s, "-o", o]) for s, o in zip(srcs, objs)]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", "-Xarch_host", "-shared-libasan", *SAN, *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
