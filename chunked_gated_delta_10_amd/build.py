"""Build libkda.so (all HIP sources of csrc/) for gfx950 with hipcc, in-tree."""

from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkda.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions are kept off: the compiler must not form them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build (device code
# is compiled as usual; every -fsanitize= applies to the host pass only).
# Loading it needs clang's ASan runtime preloaded (sanitizer_runtime()).
SANITIZE_FLAGS = [
    "--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-shared-libasan",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, what, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building " + what)


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    cmd += sources() + ["-o", tmp]
    _run(cmd, "libkda.so", verbose)
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(out: str, jobs: int = 8, verbose: bool = False) -> str:
    """The host-sanitizer build of the library, to ``out`` (sources compiled in parallel)."""
    from concurrent.futures import ThreadPoolExecutor
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    objs = [out + "." + os.path.basename(s) + ".o" for s in sources()]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _run([_hipcc()] + SANITIZE_FLAGS + inc + ["-c", so[0], "-o", so[1]], so[0], verbose),
                    zip(sources(), objs)))
    _run([_hipcc()] + SANITIZE_FLAGS + ["-shared"] + objs + ["-o", out], out, verbose)
    for o in objs:
        os.remove(o)
    return out


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime the sanitized build links against."""
    res = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return res.stdout.strip()


if __name__ == "__main__":
    print(build(verbose=True))
