"""Build liboasis.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "liboasis")
LIB = os.path.join(PKG, "liboasis.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed fp32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build (device code
# unchanged): each sanitizer flag applies to the host pass only.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SAN_OBJ = os.path.join(ROOT, "_build", "liboasis_san")
SAN_LIB = os.path.join(ROOT, "_build", "san", "liboasis_san.so")


def _compile(src, san=False):
    obj = os.path.join(SAN_OBJ if san else OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(SAN_HOST if san else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    return obj, msg


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP source for gfx950 and link liboasis.so.

    sanitize=True links the host-sanitized variant into _build/san/ instead
    (loaded only through OASIS_LIBRARY, in a process that preloads clang's
    AddressSanitizer runtime)."""
    os.makedirs(SAN_OBJ if sanitize else OBJ, exist_ok=True)
    with ThreadPoolExecutor(min(8, os.cpu_count() or 4)) as ex:
        results = list(ex.map(lambda s: _compile(s, sanitize), sources()))
    for obj, msg in results:
        if verbose and msg.strip():
            print(msg)
    out = SAN_LIB if sanitize else LIB
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
           *[o for o, _ in results], "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
