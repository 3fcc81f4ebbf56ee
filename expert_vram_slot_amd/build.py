"""Build libmoeslot.so for gfx950 with hipcc and check its exports.

The library is built in-tree (``expert_vram_slot_amd/lib/libmoeslot.so``) so
it travels with the source tree; objects go to ``_build/``.  After linking,
every function declared in include/moe_slot.h must be exported -- a build
that silently lost an entry point would otherwise only show up later as a
failed symbol lookup.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
HEADER = os.path.join(ROOT, "include", "moe_slot.h")
OUT_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(OUT_DIR, "libmoeslot.so")
OBJ_DIR = os.path.join(ROOT, "_build", "moeslot")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-I" + os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]
# gfx950 device code: no packed-fp32 instructions
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffp-contract=fast"]
HOST = ["-x", "c++", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-mf16c", "-mavx2", "-mfma", "-pthread"]
# AddressSanitizer + UndefinedBehaviorSanitizer on the host code only (the CPU
# host pass, the driver, argument checks); device code is built as usual.
# Each -fsanitize= goes right after -Xarch_host so that no GPU code is built
# with it.  The sanitized library is for CPU test runs, never for a GPU run.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_DIR = os.path.join(ROOT, "_build", "sanitized")
SAN_LIB = os.path.join(SAN_DIR, "libmoeslot.so")


def exported_api() -> list[str]:
    """Function names declared in the public header."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "return")))


def _compile(src: str, obj_dir: str = OBJ_DIR, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    flags = COMMON + (DEVICE if src.endswith(".hip") else HOST) + list(extra)
    cmd = [HIPCC] + flags + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build the library; sanitize=True builds the host code under ASan/UBSan
    into _build/sanitized/ instead (load it with the sanitizer runtime
    preloaded; MOE_SLOT_LIB points the binding at it)."""
    out = SAN_LIB if sanitize else LIB
    obj_dir = os.path.join(SAN_DIR, "obj") if sanitize else OBJ_DIR
    extra = SANITIZE if sanitize else []
    os.makedirs(os.path.dirname(out), exist_ok=True)
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, obj_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + ["-pthread"]
    if sanitize:
        cmd += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    check_exports(tmp)
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def check_exports(path: str) -> None:
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    have = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in exported_api() if n not in have]
    if missing:
        raise RuntimeError(f"{path} does not export {missing}")


if __name__ == "__main__":
    build(verbose=True)
    print("exports ok:", ", ".join(exported_api()))
    sys.exit(0)
