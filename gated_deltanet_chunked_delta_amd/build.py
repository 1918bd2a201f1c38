"""Build the HIP library ``libgdn.so`` for gfx950 with hipcc (in-tree).

Every translation unit is compiled separately (in parallel) and linked into one
shared library next to this file.  Packed-fp32 instruction selection is turned
off for all device code.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INC = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgdn.so")
# The same kernels with per-phase cycle counters (bench.py --phase-clock)
LIB_CLOCK = os.path.join(HERE, "libgdn_clock.so")
OBJ = os.path.join(HERE, "_build")
SOURCES = ["gdn_api.hip", "gdn_plan.hip", "gdn_tsolve.hip", "gdn_fwd.hip", "gdn_bwd.hip", "gdn_decode.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INC, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


# Host-side sanitizers only (the device code is built as always): for CPU runs of
# the argument checks and the workspace layout, with clang's ASan runtime preloaded.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, obj_dir: str = OBJ, extra=()) -> str:
    obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
    cmd = ["hipcc", "-c", *FLAGS, *extra, os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False, phase_clock: bool = False) -> str:
    """Compile every source and link `out`.  sanitize: host code with AddressSanitizer and
    UndefinedBehaviorSanitizer (objects in a separate folder; load with GDN_LIB=out).
    phase_clock: the kernels also sum the shader clock per phase of each workgroup
    (GDN_PHASE_CLOCK; objects in a separate folder, default output LIB_CLOCK)."""
    obj_dir = OBJ + ("_san" if sanitize else "") + ("_clock" if phase_clock else "")
    os.makedirs(obj_dir, exist_ok=True)
    extra = (SAN_FLAGS if sanitize else ()) + (("-DGDN_PHASE_CLOCK",) if phase_clock else ())
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s_: _compile(s_, obj_dir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = ["hipcc", "-shared", f"--offload-arch={ARCH}", "-fPIC", *(SAN_FLAGS if sanitize else ()), *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--sanitize", action="store_true")
    ap.add_argument("--phase-clock", action="store_true")
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    out = a.out or (LIB_CLOCK if a.phase_clock else LIB)
    build(verbose=True, out=os.path.abspath(out), sanitize=a.sanitize, phase_clock=a.phase_clock)
    sys.exit(0)
