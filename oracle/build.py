"""Compile the fp64 oracle (``gdn_oracle.c``) with gcc.  Test infrastructure only."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True, out: str = LIB, sanitize: bool = False) -> str:
    """Compile to `out`.  sanitize: with AddressSanitizer and UndefinedBehaviorSanitizer
    (load it with gcc's libasan preloaded and GDN_ORACLE_LIB=out)."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
        return out
    tmp = out + ".tmp"
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g"] if sanitize else []
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", *san, "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--sanitize", action="store_true")
    ap.add_argument("--out", default=LIB)
    a = ap.parse_args()
    print(build(out=a.out, sanitize=a.sanitize))
