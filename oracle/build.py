"""Builds the CPU oracle library (test infrastructure) with gcc."""
import os
import subprocess
from pathlib import Path

HERE = Path(__file__).resolve().parent
LIB = HERE / "liboracle.so"


SAN_LIB = HERE / "liboracle_asan.so"
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> Path:
    """liboracle.so, or with sanitize=True liboracle_asan.so (AddressSanitizer
    and UndefinedBehaviorSanitizer; load it with libasan preloaded)."""
    out = SAN_LIB if sanitize else LIB
    cmd = ["gcc", "-O1" if sanitize else "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", *(SANITIZE if sanitize else []), "-o", str(out),
           str(HERE / "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    build(verbose=True)
