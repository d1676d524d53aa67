"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, -O2, no fast-math, no FP contraction, no intrinsics: the oracle is
meant to be read against its definitions, not to be fast.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, sanitize: bool = False, out: str = None) -> str:
    """sanitize: an AddressSanitizer + UndefinedBehaviorSanitizer build (to
    `out`, for the sanitizer test; load it with the ASan runtime preloaded)."""
    lib = out or LIB
    cmd = [
        "gcc", "-std=c11", "-O2", "-fPIC", "-shared",
        "-fno-fast-math", "-ffp-contract=off", "-fno-strict-aliasing",
        "-Wall", "-Wextra",
    ]
    if sanitize:
        cmd += ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    cmd += [os.path.join(HERE, "oracle.c"), "-o", lib + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
