"""Build libpulse.so (HIP, gfx950) in-tree.

Every source is compiled for gfx950 only, with packed-FP32 instructions turned
off, FP32 denormals kept and no FP contraction (the FP8 quantiser's divisions
and rounding must be IEEE-exact).  Objects go to sparse_delta_codec_amd/_build/.
"""
import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpulse.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["capi.cpp", "util.hip", "cast_diff.hip", "apply.hip", "lz4_encode.hip", "lz4_decode.hip",
           "fp8_quant.hip", "delta_compact.hip",
           "patch_pack.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off", "-fno-fast-math",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE,
]


# host-side sanitizers (the sanitizer test): each flag behind -Xarch_host, so
# only the host code of every source is instrumented
HOST_SANITIZE = ["-g", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
                 "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all"]


def _compile(src, verbose, out=None, extra=()):
    obj = os.path.join(out or OUT, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(SRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return obj, warn


def build_host_sanitized(out_dir: str) -> str:
    """libpulse.so with its host code built with AddressSanitizer and
    UndefinedBehaviorSanitizer, into out_dir (load it with clang's ASan runtime
    preloaded).  The device code is built as usual."""
    os.makedirs(out_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, False, out_dir, HOST_SANITIZE), SOURCES))
    lib = os.path.join(out_dir, "libpulse.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", lib, *[o for o, _ in results]]
    subprocess.run(cmd, check=True, capture_output=True)
    return lib


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    for obj, warn in results:
        if verbose and warn:
            print(warn)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *[o for o, _ in results]]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    build_probe(verbose)
    return LIB


PROBE_LIB = os.path.join(HERE, "libpulse_probe.so")


def build_probe(verbose: bool = False) -> str:
    """The bandwidth probes the benchmark sets the kernels against (csrc/probe.hip),
    in a library of their own: the codec's library does not contain them."""
    cmd = [HIPCC, *FLAGS, "-shared", os.path.join(SRC, "probe.hip"), "-o", PROBE_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for probe.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose=True))
