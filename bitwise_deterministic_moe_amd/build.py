"""Builds libmoedet.so (the HIP kernels and the C ABI) for gfx950 in-tree.

    python -m bitwise_deterministic_moe_amd.build
"""
import glob
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
HEADER = os.path.join(HERE, "..", "include", "moedet.h")
LIB = os.path.join(HERE, "libmoedet.so")
SOURCES = ["moedet.hip", "route.hip", "gemm.hip", "combine.hip", "fingerprint.hip", "mfma_rate.hip", "router.hip", "train.hip", "mx.hip", "nvfp4.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-mcode-object-version=5",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-inline-asm",  # m0 is set inside the DMA asm and listed as clobbered
    # per-kernel register / LDS / scratch report, checked below
    "-Rpass-analysis=kernel-resource-usage",
    "-fno-caret-diagnostics",
]


def source_hash() -> str:
    """First 16 hex digits of SHA-256 over the library's sources (every file
    of csrc/ in name order, each name then its bytes, then the C header),
    compiled into the library as moe_source_hash()."""
    m = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))) + [HEADER]:
        m.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            m.update(fh.read())
    return m.hexdigest()[:16]


def _scratch_kernels(stderr: str) -> list:
    """Kernels whose resource report shows per-lane scratch (register spills
    or stack), from the compiler's kernel-resource-usage remarks."""
    bad, name = [], None
    for line in stderr.splitlines():
        if "remark: Function Name:" in line:
            name = line.split("Function Name:")[1].split("[")[0].strip()
        elif "ScratchSize [bytes/lane]:" in line and name:
            n = int(line.split("ScratchSize [bytes/lane]:")[1].split("[")[0])
            if n:
                bad.append((name, n))
    return bad


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = ([hipcc] + FLAGS + [f'-DMOEDET_SOURCE_HASH="{source_hash()}"'] + [os.path.join(CSRC, s) for s in SOURCES]
           + ["-o", tmp])
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    bad = _scratch_kernels(res.stderr)
    if bad:
        raise RuntimeError(f"kernels use per-lane scratch (spills): {bad}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
