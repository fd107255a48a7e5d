"""Build libdsp.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

    python -m block_drafting_verification_amd.build

Every source under csrc/ is compiled to an object in _build/ and linked into
block_drafting_verification_amd/libdsp.so. Floating-point contraction is off
(decisions compare products such as E_j * c(j-1) exactly as written; fused
multiply-adds are requested explicitly where wanted) and packed fp32 VALU
instructions are disabled.
"""
import concurrent.futures
import glob
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdsp.so")
ARCH = os.environ.get("DSP_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wno-unused-result", "-Werror=return-type",
]


# Kernels whose streaming loads are issued asynchronously from inline assembly must not
# spill registers (a spill could copy a register before its load lands): the Markov GEMM
# instantiations with rank up to 256 (k-steps 2..16) and the scheduled tree and chain GEMMs.
ASYNC_KERNELS = re.compile(r"markov_gemm_kernelILi\dELi(2|4|8|16)ELb[01]E|(?:tree|chain)_gemm_kernelILi(2|4|8|16)E")


def _spills(stderr):
    """(function, vgpr spills + scratch bytes per lane) from hipcc's kernel-resource-usage
    remarks: either means values may live in memory instead of registers."""
    out, name = {}, None
    for line in stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out.setdefault(name, 0)
        m = re.search(r"(VGPRs Spill|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and name:
            out[name] += int(m.group(2))
    return list(out.items())


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("is not a recognized feature for this target", "remark:")
    err = "\n".join(l for l in (r.stderr or "").splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    bad = [(n, c) for n, c in _spills(r.stderr or "") if c and ASYNC_KERNELS.search(n)]
    if bad:
        raise RuntimeError(f"{src}: kernels with asynchronous loads spill or use scratch: {bad}")
    return obj, err


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for _, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
