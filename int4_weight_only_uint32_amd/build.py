"""Build the HIP libraries in-tree for gfx950 with hipcc: libqgemm.so (the
GEMM library) and libqgprobe.so (achievable-peak probes for the benchmark)."""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqgemm.so")
# the same sources with QG_DEBUG_SYNC=1 (every pipeline stage waits for all
# outstanding memory operations): a race check compares its results with
# libqgemm.so's, bit for bit
DEBUG_SYNC_LIB = os.path.join(HERE, "libqgemm_debugsync.so")
PROBE_LIB = os.path.join(HERE, "libqgprobe.so")
PROBE_SRC = [os.path.join(HERE, "probe", "qg_probe.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no packed fp32 VALU instructions are generated.
# -amdgpu-mfma-vgpr-form: MFMA results and accumulators in ordinary VGPRs.  The
# compiler's own choice put the decode and the 32-80-row skinny kernels'
# results in accumulation registers and copied each one back before the
# scaling FMAs (12 copies per k-tile and wave in the decode kernel); without
# the copies, measured on MI355X: decode 1.5-3 % and skinny 6-10 % faster,
# the other kernels unchanged (they already used the VGPR form).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-result"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "qg_api.cpp")]


def _hipcc(srcs, out, verbose, defines=()):
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + list(defines) + ["-I", os.path.join(HERE, "..", "include")] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("hipcc failed building " + os.path.basename(out))
    if verbose and err.strip():
        sys.stderr.write(err + "\n")
    os.replace(tmp, out)
    return out


def build(verbose=False):
    """Build the three libraries (in parallel); returns the path of libqgemm.so."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(3) as ex:
        jobs = [ex.submit(_hipcc, PROBE_SRC, PROBE_LIB, verbose),
                ex.submit(_hipcc, sources(), DEBUG_SYNC_LIB, verbose, ["-DQG_DEBUG_SYNC=1"]),
                ex.submit(_hipcc, sources(), LIB, verbose)]
        for j in jobs:
            j.result()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
