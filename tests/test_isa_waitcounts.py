"""The counted memory waits of the pipelined mid-batch kernels, checked on
their gfx950 assembly (no GPU needed).

Each pipeline step of w4a16_mid_kernel and w4a16_mid2_kernel issues L loads
(activations straight to LDS, codes, scales, deltas) and, before its barrier,
waits until at most (SG - 2) L loads are in flight, so the loads of the step
being computed -- including every wave's direct-to-LDS activation rows, which
the barrier then publishes -- have landed.  That holds only if the compiled
code issues exactly (SG - 1) L loads before the first barrier and L per step
in the loop.  Two ways the compiler broke it: merging the scale loads of
k-tiles that read the same group row (one group over K), and dropping the
unread loads of the steps after the main loop.  Either leaves a wave's
activation rows in flight when another wave reads them (a race that corrupts
a few tiles now and then), so this test reads the instruction stream."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "int4_weight_only_uint32_amd", "csrc", "qg_w4a16_mid.hip")
HIPCC = "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


def _vmcnt(line):
    m = re.search(r"s_waitcnt\s.*vmcnt\((\d+)\)", line)
    return int(m.group(1)) if m else None


def _kernels(asm_text):
    """{mangled name: list of (loads since the previous barrier, vmcnt of the
    last wait before this barrier)} for every barrier of every function."""
    out, cur, loads, wait = {}, None, 0, None
    for ln in asm_text.split("\n"):
        m = re.match(r"^(_Z\S+):\s", ln)
        if m:
            cur, loads, wait = m.group(1), 0, None
            out[cur] = []
            continue
        if cur is None:
            continue
        if "s_endpgm" in ln:
            cur = None
            continue
        if re.search(r"\b(buffer_load|global_load)", ln):
            loads += 1
        w = _vmcnt(ln)
        if w is not None:
            wait = w
        if "s_barrier" in ln:
            out[cur].append((loads, wait))
            loads, wait = 0, None
    return out


def _demangle(names):
    r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True,
                       check=True)
    return r.stdout.strip().split("\n")


@pytest.fixture(scope="module")
def mid_asm():
    d = tempfile.mkdtemp(prefix="qg_isa_")
    try:
        out = os.path.join(d, "mid.s")
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-mllvm", "-amdgpu-mfma-vgpr-form", "-I", os.path.join(ROOT, "include"),
                        "--cuda-device-only", "-S", "-o", out, SRC],
                       check=True, capture_output=True, timeout=600)
        with open(out) as f:
            return f.read()
    finally:
        shutil.rmtree(d, ignore_errors=True)


def _loads_per_step(kind, delta, gk):
    wn = 2
    if kind == "mid":
        return 4 + wn + wn + (wn if delta else 0)
    ns = 2 if gk == 4 else 1
    return 4 + wn + ns * wn + (ns * wn if delta else 0)


def test_mid_kernels_counted_waits(mid_asm):
    kern = _kernels(mid_asm)
    names = list(kern)
    seen = 0
    for mangled, dem in zip(names, _demangle(names)):
        m = re.search(r"w4a16_(mid2?)_kernel<(\d+), (true|false), (\d+), (true|false)>", dem)
        if not m:
            continue
        kind, sg, delta, gk = m.group(1), int(m.group(2)), m.group(3) == "true", int(m.group(4))
        L = _loads_per_step(kind, delta, gk)
        counted = (sg - 2) * L
        bars = kern[mangled]
        assert bars, dem
        # prologue: SG - 1 steps' loads, closed by a counted wait
        assert bars[0] == ((sg - 1) * L, counted), (dem, bars[0])
        drained = False
        for i, (n, w) in enumerate(bars[1:], 1):
            if w == counted:
                # a main-loop step: exactly L loads since the previous barrier
                assert n == L, (dem, i, bars)
            elif w is None and n == 0 and drained:
                pass    # the epilogue's exchanges: nothing loaded since the drain
            else:
                # anything else must wait for every load in flight
                assert w == 0, (dem, i, bars)
                drained = True
        assert sum(1 for _, w in bars if w == counted) >= sg, (dem, bars)
        seen += 1
    # both kernels x symmetric/delta x gated/plain x their group forms
    assert seen == 2 * 2 * 4 + 2 * 2 * 5, seen
