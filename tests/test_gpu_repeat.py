"""Repeatability and stream probes (the same inputs under every kernel path,
repeated, on several streams at once).

A synchronisation race typically corrupts a varying subset of output tiles
from run to run (the SGLang w4a8 article's race did: a quarter of the
elements mismatched).  Every kernel here is deterministic -- the split-K
reduction sums the partial results in a fixed order -- so each repeat must
be bitwise identical to the first, whichever stream it ran on and whatever
ran beside it.  The first result is also checked against the oracle."""
import numpy as np
import pytest
import torch

import int4_weight_only_uint32_amd as qg
import oracle
import synth
from tests.gpu_util import dev, elementwise_guard, host, note, pack_case, rel_fro

pytestmark = pytest.mark.gpu

REPEATS = 20


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available()
    assert qg.qg_device_supported(0), "GPU visible but not gfx950"
    oracle.build(force=False)


# one shape per kernel path: decode split 8 ways, decode unsplit, skinny,
# mid-size M, 64x128 tiles with the fused delta, 128x256 symmetric tiles with
# the row split, the separate correction launch, and two shapes with tails
CASES = [
    (16, 16384, 4096, 128, True, 0),
    (4, 1024, 32768, 128, False, 0),
    (40, 2048, 1024, 128, True, 0),
    (256, 4096, 2048, 256, True, 0),
    (512, 1024, 8192, 128, True, 0),
    (1000, 640, 16256, 128, False, 0),
    (16, 1024, 1024, 128, True, 1),
    (16, 1000, 1000, 128, True, 0),        # tails: A padded, C cropped
    (300, 1000, 520, 256, False, 0),
]


@pytest.mark.parametrize("M,K,N,g,asym,flags", CASES)
def test_w4a16_repeats_bitwise_across_streams(M, K, N, g, asym, flags):
    note(f"repeat w4a16 M={M} K={K} N={N} g={g} asym={asym} flags={flags}")
    c = synth.w4a16_case(M, K, N, g, asym=asym, signed_scales=not asym, stream=91,
                         case_id=M + K + N, name="repeat")
    pw = pack_case(c)
    A = dev(c.A)
    first = qg.w4a16(A, pw, flags=flags)
    torch.cuda.synchronize()
    ref = oracle.w4a16(c.A, c.q, c.s, c.z, c.g)
    got = host(first).astype(np.float64)
    assert rel_fro(got, ref) <= 2e-3
    assert elementwise_guard(got, ref) <= 0

    streams = [torch.cuda.current_stream(), torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for i in range(REPEATS):
        s = streams[i % len(streams)]
        with torch.cuda.stream(s):
            # each stream has its own cached workspace; outputs are distinct
            outs.append(qg.w4a16(A, pw, flags=flags))
    torch.cuda.synchronize()
    want = host(first)
    for i, o in enumerate(outs):
        assert np.array_equal(host(o), want), f"repeat {i} (stream {i % len(streams)}) differs"


def test_w4a8_repeats_bitwise_across_streams():
    c = synth.w4a8_case(8, 64, 2048, 1024, 128, stream=92, case_id=0)
    note(f"repeat w4a8 E={c.E} rows=64 K={c.K} N={c.N}")
    packs = [qg.pack(dev(c.q[e]), dev(c.s[e]), None, c.g, fold=True) for e in range(c.E)]
    W = torch.stack([p.w for p in packs]).contiguous()
    S = torch.stack([p.scale for p in packs]).contiguous()
    Aq, asc, off = dev(c.Aq), dev(c.a_scale), dev(c.offsets)
    first = qg.w4a8(Aq, asc, W, S, off, c.E, 64, c.N, c.g)
    torch.cuda.synchronize()
    ref, _ = oracle.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, c.g)
    got = host(first).astype(np.float64)
    assert rel_fro(got, ref) <= 1e-2
    assert elementwise_guard(got, ref) <= 0
    streams = [torch.cuda.current_stream(), torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for i in range(REPEATS):
        with torch.cuda.stream(streams[i % len(streams)]):
            outs.append(qg.w4a8(Aq, asc, W, S, off, c.E, 64, c.N, c.g))
    torch.cuda.synchronize()
    want = host(first)
    for i, o in enumerate(outs):
        assert np.array_equal(host(o), want), f"repeat {i} differs"


@pytest.mark.parametrize("M,K,N", [(16, 17408, 5120), (64, 1024, 1024)])
def test_swiglu_repeats_bitwise_across_streams(M, K, N):
    """The gated decode kernel (split-K) and the GEMM-then-elementwise path."""
    note(f"repeat swiglu M={M} K={K} N={N}")
    c = synth.w4a16_case(M, K, 2 * N, 128, asym=True, stream=91, case_id=7000 + M)
    pair = qg.pack(dev(c.q), dev(c.s), dev(c.z), 128)
    A = dev(c.A)
    first = qg.w4a16_swiglu(A, pair)
    torch.cuda.synchronize()
    ref = oracle.w4a16_swiglu(c.A, c.q, c.s, c.z, 128)
    assert rel_fro(host(first).astype(np.float64), ref) <= 2e-3
    streams = [torch.cuda.current_stream(), torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for i in range(REPEATS):
        with torch.cuda.stream(streams[i % len(streams)]):
            outs.append(qg.w4a16_swiglu(A, pair))
    torch.cuda.synchronize()
    want = host(first)
    for i, o in enumerate(outs):
        assert np.array_equal(host(o), want), f"repeat {i} differs"


def test_quantize_then_w4a8_asym_repeats_bitwise_across_streams():
    """The quantizer and the zero-point W4A8 GEMM, chained on each stream."""
    c = synth.w4a8_case(8, 64, 2048, 1024, 128, stream=92, case_id=1, asym=True)
    note(f"repeat quantize + w4a8 asym E={c.E} K={c.K} N={c.N}")
    packs = [qg.pack(dev(c.q[e]), dev(c.s[e]), dev(c.z[e]), c.g) for e in range(c.E)]
    W = torch.stack([p.w for p in packs]).contiguous()
    S = torch.stack([p.scale for p in packs]).contiguous()
    D = torch.stack([p.delta for p in packs]).contiguous()
    A16, off = dev(c.A16), dev(c.offsets)

    def run():
        Aq, asc = qg.quantize_rows(A16)
        return qg.w4a8(Aq, asc, W, S, off, c.E, 64, c.N, c.g, w_delta=D)

    first = run()
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.quantize_rows_int8(c.A16)
    ref, _ = oracle.w4a8(ref_q, ref_s, c.q, c.s, c.offsets, c.g, z=c.z)
    assert rel_fro(host(first).astype(np.float64), ref) <= 1e-2
    streams = [torch.cuda.current_stream(), torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for i in range(REPEATS):
        with torch.cuda.stream(streams[i % len(streams)]):
            outs.append(run())
    torch.cuda.synchronize()
    want = host(first)
    for i, o in enumerate(outs):
        assert np.array_equal(host(o), want), f"repeat {i} differs"
