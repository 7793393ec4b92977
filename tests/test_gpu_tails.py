"""GPU parity on shapes whose K or N is not a multiple of 128 (the padded
pack; A padded and C cropped through the workspace): a 50257-wide vocabulary
head on sampled cells, and dense checks of K tails with a partial last group,
per-column scales, and every GEMM kernel the padded shape selects."""
import numpy as np
import pytest
import torch

import int4_weight_only_uint32_amd as qg
import oracle
import synth
from tests.gpu_util import dev, elementwise_guard, host, note, rel_fro

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available()
    assert qg.qg_device_supported(0), "GPU visible but not gfx950"
    oracle.build(force=False)


def _run(c, asym):
    pw = qg.pack(dev(c.q), dev(c.s), dev(c.z) if asym else None, c.g, fold=True)
    C = qg.w4a16(dev(c.A), pw)
    torch.cuda.synchronize()
    return pw, host(C).astype(np.float64)


@pytest.mark.parametrize("M,K,N,g,asym,signed", [
    (3, 1000, 300, 128, True, False),      # K and N tails, partial last group (104 of 128)
    (7, 1000, 300, -1, True, False),       # one group per column over a K tail
    (16, 1000, 1024, 384, False, True),    # groups of 384, the last of 232; decode batch
    (16, 130, 200, 128, True, False),      # a group of 2
    (64, 1000, 1000, 128, True, False),    # mid batch
    (300, 1000, 520, 256, False, True),    # tiled kernels
])
def test_tails_dense(M, K, N, g, asym, signed):
    c = synth.w4a16_case(M, K, N, g, asym=asym, signed_scales=signed, stream=92,
                         case_id=M * 7 + N)
    note(f"tails M={M} K={K} N={N} g={g} asym={asym}")
    pw, got = _run(c, asym)
    ref = oracle.w4a16(c.A, c.q, c.s, c.z if asym else None, c.g, fold=True)
    assert got.shape == (M, N)
    assert rel_fro(got, ref) <= TOL
    assert elementwise_guard(got, ref) <= 0
    Np = pw.scale.shape[1]
    if Np > N:   # padded columns hold scale 0
        assert int(pw.scale[:, N:].count_nonzero()) == 0


@pytest.mark.parametrize("M", [1, 16])
def test_vocab_head_dense(M):
    """K 5120 -> a 50257-token vocabulary (N = 50304 padded), asymmetric g128,
    in the benchmark's launch shape, checked densely: every output, so every
    column group of the decode kernel, both of its k-splits and the cropped
    tail tile."""
    K, N = 5120, 50257
    c = synth.w4a16_case(M, K, N, 128, asym=True, stream=92, case_id=1000 + M)
    note(f"vocab head M={M} K={K} N={N}")
    _, got = _run(c, True)
    ref = oracle.w4a16(c.A, c.q, c.s, c.z, 128, fold=True)
    assert rel_fro(got, ref) <= TOL
    assert elementwise_guard(got, ref) <= 0


@pytest.mark.parametrize("asym", [False, True])
def test_w4a8_tails(asym):
    """Grouped W4A8 with K = 1000 (a partial last group) and N = 300 over
    ragged experts (one empty): padded packs, A_q padded and C cropped through
    the workspace."""
    c = synth.w4a8_case(3, 0, 1000, 300, 128, signed_scales=not asym, stream=92, case_id=2000,
                        rows=[40, 0, 75], asym=asym)
    note(f"w4a8 tails asym={asym} rows={np.diff(c.offsets).tolist()} K=1000 N=300")
    packs = [qg.pack(dev(c.q[e]), dev(c.s[e]), dev(c.z[e]) if asym else None, c.g, fold=True)
             for e in range(c.E)]
    W = torch.stack([p.w for p in packs]).contiguous()
    S = torch.stack([p.scale for p in packs]).contiguous()
    D = torch.stack([p.delta for p in packs]).contiguous() if asym else None
    C = qg.w4a8(dev(c.Aq), dev(c.a_scale), W, S, dev(c.offsets), c.E, 75, c.N, c.g, w_delta=D)
    torch.cuda.synchronize()
    got = host(C).astype(np.float64)
    ref, _ = oracle.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, c.g, fold=True, z=c.z,
                         want_acc=False)
    assert rel_fro(got, ref) <= 1e-2
    assert elementwise_guard(got, ref) <= 0


def test_w4a8_tail_then_split_k_decode_shared_workspace():
    """A W4A8 call on a tail shape and a split-K W4A16 decode call share the
    binding's cached workspace on one stream: the W4A8 call must leave the
    split-K counters (the workspace's first QG_W4A16_WS_COUNTER_BYTES) at
    zero, or the decode call's partial sums never meet and C is not written."""
    c8 = synth.w4a8_case(3, 0, 1000, 300, 128, stream=92, case_id=2001, rows=[40, 0, 75])
    packs = [qg.pack(dev(c8.q[e]), dev(c8.s[e]), None, c8.g, fold=True) for e in range(c8.E)]
    W = torch.stack([p.w for p in packs]).contiguous()
    S = torch.stack([p.scale for p in packs]).contiguous()
    c16 = synth.workload("w4a16-decode-M16-K5120-N17408-g128-asym")
    pw = qg.pack(dev(c16.q), dev(c16.s), dev(c16.z), c16.g, fold=True)
    A16 = dev(c16.A)
    ref16 = oracle.w4a16(c16.A, c16.q, c16.s, c16.z, c16.g)
    ref8, _ = oracle.w4a8(c8.Aq, c8.a_scale, c8.q, c8.s, c8.offsets, c8.g, want_acc=False)
    for rep in range(2):
        note(f"shared workspace: w4a8 tail then split-K decode, rep {rep}")
        C8 = qg.w4a8(dev(c8.Aq), dev(c8.a_scale), W, S, dev(c8.offsets), c8.E, 75, c8.N, c8.g)
        C16 = torch.full((c16.M, c16.N), float("nan"), dtype=torch.float16, device="cuda")
        qg.w4a16(A16, pw, C=C16)
        torch.cuda.synchronize()
        got8 = host(C8).astype(np.float64)
        got16 = host(C16).astype(np.float64)
        assert rel_fro(got8, ref8) <= 1e-2
        assert np.all(np.isfinite(got16))
        assert rel_fro(got16, ref16) <= TOL
        assert elementwise_guard(got16, ref16) <= 0
