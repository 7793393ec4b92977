"""GPU parity of the grouped W4A8 GEMM over a seeded sweep of expert batches:
1 to 8 experts with ragged row counts (empty experts included), K and N with
and without tails, groups of 32, 64, 128, 256 and one group over K, symmetric
weights with random-sign scales and AWQ-style zero-points.  The integer group
products (acc_debug, where the shape has no tail) are compared bit for bit
and C to the W4A8 bar against the oracle ("HyperQwen ...", "int8 张量核实战数值
验证怎么做"; the SGLang w4a8 article's grouped layout, "任务切分")."""
import numpy as np
import pytest
import torch

import int4_weight_only_uint32_amd as qg
import oracle
import synth
from tests.gpu_util import dev, elementwise_guard, host, note, rel_fro

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _cases(n=40, seed=7168, groups=(64, 128, 256, -1)):
    r = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        E = int(r.choice([1, 2, 5, 8]))
        rows = [int(x) if r.rand() > 0.15 else 0 for x in r.randint(1, 200, size=E)]
        K = int(r.choice([256, 512, 1000, 2048]))
        N = int(r.choice([128, 300, 1024, 2048]))
        g = int(r.choice(list(groups)))
        g = K if g == -1 else g
        if g > K or (g >= 128 and g % 128 and g != K) or sum(rows) * K * N > (1 << 29):
            continue
        if sum(rows) == 0:
            continue                      # at least one row in the batch
        out.append((tuple(rows), K, N, g, bool(r.rand() < 0.5)))
    return out


# the 40 mixed-group batches, then 12 with groups of 32
@pytest.mark.parametrize("rows,K,N,g,asym", _cases() + _cases(12, 3232, (32,)))
def test_w4a8_sweep(rows, K, N, g, asym):
    E = len(rows)
    c = synth.w4a8_case(E, 0, K, N, g, signed_scales=not asym, stream=87,
                        case_id=sum(rows) + K + N + g, rows=list(rows), asym=asym)
    note(f"w4a8 sweep rows={list(rows)} K={K} N={N} g={g} asym={asym}")
    packs = [qg.pack(dev(c.q[e]), dev(c.s[e]), dev(c.z[e]) if asym else None, g, fold=True)
             for e in range(E)]
    W = torch.stack([p.w for p in packs]).contiguous()
    S = torch.stack([p.scale for p in packs]).contiguous()
    D = torch.stack([p.delta for p in packs]).contiguous() if asym else None
    exact = K % 128 == 0 and N % 128 == 0
    acc = (torch.full((c.M_total, K // g, N), -7, dtype=torch.int32, device="cuda")
           if exact else None)
    mr = max(max(rows), 1)
    C = qg.w4a8(dev(c.Aq), dev(c.a_scale), W, S, dev(c.offsets), E, mr, N, g, acc_debug=acc,
                w_delta=D)
    torch.cuda.synchronize()
    got = host(C).astype(np.float64)
    assert np.all(np.isfinite(got))
    ref, ref_acc = oracle.w4a8(c.Aq, c.a_scale, c.q, c.s, c.offsets, g, fold=True, z=c.z)
    if exact:
        assert np.array_equal(host(acc).astype(np.int64), ref_acc)
    assert rel_fro(got, ref) <= TOL
    assert elementwise_guard(got, ref) <= 0
