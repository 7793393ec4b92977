"""GPU parity of the per-row int8 activation quantizer against the oracle:
bit-exact codes and scales (both sides take the binary32 decisions), over
every register-resident variant and the two-pass one, ragged chunk counts, the
degenerate rows, and the W4A8 workload's inputs."""
import numpy as np
import pytest
import torch

import int4_weight_only_uint32_amd as qg
import oracle
import synth
from tests.gpu_util import dev, host, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available()
    assert qg.qg_device_supported(0), "GPU visible but not gfx950"
    oracle.build(force=False)


def _rows(M, K, seed):
    """fp16 rows of N(0,1) times a per-row magnitude spread over 1e-4 .. 1e3,
    with the degenerate rows planted: zeros, a single entry, binary16
    subnormals, exact ties at scale 1 and a constant row."""
    rng = np.random.default_rng(seed)
    mag = 10.0 ** rng.uniform(-4, 3, size=(M, 1))
    A = (rng.standard_normal((M, K)) * mag).astype(np.float16)
    if M >= 6:
        A[0] = 0
        A[1] = 0
        A[1, K // 2] = -3.0
        A[2] = np.float16(3e-7)
        A[3] = 0
        A[3, 0] = 127
        A[3, 1:] = (np.arange(1, K) % 254 - 127 + 0.5).astype(np.float16)
        A[4] = -1.5
    return A


def _check(M, K, seed=0):
    note(f"quantize_rows M={M} K={K} seed={seed}")
    A = _rows(M, K, seed)
    Aq, sc = qg.quantize_rows(dev(A))
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.quantize_rows_int8(A)
    assert np.array_equal(host(sc).view(np.uint32), ref_s.view(np.uint32))
    got = host(Aq)
    bad = np.argwhere(got != ref_q)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:4].tolist()}"


# A row has four waves (256 lanes); its chunks of 8 values per lane decide the
# variant: up to 1, 2, 4, 8 or 16 of them stay in registers, more are read
# twice.  Row counts past 2048 check many rows at once.
@pytest.mark.parametrize("M,K", [
    (1, 8), (3, 520), (7, 1032), (512, 2048),          # 1 chunk a lane
    (2, 4096), (16, 5120), (5, 12288), (16, 17408),     # 2, 3->4, 6->8, 9->16
    (2, 40000),                                         # 20: two passes
    (4100, 264), (2049, 1024), (2048, 2048),            # 1
    (2050, 4096), (2048, 8192), (2051, 8200)])          # 2, 4, 5->8
def test_quantize_rows_bit_exact(M, K):
    _check(M, K, seed=M * 7 + K)


def test_quantize_rows_w4a8_workload_inputs():
    """On the fp16 rows of the W4A8 expert-batch workload (8 x 64 rows, K
    2048) the GPU codes and scales equal the oracle's bit for bit."""
    c = synth.workload("w4a8-moe-E8x64-K2048-N7168-g128")
    note("quantize_rows w4a8 workload")
    Aq, sc = qg.quantize_rows(dev(c.A16))
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.quantize_rows_int8(c.A16)
    assert np.array_equal(host(Aq), ref_q)
    assert np.array_equal(host(sc).view(np.uint32), ref_s.view(np.uint32))


def test_quantize_rows_into_given_buffers_and_repeat():
    A = dev(_rows(40, 2048, 3))
    Aq = torch.full((40, 2048), 99, dtype=torch.int8, device="cuda")
    sc = torch.full((40,), -1.0, dtype=torch.float32, device="cuda")
    qg.quantize_rows(A, Aq, sc)
    first = (Aq.clone(), sc.clone())
    for _ in range(5):
        qg.quantize_rows(A, Aq, sc)
    torch.cuda.synchronize()
    assert torch.equal(first[0], Aq) and torch.equal(first[1], sc)
    ref_q, ref_s = oracle.quantize_rows_int8(host(A))
    assert np.array_equal(host(Aq), ref_q)
    with pytest.raises(ValueError):
        qg.quantize_rows(A, Aq[:39], sc)
