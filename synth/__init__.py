"""Seeded synthetic inputs for the packed-int4 weight GEMM.

Shared by the tests, the benchmark and the smoke check; used by both the HIP
path and the CPU oracle.  It holds no arithmetic of the method itself: it only
draws random tensors.  The W4A8 variant's int8 activation codes and per-row
scales are drawn directly, shaped like per-token codes of Gaussian rows; the
fp16 rows the quantizer reads are drawn separately.

Seeds: ``np.random.SeedSequence([20261202, stream, case_id])``; tensors are
drawn in the fixed order A, q, |s|, sign, zero-noise (W4A8: A16, q, |s|,
sign, codes, row scales, zero-points).

Value distributions of the named workloads (see WORKLOADS below):
  * A ~ N(0, 1) rounded to fp16;
  * q ~ uniform integers in [0, 15];
  * |scale| ~ U[1e-3, 2e-2] rounded to fp16;
  * asymmetric zero = fp16(-8 * scale + N(0, 1e-3)), rounded once from fp64;
  * symmetric prefill case: scale sign negative with probability 1/2.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED_ROOT = 20261202


def rng_for(stream: int, case_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, stream, case_id])))


@dataclass
class W4A16Case:
    A: np.ndarray            # fp16 [M, K]
    q: np.ndarray            # uint8 [K, N], codes 0..15
    s: np.ndarray            # fp16 [G, N]
    z: Optional[np.ndarray]  # fp16 [G, N] or None (symmetric)
    g: int
    name: str = ""

    @property
    def M(self):
        return self.A.shape[0]

    @property
    def K(self):
        return self.A.shape[1]

    @property
    def N(self):
        return self.q.shape[1]

    @property
    def G(self):
        return self.K // self.g


def w4a16_case(M, K, N, g, asym=True, signed_scales=False, stream=0, case_id=0,
               name="", zero_points="noise") -> W4A16Case:
    """zero_points (asymmetric cases): "noise", z = fp16(-8 s + N(0, 1e-3)),
    the configs' recipe (delta = z + 8 s is tiny); or "awq", an integer
    zero-point per group and column, z = fp16(-zp * s) with zp ~ U{0..15}
    drawn in place of the noise (delta as large as 8 |s|)."""
    if g == -1:
        g = K
    G = -(-K // g)            # groups of g consecutive k; the last may be partial
    r = rng_for(stream, case_id)
    A = r.standard_normal((M, K)).astype(np.float16)
    q = r.integers(0, 16, size=(K, N), dtype=np.uint8)
    s_abs = r.uniform(1e-3, 2e-2, size=(G, N))
    s = s_abs.astype(np.float16)
    if signed_scales:
        neg = r.random((G, N)) < 0.5
        s = np.where(neg, -s, s).astype(np.float16)
    z = None
    if asym and zero_points == "awq":
        zp = r.integers(0, 16, size=(G, N))
        z = (-zp * s.astype(np.float64)).astype(np.float16)
    elif asym:
        assert zero_points == "noise", zero_points
        noise = r.standard_normal((G, N)) * 1e-3
        z = (-8.0 * s.astype(np.float64) + noise).astype(np.float16)
    return W4A16Case(A=A, q=q, s=s, z=z, g=g, name=name)


@dataclass
class W4A8Case:
    A16: np.ndarray          # fp16 [M_total, K] (input of the int8 quantizer)
    Aq: np.ndarray           # int8 [M_total, K] (drawn, not quantized from A16)
    a_scale: np.ndarray      # fp32 [M_total]
    q: np.ndarray            # uint8 [E, K, N]
    s: np.ndarray            # fp16 [E, G, N]
    offsets: np.ndarray      # int32 [E + 1]
    g: int
    name: str = ""
    z: Optional[np.ndarray] = None   # fp16 [E, G, N] zero-points, or None (symmetric)

    @property
    def E(self):
        return self.q.shape[0]

    @property
    def K(self):
        return self.q.shape[1]

    @property
    def N(self):
        return self.q.shape[2]

    @property
    def M_total(self):
        return self.Aq.shape[0]


def w4a8_case(E, rows_per_expert, K, N, g, signed_scales=False, stream=4, case_id=0,
              rows=None, name="", asym=False) -> W4A8Case:
    """rows: optional explicit per-expert row counts (ragged groups).
    asym: also zero-points z = fp16(-zp * s), zp ~ U{0..15} per group and
    column (an AWQ-style integer zero-point), drawn after everything else."""
    if rows is None:
        rows = [rows_per_expert] * E
    assert len(rows) == E
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(rows)
    M_total = int(offsets[-1])
    G = -(-K // g)
    r = rng_for(stream, case_id)
    A16 = r.standard_normal((M_total, K)).astype(np.float16)
    q = r.integers(0, 16, size=(E, K, N), dtype=np.uint8)
    s = r.uniform(1e-3, 2e-2, size=(E, G, N)).astype(np.float16)
    if signed_scales:
        neg = r.random((E, G, N)) < 0.5
        s = np.where(neg, -s, s).astype(np.float16)
    # int8 activation codes ~ N(0, 36^2) rounded and clipped to [-127, 127]
    # (the spread of per-row absmax codes of Gaussian rows: max|row| ~ 3.5
    # sigma maps to 127), and per-row scales ~ U[0.025, 0.032] in fp32
    # (max|row| / 127 for N(0, 1) rows of a few thousand elements)
    Aq = np.clip(np.rint(r.standard_normal((M_total, K)) * 36.0), -127, 127).astype(np.int8)
    a_scale = r.uniform(0.025, 0.032, size=M_total).astype(np.float32)
    z = None
    if asym:
        zp = r.integers(0, 16, size=(E, G, N))
        z = (-zp * s.astype(np.float64)).astype(np.float16)
    return W4A8Case(A16=A16, Aq=Aq, a_scale=a_scale, q=q, s=s, offsets=offsets, g=g, name=name,
                    z=z)


# The named workloads: shapes, value recipe and seed stream of each.
#   small-asym  16 x 1024 x 1024, group 128, asymmetric (parity and smoke size)
#   decode      M in {1, 4, 16}; K5120/N17408 and K17408/N5120; group 128 asym;
#               M=64 on K5120/N17408 (a batched decode step)
#   midbatch    M=256, K=4096, N=8192; group 256 and per-column; asymmetric
#   prefill     M=4096, K=5120, N=17408; group 128 symmetric, half the scales
#               negative (the sign fold matters)
#   w4a8-moe    8 experts x 64 tokens, K=2048, N=7168, group 128
WORKLOADS = {}


def activations(M, K, stream=5, case_id=0) -> np.ndarray:
    """Seeded fp16 N(0,1) activations [M,K] (the quantizer's prefill-size input)."""
    return rng_for(stream, case_id).standard_normal((M, K), dtype=np.float32).astype(np.float16)


def _add(name, kind, stream, case_id, **spec):
    WORKLOADS[name] = dict(kind=kind, stream=stream, case_id=case_id, spec=spec)


_add("w4a16-small-asym-M16-K1024-N1024-g128", "w4a16", 0, 0, M=16, K=1024, N=1024, g=128, asym=True)
for _i, (_k, _n, _m) in enumerate([(k, n, m) for (k, n) in ((5120, 17408), (17408, 5120))
                                   for m in (1, 4, 16)]):
    _add(f"w4a16-decode-M{_m}-K{_k}-N{_n}-g128-asym", "w4a16", 1, _i, M=_m, K=_k, N=_n, g=128,
         asym=True)
# a batched decode step (64 tokens) on the first weight shape
_add("w4a16-decode-M64-K5120-N17408-g128-asym", "w4a16", 1, 6, M=64, K=5120, N=17408, g=128,
     asym=True)
_add("w4a16-midbatch-M256-K4096-N8192-g256-asym", "w4a16", 2, 0, M=256, K=4096, N=8192, g=256,
     asym=True)
_add("w4a16-midbatch-M256-K4096-N8192-percol-asym", "w4a16", 2, 1, M=256, K=4096, N=8192,
     g=4096, asym=True)
_add("w4a16-prefill-M4096-K5120-N17408-g128-sym-signed", "w4a16", 3, 0, M=4096, K=5120,
     N=17408, g=128, asym=False, signed_scales=True)
_add("w4a8-moe-E8x64-K2048-N7168-g128", "w4a8", 4, 0, E=8, rows_per_expert=64, K=2048, N=7168,
     g=128)


def workload(name: str):
    w = WORKLOADS[name]
    if w["kind"] == "w4a16":
        return w4a16_case(stream=w["stream"], case_id=w["case_id"], name=name, **w["spec"])
    return w4a8_case(stream=w["stream"], case_id=w["case_id"], name=name, **w["spec"])


def names(prefix: str):
    return [n for n in WORKLOADS if n.startswith(prefix)]
