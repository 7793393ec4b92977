"""Helpers shared by the GPU parity tests (marshalling and error metrics)."""
import sys

import numpy as np
import torch

import int4_weight_only_uint32_amd as qg


def note(msg):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def rel_fro(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def elementwise_guard(got, ref, atol=0.1, rtol=1e-2):
    """max over elements of |got-ref| - (atol + rtol |ref|); <= 0 passes.
    The tolerances are the elementwise ones of the SGLang w4a8 test that
    caught a synchronisation race corrupting a subset of output tiles."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref) - (atol + rtol * np.abs(ref))))


def pack_case(case, fold=True):
    q = dev(case.q)
    s = dev(case.s)
    z = dev(case.z) if case.z is not None else None
    pw = qg.pack(q, s, z, case.g, fold=fold)
    return pw


def run_w4a16(case, flags=0, fold=True):
    pw = pack_case(case, fold=fold)
    A = dev(case.A)
    C = qg.w4a16(A, pw, flags=flags)
    torch.cuda.synchronize()
    return host(C).astype(np.float64), pw
