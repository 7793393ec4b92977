"""Generator determinism (CPU): every named synthetic workload regenerates
bit for bit -- each tensor's SHA-256 equals the one recorded in
tests/golden/synth_sha256.json (written by tests/golden/make_synth_sha256.py,
which calls only the seeded generators)."""
import json
import os

import pytest

from tests.golden.make_synth_sha256 import OUT, digests

import synth

with open(OUT) as f:
    RECORDED = json.load(f)


def test_every_workload_is_recorded():
    assert sorted(RECORDED) == sorted(synth.WORKLOADS)


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_workload_regenerates_identically(name):
    assert digests(name) == RECORDED[name]
