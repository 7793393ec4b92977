"""Write synth_sha256.json: the SHA-256 of every tensor of every named
synthetic workload (generator determinism fixture).

Run from the repository root:  python tests/golden/make_synth_sha256.py
It calls only the seeded input generators in synth/ -- nothing of the GEMM
library or the oracle.
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "synth_sha256.json")


def digests(name):
    c = synth.workload(name)
    out = {}
    for field, v in sorted(vars(c).items()):
        if isinstance(v, np.ndarray):
            a = np.ascontiguousarray(v)
            out[field] = {"dtype": str(a.dtype), "shape": list(a.shape),
                          "sha256": hashlib.sha256(a.tobytes()).hexdigest()}
    return out


def main():
    rec = {n: digests(n) for n in synth.WORKLOADS}
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(OUT)


if __name__ == "__main__":
    main()
