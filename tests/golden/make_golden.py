"""Writes oracle_digest.json: the oracle's keep-mask digest and sampled outputs per workload.

Calls only the oracle and the seeded input generator.  Run from the repository root:
    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workload import ORDER, WORKLOADS, make_inputs  # noqa: E402


def main():
    out = {"_about": "written by tests/golden/make_golden.py from oracle/ only"}
    for name in ORDER:
        w = WORKLOADS[name]
        inp = make_inputs(name)
        keep = oracle.keep_mask(w.M, w.N, inp["p_drop"], w.seed)
        rows = [0, 1, w.M // 2 + 3, w.M - 1]
        cols = [0, 1, 2, 3, 37, w.N - 1]
        o, _ = oracle.run_inputs(inp, rows=rows, cols=cols)
        out[name] = {"M": w.M, "N": w.N, "K": w.K, "P": w.P, "seed": w.seed,
                     "keep_sha256": hashlib.sha256(np.packbits(keep).tobytes()).hexdigest(),
                     "kept": int(keep.sum()), "rows": rows, "cols": cols,
                     "out": [[float(v) for v in r] for r in o]}
        print(name, out[name]["kept"], flush=True)
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_digest.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
