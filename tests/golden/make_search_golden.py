"""Write tests/golden/search_4096.json: the oracle's alpha search on the
4096-token x 4096 x 4096 search layer.  Calls only the oracle and the seeded
input generators.  Run from the repository root:

    python tests/golden/make_search_golden.py
"""

import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402
from oracle import QuantConfig, scale_search  # noqa: E402


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def main():
    case = wl.search_case()
    X = case.activation()
    W = case.weight()
    t0 = time.time()
    res = scale_search(X, W, QuantConfig(group_size=case.group_size))
    dt = time.time() - t0
    out = {
        "about": "Oracle alpha-grid search (alpha_j = j/20, j=0..19, g128, zero point) on the "
                 "search layer: X [4096][4096] fp16 N(0,1) with 41 channels x20, W [4096][4096] "
                 "N(0,0.02), seeds from workloads.search_case(). Written by "
                 "tests/golden/make_search_golden.py (oracle only).",
        "case": case.name,
        "best_index": res["best_index"],
        "losses": [float(v) for v in res["losses"]],
        "sha256_s": sha(res["s"].view(np.uint32)),
        "sha256_qweight": sha(res["qweight"]),
        "sha256_scales": sha(res["scales"].view(np.uint16)),
        "sha256_zeros": sha(res["zeros"]),
        "oracle_seconds": round(dt, 1),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "search_4096.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: out[k] for k in ("best_index", "oracle_seconds")}))


if __name__ == "__main__":
    main()
