"""Write tests/golden/tiny_compose.json from the CPU oracle.

Calls only oracle/ (and the seeded input generators): the tiny workload's
metadata (seed 0), tagged row values (numpy seed 1234, tests/pins.py), the
oracle's plan arrays, and SHA-256 digests of the oracle's dense buffer and
staging region after one layer.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path[:0] = [ROOT, os.path.dirname(HERE)]

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import pins  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(HERE, "tiny_compose.json")


def golden():
    b = workloads.make_batch("tiny")
    pool, cur = pins.tagged_values(b)
    pl = oracle.plan_for(b)
    staging = np.zeros(b.staging_rows_total * b.row_bytes, np.uint8)
    dense, bad = oracle.layer_for(b, pl, pool.reshape(-1), cur, staging)
    assert not bad
    return {
        "what": "tiny workload (P = (3, 5) pages, c = (100, 37) tokens, 64-token pages, "
                "1152-byte rows): the CPU oracle's plan and one layer's output digests",
        "written_by": "tests/golden/make_golden.py (oracle only)",
        "batch": {"prefix_pages": b.prefix_pages.tolist(), "cur_tokens": b.cur_tokens.tolist(),
                  "req_pages": b.req_pages.tolist(), "n_pool_pages": b.n_pool_pages,
                  "staging_cap_pages": b.staging_cap_pages},
        "values": "tests/pins.py tagged_values(batch), numpy seed 1234",
        "plan": {k: v.tolist() for k, v in pl.items()
                 if k not in ("page_inverse", "staging_page_inverse")},
        "page_inverse_set": {str(p): int(pl["page_inverse"][p])
                             for p in np.nonzero(pl["page_inverse"] >= 0)[0]},
        "staging_page_inverse_set": {str(p): int(pl["staging_page_inverse"][p])
                                     for p in np.nonzero(pl["staging_page_inverse"] >= 0)[0]},
        "dense_sha256": hashlib.sha256(dense.tobytes()).hexdigest(),
        "staging_sha256": hashlib.sha256(staging.tobytes()).hexdigest(),
    }


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(golden(), f, indent=1, sort_keys=True)
        f.write("\n")
    print(OUT)
