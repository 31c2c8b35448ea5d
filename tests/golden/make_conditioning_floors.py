"""Writes tests/golden/conditioning_floors.json: the oracle's own conditioning
floor for every full-size parity case whose bar is derived from it
(tests.helpers.DERIVED_BAR_CASES).  Calls only the oracle and the seeded input
generators, never the library.

The floor of a case is the (rel-L2, max-abs) change of the oracle's output
(bf16 storage) on the case's compared rows (the first 96 of them at full
size) when its input x is multiplied by 1 + eps N(0, 1) (seed 0), eps = 1e-7
for an fp32-level difference and 2^-13 for the FP8 MFMA's summation error.

    python -m tests.golden.make_conditioning_floors [case ...]
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import hybrid_layer as O  # noqa: E402
from tests.helpers import (DERIVED_BAR_CASES, FLOOR_ROWS, FLOORS_JSON, conditioning_floor,  # noqa: E402
                           rows_digest, sample_rows)


def floor_of(name):
    build, n_random, eps, _ = DERIVED_BAR_CASES[name]
    t0 = time.time()
    wl = build()
    if n_random is None:
        rows, seqs, tag = None, None, "all"
    else:
        rows = sample_rows(wl, n_random=n_random)[:FLOOR_ROWS]
        lay = O.token_layout(wl.batch.chunk_len, wl.batch.chunk_prefix, wl.batch.decode_ctx)
        seqs = sorted(set(int(s) for s in lay.seq[rows]))
        tag = rows_digest(rows)
    rel, mx = conditioning_floor(wl, rows, seqs, eps=eps)
    print(f"{name}: eps {eps:.2e} rows {tag}: floor rel_l2 {rel:.4e} max_abs {mx:.4e} ({time.time() - t0:.0f} s)",
          flush=True)
    return dict(eps=eps, rows=tag, n_rows=(wl.batch.n_tokens if rows is None else len(rows)),
                floor_rel_l2=rel, floor_max_abs=mx)


def main(names):
    out = {}
    if os.path.exists(FLOORS_JSON):
        with open(FLOORS_JSON) as f:
            out = json.load(f)
    for n in names or list(DERIVED_BAR_CASES):
        out[n] = floor_of(n)
        with open(FLOORS_JSON, "w") as f:
            json.dump({k: out[k] for k in sorted(out)}, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:])
