#!/usr/bin/env python3
"""Write tests/golden/certified_subseeds.json: for every full-vocabulary parity case, the
per-request block-logit sub-seeds with which the oracle measures every decision margin at
or above the policy's threshold (1e-3).  Only the oracle and the seeded input generator
run here; the GPU tests re-measure every margin with the oracle before comparing.

    python tests/golden/make_certified_subseeds.py [key ...]
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import parity_helpers as ph  # noqa: E402


def main(keys):
    out = {}
    if os.path.exists(ph.GOLDEN_SUBSEEDS):
        with open(ph.GOLDEN_SUBSEEDS) as fh:
            out = json.load(fh)
    for key in keys or list(ph.FULL_CASES):
        t0 = time.time()
        inst, _ = ph.certify_case(key)
        out[key] = [int(x) for x in inst.subseed]
        print("%-28s %5.1f s  redrawn %d of %d" % (
            key, time.time() - t0, sum(int(a) != i for i, a in enumerate(inst.subseed)), inst.R),
            flush=True)
        with open(ph.GOLDEN_SUBSEEDS, "w") as fh:
            json.dump(out, fh, indent=0, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:])
