"""Writes tests/golden/*.json. Calls only the seeded input generator and the
CPU oracle (oracle/); nothing here touches the HIP path.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from software_pipelining_fmha_amd import inputs  # noqa: E402


def main():
    digests = {}
    for idx in (0, 1):
        w = inputs.WORKLOADS[idx]
        q, k, v, scale = inputs.workload_inputs(idx)
        digests[w.name] = {"q": inputs.sha256(q), "k": inputs.sha256(k),
                           "v": inputs.sha256(v), "scale": float(scale)}
    with open(os.path.join(HERE, "inputs_sha256.json"), "w") as f:
        json.dump(digests, f, indent=1, sort_keys=True)

    # the tiny workload's oracle output, as a regression fixture
    q, k, v, scale = inputs.workload_inputs(0)
    out = {}
    for causal in (False, True):
        o, lse = oracle.fmha_all(q, k, v, causal=causal, scale=scale)
        rows = [0, 1, 63, 64, 127]
        out["causal" if causal else "full"] = {
            "lse": [float.hex(float(x)) for x in lse[0, 0]],
            "o_rows": {str(i): [float.hex(float(x)) for x in o[0, 0, i]] for i in rows},
        }
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(out, f, indent=0, sort_keys=True)


if __name__ == "__main__":
    main()
