"""Digests of the device path's results on fixed seeded inputs, for the
bitwise-repeatability test (repeat runs in one process and in a fresh one).

Run as a script it prints the digests as one JSON line.  The inputs are the
conv-fed 27-node workload at 8 requests (two steps: the previous step's
accepted path is committed and its conv history published inside the fused
calls and inside the one-launch layer step) and the 27-node workload at 8
requests through the separate verify and commit calls.
"""
from __future__ import annotations

import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def _digest(res):
    import numpy as np
    h = hashlib.sha256()
    for key in sorted(res):
        v = res[key]
        if isinstance(v, np.ndarray):
            h.update(key.encode())
            h.update(np.ascontiguousarray(v).tobytes())
        elif isinstance(v, (int, float)):
            h.update(f"{key}={v}".encode())
    return h.hexdigest()


def digests() -> dict:
    import gdn_inputs as gi
    from harness import run_gpu, run_gpu_layer, run_gpu_two_steps, two_step_case

    c1, c2 = two_step_case(gi.CONFIGS[4], seed=77, B=8, extra_slots=1)
    case = gi.make_case(gi.CONFIGS[3], seed=78, B=8)
    return {
        "fused_conv4": _digest(run_gpu_two_steps(c1, c2)),
        "layer_conv4": _digest(run_gpu_layer(c1, c2, prepare=True)),
        "separate_tree27": _digest(run_gpu(case)),
    }


if __name__ == "__main__":
    print(json.dumps(digests()), flush=True)
