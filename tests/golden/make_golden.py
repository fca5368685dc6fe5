"""Writes tests/golden/tiny_oracle_samples.json: sampled outputs of the fp64
oracle (oracle/) on the seeded tiny workload (1 sequence x 64 tokens,
H_k = H_v = 2, d_k = d_v = 32, fp32, zero initial state and window, seed 0).

The pages print no worked example of the layer core, so no stored value here
comes from them: these values are the oracle's, stored so that a later change
to the oracle's arithmetic shows up as a change of stored numbers (and the
GPU path can be checked against them without running the oracle).  Nothing
from the GPU path is read.  Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import gdn_workloads as wk  # noqa: E402
import oracle  # noqa: E402

TOKENS = (0, 1, 2, 15, 31, 32, 63)
HEADS = (0, 1)


def samples():
    wl = wk.TINY
    inp = wk.make_sequence_inputs(wl)
    dm = oracle.dims_of(wl)
    o, win, S = oracle.layer(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"], inp["b"],
                             inp["cu_seqlens"], inp["window0"], inp["S0"])
    out = {"workload": "tiny: 1 x 64 tokens, H_k=H_v=2, d_k=d_v=32, conv width 4, fp32, S0=0, seed 0",
           "source": "oracle/ (fp64), written by tests/golden/make_golden.py; the pages print no worked example",
           "o": {f"t{t}_h{h}": [float(v) for v in o[t, h, :8]] for t in TOKENS for h in HEADS},
           "S_final": {f"h{h}_row{r}": [float(v) for v in S[0, h, r, :8]] for h in HEADS for r in (0, 17, 31)},
           "window_final_row2": [float(v) for v in win[0, 2, :8]]}
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle_samples.json")
    with open(path, "w") as f:
        json.dump(samples(), f, indent=1)
        f.write("\n")
    print("wrote", path)
