"""The stored oracle samples of tests/golden/ (tiny workload): the oracle
still reproduces them (a change to its arithmetic changes stored numbers),
and the GPU path matches them within the tiny workload's 1e-4."""
import json
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "tiny_oracle_samples.json")


def _stored():
    with open(GOLDEN) as f:
        return json.load(f)


def test_oracle_reproduces_stored_samples(ora):
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "golden", "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    now, stored = mg.samples(), _stored()
    for part in ("o", "S_final"):
        assert now[part].keys() == stored[part].keys()
        for k in stored[part]:
            np.testing.assert_allclose(now[part][k], stored[part][k], rtol=1e-12, atol=1e-15)
    assert now["window_final_row2"] == stored["window_final_row2"]


@pytest.mark.gpu
def test_gpu_tiny_matches_stored_samples():
    import gdn_workloads as wk
    from gpu_util import host, run_seq
    stored = _stored()
    wl = wk.TINY
    inp = wk.make_sequence_inputs(wl)
    o, conv, state = run_seq(wl, inp)
    o, S, win = host(o), host(state.buf), host(conv.buf)
    for h in (0, 1):
        ref = {k: np.asarray(v) for k, v in stored["o"].items() if k.endswith(f"_h{h}")}
        scale = max(np.abs(v).max() for v in ref.values())
        for k, v in ref.items():
            t = int(k.split("_")[0][1:])
            assert np.abs(o[t, h, :8] - v).max() <= 1e-4 * scale, k
        refS = {k: np.asarray(v) for k, v in stored["S_final"].items() if k.startswith(f"h{h}_")}
        scaleS = max(np.abs(v).max() for v in refS.values())
        for k, v in refS.items():
            r = int(k.split("row")[1])
            assert np.abs(S[0, h, r, :8] - v).max() <= 1e-4 * scaleS, k
    np.testing.assert_array_equal(win[0, 2, :8], np.asarray(stored["window_final_row2"], np.float32))
