"""Write tests/golden/oracle_regression.json: outputs of the fp64 oracle on tiny
seeded cases of the three paths (regression guard for the oracle itself; the
oracle's correctness is pinned by tests/test_oracle_pins.py).

Calls only oracle/ and the seeded generators. Run from the repository root:
    python tests/golden/make_oracle_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as wl  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")
CASES = {
    "dense_gdn": (wl.custom(wl.WORKLOADS[1], B=1, H=2, steps=3), "dense"),
    "dense_kda": (wl.custom(wl.WORKLOADS[3], B=1, H=2, steps=3, qkv="f32"), "dense"),
    "window_gdn_w4": (wl.custom(wl.WORKLOADS[4], B=1, H=2, W=4, steps=6, qkv="f32"), "window"),
    "log_gdn_m4": (wl.custom(wl.WORKLOADS[5], B=1, H=2, M=4, steps=6, qkv="f32"), "log"),
}


def run(w, path):
    S0 = wl.initial_state(w).astype(np.float64)
    ys = []
    if path == "dense":
        S = S0.copy()
        for t in range(w.steps):
            x = wl.step_inputs(w, t)
            ys.append(oracle.dense_step(S, x["q"], x["k"], x["v"], x["gate"], x["beta"]))
        final = S
    elif path == "window":
        Z, a = oracle.q8_quantize(S0)
        st = oracle.WindowState(Z, a, w.W, w.per_key_gate)
        for t in range(w.steps):
            x = wl.step_inputs(w, t)
            ys.append(st.step(x["q"], x["k"], x["v"], x["gate"], x["beta"]))
        final = oracle.dequant(st.Z, st.a)
    else:
        st = oracle.LogState(S0, w.M - 1, w.per_key_gate)
        for t in range(w.steps):
            x = wl.step_inputs(w, t)
            ys.append(st.step(x["q"], x["k"], x["v"], x["gate"], x["beta"]))
        final = st.logical_state()
    return np.array(ys), final


def main():
    out = {"_about": "fp64 oracle outputs on tiny seeded cases; written by make_oracle_golden.py"}
    for name, (w, path) in CASES.items():
        ys, final = run(w, path)
        out[name] = {"y_first_step_head0": [float(v) for v in ys[0, 0, :8]],
                     "y_last_step_head1": [float(v) for v in ys[-1, 1, :8]],
                     "y_sum": float(ys.sum()), "y_abs_sum": float(np.abs(ys).sum()),
                     "final_state_sum": float(final.sum()), "final_state_abs_sum": float(np.abs(final).sum())}
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
