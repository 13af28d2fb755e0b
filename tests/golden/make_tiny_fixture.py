"""Write the tiny workload's expected outputs from the CPU oracle.

Inputs: the "tiny" workload of ``kda_synth`` (1 stream, 1 layer, 4 heads,
dk = dv = 16, 16 sequential steps, seed 0), drawn on the CPU.  Expected
values: ``oracle`` only, in double precision, free-running over the 16 steps
from the BF16-rounded initial state.

Output: ``tiny_oracle.txt`` next to this script, one value per line with 17
significant digits: the 16 x 4 x 16 outputs (step-major), then the final
4 x 16 x 16 state.

    python tests/golden/make_tiny_fixture.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import kda_synth  # noqa: E402
import oracle  # noqa: E402

OUT = os.path.join(HERE, "tiny_oracle.txt")


def tiny_inputs():
    """CPU-drawn inputs of the tiny workload, as float64 numpy arrays."""
    wl = kda_synth.WORKLOADS["tiny"]
    li = kda_synth.layer_inputs(wl, 0, "cpu", "f32")
    steps = [kda_synth.step_inputs(wl, 0, t, "cpu") for t in range(wl.steps)]
    to = lambda t: t.double().numpy()  # noqa: E731
    return wl, {k: to(v) for k, v in li.items()}, [{k: to(v) for k, v in s.items()} for s in steps]


def run_oracle():
    wl, li, steps = tiny_inputs()
    orc = oracle.get()
    S, cs = li["state"], li["conv_state"]
    outs = []
    for s in steps:
        S, cs, o = orc.decode_step(S, s["x"], li["conv_w"], cs, s["alpha"], s["beta"], wl.scale)
        outs.append(o)
    return np.stack(outs), S


def main():
    o, S = run_oracle()
    with open(OUT, "w") as f:
        f.write("# tiny workload, oracle outputs [16][4][16] then final state [4][16][16]\n")
        for v in np.concatenate([o.ravel(), S.ravel()]):
            f.write(f"{v:.17g}\n")
    print(f"wrote {OUT}: {o.size} outputs + {S.size} state values")


if __name__ == "__main__":
    main()
