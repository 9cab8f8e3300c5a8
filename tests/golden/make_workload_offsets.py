"""Writes tests/golden/offsets_<workload>.txt: the expert group offsets of each full-size
layer workload and of the reduced workloads of the GPU layer tests, from the oracle's routing
and permutation of the workload's seeded inputs.

The host-side replay of the grouped GEMM's index math reads them, so the CPU tests check the
launches the GPU path makes at these sizes without regenerating the inputs every run. Calls
only the oracle and the input generator. Run from the repository root:

    python tests/golden/make_workload_offsets.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import moe_inputs as mi  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402

NAMES = ("dsv3", "dsv3_ep8", "mixtral", "qwen3", "small_softmax", "small_sigmoid", "small_mxfp8", "mid_mxfp8",
         "small_mxfp4")


def main():
    for name in NAMES:
        w = mi.WORKLOADS[name]
        idx, _, _ = O.route(mi.x_np(w), mi.w_router_np(w), mi.expert_bias(w), w.k, w.score)
        off, _, _ = O.permutation(idx, w.E, w.T if w.shared_f else 0)
        path = os.path.join(ROOT, "tests", "golden", f"offsets_{name}.txt")
        with open(path, "w") as f:
            f.write(f"# expert group offsets of workload {name} (T={w.T}, d={w.d}, f={w.f}, E={w.E}, k={w.k}, "
                    f"shared f={w.shared_f}), {len(off)} entries; written by make_workload_offsets.py from the "
                    f"oracle's routing and permutation\n")
            f.write(" ".join(str(int(v)) for v in off) + "\n")
        print(name, len(off), int(np.diff(off).max()), int(np.diff(off).min()))


if __name__ == "__main__":
    main()
