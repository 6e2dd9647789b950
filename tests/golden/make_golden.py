"""Write the stored expected values under tests/golden/.

Calls only the input generator and the oracle:
  manifest.json        SHA-256 of every generated tensor of the two fp32
                       workloads and of the 16K bf16 workload, so that a run
                       on another host can check it draws the same inputs;
  tiny_gdn_f32.json    the oracle's o and S_final on the tiny GDN workload
                       (a regression fixture for the oracle itself).
Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    man = {}
    for name in ["tiny_gdn_f32", "small_rankL_f32", "rec16k_bf16"]:
        man[name] = workloads.manifest(workloads.generate(workloads.workload(name)))
    with open(os.path.join(HERE, "manifest.json"), "w") as f:
        json.dump(man, f, indent=1, sort_keys=True)

    w = workloads.workload("tiny_gdn_f32")
    x = workloads.generate(w)
    o, S = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], None, None, None, x["conv_w"], w.L)
    with open(os.path.join(HERE, "tiny_gdn_f32.json"), "w") as f:
        json.dump({"o": np.asarray(o).ravel().tolist(), "S_final": np.asarray(S).ravel().tolist()}, f)


if __name__ == "__main__":
    main()
