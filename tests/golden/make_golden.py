"""Write tests/golden/tiny_oracle.json from the oracle (and only the oracle).

Run from the repository root:  python tests/golden/make_golden.py
The stored values pin the oracle against accidental change; the inputs come
from the seeded generators on the CPU (tiny workload, seed 0).
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import accept_greedy, accept_stochastic, verify_attention  # noqa: E402
from workloads import generate, preset  # noqa: E402
from tests.oracle_io import accept_args, attention_args  # noqa: E402

SAMPLE_IDX = [(0, 0, 0), (3, 7, 63), (4, 2, 31), (7, 5, 5), (5, 6, 40), (2, 1, 17), (6, 3, 0), (1, 4, 62)]


def build():
    inp = generate(preset("tiny"))
    out = verify_attention(**attention_args(inp))
    a = accept_args(inp)
    al_s, tok_s = accept_stochastic(**a)
    al_g, tok_g = accept_greedy(a["target_logits"], a["draft_tokens"], a["q_start"])
    return {
        "workload": inp.spec.name,
        "seed": 0,
        "attention": {
            "shape": list(out.shape),
            "sum": float(out.sum()),
            "sum_sq": float((out * out).sum()),
            "samples": [[list(ix), float(out[ix])] for ix in SAMPLE_IDX],
        },
        "stochastic": {"accept_len": al_s.tolist(), "out_tokens": tok_s.tolist()},
        "greedy": {"accept_len": al_g.tolist(), "out_tokens": tok_g.tolist()},
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(build(), f, indent=1)
    print("wrote", path)
