"""Writes oracle_small.json: oracle outputs on a small seeded case (calls only oracle/ and synth/).

The pages print no worked attention example, so the stored values pin the oracle against
its own earlier self only (a regression guard); the mathematical pins are in test_oracle.py.
Run: python -m tests.golden.make_golden
"""
import json
import os

import numpy as np

import oracle
from synth import WORKLOADS, prefill_inputs


def compute():
    wl = WORKLOADS["prefill_f32_s128"]
    x = prefill_inputs(wl)
    o, lse = oracle.attention(x["q"], x["k"], x["v"], wl.scale, True, 0)
    ow, _ = oracle.attention(x["q"], x["k"], x["v"], wl.scale, True, 16)
    rows = [0, 1, 2, 63, 64, 127]
    return {
        "prefill_f32_s128_rows_0_1_2_63_64_127_dims_0_to_7": o[0, rows, 0, :8].tolist(),
        "prefill_f32_s128_lse_rows_0_1_2_63_64_127": lse[0, 0, rows].tolist(),
        "prefill_f32_s128_window16_rows_0_1_2_63_64_127_dims_0_to_7": ow[0, rows, 0, :8].tolist(),
        "quantize_int8_first_row_of_q": [int(c) for c in oracle.quantize_int8(x["q"][0, 0, 0][None])[0][0]],
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(out, "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", out)
