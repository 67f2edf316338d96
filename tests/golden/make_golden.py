"""Writes tests/golden/tiny_fp32_oracle.json: the oracle's output on the tiny
fp32 workload (B=1, T=16, H=2, dk=dv=4, short-conv kernel 2, seed 0).

The public pages print no KDA worked example, so this fixture is not a page
value: it is a regression record produced by the oracle alone (this script
imports nothing but the oracle and the seeded input generator).
Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import kda_inputs as ki  # noqa: E402
import oracle  # noqa: E402

r = oracle.get().prefill(ki.config_prefill(0))
out = dict(
    workload="tiny fp32: B=1 T=16 H=2 dk=dv=4 K=2, zero state, seed 0, SiLU conv, eps 1e-6, scale 1",
    y=r["y"].tolist(), final_state=r["final_state"].tolist(), conv_cache=r["conv_cache"].tolist(),
)
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32_oracle.json"), "w") as f:
    json.dump(out, f, indent=1)
print("wrote tiny_fp32_oracle.json")
