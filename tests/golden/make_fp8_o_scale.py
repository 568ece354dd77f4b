"""Writes fp8_o_scale.json: the output quantisation scale of the dense FP8
workload, o_scale = amax|O| / 448 with O from the f64 oracle over the whole
workload (B=8, H=32, Hkv=8, S=4096, D=128, causal).

Calls only the oracle (and the seeded input generator).  Run from the repo root:
    python tests/golden/make_fp8_o_scale.py
"""

import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from oracle.attention import default_workers  # noqa: E402
from variable_length_gqa_amd import workloads as W  # noqa: E402


def input_digest(d) -> str:
    h = hashlib.sha256()
    for t in (d.q, d.k, d.v):
        h.update(t.contiguous().numpy().tobytes())
    return h.hexdigest()


def main():
    d = W.workload("dense_fp8")
    s = d.scales
    t0 = time.time()
    _, _, O = oracle.flash_attention_fwd_fp8(d.q, d.k, d.v, d.num_heads, d.num_kv_heads,
                                             d.causal, s["q_scale"], s["k_scale"], s["v_scale"],
                                             1.0, workers=default_workers())
    amax = float(np.abs(O).max())
    out = {
        "workload": "dense_fp8 (B=8, H=32, Hkv=8, S=4096, D=128, causal, seed 1004)",
        "how": "amax|O_oracle| / 448 over every output element, f64 oracle",
        "o_scale": amax / 448.0,
        "amax_O": amax,
        "q_scale": s["q_scale"], "k_scale": s["k_scale"], "v_scale": s["v_scale"],
        "input_sha256": input_digest(d),
        "oracle_seconds": round(time.time() - t0, 1),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_o_scale.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=2)
    print(json.dumps(out, indent=2))


if __name__ == "__main__":
    main()
