"""Write tests/golden/tiny_oracle.json from the CPU oracle.

The fixture records the oracle's results for the tiny verify workload
(M=8, K=512, N=1024, bf16 activations, seed 1; then a verify block of T=8
with 7 drafts whose first 3 are forced to the oracle's argmax). It calls
only ``gen`` (inputs) and ``oracle`` (results). ``tests/test_golden.py``
recomputes it to catch any drift in either.

Run from the repository root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import gen  # noqa: E402
from oracle import qgemm_ref, verify_ref  # noqa: E402

SAMPLE_COLS = [0, 1, 2, 15, 16, 63, 64, 255, 256, 511, 512, 767, 1000, 1022, 1023]


def build():
    c = gen.make_config("tiny")
    y = qgemm_ref(c["x"], c["act"], c["wq"], c["scales"], c["biases"])
    a0, _ = verify_ref(y.astype(np.float32), None if c["T"] == 1 else
                       np.zeros((1, c["T"] - 1), np.int32), c["B"], c["T"])
    draft = gen.make_drafts(a0, c["B"], c["T"], c["N"], c["seed"], force_first=3)
    a, acc = verify_ref(y.astype(np.float32), draft, c["B"], c["T"])
    return dict(
        workload="tiny: M=8 K=512 N=1024 bf16 seed 1, verify T=8 (first 3 drafts forced)",
        source="CPU oracle (oracle/vqv_ref.py) on gen.make_config('tiny')",
        sample_cols=SAMPLE_COLS,
        y_sample=[[repr(float(v)) for v in y[m, SAMPLE_COLS]] for m in range(c["M"])],
        y_row_sums=[repr(float(v)) for v in y.sum(axis=1)],
        draft=draft.tolist(),
        argmax=a.tolist(),
        accept_len=acc.tolist(),
    )


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(out, "w") as f:
        json.dump(build(), f, indent=1)
        f.write("\n")
    print("wrote", out)
