"""Write oracle_snapshot_tiny_f32.json from the fp64 oracle alone.

    python tests/golden/make_snapshot.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from long_context_decode_fd_amd import workloads as wl  # noqa: E402
from oracle import oracle  # noqa: E402

NAME = "tiny_mha_f32_b1_h8_d64_l1024"


def main():
    w = wl.WORKLOADS[NAME]
    q, k, v, seqlens = wl.gen_all(w)
    out, lse = oracle.decode(q, k, v, seqlens, w.scale)
    doc = {"workload": NAME, "scale": w.scale,
           "out": [repr(float(x)) for x in out.ravel()],
           "lse": [repr(float(x)) for x in lse.ravel()]}
    with open(os.path.join(HERE, "oracle_snapshot_tiny_f32.json"), "w") as f:
        json.dump(doc, f, indent=0)


if __name__ == "__main__":
    main()
