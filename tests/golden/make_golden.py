"""Writes the stored expected values under tests/golden/.

Calls only the fp64 oracle (oracle/decode_ref.py) on the seeded inputs of
workloads/; no value here comes from the HIP library.  Run from the repo root:

    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.decode_ref import gqa_decode_ref  # noqa: E402
from workloads import make_inputs, make_case  # noqa: E402


def write(name, out, note):
    path = os.path.join(HERE, name)
    S, T, H, D = out.shape
    with open(path, "w") as f:
        f.write(f"# {note}\n# shape {S} {T} {H} {D}; one output row (s, t, h) per line, %.17g\n")
        for s in range(S):
            for t in range(T):
                for h in range(H):
                    f.write(" ".join("%.17g" % x for x in out[s, t, h]) + "\n")


def main():
    inp = make_inputs("tiny_f16")
    write("tiny_f16.txt", gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale),
          "oracle output of the tiny_f16 workload (1 seq, 8/2 heads, hd 64, 256 cells, scale 1/8)")
    inp = make_case(2, 3, 4, 1, 64, 70, [70, 2], kv="i8", budget=24, seed=21, scale=1.0 / 8.0)
    write("small_i8_ids_causal.txt",
          gqa_decode_ref(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.k_scales, inp.v_scales, inp.ids),
          "oracle output of make_case(2, 3, 4, 1, 64, 70, [70, 2], kv='i8', budget=24, seed=21, scale=1/8)")


if __name__ == "__main__":
    main()
