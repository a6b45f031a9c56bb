"""Writes the stored expected values under tests/golden/ from the oracle only.

The pages print no worked numeric example of block scores, selections or
attention outputs, so every fixture here is produced by this script, which
calls nothing but `oracle` and the seeded input recipe in `workloads`.

  decode_1x4k_int.txt : the 1-stream, 4096-slot decode workload with integer
      indexer inputs (integers -8..8 stored as f32), query at position 4095.
      All scores are integers, exact in f32 and fp64, so the block maxima and
      the top-16 selection (local block forced, ties to the lower block id)
      are unique and must be reproduced bit for bit by any correct path.

Run:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    wl = W.CONFIGS["decode_1x4k_int"]
    ck = W.caches(wl)
    qs = W.queries(wl)
    bs, sel, n_sel = oracle.msa_select(ck["idx_k"], qs["stream"], qs["pos"], qs["idx_q"])
    lines = ["# decode_1x4k_int: stream 0, position 4095, 32 blocks of 128; seed 0",
             "# produced by tests/golden/make_golden.py (oracle only)",
             "# per group: 'bs g' then 32 integer block maxima; 'sel g' then the 16 ids"]
    for g in range(W.N_GROUP):
        assert np.all(bs[0, g] == np.round(bs[0, g]))
        lines.append(f"bs {g} " + " ".join(str(int(x)) for x in bs[0, g]))
        lines.append(f"sel {g} " + " ".join(str(int(x)) for x in sel[0, g]))
    with open(os.path.join(HERE, "decode_1x4k_int.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
