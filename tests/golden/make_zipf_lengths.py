"""Write zipf_lengths_workload4.json: the sequence lengths of the Zipf batch
(64 sequences, 65,536 tokens, exponent 1), computed here in exact rational
arithmetic so that the floating-point generator in workloads.py is pinned by
an independent computation.

Only the rank permutation is taken from numpy (PCG64, seed 1004, the
workload's length seed); everything else is fractions.Fraction: every
sequence keeps one token and the remaining tokens are apportioned in
proportion to 1/rank by the largest-remainder rule (ties in index order).

Usage: python tests/golden/make_zipf_lengths.py
"""

import json
import os
from fractions import Fraction

import numpy as np

TOTAL, SEQS, SEED = 65536, 64, 1004


def main() -> None:
    rank = [int(r) + 1 for r in np.random.default_rng(SEED).permutation(SEQS)]
    spare = TOTAL - SEQS
    harmonic = sum(Fraction(1, r) for r in rank)
    quota = [Fraction(spare, r) / harmonic for r in rank]
    base = [q.numerator // q.denominator for q in quota]
    left = spare - sum(base)
    order = sorted(range(SEQS), key=lambda i: (-(quota[i] - base[i]), i))
    for i in order[:left]:
        base[i] += 1
    lengths = [b + 1 for b in base]
    assert sum(lengths) == TOTAL and min(lengths) >= 1
    doc = {
        "source": "So you wanna CUDA Graph, section 'Hello World' (Zipf token split), with exponent 1 and "
                  "65,536 tokens over 64 sequences as in the Zipf decoder batch",
        "seed": SEED,
        "ranks": rank,
        "lengths": lengths,
        "note": "exact rational largest-remainder apportionment of the tokens beyond one per sequence, "
                "weights 1/rank; written by tests/golden/make_zipf_lengths.py",
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_lengths_workload4.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(path)


if __name__ == "__main__":
    main()
