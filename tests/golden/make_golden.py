"""Writes tests/golden/tiny_oracle.json from the fp64 oracle alone.

Inputs come from the seeded generator (`synthetic.make("tiny")`: T=8, H=256,
E=16, k=2, I=128); every stored value is computed by `oracle/` with the exact
(math.fsum) router.  The definition followed is the sparse-MoE block of the
grouped_mm path: router -> top-k (ties to the lower index) -> renormalised
softmax weights -> histogram / exclusive scan / stable permutation -> SwiGLU
experts -> per-token weighted sum [unsloth commit 80aaf1121b page, third and
last paragraphs; unsloth commit 4f2bfe7f69 page, second paragraph].

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synthetic as S  # noqa: E402


def main():
    inp = S.make("tiny")
    out, r = O.forward_per_token(inp, exact_router=True)
    counts, offsets, perm, pos = O.permute(r["ids"], inp.E)
    doc = {
        "about": __doc__.strip().splitlines()[0],
        "workload": {"name": "tiny", "T": inp.T, "H": inp.H, "E": inp.E, "k": inp.k, "I": inp.I},
        "ids": r["ids"].tolist(),
        "weights": [[float(v) for v in row] for row in r["w"]],
        "counts": counts.tolist(),
        "offsets": offsets.tolist(),
        "perm": perm.tolist(),
        "out_rms": O.rms(out),
        "out_first_row_first_16": [float(v) for v in out[0, :16]],
        "out_row_sums": [float(v) for v in out.sum(axis=1)],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
