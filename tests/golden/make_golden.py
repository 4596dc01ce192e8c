"""Writes tests/golden/tiny_oracle.json and tests/golden/tiny_variants.json
from the fp64 oracle alone.

Inputs come from the seeded generator (`synthetic.make("tiny")`: T=8, H=256,
E=16, k=2, I=128); every stored value is computed by `oracle/` with the exact
(math.fsum) router.  The definition followed is the sparse-MoE block of the
grouped_mm path: router -> top-k (ties to the lower index) -> renormalised
softmax weights -> histogram / exclusive scan / stable permutation -> SwiGLU
experts -> per-token weighted sum [unsloth commit 80aaf1121b page, third and
last paragraphs; unsloth commit 4f2bfe7f69 page, second paragraph].

tiny_variants.json holds the same block's variants: top-k weights without
renormalisation, rank-16 LoRA adapters (synthetic.lora_adapters) on the
experts [unsloth commit 4f2bfe7f69 page, bench table], and the pre-block
residual add + RMSNorm on synthetic.prenorm_inputs(8, 256) [unsloth commit
a1bc5cbd page, first paragraph].

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

    # variants of the same block
    out_s, rs = O.forward_per_token(inp, exact_router=True, renorm=False)
    lora = O.LoRA(**S.lora_adapters(inp.E, inp.H, inp.I))
    out_l, _ = O.forward_per_token(inp, exact_router=True, lora=lora)
    p = S.prenorm_inputs(8, 256)
    r_bits, x64 = O.residual_rmsnorm(p["residual"], p["delta"], p["gamma"], p["eps"])
    doc = {
        "about": "tiny block variants and the pre-block step, from the fp64 oracle alone",
        "softmax_weights": [[float(v) for v in row] for row in rs["w"]],
        "softmax_out_row_sums": [float(v) for v in out_s.sum(axis=1)],
        "lora_out_rms": O.rms(out_l),
        "lora_out_first_row_first_16": [float(v) for v in out_l[0, :16]],
        "lora_out_row_sums": [float(v) for v in out_l.sum(axis=1)],
        "prenorm_r_bits_row0_first_16": [int(v) for v in r_bits[0, :16]],
        "prenorm_x_bits_row0_first_16": [int(v) for v in O.f64_to_bf16_rne(x64)[0, :16]],
        "prenorm_x_row_sums": [float(v) for v in x64.sum(axis=1)],
        "prenorm_x_row_sumsq": [float(v) for v in (x64 * x64).sum(axis=1)],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_variants.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
