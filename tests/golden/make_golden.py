"""Writes tests/golden/tiny_rows.json from the 50-digit brute force in oracle/.

Run from the repository root:  python tests/golden/make_golden.py
The inputs are stored as exact float64 values; the expected KL is the brute
force's 50-digit decimal result, the argmaxes come from its explicit scan.
"""
import json
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle.bruteforce import bruteforce  # noqa: E402

CASES = [
    dict(name="page_example_three_named_tokens",
         cite="Qwen3.6 27B Quantization Benchmark (huy.rocks), section 'Understand KLD and "
              "Same Top P': base 90% homework / 5% bike / 1% banana, a poor quant 50% / 30% / 20%; "
              "both still pick 'homework'. Reading: only the three named tokens, logits = log of "
              "the quoted confidences, renormalised by the softmax (the base's 96% need not sum to 1).",
         base=[math.log(0.90), math.log(0.05), math.log(0.01)],
         quant=[math.log(0.50), math.log(0.30), math.log(0.20)]),
    dict(name="constructed_top_token_changes",
         cite="Constructed case (not on the pages): the first case's base row against a quant row "
              "whose two leading confidences are swapped (30% / 50% / 20%), so the top tokens differ "
              "and the match is 0.",
         base=[math.log(0.90), math.log(0.05), math.log(0.01)],
         quant=[math.log(0.30), math.log(0.50), math.log(0.20)]),
    dict(name="identical_rows", cite="KL(p||p) = 0",
         base=[1.5, -2.0, 0.25, 3.0], quant=[1.5, -2.0, 0.25, 3.0]),
    dict(name="two_tokens", cite="V = 2 closed form",
         base=[0.75, -0.5], quant=[-0.25, 0.5]),
    dict(name="base_tie_lowest_index", cite="argmax tie broken toward the lowest index",
         base=[2.0, 7.0, 7.0, -1.0, 7.0], quant=[2.0, 6.5, 7.0, -1.0, 7.0]),
    dict(name="large_offsets", cite="shift-safe evaluation",
         base=[80.0, 79.0, -30.0, 0.0, 12.5], quant=[-40.0, 79.5, 81.0, 0.0, 12.0]),
]


def main():
    out = []
    for c in CASES:
        kl, ib, iq = bruteforce(c["base"], c["quant"])
        out.append(dict(name=c["name"], cite=c["cite"],
                        base=[float(v) for v in c["base"]], quant=[float(v) for v in c["quant"]],
                        kl=format(kl, "f") if abs(kl) > 0 else "0", argmax_base=ib, argmax_quant=iq,
                        match=int(ib == iq)))
    doc = dict(generator="tests/golden/make_golden.py (oracle.bruteforce, 50 digits)", cases=out)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_rows.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(f"wrote {path}")


if __name__ == "__main__":
    main()
