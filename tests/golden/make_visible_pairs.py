"""Write visible_pairs.json from the closed form of the pages.

"Fast Diffusion Attention", section "The right yardstick": a sample of 2n
tokens with block size b has n^2 + n*b visible pairs (per head) when b
divides n.  With a shorter last block the diagonal squares are
size_i^2, so the count is n^2 + sum_i size_i^2.  This script uses only
that arithmetic and the workload table.
"""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from workloads import WORKLOADS  # noqa: E402


def closed_form(n, b):
    if n % b == 0:
        return n * n + n * b
    full, rest = divmod(n, b)
    return n * n + full * b * b + rest * rest


def main():
    rows = {name: {"n": w.n, "b": w.b, "pairs": closed_form(w.n, w.b)} for name, w in WORKLOADS.items()}
    out = {"source": "Fast Diffusion Attention, section 'The right yardstick' (n^2 + n*b); "
                     "n^2 + sum of squared block sizes when b does not divide n",
           "workloads": rows}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "visible_pairs.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
