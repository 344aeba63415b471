"""Loaders for the hand-derived fixtures under tests/golden (test-only)."""

import os

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def limiter_goldens():
    """(name, counts, expected lengths) from golden/limiter_cases.txt: the
    hand-derived outcomes of the K3 page's length limit (section "canonical
    code assignment and Kraft check") under readings C2/C10 and the repay."""
    out = []
    for line in open(os.path.join(GOLD, "limiter_cases.txt")):
        if line.strip() and not line.startswith("#"):
            name, counts, lens = (f.split() for f in line.split("|"))
            out.append((name[0], [int(c) for c in counts], [int(l) for l in lens]))
    return out
