"""Readers for the text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            s = raw.strip()
            if s and not s.startswith("#"):
                yield s


def page_numbers():
    out = {}
    for s in lines("page_numbers.txt"):
        key, val = s.split()[:2]
        out[key] = float(val)
    return out
