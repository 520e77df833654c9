"""Readers for the hand-transcribed fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def worked_example():
    ex = {"q": {}, "w": {}, "k": {}, "h": {}, "I": {}, "select": None}
    for tok in _lines("worked_example_t10.txt"):
        tag, rest = tok[0], tok[1:]
        if tag == "select":
            ex["select"] = [int(x) for x in rest]
        elif tag in ("q", "k"):
            ex[tag][int(rest[0])] = [float(x) for x in rest[1:]]
        elif tag == "h":
            ex["h"][int(rest[0])] = [float(x) for x in rest[1:]]
        else:
            ex[tag][int(rest[0])] = float(rest[1])
    return ex


def counts():
    return [tuple(int(x) for x in tok) for tok in _lines("counts.txt")]
