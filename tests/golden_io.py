"""Reader for the small text fixtures under tests/golden/ ("key: v1 v2 ..." lines, '#' comments)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = val.split()
    return out


def floats(vals):
    return [float(v) for v in vals]


def ints(vals):
    return [int(v) for v in vals]
