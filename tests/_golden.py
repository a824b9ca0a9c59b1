"""Reader for the plain-text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read(name):
    """Return the fixture's "key = values" lines as an ordered list of (key, [tokens])."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split("=", 1)
            out.append((key.strip(), val.split()))
    return out


def table(name):
    return {k: v for k, v in read(name)}


def floats(tokens):
    return [float(t) for t in tokens]


def hexbytes(tokens):
    return [int(t, 16) for t in tokens]
