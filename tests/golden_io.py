"""Reader for the key = value fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            out[k] = float(v) if any(ch in v for ch in ".eE") else int(v)
    return out
