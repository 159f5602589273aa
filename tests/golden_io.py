"""Reader for the small text fixtures under tests/golden/.

Each fixture is ``key value value ...`` lines; ``#`` lines hold the citation.
Repeated keys are returned as a list of rows.
"""
import os
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(tok):
    if tok == "-":
        return None
    if "/" in tok:
        return Fraction(tok)
    try:
        return int(tok)
    except ValueError:
        return float(tok)


def read(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            vals = [_num(v) for v in vals]
            val = vals[0] if len(vals) == 1 else vals
            if key in out:
                if not isinstance(out[key], list) or not out[key] or not isinstance(out[key][0], list):
                    out[key] = [out[key]]
                out[key].append(val)
            else:
                out[key] = val
    return out
