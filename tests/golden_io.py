"""Readers for the small text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def num(tok: str) -> float:
    t = tok.lower()
    if t in ("nan", "inf", "-inf"):
        return float(t)
    if "x" in t:
        return float.fromhex(tok)
    return float(tok)


def read_points(name):
    """Lines of '<code hex> <value> <comment...>' -> list of (code, value)."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            out.append((int(parts[0], 16), num(parts[1])))
    return out


def read_blocks(name):
    """'block <name>' records with z / q / optional d lines -> dict name -> record."""
    blocks = {}
    cur = None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "block":
                cur = {}
                blocks[vals[0]] = cur
            elif key == "z":
                cur["z"] = [num(v) for v in vals]
            elif key == "q":
                cur["q"] = [int(v) for v in vals]
            elif key == "d":
                cur["d"] = num(vals[0])
    return blocks
