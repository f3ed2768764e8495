"""Reader for the small text fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(tok: str) -> float:
    return float(int(tok, 16)) if tok.lower().startswith("0x") else float(tok)


def load(name: str) -> dict:
    blocks, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or (line.startswith("#") and not line.startswith("##")):
                continue
            if line.startswith("##"):
                cur = line[2:].strip()
                blocks[cur] = []
                continue
            blocks[cur].append([_num(t) for t in line.split()])
    return {k: np.array(v, dtype=np.float64) for k, v in blocks.items()}
