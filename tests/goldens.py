"""Readers of the hand-worked fixtures in tests/golden/."""
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def to_bf16_bits(values) -> np.ndarray:
    t = torch.tensor([float(v) for v in values], dtype=torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def read_groups(name: str, group: int):
    """[(case, bf16 bits [group], scale byte, payload bytes [group // 2])]."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            case, vals, sc, pay = [p.strip() for p in line.split("|")]
            v = vals.split()
            v = v + ["0"] * (group - len(v))
            p = [int(x, 16) for x in pay.split()]
            p = p + [0] * (group // 2 - len(p))
            out.append((case, to_bf16_bits(v), int(sc, 16), np.array(p, dtype=np.uint8)))
    return out
