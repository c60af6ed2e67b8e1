"""Readers for the hand-written fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_visibility_fixture(name="grouped_visibility_tiny.txt"):
    groups, positions, pairs, rows = None, None, None, []
    in_matrix = False
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if in_matrix:
                rows.append([int(c) for c in line])
            elif line.startswith("groups:"):
                groups = []
                for tok in line.split(":", 1)[1].split():
                    p, rs = tok.split(":")
                    groups.append((int(p), [int(r) for r in rs.split(",")]))
            elif line.startswith("positions:"):
                positions = np.array([int(x) for x in line.split(":", 1)[1].split()])
            elif line.startswith("pairs:"):
                pairs = tuple(int(x) for x in line.split(":", 1)[1].split())
            elif line.startswith("visible:"):
                in_matrix = True
    return groups, positions, pairs, np.array(rows, dtype=bool)
