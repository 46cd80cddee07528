"""Reader for tests/golden/q4k_blocks.txt and exact closed-form weights."""
from __future__ import annotations

import os
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "q4k_blocks.txt")

Q_RULES = {
    "twice_subblock_plus_parity": lambda t: 2 * (t // 32) + (t % 2),
    "all_one": lambda t: 1,
    "all_three": lambda t: 3,
    "all_zero": lambda t: 0,
    "t_mod_16": lambda t: t % 16,
}


def half_bits_to_fraction(bits: int) -> Fraction:
    """Exact value of a binary16 pattern (finite only), via numpy's decoder."""
    v = np.array([bits], np.uint16).view(np.float16)[0]
    assert np.isfinite(v)
    return Fraction(float(v))  # float16 -> double is exact


@dataclass
class GoldenBlock:
    name: str
    dbits: int
    mbits: int
    sc: list
    m: list
    q: list
    raw: np.ndarray  # 144 uint8

    def weights_exact(self):
        """Exact rational weights w[t] = d*sc_j*q[t] - dmin*m_j from the fields."""
        d = half_bits_to_fraction(self.dbits)
        dmin = half_bits_to_fraction(self.mbits)
        return [d * self.sc[t // 32] * self.q[t] - dmin * self.m[t // 32] for t in range(256)]

    def weights_f32(self) -> np.ndarray:
        return np.array([np.float32(float(v)) for v in self.weights_exact()], np.float32)


def load_golden_blocks():
    blocks = []
    cur = None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "block":
                cur = {"name": rest, "hex": ""}
            elif key == "d":
                parts = rest.split()
                cur["d"] = int(parts[0], 16)
                assert parts[1] == "dmin"
                cur["dmin"] = int(parts[2], 16)
            elif key == "sc":
                cur["sc"] = [int(v) for v in rest.split()]
            elif key == "m":
                cur["m"] = [int(v) for v in rest.split()]
            elif key == "q":
                cur["q"] = [Q_RULES[rest](t) for t in range(256)]
            elif key == "hex":
                cur["hex"] += "".join(rest.split())
            elif key == "end":
                raw = np.frombuffer(bytes.fromhex(cur["hex"]), np.uint8).copy()
                assert raw.size == 144, (cur["name"], raw.size)
                blocks.append(GoldenBlock(cur["name"], cur["d"], cur["dmin"], cur["sc"], cur["m"],
                                          cur["q"], raw))
                cur = None
            else:
                raise ValueError(f"bad golden line: {line}")
    return blocks
