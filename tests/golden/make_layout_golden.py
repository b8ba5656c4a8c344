"""Writes tests/golden/q2_block_d128.hex: one 2-bit (layer, head) block of
128 dims filled from a fixed code pattern through the oracle's layout
(oracle/layout.py) only.  The file freezes the whole byte image of the block
format; tests/test_oracle_layout.py rebuilds it and compares.

    python tests/golden/make_layout_golden.py
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import layout  # noqa: E402

D = 128


def pattern_block() -> np.ndarray:
    """Codes K[t][d] = (t + 3d) % 4, V[t][d] = (2t + d + t // 16) % 4;
    metadata K (scale t + 1, min -t / 8), V (scale 1 / (t + 1), min t / 4)."""
    buf = np.zeros(layout.q2_block_bytes(D), np.uint8)
    blk = layout.Q2Block(buf, D)
    d = np.arange(D)
    for t in range(layout.PAGE):
        blk.write_k(t, ((t + 3 * d) % 4).astype(np.uint8), np.float32(t + 1), np.float32(-t / 8))
        blk.write_v(t, ((2 * t + d + t // 16) % 4).astype(np.uint8), np.float32(1.0 / (t + 1)), np.float32(t / 4))
    return buf


def main():
    buf = pattern_block()
    path = os.path.join(HERE, "q2_block_d128.hex")
    with open(path, "w") as f:
        f.write("# 2-bit block, D = 128, written by tests/golden/make_layout_golden.py (oracle/layout.py only)\n")
        for off in range(0, buf.size, 64):
            f.write(f"{off:05d} {buf[off:off + 64].tobytes().hex()}\n")
    print(path)


if __name__ == "__main__":
    main()
