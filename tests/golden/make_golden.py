"""Writes tests/golden/*.txt from the CPU oracle only (no GPU code involved).

The fixtures freeze small worked examples so that a later change to the
oracle's arithmetic shows up as a diff here.  Re-run only together with a
change to the oracle whose commit message names the passage or reading that
justifies it:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402

# A routing table small enough to check by hand: T=5 tokens, k=3, E=4, with a
# duplicate id in a row (token 2), an id below range (-1) and one past the
# end (4).
IDX = np.array([[2, 0, 3], [0, 0, 1], [3, 3, -1], [1, 4, 0], [2, 1, 0]], np.int32)


def write_layout():
    lines = ["# oracle layout of a hand-checkable routing table (E=4)",
             "topk_idx: " + " ".join(map(str, IDX.ravel()))]
    for cap in (0, 2):
        lay = oracle.layout(IDX, 4, cap)
        lines.append(f"[capacity {cap}]")
        for name in ("count", "offset", "slot_of", "src_of_slot", "status"):
            lines.append(f"{name}: " + " ".join(map(str, np.asarray(lay[name]).ravel())))
    with open(os.path.join(HERE, "layout_small.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


def write_fp8_row():
    # one 128-channel block: values chosen to hit ties, zeros and the maximum
    vals = np.zeros(128, np.float32)
    vals[0] = 448.0
    vals[1] = -448.0
    vals[2] = 1.0625          # tie 1.0 / 1.125 -> 1.0
    vals[3] = 3 * 2.0 ** -10  # tie 2^-9 / 2^-8 -> 2^-8
    vals[4] = -(2.0 ** -10)   # tie 0 / 2^-9 -> -0
    vals[5] = -0.0
    vals[6] = 232.0           # tie 224 / 240 -> 224
    vals[7:] = np.linspace(-300, 300, 121, dtype=np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)   # all values are exact in bf16
    q, s = oracle.dispatch(bits[None, :], np.zeros((1, 1), np.int32), 1, True)
    lines = ["# oracle E4M3FN quantisation of one 128-channel bf16 block (scale = 448/448 = 1)",
             "x_bf16_hex: " + " ".join(f"{b:04x}" for b in bits),
             f"scale_hex: {s.view(np.uint32)[0, 0]:08x}",
             "codes_hex: " + " ".join(f"{c:02x}" for c in q[0])]
    with open(os.path.join(HERE, "fp8_block.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    write_layout()
    write_fp8_row()
