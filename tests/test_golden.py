"""Stored worked examples (tests/golden/, written by make_golden.py from the
oracle only) against the oracle as it stands, and against values derived by
hand from the definitions."""
import os

import numpy as np

import oracle

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read(name):
    out, section = {}, None
    for line in open(os.path.join(HERE, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            section = line.strip("[]")
            continue
        key, _, val = line.partition(":")
        out[(section, key.strip())] = val.split()
    return out


def test_layout_small_matches_oracle_and_hand_derivation():
    g = _read("layout_small.txt")
    idx = np.array(g[(None, "topk_idx")], np.int32).reshape(5, 3)
    for cap in (0, 2):
        lay = oracle.layout(idx, 4, cap)
        for name in ("count", "offset", "slot_of", "src_of_slot", "status"):
            want = np.array(g[(f"capacity {cap}", name)], np.int32)
            np.testing.assert_array_equal(np.asarray(lay[name]).ravel(), want, err_msg=(cap, name))
    # by hand: expert 0 appears at entries 1, 3, 4, 11, 14; with 2 rows per
    # expert the 3rd-5th are dropped, together with entries 7 (3rd of expert
    # 3) and 13 (3rd of expert 1): five drops, two invalid ids (-1 and 4).
    assert g[("capacity 2", "status")] == ["2", "5"]
    assert g[("capacity 0", "slot_of")][:5] == ["8", "0", "10", "1", "2"]


def test_fp8_block_matches_oracle_and_named_codes():
    g = _read("fp8_block.txt")
    bits = np.array([int(h, 16) for h in g[(None, "x_bf16_hex")]], np.uint16)
    q, s = oracle.dispatch(bits[None, :], np.zeros((1, 1), np.int32), 1, True)
    assert f"{s.view(np.uint32)[0, 0]:08x}" == g[(None, "scale_hex")][0]
    codes = [int(h, 16) for h in g[(None, "codes_hex")]]
    assert q[0].tolist() == codes
    # scale is exactly 1, so the codes are the OCP encodings of x itself:
    # 448 -> 0x7E, -448 -> 0xFE, 1.0625 -> 0x38 (tie to even), 3*2^-10 -> 0x02,
    # -2^-10 -> 0x80 (tie to zero keeps the sign), -0 -> 0x80, 232 -> 0x76
    assert codes[:7] == [0x7E, 0xFE, 0x38, 0x02, 0x80, 0x80, 0x76]
