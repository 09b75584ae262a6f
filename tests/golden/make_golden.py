"""Writes the oracle regression fixtures in this folder. Calls only ``oracle``.

The pages print no numeric worked example, so these files are not independent pins: they
freeze the oracle's output on a tiny, formula-defined input (three documents of lengths 1, 5
and 17; hq=2, hkv=1, d=8; scale 0.35) so that any later change to the oracle's arithmetic
shows up as a diff. Regenerate only together with a change that names its justification.

    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import attention, mx  # noqa: E402


def tiny_inputs():
    lengths = [1, 5, 17]
    cu = np.array([0, 1, 6, 23])
    T, hq, hkv, d = 23, 2, 1, 8
    t = np.arange(T)[:, None, None]
    r = np.arange(d)[None, None, :]
    hq_i = np.arange(hq)[None, :, None]
    hk_i = np.arange(hkv)[None, :, None]
    q = (((7 * t + 3 * hq_i + 5 * r) % 11) - 5) / 4.0
    k = (((5 * t + 2 * hk_i + 3 * r) % 13) - 6) / 4.0
    v = (((3 * t + hk_i + 7 * r) % 9) - 4) / 2.0
    do = (((11 * t + 5 * hq_i + r) % 7) - 3) / 2.0
    return lengths, cu, q, k, v, do, 0.35


def main():
    _, cu, q, k, v, do, sc = tiny_inputs()
    o, lse = attention.attn_fwd(q, k, v, cu, sc)
    dq, dk, dv = attention.attn_bwd(q, k, v, do, cu, sc)
    with open(os.path.join(HERE, "tiny_attention.txt"), "w") as f:
        f.write("# oracle.attention on tests/golden/make_golden.py:tiny_inputs(); one array per line\n")
        for name, a in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            f.write(name + " " + " ".join(repr(float(x)) for x in a.ravel()) + "\n")
    with open(os.path.join(HERE, "e4m3_table.txt"), "w") as f:
        f.write("# code value (oracle.mx.e4m3_decode), all 256 E4M3 codes\n")
        for c in range(256):
            f.write(f"{c} {float(mx.e4m3_decode(c))!r}\n")


if __name__ == "__main__":
    main()
