"""Writes rope_closed_form.txt: rotary-embedding outputs derived by hand.

Rotary embedding as defined by RoFormer (cited by "FlashDecoder: Real-Time
Latent-to-Pixel Streaming Decoder with Transformers", Sec. 3.2 "Base
Architecture"): a channel pair (x0, x1) at angle a becomes
(x0 cos a - x1 sin a, x0 sin a + x1 cos a).  Each axis block of P_a pairs
uses frequencies theta^(-2j/(2 P_a)), j = 0..P_a-1.  The angles below were
worked out by hand for the listed positions and are written as literals, so
the file does not depend on the oracle.  Run: python tests/golden/make_golden.py
"""
import math
import os

CASES = [
    # pairs (t,h,w), theta, position (t,h,w), x, angles per pair (hand-derived)
    # case A: t-block of 2 pairs: omegas 1, 10000^(-1/2)=0.01 -> angles 3, 0.03;
    #         h-block 1 pair: angle 2; w-block 1 pair: angle 5.
    ((2, 1, 1), 10000.0, (3, 2, 5), [1, 0, 1, 0, 0, 1, 1, 1], [3.0, 0.03, 2.0, 5.0]),
    # case B: t-block 1 pair: angle 1; h-block 2 pairs: omegas 1, 100^(-1/2)=0.1 -> 4, 0.4;
    #         w-block 1 pair: angle 7.
    ((1, 2, 1), 100.0, (1, 4, 7), [0.5, -2, 1, 3, -1, 0.25, 2, 2], [1.0, 4.0, 0.4, 7.0]),
]


def main():
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "rope_closed_form.txt")
    with open(out, "w") as f:
        f.write("# Rotary embedding closed-form cases (RoFormer rotation, cited by FlashDecoder Sec. 3.2).\n")
        f.write("# pairs_t pairs_h pairs_w | theta | t h w | x[8] | y[8]\n")
        for pairs, theta, pos, x, ang in CASES:
            y = []
            for p, a in enumerate(ang):
                x0, x1 = x[2 * p], x[2 * p + 1]
                y += [x0 * math.cos(a) - x1 * math.sin(a), x0 * math.sin(a) + x1 * math.cos(a)]
            f.write("%s | %r | %s | %s | %s\n" % (
                " ".join(map(str, pairs)), theta, " ".join(map(str, pos)),
                " ".join(repr(float(v)) for v in x), " ".join(repr(v) for v in y)))


if __name__ == "__main__":
    main()
