"""The select kernel's clipped z-score divides by sqrt((double) D) where D is an
exact 128-bit integer; the kernel converts D to double by taking its top 64
bits with the rest folded into a sticky bit, converting those (one IEEE
rounding), and scaling by a power of two. That equals the correctly rounded
conversion (what the oracle's (double) of an unsigned __int128 gives) only if
the sticky bit sits below the rounding position; this checks the identity on
the CPU, step for step in exact integer arithmetic against Python's correctly
rounded int -> float, over random and edge-case values of up to 81 bits."""
import random


def sticky_to_double(v: int) -> float:
    hi = v >> 64
    if hi == 0:
        return float(v)  # an exact u64 -> double conversion, correctly rounded
    sh = hi.bit_length()
    m = v >> sh
    if v & ((1 << sh) - 1):
        m |= 1
    return float(m) * 2.0 ** sh  # m < 2^64: one rounding; the scaling is exact


def test_sticky_conversion_is_correctly_rounded():
    rng = random.Random(11)
    cases = []
    for bits in range(60, 82):
        for _ in range(3000):
            cases.append(rng.getrandbits(bits) | (1 << (bits - 1)))
    # halfway cases and their neighbours: 53 significant bits, then a 1, then
    # zeros or a single low 1 far below (only the sticky bit sees it)
    for bits in range(65, 82):
        for _ in range(500):
            top = rng.getrandbits(53) | (1 << 52)
            sh = bits - 54
            half = (top << 1 | 1) << sh
            cases += [half, half + 1, half - 1, (top << 1) << sh, ((top << 1) << sh) + 1]
    for v in cases:
        assert sticky_to_double(v) == float(v), v
