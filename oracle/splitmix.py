"""SplitMix64 and the per-row systematic-sampling offset (oracle side).

Test infrastructure only (see ``oracle/__init__``).

SplitMix64 is the counter-based generator of Steele, Lea and Flood,
"Fast splittable pseudorandom number generators" (OOPSLA 2014): output i of
the stream seeded with ``seed`` mixes the state ``seed + (i + 1) * gamma``
(gamma = 0x9E3779B97F4A7C15) with two xor-shift-multiply rounds.  It is
written here from that published definition.  The HIP library carries its
own implementation; the two share no code.

The pages say only that the sample is systematic (AB-Attention page, section
"어떻게 쓰나"); the offset recipe below is this project's reading: a 44-bit
fixed-point offset U in [0, 2^44 - 2^16) for row (b * H + h) * nQB + i.
"""

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

UNIT_BITS = 44
UNIT = 1 << UNIT_BITS           # fixed-point 1.0 of an inclusion probability
OFFSET_LIMIT = UNIT - (1 << 16)  # offsets lie in [0, OFFSET_LIMIT)


def splitmix64(seed: int, i: int) -> int:
    """Output number ``i`` (0-based) of SplitMix64 seeded with ``seed``."""
    z = (seed + (i + 1) * GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def sampling_offset(seed: int, row: int) -> int:
    """U_row = floor((x >> 20) * (2^44 - 2^16) / 2^44), x = splitmix64(seed, row)."""
    x = splitmix64(seed & MASK64, row) >> 20
    return (x * OFFSET_LIMIT) >> UNIT_BITS
