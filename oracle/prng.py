"""Parameter random streams for the oracle (test infrastructure only).

The pages draw three random objects and never say how: the per-group rotors
("normalized random bivector exponentials"), TurboQuant's Gaussian matrix that
QR turns into Pi, and QJL's Gaussian projection S (README "How TurboQuant
Works", blog section on QJL).  Both the oracle and the library must draw the
same numbers from a seed, so each side implements the same published
generator independently:

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): state += 0x9E3779B97F4A7C15, then the two
  xor-shift-multiply rounds of the published finaliser.
* One stream per (seed, tag); the stream starts from state
  seed XOR (tag * 0xD1B54A32D192ED03 mod 2**64).  Tags: 1 rotors, 2 Pi, 3 S.
* Uniform u = ((w >> 11) + 0.5) * 2**-53, strictly inside (0, 1).
* Normals by the Box-Muller transform (Box and Muller 1958): from u1, u2,
  z0 = sqrt(-2 ln u1) cos(2 pi u2), then z1 = sqrt(-2 ln u1) sin(2 pi u2).
  Scalar libm functions (Python ``math``) are used, never numpy's vectorised
  transcendental kernels, so the values are those of the C library.
"""
import math

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15
STREAM_MUL = 0xD1B54A32D192ED03
TWO_PI = 2.0 * math.pi

TAG_ROTORS = 1
TAG_PI = 2
TAG_S = 3


class SplitMix64:
    """SplitMix64 generator over Python integers (exact 64-bit arithmetic)."""

    def __init__(self, state):
        self.state = state & MASK64

    def next_u64(self):
        self.state = (self.state + GOLDEN_GAMMA) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)

    def uniform(self):
        return ((self.next_u64() >> 11) + 0.5) * (2.0 ** -53)


def stream(seed, tag):
    """The SplitMix64 stream for (seed, tag)."""
    return SplitMix64((seed & MASK64) ^ ((tag * STREAM_MUL) & MASK64))


def normals(seed, tag, count):
    """`count` standard normals of stream (seed, tag), in draw order."""
    g = stream(seed, tag)
    out = []
    while len(out) < count:
        u1 = g.uniform()
        u2 = g.uniform()
        rad = math.sqrt(-2.0 * math.log(u1))
        ang = TWO_PI * u2
        out.append(rad * math.cos(ang))
        out.append(rad * math.sin(ang))
    return out[:count]
