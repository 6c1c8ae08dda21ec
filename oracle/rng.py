"""Counter-based random numbers for the codec's random matrices.  Test infrastructure only.

The method draws two random matrices: the Gaussian matrix whose QR factor is the
rotation Pi (7minutos.es TurboQuant walkthrough, "Etapa 1 (PolarQuant)": y = R*x with R a
random orthogonal matrix) and the Gaussian projection S of the QJL stage ("Etapa 2
(Corrección Residual)": a random projection matrix S).  Both sides of the parity check
generate them from a seed with the same published generator, each in its own code:

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014): output k (k = 0, 1, ...) of stream ``seed`` is
  mix(seed + (k + 1) * 0x9E3779B97F4A7C15 mod 2**64), with mix the 64-bit finaliser
  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31.
* a uniform double u = (x >> 11) * 2**-53 in [0, 1);
* Box-Muller (Box and Muller, 1958): Gaussian pair j uses outputs 2j and 2j+1,
  u1 = 1 - uniform(out 2j) in (0, 1], u2 = uniform(out 2j+1),
  rho = sqrt(-2 ln u1), g[2j] = rho * cos(2 pi u2), g[2j+1] = rho * sin(2 pi u2).

Python's ``math`` functions are used (the platform libm), in pure Python loops; the
matrices are at most 200 x 200.
"""

import math

import numpy as np

_MASK = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed: int, k: int) -> int:
    """Output ``k`` of the SplitMix64 stream started at ``seed`` (a 64-bit integer)."""
    z = (seed + (k + 1) * _GAMMA) & _MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def uniform01(x: int) -> float:
    """Top 53 bits of a 64-bit word as a double in [0, 1)."""
    return (x >> 11) * (1.0 / 9007199254740992.0)


def gaussians(seed: int, count: int) -> np.ndarray:
    """``count`` standard normal doubles from stream ``seed`` (Box-Muller pairs, in order)."""
    out = np.empty(count, dtype=np.float64)
    two_pi = 2.0 * math.pi
    seed &= _MASK
    for j in range((count + 1) // 2):
        u1 = 1.0 - uniform01(splitmix64(seed, 2 * j))
        u2 = uniform01(splitmix64(seed, 2 * j + 1))
        rho = math.sqrt(-2.0 * math.log(u1))
        ang = two_pi * u2
        out[2 * j] = rho * math.cos(ang)
        if 2 * j + 1 < count:
            out[2 * j + 1] = rho * math.sin(ang)
    return out
