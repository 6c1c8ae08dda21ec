"""Codec construction: rotation Pi, QJL sketch S, Lloyd-Max codebook.  Test infrastructure only.

Sources (page title, section):

* Rotation.  7minutos.es TurboQuant walkthrough, "Etapa 1 (PolarQuant)": y = R*x with R a
  random orthogonal matrix; the norm is unchanged and the outlier energy is spread over
  all coordinates.  TurboESM summary, section 2.A: Pi^T Pi = I.  A Haar-distributed
  orthogonal matrix is the QR factor of a Gaussian matrix with the signs of R's diagonal
  moved into Q (Mezzadri, "How to generate random matrices from the classical compact
  groups", 2007).
* Per-head rotations.  TurboESM summary, section 2.B: one rotation per layer and head.
  Here a seeded orthogonal basis B_h is composed before Pi: y = Pi (B_h x), so the
  stored rotation is Pi @ B_h.
* Sketch.  Same walkthrough, "Etapa 2 (Corrección Residual)": a random projection S whose
  entries are standard Gaussian; here S has m rows and d columns and z = S r.
* Codebook.  Same walkthrough, "Etapa 1": after the rotation a coordinate u_i of the unit
  direction satisfies u_i^2 ~ Beta(1/2, (d-1)/2) (the chi-square ratio theorem), so u_i has
  density f_d(x) = (1 - x^2)^((d-3)/2) / B(1/2, (d-1)/2) on [-1, 1].  Lloyd-Max places the
  2^b levels to minimise mean squared error: boundaries are midpoints between adjacent
  levels and each level is the mean of its cell; the codebook depends only on (d, b) and
  is computed once, offline.

The Lloyd-Max cell integrals use closed forms:
  mass  = F(b) - F(a) with F(x) = 1/2 + sgn(x)/2 * I_{x^2}(1/2, (d-1)/2)  (regularised
          incomplete beta, scipy.special.betainc);
  first moment = [(1 - a^2)^((d-1)/2) - (1 - b^2)^((d-1)/2)] / ((d-1) B(1/2, (d-1)/2)).
The Gaussian (d -> infinity) codebook uses Phi and phi the same way.
"""

from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np
from scipy import integrate, special

from . import rng


# --------------------------------------------------------------------------- rotation


def haar_rotation64(seed: int, d: int) -> np.ndarray:
    """Haar orthogonal d x d matrix in fp64: QR of a seeded Gaussian matrix, sign-fixed."""
    g = rng.gaussians(seed, d * d).reshape(d, d)  # row-major fill
    q, r = np.linalg.qr(g)
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return q * s[None, :]


def haar_rotation(seed: int, d: int) -> np.ndarray:
    """The stored rotation: fp32 (round to nearest even) of ``haar_rotation64``."""
    return haar_rotation64(seed, d).astype(np.float32)


def head_rotations(seed_pi: int, basis_seeds, d: int) -> np.ndarray:
    """Per-head rotations Pi @ B_h (fp64 product of the fp64 Haar factors), stored fp32."""
    pi = haar_rotation64(seed_pi, d)
    out = np.empty((len(basis_seeds), d, d), dtype=np.float32)
    for h, s in enumerate(basis_seeds):
        out[h] = (pi @ haar_rotation64(int(s), d)).astype(np.float32)
    return out


def gaussian_sketch(seed: int, m: int, d: int) -> np.ndarray:
    """QJL projection S (m x d), standard Gaussian entries, stored fp32."""
    return rng.gaussians(seed, m * d).reshape(m, d).astype(np.float32)


# --------------------------------------------------------------------------- densities


def beta_coord_density(d: int) -> Callable[[np.ndarray], np.ndarray]:
    """Density of one coordinate of a uniform point on the unit sphere in R^d."""
    logc = -special.betaln(0.5, 0.5 * (d - 1))

    def f(x):
        x = np.asarray(x, dtype=np.float64)
        return np.exp(logc) * np.power(np.clip(1.0 - x * x, 0.0, None), 0.5 * (d - 3))

    return f


def _beta_cell_stats(d: int):
    logc = -special.betaln(0.5, 0.5 * (d - 1))
    c = np.exp(logc)

    def cdf(x):
        x = np.asarray(x, dtype=np.float64)
        return 0.5 + 0.5 * np.sign(x) * special.betainc(0.5, 0.5 * (d - 1), np.minimum(x * x, 1.0))

    def mass(a, b):
        return cdf(b) - cdf(a)

    def moment(a, b):
        ea = np.power(np.clip(1.0 - a * a, 0.0, None), 0.5 * (d - 1))
        eb = np.power(np.clip(1.0 - b * b, 0.0, None), 0.5 * (d - 1))
        return c * (ea - eb) / (d - 1)

    return mass, moment


def _gauss_cell_stats():
    def mass(a, b):
        return special.ndtr(b) - special.ndtr(a)

    def moment(a, b):
        phi = lambda x: np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)  # noqa: E731
        return phi(a) - phi(b)

    return mass, moment


# --------------------------------------------------------------------------- Lloyd-Max


def lloyd_step(levels: np.ndarray, mass, moment, lo: float, hi: float) -> np.ndarray:
    """One Lloyd-Max update: midpoint boundaries, then each level moves to its cell mean."""
    t = 0.5 * (levels[:-1] + levels[1:])
    a = np.concatenate(([lo], t))
    b = np.concatenate((t, [hi]))
    return moment(a, b) / mass(a, b)


def lloyd_step_samples(levels, samples) -> np.ndarray:
    """The same update on a finite sample: assign to the nearest level, replace by the mean."""
    levels = np.asarray(levels, dtype=np.float64)
    samples = np.asarray(samples, dtype=np.float64)
    t = 0.5 * (levels[:-1] + levels[1:])
    cell = np.searchsorted(t, samples, side="right")
    out = levels.copy()
    for j in range(len(levels)):
        sel = samples[cell == j]
        if sel.size:
            out[j] = sel.mean()
    return out


def lloyd_max(mass, moment, lo, hi, init, rel_tol=1e-14, floor_tol=1e-12, max_iter=400000):
    """Iterate ``lloyd_step`` until no level moves by more than ``rel_tol`` of the largest.

    When the cell integrals' rounding noise keeps the step above ``rel_tol`` (very large d),
    stop once the step is below ``floor_tol`` and has not shrunk for 200 iterations.
    Returns (levels, iterations).
    """
    c = np.asarray(init, dtype=np.float64)
    best, since = np.inf, 0
    for it in range(1, max_iter + 1):
        nc = lloyd_step(c, mass, moment, lo, hi)
        step = np.max(np.abs(nc - c)) / np.max(np.abs(nc))
        if step <= rel_tol:
            return nc, it
        if step < best:
            best, since = step, 0
        else:
            since += 1
            if best <= floor_tol and since >= 200:
                return nc, it
        c = nc
    raise RuntimeError("Lloyd-Max did not converge")


@dataclass
class Codebook:
    d: int
    bits: int
    centroids64: np.ndarray
    thresholds64: np.ndarray
    centroids: np.ndarray  # fp32, ascending
    thresholds: np.ndarray  # fp32 midpoints
    mse: float  # per-coordinate E[(u - Q(u))^2] under f_d
    iterations: int


def _finish(c64):
    c64 = 0.5 * (c64 - c64[::-1])  # exact symmetry of a symmetric density's optimum
    t64 = 0.5 * (c64[:-1] + c64[1:])
    return c64, t64


def lloyd_max_beta(d: int, bits: int) -> Codebook:
    """Lloyd-Max codebook with 2^bits levels for the rotated-coordinate density f_d."""
    if d < 3:
        raise ValueError("the rotated-coordinate law needs d >= 3")
    L = 1 << bits
    mass, moment = _beta_cell_stats(d)
    span = min(2.0 / np.sqrt(d), 0.9)
    init = span * (2.0 * np.arange(L) + 1.0 - L) / L
    c64, it = lloyd_max(mass, moment, -1.0, 1.0, init)
    c64, t64 = _finish(c64)
    f = beta_coord_density(d)
    mse = _cell_mse(f, c64, t64, -1.0, 1.0)
    return Codebook(d, bits, c64, t64, c64.astype(np.float32), t64.astype(np.float32), mse, it)


def lloyd_max_gauss(bits: int):
    """Lloyd-Max levels and MSE for N(0, 1) (Max, 1960): the d -> infinity limit of f_d."""
    L = 1 << bits
    mass, moment = _gauss_cell_stats()
    init = 2.0 * (2.0 * np.arange(L) + 1.0 - L) / L
    c64, _ = lloyd_max(mass, moment, -np.inf, np.inf, init)
    c64, t64 = _finish(c64)
    phi = lambda x: np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)  # noqa: E731
    mse = _cell_mse(phi, c64, t64, -np.inf, np.inf)
    return c64, t64, mse


def _cell_mse(f, c, t, lo, hi) -> float:
    edges = np.concatenate(([lo], t, [hi]))
    total = 0.0
    for j in range(len(c)):
        val, _ = integrate.quad(lambda x: (x - c[j]) ** 2 * float(f(x)), edges[j], edges[j + 1],
                                epsabs=1e-15, epsrel=1e-12, limit=200)
        total += val
    return total


# --------------------------------------------------------------------------- codec bundle


@dataclass
class Codec:
    """Everything the encoder and decoder share for one (d, bits, m) configuration."""

    d: int
    bits: int
    m: int
    rot: np.ndarray  # [n_rot, d, d] fp32, y = rot @ x
    sketch: Optional[np.ndarray]  # [m, d] fp32 or None when m == 0
    centroids: np.ndarray  # [2^bits] fp32 ascending
    thresholds: np.ndarray  # [2^bits - 1] fp32
    vecs_per_rot: int = 0  # consecutive vectors sharing one rotation (0: all share rot[0])
    # > 0: the high half of a record's norm word holds fp16(nbar * resid_scale) instead of the
    # residual norm (the TurboESM residual-sign correction, oracle/calibrate.py)
    resid_scale: float = 0.0
    extra: dict = field(default_factory=dict)

    @property
    def n_rot(self) -> int:
        return self.rot.shape[0]

    def rot_index(self, n_vec: int, first: int = 0) -> np.ndarray:
        ids = np.arange(first, first + n_vec, dtype=np.int64)
        if self.n_rot == 1 or self.vecs_per_rot <= 0:
            return np.zeros(n_vec, dtype=np.int64)
        return np.minimum(ids // self.vecs_per_rot, self.n_rot - 1)


def make_codec(d: int, bits: int, m: int, rot_seed: int, sketch_seed: int,
               basis_seeds=None, vecs_per_rot: int = 0) -> Codec:
    """Build a codec from seeds: Haar Pi (optionally composed with per-head bases), S, codebook."""
    if basis_seeds is None:
        rot = haar_rotation(rot_seed, d)[None]
    else:
        rot = head_rotations(rot_seed, basis_seeds, d)
    sk = gaussian_sketch(sketch_seed, m, d) if m > 0 else None
    cb = lloyd_max_beta(d, bits)
    return Codec(d, bits, m, rot, sk, cb.centroids, cb.thresholds, vecs_per_rot)
