"""Codebooks calibrated on data, and the TurboESM residual-sign codec.  Test infrastructure
only: the tests, __graft_entry__.smoke() and bench.py's cpu_baseline use it; the library does
not.

Sources (gist.science TurboESM page, Spanish and Korean summaries):
  * section 2.C, "dual LUT": K and V get their own 8-level Lloyd-Max tables, each fitted to
    that matrix's statistics (K after the rotation is near-Gaussian with heavier tails, V has
    a lower variance);
  * section 2.D, "1-bit residual correction": only the sign of the quantisation residual
    x - x^ is stored, one bit, and the decoder adds a first-order correction
    x~ = x^ + sign * e, e the mean residual magnitude calibrated beforehand.
The walkthrough (7minutos.es, "Etapa 1 (PolarQuant)") gives the Lloyd rule itself: midpoint
boundaries, each level moved to the mean of its cell, repeated until nothing improves; on a
finite sample that is 1-D k-means (its worked example is pinned in the tests).

Readings (the pages leave these open):
  * the samples are the rotated directions u = Pi x / ||x|| of calibration vectors, the
    quantity the encoder compares with the thresholds;
  * the Lloyd iteration starts from a given codebook (the law's own Lloyd-Max levels) and
    stops when no level moves by more than rel_tol of the largest, or after max_iter rounds;
    an empty cell keeps its level;
  * e is one number per table: the mean over the samples of |u_i - c[idx(u_i)]| with the
    final levels and their midpoints;
  * the sign is taken per coordinate of the rotated residual r = y - nbar c[idx] (the
    residual of reading 7), i.e. the QJL sign bits with S = I and m = d; the record keeps
    n16 and, in the high half of the norm word, fp16(nbar * resid_scale) with
    resid_scale = fl32(e * m / sqrt(pi/2)), so that the estimator's sign term
    rnbar sqrt(pi/2)/m <S q~, 2b - 1> is nbar e <q~, 2b - 1>, the pages' correction.
"""

import math
from dataclasses import dataclass, replace

import numpy as np

from .codec import Codec


@dataclass
class Calibrated:
    centroids: np.ndarray   # fp32 ascending
    thresholds: np.ndarray  # fp32 midpoints
    ebar: float             # mean |u - c[idx(u)]| (fp64)
    iterations: int


def rotated_directions(x: np.ndarray, codec: Codec, first: int = 0) -> np.ndarray:
    """u = Pi x / ||x|| per row (fp64; each row with its rotation block's Pi)."""
    x64 = np.asarray(x, dtype=np.float64)
    rid = codec.rot_index(x64.shape[0], first)
    y = np.einsum("nij,nj->ni", codec.rot.astype(np.float64)[rid], x64)
    nrm = np.linalg.norm(x64, axis=1)
    return y / np.where(nrm > 0, nrm, 1.0)[:, None]


def cells(levels: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Cell of each sample: the number of midpoints it reaches (u >= t_j)."""
    t = 0.5 * (levels[:-1] + levels[1:])
    return np.searchsorted(t, u, side="right")


def calibrate_codebook(u, init, max_iter: int = 200, rel_tol: float = 1e-12) -> Calibrated:
    """Lloyd's rule on the samples u (any shape), starting from the levels ``init``."""
    u = np.asarray(u, dtype=np.float64).ravel()
    lv = np.asarray(init, dtype=np.float64).copy()
    it = 0
    while it < max_iter:
        cell = cells(lv, u)
        new = lv.copy()
        for j in range(len(lv)):
            sel = u[cell == j]
            if sel.size:
                new[j] = np.sum(sel) / sel.size
        it += 1
        moved = np.max(np.abs(new - lv))
        lv = new
        if moved <= rel_tol * np.max(np.abs(lv)):
            break
    cell = cells(lv, u)
    ebar = float(np.sum(np.abs(u - lv[cell])) / u.size)
    c32 = lv.astype(np.float32)
    t32 = (0.5 * (lv[:-1] + lv[1:])).astype(np.float32)
    return Calibrated(c32, t32, ebar, it)


def resid_scale(ebar: float, m: int) -> float:
    """The value stored with the codec: fl32(e * m / sqrt(pi/2))."""
    return float(np.float32(ebar * m / math.sqrt(math.pi / 2.0)))


def turboesm_codec(codec: Codec, cal: Calibrated) -> Codec:
    """The codec with a calibrated table and the residual-sign correction (S = I, m = d)."""
    d = codec.d
    return replace(codec, m=d, sketch=np.eye(d, dtype=np.float32), centroids=cal.centroids,
                   thresholds=cal.thresholds, resid_scale=resid_scale(cal.ebar, d))
