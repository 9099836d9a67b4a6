"""Seeded synthetic particle sets with the shapes of the jz-fmm and jaccpot pages'
workloads.

This module holds only input generation (no step of the multipole method), so
that the GPU path and the CPU oracle can be fed identical inputs without sharing
any of the method's arithmetic.  All positions are generated in fp64 with
numpy's PCG64 generator and equal masses 1/N (G = 1, no softening).

Distributions:
  uniform    -- iid in the unit cube [0, 1)^3.
  plummer    -- Plummer sphere: radii from the inverse of the cumulative mass
                profile M(<r)/M = r^3 / (r^2 + a^2)^(3/2), truncated at 20 a,
                isotropic directions (a normalised 3-d standard normal).
  clustered  -- 64 Plummer spheres, centres uniform in the unit cube, scale
                radii log-uniform in [0.002, 0.05], occupancies from a
                multinomial draw with Dirichlet(1) weights, shuffled.
  hernquist  -- Hernquist sphere (scale a = 1): radii from the inverse of the
                cumulative mass profile M(<r)/M = r^2 / (r + a)^2, truncated
                at 100 a (98 % of the mass), isotropic directions.
  lattice    -- 256^3 cell-centred lattice of the unit cube displaced by a
                Gaussian random field with power spectrum P(k) ~ k^-2 per
                component (rms displacement 0.3 lattice spacings), wrapped
                periodically into [0, 1).
The jz-fmm page measures a 40-million-particle Hernquist sphere (its
accuracy-runtime figure) and jaccpot a distribution it does not state; the
hernquist set replays the former's shape, the others stand in for the rest.
"""
from __future__ import annotations

import numpy as np

__all__ = ["uniform", "plummer", "clustered", "hernquist", "lattice", "CONFIGS", "make",
           "lattice_state", "LATTICE_DX", "LATTICE_DV"]


def uniform(n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.random((n, 3))


def _plummer_radii(rng, n, a, trunc):
    frac = trunc ** 3 / (1.0 + trunc ** 2) ** 1.5  # mass fraction inside trunc*a
    u = 1.0 - rng.random(n)  # (0, 1]
    v = frac * u
    return a / np.sqrt(v ** (-2.0 / 3.0) - 1.0)


def _directions(rng, n):
    d = rng.standard_normal((n, 3))
    return d / np.linalg.norm(d, axis=1, keepdims=True)


def plummer(n: int, seed: int, a: float = 1.0, trunc: float = 20.0,
            centre=(0.0, 0.0, 0.0)) -> np.ndarray:
    rng = np.random.default_rng(seed)
    r = _plummer_radii(rng, n, a, trunc)
    return np.asarray(centre, dtype=np.float64) + r[:, None] * _directions(rng, n)


def clustered(n: int, seed: int, n_clusters: int = 64, a_min: float = 0.002,
              a_max: float = 0.05, trunc: float = 20.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    centres = rng.random((n_clusters, 3))
    scales = np.exp(rng.uniform(np.log(a_min), np.log(a_max), n_clusters))
    weights = rng.dirichlet(np.ones(n_clusters))
    counts = rng.multinomial(n, weights)
    parts = []
    for c in range(n_clusters):
        k = int(counts[c])
        if k == 0:
            continue
        r = _plummer_radii(rng, k, scales[c], trunc)
        parts.append(centres[c] + r[:, None] * _directions(rng, k))
    pos = np.concatenate(parts, axis=0)
    return pos[rng.permutation(n)]


def hernquist(n: int, seed: int, a: float = 1.0, trunc: float = 100.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    frac = (trunc / (1.0 + trunc)) ** 2  # mass fraction inside trunc*a
    u = 1.0 - rng.random(n)  # (0, 1]
    s = np.sqrt(frac * u)  # r / (r + a)
    r = a * s / (1.0 - s)
    return r[:, None] * _directions(rng, n)


def lattice(ngrid: int, seed: int, rms_cells: float = 0.3, slope: float = -2.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    q1 = (np.arange(ngrid) + 0.5) / ngrid
    kf = 2.0 * np.pi * np.fft.fftfreq(ngrid, d=1.0 / ngrid)
    kr = 2.0 * np.pi * np.fft.rfftfreq(ngrid, d=1.0 / ngrid)
    k2 = kf[:, None, None] ** 2 + kf[None, :, None] ** 2 + kr[None, None, :] ** 2
    k2[0, 0, 0] = 1.0
    amp = np.sqrt(k2 ** (slope / 2.0))
    amp[0, 0, 0] = 0.0  # no mean displacement
    psi = np.empty((3, ngrid, ngrid, ngrid))
    for c in range(3):
        white = rng.standard_normal((ngrid, ngrid, ngrid))
        psi[c] = np.fft.irfftn(np.fft.rfftn(white) * amp, s=(ngrid, ngrid, ngrid), axes=(0, 1, 2))
    rms = np.sqrt(np.mean(np.sum(psi ** 2, axis=0)))
    psi *= (rms_cells / ngrid) / rms
    gx, gy, gz = np.meshgrid(q1, q1, q1, indexing="ij")
    pos = np.stack([gx + psi[0], gy + psi[1], gz + psi[2]], axis=-1).reshape(-1, 3)
    del psi
    pos = np.mod(pos, 1.0)
    return pos[rng.permutation(pos.shape[0])]


# Named workloads: the five configurations the pages' problem statement is
# measured on (sizes, distributions, precision, order, theta, leaf size).
CONFIGS = {
    "uniform_4096": dict(dist="uniform", n=4096, seed=1001, dtype="f64", order=4, theta=0.7, leaf=32),
    "plummer_1e4": dict(dist="plummer", n=10_000, seed=1002, dtype="f64", order=4, theta=0.7, leaf=32),
    "plummer_1e5": dict(dist="plummer", n=100_000, seed=1003, dtype="f64", order=4, theta=0.7, leaf=32),
    "uniform_1e5": dict(dist="uniform", n=100_000, seed=1004, dtype="f64", order=4, theta=0.7, leaf=32),
    "clustered_1e6_p4": dict(dist="clustered", n=1_000_000, seed=1005, dtype="f64", order=4, theta=0.7, leaf=32),
    "clustered_1e6_p6": dict(dist="clustered", n=1_000_000, seed=1005, dtype="f64", order=6, theta=0.5, leaf=32),
    "clustered_1e6_f32": dict(dist="clustered", n=1_000_000, seed=1005, dtype="f32", order=4, theta=0.7, leaf=32),
    "hernquist_1e5": dict(dist="hernquist", n=100_000, seed=1007, dtype="f64", order=4, theta=0.7, leaf=32),
    "hernquist_4e7": dict(dist="hernquist", n=40_000_000, seed=1007, dtype="f64", order=4, theta=0.7,
                          leaf=32),
    "lattice_256_f32": dict(dist="lattice", n=256 ** 3, seed=1006, dtype="f32", order=4, theta=0.7, leaf=64),
    "lattice_256_p8": dict(dist="lattice", n=256 ** 3, seed=1006, dtype="f64", order=8, theta=0.5, leaf=64),
}


def make(dist: str, n: int, seed: int):
    """(positions [n,3] fp64, masses [n] fp64) for a distribution name."""
    if dist == "uniform":
        pos = uniform(n, seed)
    elif dist == "plummer":
        pos = plummer(n, seed)
    elif dist == "clustered":
        pos = clustered(n, seed)
    elif dist == "hernquist":
        pos = hernquist(n, seed)
    elif dist == "lattice":
        g = round(n ** (1.0 / 3.0))
        if g ** 3 != n:
            raise ValueError("lattice needs a cube number of particles")
        pos = lattice(g, seed)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return pos, np.full(n, 1.0 / n)


# Integer-lattice state for the reversible integrator: positions x = q dx and
# velocities v = u dv with q, u int64.  Powers of two, so that q dx is exact in
# fp64 for |q| < 2^53.
LATTICE_DX = 2.0 ** -32
LATTICE_DV = 2.0 ** -32


def lattice_state(pos: np.ndarray, seed: int, sigma_v: float = 0.1, dx: float = LATTICE_DX,
                  dv: float = LATTICE_DV):
    """q = round(pos / dx) and u = round(v / dv) with v ~ N(0, sigma_v) per component."""
    rng = np.random.default_rng(seed)
    q = np.rint(np.asarray(pos, dtype=np.float64) / dx).astype(np.int64)
    u = np.rint(sigma_v * rng.standard_normal(q.shape) / dv).astype(np.int64)
    return q, u
