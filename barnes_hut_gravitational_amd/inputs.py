"""Seeded synthetic particle sets for the force evaluation.

This module draws inputs only. It holds none of the tree method's arithmetic,
so both the HIP path and the CPU oracle take their particles from here.

Workloads follow the orrery performance page ("docs/performance/sycl_tree.md",
table "The machine and the device"): a Plummer sphere, seed 20260811, softening
0.05, opening angle 0.5, leaf capacity 32, monopole only. The pages give the
seed but not the generator, so the particle sets here are not the pages' own:

* random numbers: NumPy ``Generator(PCG64(seed)).random((n, 3))`` in float64,
  one row (u, v, w) per particle, rows in particle order;
* Plummer radius from the inverted cumulative mass of a unit Plummer sphere,
  r = 1 / sqrt(u^(-2/3) - 1), capped at 10 scale radii;
* isotropic direction: cos(polar) = 2v - 1, azimuth = 2 pi w;
* positions computed in float64 and rounded once to float32;
* every mass is 1/N in float32 (exact, since every N used is a power of two).
"""

from __future__ import annotations

import numpy as np

SEED = 20260811
PLUMMER_R_CAP = 10.0

# name -> (kind, n). The first is the small case used for oracle parity; the
# fourth is the headline measurement.
CONFIGS = {
    "plummer_16k": ("plummer", 16384),
    "plummer_131k": ("plummer", 131072),
    "uniform_262k": ("uniform", 262144),
    "plummer_1m": ("plummer", 1048576),
    "merger_8m": ("merger", 8388608),
}

# Softened force law and tree parameters of every workload.
EPS = 0.05
THETA = 0.5
LEAF_CAP = 32


def _draws(n: int, seed: int) -> np.ndarray:
    return np.random.Generator(np.random.PCG64(seed)).random((n, 3))


def _unit_plummer(draws: np.ndarray) -> np.ndarray:
    """Positions (float64) of a unit-mass, unit-scale-radius Plummer sphere."""
    u, v, w = draws[:, 0], draws[:, 1], draws[:, 2]
    with np.errstate(divide="ignore"):
        r = 1.0 / np.sqrt(u ** (-2.0 / 3.0) - 1.0)
    r = np.minimum(r, PLUMMER_R_CAP)
    cos_t = 2.0 * v - 1.0
    sin_t = np.sqrt(np.maximum(0.0, 1.0 - cos_t * cos_t))
    phi = 2.0 * np.pi * w
    return np.stack([r * sin_t * np.cos(phi), r * sin_t * np.sin(phi), r * cos_t], axis=1)


def plummer(n: int, seed: int = SEED) -> tuple[np.ndarray, np.ndarray]:
    pos = _unit_plummer(_draws(n, seed)).astype(np.float32)
    return pos, np.full(n, 1.0 / n, dtype=np.float32)


def uniform_cube(n: int, seed: int = SEED) -> tuple[np.ndarray, np.ndarray]:
    """Positions uniform in [-1, 1)^3."""
    pos = (2.0 * _draws(n, seed) - 1.0).astype(np.float32)
    return pos, np.full(n, 1.0 / n, dtype=np.float32)


def merger(n: int, seed: int = SEED) -> tuple[np.ndarray, np.ndarray]:
    """Two Plummer spheres of n/2 particles each drawn from one stream.

    Sphere A (scale radius 1, centre at the origin) takes the first n/2 rows
    of draws, sphere B (scale radius 0.5, centre (6, 0, 0)) the rest. The
    radius cap applies in scale radii, before scaling.
    """
    half = n // 2
    unit = _unit_plummer(_draws(n, seed))
    unit[half:] = 0.5 * unit[half:] + np.array([6.0, 0.0, 0.0])
    return unit.astype(np.float32), np.full(n, 1.0 / n, dtype=np.float32)


def make(kind: str, n: int, seed: int = SEED) -> tuple[np.ndarray, np.ndarray]:
    """Contiguous float32 positions [n, 3] and masses [n] for a workload kind."""
    gen = {"plummer": plummer, "uniform": uniform_cube, "merger": merger}[kind]
    pos, mass = gen(n, seed)
    return np.ascontiguousarray(pos), np.ascontiguousarray(mass)


def make_config(name: str, seed: int = SEED) -> tuple[np.ndarray, np.ndarray]:
    kind, n = CONFIGS[name]
    return make(kind, n, seed)
