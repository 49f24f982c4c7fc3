"""Noise schedule and DDIM timestep grid — oracle, test infrastructure.

Linear beta schedule over T training steps (DDPM, Ho et al., ref. [19] of the
ParaChromo paper):  beta_s = beta_start + (beta_end - beta_start) * s / (T - 1)
for s = 0 .. T-1, and abar_t = prod_{s <= t} (1 - beta_s).

(The paper's own runs use a cosine schedule, section 4.3.2; the workloads here
fix the linear one.)

DDIM grid (Song et al., ref. [7]): n reverse steps with stride d = T / n visit
tau_i = T - d (i + 1), i = 0 .. n-1 (980, 960, ..., 0 for n = 50).  Step i
moves from abar_{tau_i} to abar_{tau_{i+1}}; after the last step (tau = 0) the
target is the clean sample, abar = 1.

DDIM noise scale for a step from abar a to abar a':
    sigma(eta) = eta * sqrt((1 - a') / (1 - a)) * sqrt(1 - a / a').

Cosine schedule (Nichol & Dhariwal, "Improved denoising diffusion
probabilistic models", ICML 2021), the schedule ChromoGen's sampler uses
(ParaChromo, section 4.3.2): with f(u) = cos^2(pi/2 (u + s)/(1 + s)),
beta_t = min(1 - f((t+1)/T) / f(t/T), beta_max) and abar_t the running
product of (1 - beta_t), as for the linear schedule.
"""

from __future__ import annotations

import math

import numpy as np


def betas(T: int = 1000, beta_start: float = 1e-4, beta_end: float = 0.02) -> np.ndarray:
    s = np.arange(T, dtype=np.float64)
    return beta_start + (beta_end - beta_start) * s / (T - 1)


def alpha_bar(T: int = 1000, beta_start: float = 1e-4, beta_end: float = 0.02) -> np.ndarray:
    """abar_t for t = 0 .. T-1, as a running product in index order."""
    b = betas(T, beta_start, beta_end)
    out = np.empty(T, dtype=np.float64)
    acc = 1.0
    for t in range(T):
        acc *= 1.0 - b[t]
        out[t] = acc
    return out


def betas_cosine(T: int = 1000, s: float = 0.008, beta_max: float = 0.999) -> np.ndarray:
    def f(u):
        return math.cos((u + s) / (1.0 + s) * math.pi / 2.0) ** 2
    return np.array([min(1.0 - f((t + 1) / T) / f(t / T), beta_max) for t in range(T)], dtype=np.float64)


def alpha_bar_from_betas(b) -> np.ndarray:
    out = np.empty(len(b), dtype=np.float64)
    acc = 1.0
    for t in range(len(b)):
        acc *= 1.0 - b[t]
        out[t] = acc
    return out


def ddim_timesteps(n_steps: int, T: int = 1000) -> np.ndarray:
    if n_steps < 1 or T % n_steps:
        raise ValueError("n_steps must divide T")
    d = T // n_steps
    return np.array([T - d * (i + 1) for i in range(n_steps)], dtype=np.int64)


def ddim_pairs(n_steps: int, T: int = 1000, beta_start: float = 1e-4, beta_end: float = 0.02, ab=None):
    """[(a_i, a'_i)] for each DDIM step i: abar before and after the step.  ``ab`` overrides the
    linear schedule with any abar table of length T."""
    if ab is None:
        ab = alpha_bar(T, beta_start, beta_end)
    tau = ddim_timesteps(n_steps, T)
    out = []
    for i in range(n_steps):
        a = float(ab[tau[i]])
        a_next = float(ab[tau[i + 1]]) if i + 1 < n_steps else 1.0
        out.append((a, a_next))
    return out


def ddim_sigma(a: float, a_next: float, eta: float) -> float:
    return eta * math.sqrt((1.0 - a_next) / (1.0 - a)) * math.sqrt(1.0 - a / a_next)
