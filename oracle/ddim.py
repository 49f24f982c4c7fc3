"""Stand-in denoiser, classifier-free guidance and the DDIM reverse step —
oracle, test infrastructure.

ChromoGen's conditional U-Net predicts the noise of a distance-map state at
every reverse step, once conditioned and once unconditioned, and the two
predictions are mixed by classifier-free guidance (ParaChromo, section 3.1;
Ho & Salimans, ref. [15]).  The trained weights are not available, so the
denoiser is replaced by the exact noise prediction for a point-mass data
distribution at a reference map x0:

    eps(x; x0, a) = (x - sqrt(a) x0) / sqrt(1 - a).

Guidance combine (w = 0 unconditional, w = 1 conditional):

    eps = eps_u + w (eps_c - eps_u).

DDIM update (Song et al., ref. [7]) from abar a to abar a' with noise z:

    x0_hat = (x - sqrt(1 - a) eps) / sqrt(a)                (no clipping)
    x'     = sqrt(a') x0_hat + sqrt(max(0, 1 - a' - sigma^2)) eps + sigma z.

All functions are elementwise over numpy arrays, float64.
"""

from __future__ import annotations

import math

import numpy as np

from .schedule import ddim_sigma


def eps_point_mass(x, x0, a: float):
    return (x - math.sqrt(a) * x0) / math.sqrt(1.0 - a)


def cfg_combine(eps_c, eps_u, w):
    return eps_u + w * (eps_c - eps_u)


def ddim_update(x, eps, a: float, a_next: float, sigma: float, z):
    x0_hat = (x - math.sqrt(1.0 - a) * eps) / math.sqrt(a)
    c_dir = math.sqrt(max(0.0, 1.0 - a_next - sigma * sigma))
    out = math.sqrt(a_next) * x0_hat + c_dir * eps
    if sigma != 0.0:
        out = out + sigma * z
    return out


def ddim_cfg_step_eps(x, eps_c, eps_u, w, a: float, a_next: float, eta: float, z):
    """The same step when the conditional and unconditional noise predictions come
    from a network (buffers), not from the point-mass stand-in."""
    eps = cfg_combine(eps_c, eps_u, w)
    return ddim_update(x, eps, a, a_next, ddim_sigma(a, a_next, eta), z)


def ddim_cfg_step(x, x0c, x0u, w, a: float, a_next: float, eta: float, z):
    """One fused guidance + DDIM step.  ``w`` broadcasts against ``x``."""
    eps_c = eps_point_mass(x, x0c, a)
    eps_u = eps_point_mass(x, x0u, a)
    eps = cfg_combine(eps_c, eps_u, w)
    return ddim_update(x, eps, a, a_next, ddim_sigma(a, a_next, eta), z)
