"""Pins for the oracle's schedule, stand-in denoiser, guidance combine and DDIM step."""

import math

import numpy as np
import pytest

from oracle import ddim, sampler, schedule
from workloads import get, reference_maps

AB = schedule.alpha_bar()
BETA = schedule.betas()


def test_beta_endpoints_and_first_alpha_bar():
    assert BETA[0] == 1e-4 and BETA[-1] == pytest.approx(0.02, rel=1e-15)
    assert AB[0] == 1.0 - 1e-4
    assert np.all(np.diff(AB) < 0)


def test_alpha_bar_between_exponential_bounds():
    # -x/(1-x) <= log(1-x) <= -x, and sum_{s<=t} beta_s is an arithmetic series
    for t in (0, 19, 499, 980, 999):
        n = t + 1
        sbeta = n * 1e-4 + (0.02 - 1e-4) * (t * (t + 1) / 2) / 999
        hi = math.exp(-sbeta)
        lo = math.exp(-sbeta / (1.0 - BETA[t]))
        assert lo <= AB[t] <= hi


def test_ddim_grids():
    assert list(schedule.ddim_timesteps(50)) == list(range(980, -1, -20))
    assert list(schedule.ddim_timesteps(1000)) == list(range(999, -1, -1))
    assert list(schedule.ddim_timesteps(250))[:3] == [996, 992, 988]
    for n in (50, 250, 500, 1000):
        pairs = schedule.ddim_pairs(n)
        assert len(pairs) == n
        assert pairs[-1][1] == 1.0 and pairs[-1][0] == AB[0]
        for (a, an), (b, _) in zip(pairs, pairs[1:]):
            assert an == b and a < an
    with pytest.raises(ValueError):
        schedule.ddim_timesteps(3)


def test_sigma_eta1_stride1_is_ddpm_posterior_std():
    # DDPM (Ho et al.) posterior variance: beta~_t = (1 - abar_{t-1}) / (1 - abar_t) * beta_t
    for t in (1, 2, 50, 500, 999):
        post = (1.0 - AB[t - 1]) / (1.0 - AB[t]) * BETA[t]
        assert schedule.ddim_sigma(AB[t], AB[t - 1], 1.0) ** 2 == pytest.approx(post, rel=1e-10)
        assert schedule.ddim_sigma(AB[t], AB[t - 1], 0.0) == 0.0
    assert schedule.ddim_sigma(AB[0], 1.0, 1.0) == 0.0


def test_point_mass_denoiser_returns_the_true_noise():
    rng = np.random.default_rng(0)
    x0 = rng.uniform(1, 20, 2016)
    eps = rng.standard_normal(2016)
    for a in (AB[999], AB[500], AB[0]):
        x = math.sqrt(a) * x0 + math.sqrt(1 - a) * eps
        assert np.allclose(ddim.eps_point_mass(x, x0, a), eps, rtol=0, atol=1e-9)


def test_cfg_endpoints():
    rng = np.random.default_rng(1)
    ec, eu = rng.standard_normal((2, 100))
    assert np.array_equal(ddim.cfg_combine(ec, eu, 0.0), eu)
    assert np.allclose(ddim.cfg_combine(ec, eu, 1.0), ec, rtol=1e-15, atol=1e-15)
    assert np.allclose(ddim.cfg_combine(ec, eu, 3.0), 3 * ec - 2 * eu)


def test_stride1_eta1_step_equals_ddpm_posterior_mean_plus_noise():
    # With the point-mass denoiser x0_hat = x0*, and DDIM(eta=1) at stride 1 is the DDPM
    # ancestral step: x_{t-1} = c0 x0_hat + ct x_t + sigma z with
    # c0 = sqrt(abar_{t-1}) beta_t / (1 - abar_t), ct = sqrt(alpha_t) (1 - abar_{t-1}) / (1 - abar_t).
    rng = np.random.default_rng(2)
    x0c, x0u = rng.uniform(1, 20, (2, 2016))
    w = 0.7
    xstar = x0u + w * (x0c - x0u)
    for t in (1, 300, 999):
        a, ap = AB[t], AB[t - 1]
        x = rng.standard_normal(2016) * 2
        z = rng.standard_normal(2016)
        got = ddim.ddim_cfg_step(x, x0c, x0u, w, a, ap, 1.0, z)
        c0 = math.sqrt(ap) * BETA[t] / (1 - a)
        ct = math.sqrt(1 - BETA[t]) * (1 - ap) / (1 - a)
        want = c0 * xstar + ct * x + math.sqrt((1 - ap) / (1 - a) * BETA[t]) * z
        assert np.allclose(got, want, rtol=1e-11, atol=1e-11)


def test_identity_when_abar_does_not_move():
    rng = np.random.default_rng(3)
    x0c, x0u, x = rng.uniform(1, 20, (3, 50))
    for a in (AB[900], AB[10]):
        y = ddim.ddim_cfg_step(x, x0c, x0u, 0.3, a, a, 0.0, 0.0)
        assert np.allclose(y, x, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("eta", [0.0, 1.0])
@pytest.mark.parametrize("w", [0.0, 1.0, 0.5, 2.0])
def test_trajectory_lands_on_guided_reference(eta, w):
    x0c, x0u = reference_maps(get("single_region"), 0)
    M = 4
    fin, _ = sampler.run_independent(np.repeat(x0c, M, 0), np.repeat(x0u, M, 0), [w] * M, np.arange(M),
                                     seed=7, n_steps=50, eta=eta)
    xstar = x0u.astype(np.float64) + w * (x0c.astype(np.float64) - x0u.astype(np.float64))
    assert np.allclose(fin, np.repeat(xstar, M, 0), rtol=0, atol=1e-9)


def test_eta0_intermediate_states_closed_form():
    x0c, x0u = reference_maps(get("single_region"), 1)
    x0c = x0c.astype(np.float64)
    x0u = x0u.astype(np.float64)
    w = np.array([0.0, 1.0, 0.25])
    M = w.size
    rec_steps = set(range(0, 51))
    _, rec = sampler.run_independent(np.repeat(x0c, M, 0), np.repeat(x0u, M, 0), w, np.arange(M),
                                     seed=3, n_steps=50, eta=0.0, record=rec_steps)
    xstar = x0u + w[:, None] * (x0c - x0u)
    pairs = schedule.ddim_pairs(50)
    a0 = pairs[0][0]
    eps_star = (rec[0] - math.sqrt(a0) * xstar) / math.sqrt(1 - a0)
    for i in range(1, 50):
        ai = pairs[i - 1][1]
        want = math.sqrt(ai) * xstar + math.sqrt(1 - ai) * eps_star
        assert np.allclose(rec[i], want, rtol=0, atol=1e-9)


def test_eta1_standardised_residual_statistics():
    # rho_i = (x_i - sqrt(a'_i) x0*) / sqrt(1 - a'_i) is Gaussian per element with unit variance
    # and mean m_i = m_{i-1} sqrt(1 - a' - sigma^2) / sqrt(1 - a'), m_{-1} = -sqrt(a_0) x0* / sqrt(1 - a_0).
    wl = get("region_ensemble")
    x0c, x0u = reference_maps(wl, 0)
    x0c = x0c.astype(np.float64)
    x0u = x0u.astype(np.float64)
    M = 200
    w = np.tile([0.0, 1.0], M // 2)
    steps = {1, 10, 25, 49}
    _, rec = sampler.run_independent(np.repeat(x0c, M, 0), np.repeat(x0u, M, 0), w, np.arange(M),
                                     seed=11, n_steps=50, eta=1.0, record=steps)
    xstar = x0u + w[:, None] * (x0c - x0u)
    pairs = schedule.ddim_pairs(50)
    a0 = pairs[0][0]
    m = -math.sqrt(a0) * xstar / math.sqrt(1 - a0)
    for i, (a, an) in enumerate(pairs[:49]):
        sig = schedule.ddim_sigma(a, an, 1.0)
        m = m * math.sqrt(1 - an - sig * sig) / math.sqrt(1 - an)
        if i + 1 in steps:
            rho = (rec[i + 1] - math.sqrt(an) * xstar) / math.sqrt(1 - an)
            r = (rho - m).reshape(-1)
            assert abs(r.mean()) < 5.0 / math.sqrt(r.size)
            assert abs(r.var() - 1.0) < 0.01


def test_cosine_schedule_telescopes():
    # without clipping, prod_{i<=t} (1 - beta_i) = prod f(i+1)/f(i) = f(t+1)/f(0)
    b = schedule.betas_cosine()
    ab = schedule.alpha_bar_from_betas(b)

    def f(u):
        return math.cos((u + 0.008) / 1.008 * math.pi / 2) ** 2

    clipped = np.nonzero(b >= 0.999)[0]
    first_clip = clipped[0] if clipped.size else len(b)
    assert first_clip >= 990   # only the very end of the schedule is clipped
    for t in (0, 1, 100, 500, 900, first_clip - 1):
        assert ab[t] == pytest.approx(f((t + 1) / 1000) / f(0.0), rel=1e-12)
    assert np.all(np.diff(ab) < 0) and np.all(b <= 0.999)
    pairs = schedule.ddim_pairs(50, ab=ab)
    assert pairs[0][0] == ab[980] and pairs[-1] == (ab[0], 1.0)


def test_eps_buffer_step():
    rng = np.random.default_rng(4)
    x0 = rng.uniform(1, 20, 2016)
    eps = rng.standard_normal(2016)
    a, an = AB[700], AB[680]
    x = math.sqrt(a) * x0 + math.sqrt(1 - a) * eps
    # true noise on both branches: x0_hat = x0 exactly, so the step is the closed form below
    for eta in (0.0, 1.0):
        z = rng.standard_normal(2016)
        sig = schedule.ddim_sigma(a, an, eta)
        want = math.sqrt(an) * x0 + math.sqrt(1 - an - sig * sig) * eps + sig * z
        got = ddim.ddim_cfg_step_eps(x, eps, eps + 3.0, 1.0, a, an, eta, z)   # w = 1 ignores eps_u
        assert np.allclose(got, want, rtol=0, atol=1e-10)
    # point-mass predictions as buffers reproduce the stand-in step
    x0c, x0u = rng.uniform(1, 20, (2, 2016))
    ec, eu = ddim.eps_point_mass(x, x0c, a), ddim.eps_point_mass(x, x0u, a)
    z = rng.standard_normal(2016)
    assert np.allclose(ddim.ddim_cfg_step_eps(x, ec, eu, 0.3, a, an, 1.0, z),
                       ddim.ddim_cfg_step(x, x0c, x0u, 0.3, a, an, 1.0, z), rtol=0, atol=1e-12)
