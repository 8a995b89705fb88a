"""Pins of the oracle's online calibration of the confidence logits (CPU only).

The oracle (oracle_calibrate_step / oracle_ece in oracle/dspark_oracle.c) takes one damped
Newton step per round on the log-loss of the tested positions.  These tests pin it to things
other than its own formulas: finite differences of a separately written loss, the minimiser
scipy finds for that loss, recovery of a known temperature from chains drawn by simulating
the verifier's sequential accept process, invariances, and a hand-computed ECE.
"""
import numpy as np
import pytest
from scipy.optimize import minimize_scalar

import oracle


def draw_chains(C, theta_true, L, rng):
    """Accepted lengths of chains whose position k passes with probability
    sigmoid(theta_true[k] * C[b, k]) once every earlier position passed (the verifier's own
    left-to-right process), stopping at the first failure or at L[b]."""
    B, K = C.shape
    p = 1.0 / (1.0 + np.exp(-theta_true[None, :] * C.astype(np.float64)))
    u = rng.random((B, K))
    a = np.empty(B, np.int32)
    for b in range(B):
        n = 0
        while n < L[b] and u[b, n] < p[b, n]:
            n += 1
        a[b] = n
    return a


def chain_loss(theta, C, L, a, k):
    """Negative log-likelihood of the observed outcomes at position k under
    P(pass) = sigmoid(theta * C): only chains that reached position k (every earlier position
    passed, and k is inside the verified length) observe it."""
    reached = (np.arange(len(L)) >= 0) & (L > k) & (a >= k)
    c = C[reached, k].astype(np.float64)
    passed = a[reached] > k
    z = theta * c
    # -log sigmoid(z) for passes, -log(1 - sigmoid(z)) for failures
    return float(np.sum(np.logaddexp(0.0, -z[passed])) + np.sum(np.logaddexp(0.0, z[~passed])))


def _data(seed, B=300, K=6):
    rng = np.random.default_rng(seed)
    C = (rng.normal(1.2, 1.3, (B, K)) - 0.1 * np.arange(K)).astype(np.float32)
    L = rng.integers(0, K + 1, B).astype(np.int32)
    a = draw_chains(C, np.full(K, 0.6), L, rng)
    return C, L, a, rng


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_step_is_damped_newton_on_the_chain_log_loss(seed):
    C, L, a, rng = _data(seed)
    K = C.shape[1]
    th0 = rng.uniform(0.4, 1.6, K)
    step, ridge = 0.7, 0.05
    th1 = oracle.calibrate_step(C, L, a, th0, step=step, ridge=ridge)
    h = 1e-4
    for k in range(K):
        f0 = chain_loss(th0[k], C, L, a, k)
        fp = chain_loss(th0[k] + h, C, L, a, k)
        fm = chain_loss(th0[k] - h, C, L, a, k)
        d1 = (fp - fm) / (2 * h)
        d2 = (fp - 2 * f0 + fm) / (h * h)
        want = np.clip(th0[k] - step * d1 / (d2 + ridge), 1 / 64, 64)
        assert th1[k] == pytest.approx(want, rel=1e-6, abs=1e-7), (k, th1[k], want)


def test_iterated_steps_reach_the_maximum_likelihood():
    C, L, a, _ = _data(7, B=2000)
    K = C.shape[1]
    th = np.ones(K)
    for _ in range(60):
        th = oracle.calibrate_step(C, L, a, th, step=1.0, ridge=1e-12)
    for k in range(K):
        res = minimize_scalar(lambda t: chain_loss(t, C, L, a, k), bounds=(1 / 64, 64),
                              method="bounded", options={"xatol": 1e-10})
        assert th[k] == pytest.approx(res.x, rel=1e-5), (k, th[k], res.x)


def test_unreached_positions_do_not_move_the_estimate():
    C, L, a, rng = _data(11, B=200)
    K = C.shape[1]
    th0 = np.full(K, 0.9)
    base = oracle.calibrate_step(C, L, a, th0, step=0.5, ridge=0.01)
    C2 = C.copy()
    for b in range(C.shape[0]):
        for k in range(K):
            if not (k < L[b] and k <= a[b]):  # never tested in this round
                C2[b, k] = rng.normal(0, 5)
    assert np.array_equal(oracle.calibrate_step(C2, L, a, th0, step=0.5, ridge=0.01), base)
    # a tested position does move it
    b = int(np.nonzero((L > 0))[0][0])
    C3 = C.copy()
    C3[b, 0] += 1.0
    assert not np.array_equal(oracle.calibrate_step(C3, L, a, th0, step=0.5, ridge=0.01), base)


def test_no_observation_keeps_theta_and_clamps_apply():
    C = np.ones((4, 3), np.float32)
    L = np.zeros(4, np.int32)  # nothing verified
    th = np.array([0.3, 1.0, 7.0])
    assert np.array_equal(oracle.calibrate_step(C, L, np.zeros(4, np.int32), th), th)
    # every chain passes every position with a huge confidence: the step is clamped at 64
    L = np.full(4, 3, np.int32)
    big = oracle.calibrate_step(np.full((4, 3), -30.0, np.float32), L, L, np.full(3, 60.0),
                                step=1.0, ridge=1e-12)
    assert np.all(big <= 64.0) and np.all(big >= 1 / 64)


def test_online_rounds_recover_the_temperature_and_cut_ece():
    """An over-confident drafter: the real pass probability is sigmoid(C / 2), the raw score
    sigmoid(C).  Online steps over rounds of fresh chains bring theta to about 1/2 and the
    calibration error on held-out chains from several percent to about one."""
    rng = np.random.default_rng(5)
    B, K, rounds = 512, 8, 30
    theta_true = np.full(K, 0.5)
    th = np.ones(K)

    def round_data():
        C = (rng.normal(1.5, 1.0, (B, K)) - 0.15 * np.arange(K)).astype(np.float32) * 2.0
        L = np.full(B, K, np.int32)
        return C, L, draw_chains(C, theta_true, L, rng)

    for _ in range(rounds):
        C, L, a = round_data()
        th = oracle.calibrate_step(C, L, a, th, step=0.5, ridge=1e-3)
    assert np.all(np.abs(th[:4] - 0.5) < 0.05), th
    # held-out chains: predictions vs outcomes on the positions they tested
    C, L, a = round_data()
    s_raw, s_cal, y = [], [], []
    for b in range(B):
        for k in range(min(a[b] + 1, L[b])):
            s_raw.append(1 / (1 + np.exp(-float(C[b, k]))))
            s_cal.append(1 / (1 + np.exp(-th[k] * float(C[b, k]))))
            y.append(1.0 if k < a[b] else 0.0)
    e_raw, e_cal = oracle.ece(s_raw, y), oracle.ece(s_cal, y)
    assert e_raw > 0.05 and e_cal < 0.02, (e_raw, e_cal)


def test_ece_by_hand():
    # bins of width 0.5: {0.1, 0.2 | y 0, 1} and {0.7, 0.9, 0.6 | y 1, 1, 0}
    s = [0.1, 0.2, 0.7, 0.9, 0.6]
    y = [0, 1, 1, 1, 0]
    want = (2 / 5) * abs(0.5 - 0.15) + (3 / 5) * abs(2 / 3 - 2.2 / 3)
    assert oracle.ece(s, y, n_bins=2) == pytest.approx(want, abs=1e-15)
    assert oracle.ece([1.0, 1.0], [1, 1], n_bins=10) == 0.0  # s = 1 lands in the last bin
    rng = np.random.default_rng(3)
    sp = rng.random(200000)
    assert oracle.ece(sp, (rng.random(200000) < sp).astype(float)) < 0.01


@pytest.mark.parametrize("theta", [0.5, 2.0, 0.25])
def test_schedule_inverse_temperature_scales_the_logits(theta):
    """Survival with inverse temperature theta equals the raw survival of theta * C (powers
    of two keep the scaled float logits exact)."""
    rng = np.random.default_rng(9)
    B, K = 24, 8
    C = rng.normal(1.0, 1.5, (B, K)).astype(np.float32)
    kt = np.array([1.0, 64.0, 256.0])
    kp = np.array([10.0, 600.0, 900.0])
    th = np.full(K, theta)
    a = oracle.schedule(C, kt, kp, True, inv_temp=th)
    b = oracle.schedule((C * np.float32(theta)).astype(np.float32), kt, kp, True)
    assert np.array_equal(a["verify_len"], b["verify_len"])
    np.testing.assert_allclose(a["expected_tokens"], b["expected_tokens"], rtol=0, atol=0)
    # theta = 1 everywhere is the raw schedule
    c = oracle.schedule(C, kt, kp, True, inv_temp=np.ones(K))
    d = oracle.schedule(C, kt, kp, True)
    assert np.array_equal(c["verify_len"], d["verify_len"])
