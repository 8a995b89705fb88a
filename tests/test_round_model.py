"""The round cost model against simulation and against the schedule's own expected tokens."""
import numpy as np
import pytest

import oracle
from draft_head_verification_amd import round_model as RM


def test_expected_tokens_match_simulated_rounds():
    """E_b = 1 + sum_{k<L_b} P: simulate the verifier's left-to-right accept process with the
    per-position pass probabilities and count what a round emits (accepted prefix + 1)."""
    rng = np.random.default_rng(4)
    B, K, n = 6, 8, 200000
    s = rng.uniform(0.3, 0.95, (B, K))
    L = np.array([0, 1, 3, 8, 5, 8])
    r = RM.round_cost(RM.prefix_survival(s), L, [1.0, 100.0], [10.0, 1000.0], 0.0)
    for b in range(B):
        u = rng.random((n, K))
        passed = u < s[b][None, :]
        # accepted = length of the leading run of passes, capped at L_b
        acc = np.where(passed[:, : L[b]].all(axis=1), L[b], np.argmin(passed[:, : L[b]], axis=1)) if L[b] else np.zeros(n)
        emitted = acc + 1
        assert r["emitted"][b] == pytest.approx(emitted.mean(), abs=5 * emitted.std() / np.sqrt(n) + 1e-12)


def test_matches_the_schedules_expected_tokens():
    rng = np.random.default_rng(8)
    B, K = 40, 12
    C = rng.normal(1.0, 1.5, (B, K)).astype(np.float32)
    kt, kp = np.array([1.0, 200.0, 400.0]), np.array([20.0, 3000.0, 3500.0])
    o = oracle.schedule(C, kt, kp, True)
    P = RM.prefix_survival(1.0 / (1.0 + np.exp(-C.astype(np.float64))))
    r = RM.round_cost(P, o["verify_len"], kt, kp, 1e-4)
    np.testing.assert_allclose(r["emitted"], o["expected_tokens"], rtol=1e-14)
    # with no drafting time the round's throughput is the schedule's objective E(n) T(N)/N:
    # over every top-n set of the (P desc, position asc, request asc) ranking, the schedule's
    # lengths reach the model's maximum
    items = sorted(((-P[b, k], k, b) for b in range(B) for k in range(K)))
    best, L = -1.0, np.zeros(B, np.int64)
    thr = [RM.round_cost(P, L, kt, kp, 0.0)["throughput"]]
    for _, k, b in items:
        L[b] += 1
        thr.append(RM.round_cost(P, L, kt, kp, 0.0)["throughput"])
    mine = RM.round_cost(P, o["verify_len"], kt, kp, 0.0)["throughput"]
    assert mine == pytest.approx(max(thr), rel=1e-12)
    assert int(np.argmax(thr)) == int(o["verify_len"].sum())


def test_single_request_numbers():
    """One request, a flat curve: four drafted positions at 2 ms each, five target positions at
    500 tokens/s (10 ms), 1 + 0.9 + 0.8 + 0.6 + 0.5 = 3.8 expected tokens: 18 ms / 3.8."""
    P = np.array([[0.9, 0.8, 0.6, 0.5]])
    r = RM.round_cost(P, [4], [1.0, 2.0], [500.0, 500.0], 4 * 2e-3)
    assert r["t_verify"] == pytest.approx(0.010) and r["tokens"] == pytest.approx(3.8)
    assert r["time_per_token"] == pytest.approx(0.018 / 3.8)


def test_measured_round_from_trace():
    recs = ([("draft_prepare", 0.006)] + [("markov_head_step", 0.04), ("draft_reduce", 0.01)] * 16
            + [("schedule", 0.008), ("verify_rows", 0.05)]) * 3
    m = RM.MeasuredRound.from_trace(recs, 3, 16, [1.0, 100.0], [10.0, 1000.0])
    assert m.t_position == pytest.approx(50e-6) and m.t_fixed == pytest.approx(14e-6)
    assert m.draft_time(4) == pytest.approx(14e-6 + 4 * 50e-6)
    P = RM.prefix_survival(np.full((8, 16), 0.9))
    r, base, ratio = m.against_one_token(P, np.full(8, 16), 16)
    assert r["t_round"] == pytest.approx(m.draft_time(16) + 8 * 17 / 1000.0)
    assert base["N"] == 16 and ratio == pytest.approx(np.mean(r["per_user"]) / np.mean(base["per_user"]))


def test_profile_is_clamped_and_linear():
    kt, kp = [4.0, 20.0], [600.0, 2200.0]
    assert RM.profile(kt, kp, 1.0) == 600.0 and RM.profile(kt, kp, 50.0) == 2200.0
    assert RM.profile(kt, kp, 12.0) == pytest.approx(600.0 + 1600.0 * 0.5)


def test_compare_against_one_token_rounds():
    """More accepted tokens per round at a modest drafting cost beat one-token rounds in
    per-user speed; a drafter whose tokens are all rejected does not."""
    kt, kp = [1.0, 2048.0, 8704.0], [1e5 / 2048, 1e5, 1e5]
    B, K = 64, 16
    good = RM.prefix_survival(np.full((B, K), 0.8))
    bad = RM.prefix_survival(np.full((B, K), 0.05))
    _, _, up = RM.compare(good, np.full(B, K), kt, kp, 2e-3, np.full(B, 0.8), 1e-3)
    _, _, down = RM.compare(bad, np.full(B, K), kt, kp, 2e-3, np.full(B, 0.05), 1e-3)
    assert up > 1.0 > down
