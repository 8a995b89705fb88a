"""GPU parity of the online calibration step and of the schedule's per-position inverse
temperatures against the CPU oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
from draft_head_verification_amd import synth

pytestmark = pytest.mark.gpu

TOL_THETA = 1e-12  # float64 sums in a different order


def _case(seed, B, K, bad=False):
    rng = np.random.default_rng(seed)
    C = (rng.normal(1.0, 2.0, (B, K)) - 0.1 * np.arange(K)).astype(np.float32)
    L = rng.integers(0, K + 1, B).astype(np.int32)
    a = np.minimum(rng.integers(0, K + 1, B), L).astype(np.int32)
    if B >= 4:  # edge rows: nothing verified, all accepted, first rejected, full length
        L[0], a[0] = 0, 0
        L[1], a[1] = K, K
        L[2], a[2] = K, 0
        L[3], a[3] = 1, 1
    if bad:
        L[1], a[2], L[3], a[3] = K + 3, -2, -1, 5
    th = rng.uniform(0.3, 2.5, K)
    return C, L, a, th


@pytest.mark.parametrize("B,K", [(1, 1), (7, 5), (256, 16), (1000, 16), (300, 64)])
def test_calibrate_step_parity(B, K):
    from draft_head_verification_amd import dspark as D
    C, L, a, th = _case(B * 131 + K, B, K)
    for step, ridge in ((1.0, 1e-3), (0.35, 0.2)):
        g_th = torch.from_numpy(th.copy()).cuda()
        out = D.calibrate(torch.from_numpy(C).cuda(), torch.from_numpy(L).cuda(),
                          torch.from_numpy(a).cuda(), g_th, step=step, ridge=ridge)
        assert D.dspark_query_device_status(out["workspace"]) == 0
        want = oracle.calibrate_step(C, L, a, th, step=step, ridge=ridge)
        np.testing.assert_allclose(g_th.cpu().numpy(), want, rtol=TOL_THETA, atol=1e-15)


def test_calibrate_flags_and_clamps_bad_lengths():
    from draft_head_verification_amd import dspark as D
    C, L, a, th = _case(3, 64, 8, bad=True)
    g_th = torch.from_numpy(th.copy()).cuda()
    out = D.calibrate(torch.from_numpy(C).cuda(), torch.from_numpy(L).cuda(),
                      torch.from_numpy(a).cuda(), g_th, step=0.8, ridge=1e-2)
    bits = D.dspark_query_device_status(out["workspace"])
    assert bits & D.DEV_BAD_LENGTH
    want = oracle.calibrate_step(C, L, a, th, step=0.8, ridge=1e-2)
    np.testing.assert_allclose(g_th.cpu().numpy(), want, rtol=TOL_THETA, atol=1e-15)


def test_online_rounds_track_the_oracle():
    """Twenty rounds of chains drawn from an over-confident drafter: the device's theta stays
    with the oracle's round after round, and both approach the true 1/2."""
    from draft_head_verification_amd import dspark as D
    rng = np.random.default_rng(17)
    B, K = 512, 8
    th_o = np.ones(K)
    th_g = torch.ones(K, dtype=torch.float64, device="cuda")
    ws = None
    for _ in range(20):
        C = ((rng.normal(1.5, 1.0, (B, K)) - 0.15 * np.arange(K)) * 2.0).astype(np.float32)
        p = 1 / (1 + np.exp(-0.5 * C.astype(np.float64)))
        u = rng.random((B, K))
        a = np.array([next((k for k in range(K) if u[b, k] >= p[b, k]), K) for b in range(B)],
                     np.int32)
        L = np.full(B, K, np.int32)
        th_o = oracle.calibrate_step(C, L, a, th_o, step=0.5, ridge=1e-3)
        ws = D.calibrate(torch.from_numpy(C).cuda(), torch.from_numpy(L).cuda(),
                         torch.from_numpy(a).cuda(), th_g, step=0.5, ridge=1e-3,
                         workspace=ws)["workspace"]
        np.testing.assert_allclose(th_g.cpu().numpy(), th_o, rtol=1e-10)
    assert np.all(np.abs(th_o[:4] - 0.5) < 0.06), th_o


@pytest.mark.parametrize("name", ["tiny", "concurrent"])
def test_schedule_with_inverse_temperatures(name):
    from draft_head_verification_amd import dspark as D
    w = synth.shrink(synth.WORKLOADS[name], V=1208)  # the schedule does not read logits
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(23)
    th = rng.uniform(0.4, 1.8, w.K)
    g = D.schedule(inp["conf_logits"].cuda(), inp["knot_tokens"].cuda(), inp["knot_tps"].cuda(),
                   True, draft_len=inp["draft_len"].cuda(),
                   inv_temp=torch.from_numpy(th).cuda())
    assert D.dspark_query_device_status(g["workspace"]) == 0
    o = oracle.schedule(inp["conf_logits"], inp["knot_tokens"], inp["knot_tps"], True,
                        draft_len=inp["draft_len"], inv_temp=th)
    gvl = g["verify_len"].cpu().numpy()
    if not np.array_equal(gvl, o["verify_len"]):
        assert o["margin"] < 1e-12, ("schedule differs away from a tie", o["margin"])
    else:
        np.testing.assert_allclose(g["expected_tokens"].cpu().numpy(), o["expected_tokens"],
                                   rtol=1e-12, atol=0)
    # the temperatures change the schedule of this workload (so the test sees them)
    o1 = oracle.schedule(inp["conf_logits"], inp["knot_tokens"], inp["knot_tps"], True,
                         draft_len=inp["draft_len"])
    assert not np.array_equal(o1["expected_tokens"], o["expected_tokens"])
