"""GPU parity of the confidence schedule across batch shapes, ties and profiles.

The schedule ranks every (request, position) item by its prefix survival probability and
cuts the ranked list where expected emitted tokens per unit of verify time peak.  These cases
cover the sizes the kernel's merge rounds see (one round per doubling of the run length, up
to the 8192-item limit), ragged draft lengths, exact ties between requests (equal confidence
rows give bit-equal products; the order is then position, then request), items whose
survival is exactly zero, and linear, knee and irregular throughput profiles.  E(n) is
rounded once from the exact sum on both sides and the objective is evaluated with the same
float64 operations, so the scheduled lengths agree bit for bit whenever the two sides' prefix
products do; the products go through each side's float64 exp, which may round differently in
the last place, so a different length is accepted only where the oracle's best objective
leads the runner-up by less than 1e-12, and every such case is counted in the parity tally.
The hand-derived tie cases (tests/golden/schedule_ties.json) must come out exactly.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from draft_head_verification_amd import synth
from parity import Tally

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "schedule_ties.json")

pytestmark = pytest.mark.gpu

PROFILES = {
    "knee": synth.KNEE_PROFILE,
    "linear": synth.LINEAR_PROFILE,
    "irregular": ((3.0, 900.0), (40.0, 5000.0), (300.0, 21000.0), (1500.0, 26000.0),
                  (6000.0, 24000.0)),
}

CASES = [  # B, K, ragged, conf kind, profile
    (1, 1, False, "normal", "linear"),
    (3, 5, True, "normal", "irregular"),
    (64, 4, False, "normal", "knee"),
    (100, 7, True, "ties", "irregular"),
    (256, 16, False, "normal", "knee"),
    (256, 16, True, "ties", "knee"),
    (512, 16, False, "normal", "knee"),
    (512, 16, True, "zeros", "irregular"),
    (8192, 1, False, "ties", "knee"),
    (1000, 8, True, "normal", "linear"),
    (128, 64, True, "ties", "knee"),   # the largest draft length, 8192 items
    (1, 64, False, "normal", "irregular"),
    (300, 3, True, "zeros", "linear"),
]


def _inputs(B, K, ragged, kind, seed):
    g = torch.Generator().manual_seed(seed)
    conf = 1.5 + torch.randn(B, K, generator=g) - 0.15 * torch.arange(K)
    if kind == "ties":
        # few distinct rows: many requests share a confidence row, so their products tie
        rows = torch.round(torch.randn(7, K, generator=g) * 2) / 2 + 1.0
        conf = rows[torch.randint(0, 7, (B,), generator=g)]
    elif kind == "zeros":
        # survival exactly 0 in float64 from some position on, for a third of the requests
        cut = torch.randint(0, K, (B,), generator=g)
        dead = (torch.arange(K)[None, :] >= cut[:, None]) & (torch.arange(B)[:, None] % 3 == 0)
        conf = torch.where(dead, torch.full_like(conf, -1000.0), conf)
    dlen = (torch.randint(0, K + 1, (B,), generator=g, dtype=torch.int32) if ragged
            else torch.full((B,), K, dtype=torch.int32))
    return conf.float().contiguous(), dlen


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}K{c[1]}{'r' if c[2] else ''}-{c[3]}-{c[4]}"
                                             for c in CASES])
def test_schedule_matches_oracle(case):
    from draft_head_verification_amd import dspark as D
    B, K, ragged, kind, prof = case
    print(f"[schedule] B={B} K={K} ragged={ragged} {kind} {prof}", flush=True)
    conf, dlen = _inputs(B, K, ragged, kind, seed=7 * B + K)
    kt = torch.tensor([p[0] for p in PROFILES[prof]], dtype=torch.float64)
    kp = torch.tensor([p[1] for p in PROFILES[prof]], dtype=torch.float64)
    o = oracle.schedule(conf, kt, kp, True, draft_len=dlen)
    gs = D.schedule(conf.cuda(), kt.cuda(), kp.cuda(), True, draft_len=dlen.cuda())
    assert D.dspark_query_device_status(gs["workspace"]) == 0
    gvl = gs["verify_len"].cpu().numpy()
    tally = Tally()
    if not np.array_equal(gvl, o["verify_len"]):
        assert o["margin"] < 1e-12, ("schedule differs away from a tie", o["margin"])
        tally.schedule_near_ties += 1
    tally.compared_positions += int(dlen.sum())
    tally.report(f"schedule-B{B}K{K}{'r' if ragged else ''}-{kind}-{prof}")
    assert np.all((gvl >= 0) & (gvl <= dlen.numpy()))
    get = gs["expected_tokens"].cpu().numpy()
    np.testing.assert_allclose(get, o["expected_tokens"], rtol=1e-12, atol=0)
    print(f"[schedule] expected tokens bit-equal for {int((get == o['expected_tokens']).sum())} "
          f"of {B} requests", flush=True)
    # with scheduling off every request verifies its whole draft
    g0 = D.schedule(conf.cuda(), kt.cuda(), kp.cuda(), False, draft_len=dlen.cuda())
    np.testing.assert_array_equal(g0["verify_len"].cpu().numpy(), dlen.numpy())
    print(f"[schedule] n*={o['n_star']} of {int(dlen.sum())} items, margin {o['margin']:.3g}",
          flush=True)


def test_schedule_off_beyond_the_item_limit():
    """With scheduling off the batch may exceed the 8192 ranked items (B = 2000, K = 64):
    every request verifies its draft and the expected tokens are formed by the
    scheduling-off kernel alone."""
    from draft_head_verification_amd import dspark as D
    B, K = 2000, 64
    conf, dlen = _inputs(B, K, True, "normal", seed=11)
    kt = torch.tensor([p[0] for p in PROFILES["knee"]], dtype=torch.float64)
    kp = torch.tensor([p[1] for p in PROFILES["knee"]], dtype=torch.float64)
    o = oracle.schedule(conf, kt, kp, False, draft_len=dlen)
    g = D.schedule(conf.cuda(), kt.cuda(), kp.cuda(), False, draft_len=dlen.cuda())
    assert D.dspark_query_device_status(g["workspace"]) == 0
    np.testing.assert_array_equal(g["verify_len"].cpu().numpy(), dlen.numpy())
    np.testing.assert_array_equal(o["verify_len"], dlen.numpy())
    np.testing.assert_allclose(g["expected_tokens"].cpu().numpy(), o["expected_tokens"],
                               rtol=1e-12, atol=0)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_tie_rules_hand_derived_gpu(case):
    """The hand-derived tie cases: ranking at equal survival (position, then request) and the
    smallest n among exactly equal objectives, through the GPU."""
    from draft_head_verification_amd import dspark as D
    conf = torch.tensor(case["conf_logits"], dtype=torch.float32, device="cuda")
    kt = torch.tensor(case["knot_tokens"], dtype=torch.float64, device="cuda")
    kp = torch.tensor(case["knot_tps"], dtype=torch.float64, device="cuda")
    g = D.schedule(conf, kt, kp, True)
    assert D.dspark_query_device_status(g["workspace"]) == 0
    np.testing.assert_array_equal(g["verify_len"].cpu().numpy(), case["verify_len"])
    np.testing.assert_array_equal(g["expected_tokens"].cpu().numpy(), case["expected_tokens"])
