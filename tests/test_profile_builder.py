"""The verify-throughput curve builder: knot assembly on the CPU, a measured curve on the GPU
that the schedule accepts."""
import numpy as np
import pytest
import torch

import oracle


def test_knots_from_timings():
    from draft_head_verification_amd.profile_builder import knots_from_timings
    kt, kp = knots_from_timings([(34, 2e-5), (17, 1e-5), (34, 4e-5), (34, 3e-5), (68, 2e-5)])
    np.testing.assert_array_equal(kt, [17.0, 34.0, 68.0])
    np.testing.assert_allclose(kp, [17 / 1e-5, 34 / 3e-5, 68 / 2e-5])
    with pytest.raises(ValueError):
        knots_from_timings([(0, 1e-5)])


@pytest.mark.gpu
def test_measured_curve_feeds_the_schedule():
    from draft_head_verification_amd import dspark as D
    from draft_head_verification_amd.profile_builder import measure_verify_curve
    kt, kp = measure_verify_curve([(1, 0), (4, 3), (16, 7), (64, 7), (128, 16)], V=19008,
                                  reps=2)
    assert np.all(np.diff(kt) > 0) and np.all(kp > 0)
    print("[verify curve] " + ", ".join(f"N={int(n)}: {t / 1e6:.2f} M tokens/s"
                                        for n, t in zip(kt, kp)), flush=True)
    rng = np.random.default_rng(2)
    C = rng.normal(1.5, 1.0, (64, 16)).astype(np.float32)
    g = D.schedule(torch.from_numpy(C).cuda(), torch.from_numpy(kt).cuda(),
                   torch.from_numpy(kp).cuda(), True)
    assert D.dspark_query_device_status(g["workspace"]) == 0
    o = oracle.schedule(C, kt, kp, True)
    gl = g["verify_len"].cpu().numpy()
    assert np.array_equal(gl, o["verify_len"]) or o["margin"] < 1e-12
