"""The round cost model built from a real measured run: the per-kernel HIP-event times of traced
rounds and the verify throughput curve measured on this GPU.  Its expected emitted tokens per
request equal the GPU schedule's expected_tokens (both 1 + sum of the verified prefix survival
products), and its predicted round time agrees with the measured round (the curve is measured
with every position accepted, so the prediction sits at or above the early-exit round).  The
measured round is the same three calls captured as one HIP graph and replayed, as a serving
loop runs it: GPU time against the model's GPU times (an eager round at this small size also
pays the host's launch gaps, about as long again as its kernels)."""
import numpy as np
import pytest
import torch

from draft_head_verification_amd import synth

pytestmark = pytest.mark.gpu


def test_model_from_measured_round():
    from draft_head_verification_amd import dspark as D
    from draft_head_verification_amd import profile_builder as PB
    from draft_head_verification_amd import round_model as RM
    w = synth.shrink(synth.WORKLOADS["headline_sched"], V=19008, B=64, K=8)
    inp = synth.make_inputs(w, device="cuda")
    Z = inp["Z_ext"][:, : w.K].contiguous()
    kt, kp = PB.measure_verify_curve([(b, l) for b in (1, 16, 64) for l in (0, 3, 7)],
                                     V=w.V, r=w.r, K=w.K, y_dtype=w.y_dtype, reps=2)
    # the schedule against the measured curve of this verifier
    kt_d, kp_d = torch.from_numpy(kt).cuda(), torch.from_numpy(kp).cuda()
    trace = D.Trace(capacity=512)
    rounds, times = 3, []
    for i in range(rounds + 1):
        tr = trace if i > 0 else None  # the first round warms up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        d = D.draft_block(Z, inp["U"], inp["W"], inp["prev_token"], inp["temperature"],
                          inp["seed"], req_id=inp["req_id"], trace=tr, want_corrected=(i == 0))
        s = D.schedule(inp["conf_logits"], kt_d, kp_d, True, trace=tr)
        if i == 0:
            corr = inp["Z_ext"].float()
            corr[:, : w.K] = d["corrected"]
            Y = synth.target_logits(corr, inp["noise"], w.y_dtype)
        v = D.verify(Y, d["tokens"], d["q_tok"], d["q_lse"], Z, inp["U"], inp["W"],
                     inp["prev_token"], s["verify_len"], inp["temperature"], inp["seed"],
                     req_id=inp["req_id"], trace=tr)
        e1.record()
        torch.cuda.synchronize()
        if i > 0:
            times.append(e0.elapsed_time(e1) * 1e-3)
    # the measured round: one captured graph of the three calls, timed over replays
    B, K = w.B, w.K
    toks = torch.empty(B, K, dtype=torch.int32, device="cuda")
    q_tok = torch.empty(B, K, device="cuda")
    q_lse = torch.empty(B, K, device="cuda")
    vlen = torch.empty(B, dtype=torch.int32, device="cuda")
    exp_tok = torch.empty(B, dtype=torch.float64, device="cuda")
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    ws_d = torch.empty(D.dspark_draft_workspace_size(B, K, w.V, w.r), dtype=torch.uint8,
                       device="cuda")
    ws_s = torch.empty(max(256, D.dspark_schedule_workspace_size(B, K)), dtype=torch.uint8,
                       device="cuda")
    ws_v = torch.empty(D.dspark_verify_workspace_size(B, K, w.V, w.r), dtype=torch.uint8,
                       device="cuda")

    def step():
        D.dspark_draft_block(Z, inp["U"], inp["W"], inp["prev_token"], inp["temperature"],
                             inp["seed"], toks, q_tok, q_lse, req_id=inp["req_id"],
                             workspace=ws_d)
        D.dspark_schedule(inp["conf_logits"], vlen, kt_d, kp_d, True, expected_tokens=exp_tok,
                          workspace=ws_s)
        D.dspark_verify(Y, toks, q_tok, q_lse, Z, inp["U"], inp["W"], inp["prev_token"], vlen,
                        inp["temperature"], inp["seed"], acc, nxt, req_id=inp["req_id"],
                        workspace=ws_v)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    n_rep = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_rep):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_time = e0.elapsed_time(e1) * 1e-3 / n_rep
    for ws in (ws_d, ws_s, ws_v):
        assert D.dspark_query_device_status(ws) == 0
    m = RM.MeasuredRound.from_trace(trace.records(), rounds, w.K, kt, kp)
    assert m.t_position > 0 and m.t_fixed > 0
    P = np.cumprod(torch.sigmoid(inp["conf_logits"].double()).cpu().numpy(), axis=1)
    L = s["verify_len"].cpu().numpy()
    r, base, ratio = m.against_one_token(P, L, w.K)
    np.testing.assert_allclose(r["emitted"], s["expected_tokens"].cpu().numpy(), rtol=1e-12)
    measured = graph_time
    print(f"[round model] predicted {r['t_round'] * 1e3:.3f} ms, measured {measured * 1e3:.3f} ms "
          f"as a graph ({float(np.median(times)) * 1e3:.3f} ms eager with per-kernel events); "
          f"per-user speed vs one-token rounds {ratio:.3f}; "
          f"{m.t_position * 1e6:.1f} us per drafting position", flush=True)
    assert 0.5 * measured < r["t_round"] < 3.0 * measured
    assert np.isfinite(ratio) and ratio > 0
    assert D.dspark_query_device_status(v["workspace"]) == 0
