"""A whole round (draft block, schedule, verify) captured as one HIP graph, as the benchmark and
a serving loop run it: every call only enqueues kernels, so the capture records the round's
launches.  Each replay (outputs overwritten before it, an eager round between replays) must
reproduce the eager round bit for bit."""
import pytest
import torch

from draft_head_verification_amd import synth

pytestmark = pytest.mark.gpu

CASES = [
    ("headline", {"V": 2392}, "token"),   # 16-wave matrix-core kernel (256 requests)
    ("moderate", {"V": 2392}, "token"),   # split pairs (64 requests)
    ("concurrent", {"V": 1208, "B": 300}, "block16"),  # scheduling on, two-level sampler
    ("tiny", {}, "token"),                # vector-ALU head
]


@pytest.mark.parametrize("name,kw,sampler", CASES, ids=lambda c: str(c))
def test_round_graph_replays_match_eager(name, kw, sampler):
    from draft_head_verification_amd import dspark as D
    w = synth.shrink(synth.WORKLOADS[name], **kw)
    print(f"[graph {name} {sampler}] B={w.B} K={w.K} V={w.V} r={w.r}", flush=True)
    inp = synth.make_inputs(w, device="cuda", strong_bias=True)
    inp = {k: (v.contiguous() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    B, K, V, r = w.B, w.K, w.V, w.r
    Z = inp["Z_ext"][:, :K].contiguous()
    # targets: the base rows plus the workload's noise (any rows do for a replay check)
    Y = synth.target_logits(inp["Z_ext"].float(), inp["noise"], w.y_dtype).contiguous()
    toks = torch.empty(B, K, dtype=torch.int32, device="cuda")
    q_tok = torch.empty(B, K, device="cuda")
    q_lse = torch.empty(B, K, device="cuda")
    vlen = torch.empty(B, dtype=torch.int32, device="cuda")
    exp_tok = torch.empty(B, dtype=torch.float64, device="cuda")
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    p_tok = torch.empty(B, K, device="cuda")
    ws_d = torch.empty(D.dspark_draft_workspace_size(B, K, V, r), dtype=torch.uint8, device="cuda")
    ws_s = torch.empty(max(256, D.dspark_schedule_workspace_size(B, K)), dtype=torch.uint8,
                       device="cuda")
    ws_v = torch.empty(D.dspark_verify_workspace_size(B, K, V, r), dtype=torch.uint8, device="cuda")
    outs = (toks, q_tok, q_lse, vlen, exp_tok, acc, nxt, p_tok)

    def step():
        D.dspark_draft_block(Z, inp["U"], inp["W"], inp["prev_token"], inp["temperature"],
                             inp["seed"], toks, q_tok, q_lse, draft_len=inp["draft_len"],
                             req_id=inp["req_id"], workspace=ws_d, sampler=sampler)
        D.dspark_schedule(inp["conf_logits"], vlen, inp["knot_tokens"], inp["knot_tps"],
                          w.schedule, draft_len=inp["draft_len"], expected_tokens=exp_tok,
                          workspace=ws_s)
        D.dspark_verify(Y, toks, q_tok, q_lse, Z, inp["U"], inp["W"], inp["prev_token"], vlen,
                        inp["temperature"], inp["seed"], acc, nxt, req_id=inp["req_id"],
                        p_tok=p_tok, workspace=ws_v, sampler=sampler)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for replay in range(3):
        for t in outs:
            t.fill_(-3)
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, outs)):
            assert torch.equal(a, b), (replay, i)
        for ws in (ws_d, ws_s, ws_v):
            assert D.dspark_query_device_status(ws) == 0
        step()  # the program's own eager work between replays
        torch.cuda.synchronize()
        for a, b in zip(ref, outs):
            assert torch.equal(a, b)
