"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

Inputs are generated on the GPU with the seeded generator.  The whole batch goes through the
library; a sample of requests is recomputed by the oracle from the generator's inputs alone
and compared position by position: one request in every wave slot of the matrix-core kernel's
first request group, in both of its 16-wide column blocks and at varied lanes, the first and
last request of each noise half, and some of a second request group when there is one.  Requests
outside the sample are checked through properties that hold at any size (valid token ids,
masking past the draft length, accept lengths within the verify lengths, and for greedy
requests the exact-match prefix and the argmax correction / bonus).
Tolerances and near-tie rules: tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
from draft_head_verification_amd import synth
from parity import Tally, compare_draft, compare_verify, oracle_targets, TOL_EXP

pytestmark = pytest.mark.gpu

FULL = ["single", "moderate", "concurrent", "ragged", "headline", "headline_sched"]


def _sample_rows(B):
    """Requests b = 256 g + 32 w + 16 q + m (group g, wave w, column block q, lane m)."""
    rows = {0, B // 2 - 1 if B > 1 else 0, B // 2, B - 1}
    for w_ in range(8):
        for q in range(2):
            rows.add(32 * w_ + 16 * q + (3 * w_ + 7 * q + 1) % 16)
    for w_ in (0, 5):
        rows.add(256 + 32 * w_ + 16 * (w_ & 1) + 9)
    rows = sorted(r for r in rows if 0 <= r < B)
    if len(rows) < 16:  # small batches: every request up to 16
        rows = sorted(set(rows) | set(range(min(B, 16))))
    return rows


@pytest.mark.parametrize("name", FULL)
def test_full_size_round(name):
    from draft_head_verification_amd import dspark as D
    w = synth.WORKLOADS[name]
    B, K, V, r = w.B, w.K, w.V, w.r
    print(f"[full {name}] B={B} K={K} V={V} r={r}", flush=True)
    g = synth.make_inputs(w, device="cuda")
    Z = g["Z_ext"][:, :K].contiguous()
    rows = _sample_rows(B)
    U_cpu, W_cpu = g["U"].cpu(), g["W"].cpu()
    host = {k: (v.cpu() if isinstance(v, torch.Tensor) and v.numel() <= 1 << 20 else v)
            for k, v in g.items()}
    temps = host["temperature"].numpy()
    dlen = host["draft_len"].numpy()
    tally = Tally()

    # ---- draft: whole batch on the GPU, sample on the oracle
    gd = D.draft_block(Z, g["U"], g["W"], g["prev_token"], g["temperature"], g["seed"],
                       draft_len=g["draft_len"], req_id=g["req_id"], want_corrected=True)
    assert D.dspark_query_device_status(gd["workspace"]) == 0
    toks = gd["tokens"].cpu().numpy()
    for b in range(B):
        kb = int(dlen[b])
        assert np.all((toks[b, :kb] >= 0) & (toks[b, :kb] < V)) and np.all(toks[b, kb:] == -1)
    od = oracle.draft_block(Z, U_cpu, W_cpu, host["prev_token"], host["temperature"], g["seed"],
                            draft_len=host["draft_len"], req_id=host["req_id"], rows=rows,
                            want_corrected=True)
    gnp = {"tokens": toks, "q_tok": gd["q_tok"].cpu().numpy(), "q_lse": gd["q_lse"].cpu().numpy()}
    idx = torch.tensor(rows, device="cuda")
    gcorr = gd["corrected"][idx].cpu().numpy()
    compare_draft(gnp, od, rows, temps, tally, g_corr=gcorr, o_corr=od["corrected"])
    print(f"[full {name}] draft ok", flush=True)

    # ---- schedule: the whole batch on both sides (cheap)
    if w.schedule:
        gs = D.schedule(g["conf_logits"], g["knot_tokens"], g["knot_tps"], True,
                        draft_len=g["draft_len"])
        os_ = oracle.schedule(host["conf_logits"], g["knot_tokens"].cpu(), g["knot_tps"].cpu(),
                              True, draft_len=host["draft_len"])
        gvl = gs["verify_len"].cpu().numpy()
        if not np.array_equal(gvl, os_["verify_len"]):
            assert os_["margin"] < 1e-12, ("schedule differs away from a tie", os_["margin"])
            tally.schedule_near_ties += 1
        np.testing.assert_allclose(gs["expected_tokens"].cpu().numpy(), os_["expected_tokens"],
                                   rtol=TOL_EXP, atol=0)
        vlen = torch.from_numpy(os_["verify_len"])
        print(f"[full {name}] schedule ok: n*={os_['n_star']} of {int(dlen.sum())}, "
              f"lengths {vlen.min().item()}..{vlen.max().item()}", flush=True)
    else:
        vlen = host["draft_len"].clone()

    # ---- verify: sampled requests get the oracle's draft and targets built from it; the
    # rest get targets from the GPU's own chain (load only)
    prev = torch.cat([g["prev_token"][:, None].long(), gd["tokens"].long()], 1)[:, : K + 1]
    prev = prev.clamp(min=0)
    corr = g["Z_ext"].float()
    Wf = g["W"].float()
    for k in range(K + 1):
        corr[:, k] += g["U"][prev[:, k]].float() @ Wf.T
    del Wf
    Y = synth.target_logits(corr, g["noise"], w.y_dtype)
    del corr
    torch.cuda.empty_cache()
    Ys = oracle_targets({**host, "Z_ext": g["Z_ext"][idx].cpu(), "noise": g["noise"][idx].cpu(),
                         "draft_len": host["draft_len"][rows], "prev_token": host["prev_token"][rows]},
                        list(range(len(rows))), od["tokens"], U_cpu, W_cpu)
    Y[idx] = Ys.cuda()
    vtoks, vq, vl = gd["tokens"].clone(), gd["q_tok"].clone(), gd["q_lse"].clone()
    vtoks[idx] = torch.from_numpy(od["tokens"]).cuda()
    vq[idx] = torch.from_numpy(od["q_tok"].astype(np.float32)).cuda()
    vl[idx] = torch.from_numpy(od["q_lse"].astype(np.float32)).cuda()
    vlen_d = vlen.cuda()
    gv = D.verify(Y, vtoks, vq, vl, Z, g["U"], g["W"], g["prev_token"], vlen_d, g["temperature"],
                  g["seed"], req_id=g["req_id"])
    assert D.dspark_query_device_status(gv["workspace"]) == 0
    ov = oracle.verify(Ys, od["tokens"], od["q_tok"].astype(np.float32),
                       od["q_lse"].astype(np.float32), Z[idx].cpu(), U_cpu, W_cpu,
                       host["prev_token"][rows], vlen[rows], host["temperature"][rows], g["seed"],
                       req_id=host["req_id"][rows])
    gvn = {k: gv[k].cpu().numpy() for k in ("accept_len", "next_token", "p_tok")}
    sub = {k: gvn[k][rows] for k in gvn}
    compare_verify(sub, ov, list(range(len(rows))), temps[rows], tally)

    # ---- properties of every request
    acc, nxt = gvn["accept_len"], gvn["next_token"]
    vl_h = vlen.numpy()
    assert np.all((acc >= 0) & (acc <= vl_h)) and np.all((nxt >= 0) & (nxt < V))
    greedy = np.where(temps == 0)[0]
    if len(greedy):
        gi = torch.from_numpy(greedy).cuda()
        am = Y[gi].float().argmax(-1).cpu().numpy()  # first maximal index
        vt = vtoks[gi].cpu().numpy()
        for j, b in enumerate(greedy):
            L = int(vl_h[b])
            match = vt[j, :L] == am[j, :L]
            a = int(np.argmin(match)) if not match.all() else L
            assert acc[b] == a and nxt[b] == am[j, a], (b, acc[b], a)
    tally.report(f"full-{name}")
    print(f"[full {name}] mean accept {acc.mean():.2f} over {B} requests", flush=True)
