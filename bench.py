#!/usr/bin/env python3
"""Benchmark: one DSpark round (draft block -> schedule -> verify) per step on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload headline]

A step is the whole hot path over one batch of synthetic inputs already resident in HBM:
the K Markov-head draft steps (gather, bias contraction, base add, temperature, softmax,
Gumbel-max sample), the confidence schedule, and the rejection-sampling verify (row
statistics over the target logits, accept scan, residual / bonus draw).  The default workload
is the headline shape: B=256 requests, K=16 draft positions, V=151936, rank 256, bf16 base
logits and factors, fp32 target logits, temperature 1, scheduling off.

Prints one JSON line: throughput in drafted positions per second (sum of draft lengths per
step / step time), the roofline of the dominant kernel (algorithmic bytes per launch over its
average HIP-event duration inside the timed region, against the MI355X HBM peak), and the
CPU oracle timed on a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
# Vector-ALU issue peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T 32-bit lane operations
# per second (a wave64 instruction issues over four cycles; packed FP32 is not used)
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# Algorithmic vector operations per vocabulary entry and request of one drafting step:
# sampled (per-token Gumbel-max) -- Philox4x32-10 (10 rounds of two 32x32->64-bit products and
# four XORs: 60 per call of four tokens, 15 per token), uniform -> E (conversion, scale,
# logarithm: 3), weight (scale-and-shift, exponential: 2), running sum and maximum (2),
# candidate test (two products, a compare, three selects: 6), bias add and base-logit decode
# (2) = 30; greedy -- bias add, decode, compare and two selects = 5
ALU_OPS_SAMPLED, ALU_OPS_GREEDY = 30, 5
METRIC = "draft+verify positions/s at V=151936,K=16,B=256; HBM GB/s vs peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--temperature", type=float, default=None,
                    help="override every request's temperature (0 = greedy)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters (optional)")
    ap.add_argument("--head", choices=("markov", "rnn"), default="markov",
                    help="sequential head: the default Markov head, or the optional recurrent "
                         "(GRU) head with seeded weights")
    ap.add_argument("--sampler", choices=("token", "block16"), default="token",
                    help="how sampled tokens are drawn: the per-token Gumbel-max (default) or the "
                         "optional two-level 16-token block race")
    ap.add_argument("--targets", choices=("noisy", "exact"), default="noisy",
                    help="target logits: the workload's (corrected draft logits plus noise), or "
                         "exactly the drafter's corrected logits, so that p = q and every verified "
                         "position is accepted (the verifier reads every target row)")
    ap.add_argument("--round-model", action="store_true",
                    help="also measure the verify throughput curve at this workload's shape and "
                         "report the round cost model built from the measured kernel times")
    ap.add_argument("--graph", action="store_true",
                    help="(the default) capture one round (all its launches) in a HIP graph and "
                         "time graph replays, each checked against an eager round first")
    ap.add_argument("--eager", action="store_true",
                    help="time the round as plain kernel launches instead of graph replays")
    ap.add_argument("--flush", action="store_true",
                    help="time every round on its own, after writing a 512 MB buffer (untimed) so "
                         "that no input is left in L2 or the Infinity Cache; reports the median")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the benchmark, run a plain device copy of BYTES bytes five "
                         "times (scales the HBM byte counters of the profiler)")
    return ap.parse_args()


def copy_calibration(nbytes: int):
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "launches": 5}), flush=True)


def build_targets_on_gpu(inp, tokens, corrected, w, exact=False):
    """Target logits for the timed GPU path: the drafter's corrected rows plus the workload's
    noise (exact: no noise, the target equals the drafter); the bonus row adds the bias of the
    last drafted token to the extra base row."""
    import torch
    from draft_head_verification_amd import synth
    B, K = w.B, w.K
    corr = inp["Z_ext"].float()
    corr[:, :K] = corrected
    last = tokens[:, K - 1].long().clamp(min=0)
    bias = inp["U"][last].float() @ inp["W"].float().T
    corr[:, K] += bias
    Y = synth.target_logits(corr, 0.0 * inp["noise"] if exact else inp["noise"], w.y_dtype)
    del corr, bias
    torch.cuda.empty_cache()
    return Y


def algorithmic_bytes(name, w, inp, acc_host, n_resid, zb, ub, yb):
    """Bytes the method must move per step, per kernel (reads of base logits, factors and
    target rows).  The draft step runs K times, each reading the base logits of one position
    and all of W.  The verifier needs the target rows up to the deciding one: a + 1 rows of a
    request whose accepted length is a (the rejected row, or the bonus row when all are
    accepted)."""
    B, K, V, r = w.B, w.K, w.V, w.r
    if name == "markov_head_step":
        return K * (B * V * zb + V * r * ub + B * r * ub)
    if name == "verify_rows":
        return int(sum((int(a) + 1) for a in acc_host)) * V * yb
    if name == "verify_residual":
        return n_resid * V * (zb + yb) + (V * r * ub if n_resid else 0) + n_resid * r * ub
    if name == "rnn_step":  # GRU weights (float32) + per request: U row, state in/out, operands
        return K * (2 * 3 * r * r * 4 + B * r * (ub + 4 + 4 + 2 + 2))
    return None


def cpu_baseline(inp, w, n_threads_hint, sampler="token"):
    """The oracle, as it stands, on a bounded sample of requests of the same workload."""
    import numpy as np
    import torch

    import oracle
    from draft_head_verification_amd import synth
    threads = oracle.num_threads()
    # up to 16 requests per host thread (about 10 s of oracle work at the headline), never
    # more than the batch
    n = min(w.B, max(8, 16 * threads))
    rows = list(range(n))
    U, W = inp["U"].cpu(), inp["W"].cpu()
    Zc = inp["Z_ext"][:n, : w.K].cpu().contiguous()
    prev, temp = inp["prev_token"][:n].cpu(), inp["temperature"][:n].cpu()
    req, dlen = inp["req_id"][:n].cpu(), inp["draft_len"][:n].cpu()
    t0 = time.perf_counter()
    od = oracle.draft_block(Zc, U, W, prev, temp, inp["seed"], draft_len=dlen, req_id=req,
                            want_corrected=True, sampler=sampler)
    t_draft = time.perf_counter() - t0
    # targets of the sample from the oracle's own chain (not timed)
    corr = inp["Z_ext"][:n].cpu().float().clone()
    corr[:, : w.K] = torch.from_numpy(od["corrected"])
    for i in range(n):
        kb = int(dlen[i])
        corr[i, kb] = torch.from_numpy(oracle.corrected_row(inp["Z_ext"][i, kb].cpu(), U, W,
                                                            int(od["tokens"][i, kb - 1])))
    Y = synth.target_logits(corr, inp["noise"][:n].cpu(), w.y_dtype)
    t1 = time.perf_counter()
    oracle.verify(Y, od["tokens"], od["q_tok"].astype(np.float32), od["q_lse"].astype(np.float32),
                  Zc, U, W, prev, dlen, temp, inp["seed"], req_id=req, rows=rows, sampler=sampler)
    t_verify = time.perf_counter() - t1
    positions = int(dlen.sum())
    # one core: the first request alone (OpenMP over one request runs on one thread)
    one = [0]
    t2 = time.perf_counter()
    oracle.draft_block(Zc, U, W, prev, temp, inp["seed"], draft_len=dlen, req_id=req, rows=one,
                       sampler=sampler)
    oracle.verify(Y, od["tokens"], od["q_tok"].astype(np.float32), od["q_lse"].astype(np.float32),
                  Zc, U, W, prev, dlen, temp, inp["seed"], req_id=req, rows=one, sampler=sampler)
    t_one = time.perf_counter() - t2
    return {"value": positions / (t_draft + t_verify), "unit": "positions/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} of {w.B} requests of the same workload ({positions} drafted positions): "
                      f"oracle draft {t_draft:.2f} s + verify {t_verify:.2f} s, OpenMP over requests",
            "one_core": {"value": int(dlen[0]) / t_one, "unit": "positions/s",
                         "sample": f"request 0 alone ({int(dlen[0])} positions, {t_one:.2f} s)"}}


def round_model_report(w, records, steps, inp, vlen, acc, ms_per_step):
    """The round cost model built from this run: per-position and fixed kernel times from the
    traced rounds, and the verify throughput curve measured at this workload's vocabulary, rank,
    draft length and target dtype (every tested position accepted, so every target row is
    read).  Reports the model's time per emitted token and per-user speed against one-token
    rounds (one drafting position, its pass probability the first survival probability), the
    model's expected tokens next to the measured ones, and the drafting cost of K = 4 against
    K = 16 positions."""
    import numpy as np
    import torch
    from draft_head_verification_amd import profile_builder as PB
    from draft_head_verification_amd import round_model as RM
    B, K = w.B, w.K
    shapes = [(b, l) for b in (1, 8, 32, 64, 128, 256, 512) for l in (0, 3, 7, K - 1)
              if b <= max(B, 8) and l <= K - 1]
    kt, kp = PB.measure_verify_curve(shapes, V=w.V, r=w.r, K=K, y_dtype=w.y_dtype, reps=2)
    m = RM.MeasuredRound.from_trace(records, steps, K, kt, kp)
    surv = torch.sigmoid(inp["conf_logits"].double()).cpu().numpy()
    P = np.cumprod(surv, axis=1)
    L = vlen.cpu().numpy()
    r, base, ratio = m.against_one_token(P, L, K)
    a = acc.cpu().numpy().astype(np.float64)
    r4 = m.round(P[:, :4], np.minimum(L, 4), 4)
    # A target model's forward of t seconds per round adds t to both rounds:
    # speed ratio(t) = (E_K / E_1) (T_1 + t) / (T_K + t), above 1 once t exceeds the break-even
    eK, e1 = float(r["emitted"].mean()), float(base["emitted"].mean())
    tK, t1 = r["t_round"], base["t_round"]
    t_even = (e1 * tK - eK * t1) / (eK - e1) if eK > e1 else float("inf")
    return {
        "t_position_us": round(m.t_position * 1e6, 2), "t_fixed_us": round(m.t_fixed * 1e6, 2),
        "verify_curve": {"tokens": [float(x) for x in kt], "tokens_per_s": [round(float(x), 1) for x in kp]},
        "model_emitted_per_request": round(float(r["emitted"].mean()), 4),
        "measured_emitted_per_request": round(float((a + 1).mean()), 4),
        "model_round_ms": round(r["t_round"] * 1e3, 4), "measured_round_ms": round(ms_per_step, 4),
        "model_time_per_token_us": round(r["time_per_token"] * 1e6, 3),
        "one_token_round_ms": round(base["t_round"] * 1e3, 4),
        "per_user_speed_vs_one_token": round(ratio, 4),
        "target_forward_break_even_ms": round(max(t_even, 0.0) * 1e3, 4),
        "per_user_speed_limit_large_target": round(eK / e1, 4),
        "drafting_K4_vs_K16": {"draft_ms_K4": round(m.draft_time(4) * 1e3, 4),
                               "draft_ms_K16": round(m.draft_time(K) * 1e3, 4),
                               "model_round_ms_K4": round(r4["t_round"] * 1e3, 4)},
        "note": "the verify curve is this library's verifier standing in for a target model's "
                "forward, which the round does not include",
    }


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the path shards by "
              "request with no exchange, so multi-GPU throughput is N x the one-GPU figure; "
              "run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    from draft_head_verification_amd import dspark as D
    from draft_head_verification_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = synth.WORKLOADS[args.workload]
    dev = "cuda"
    inp = synth.make_inputs(w, device=dev, temperature=args.temperature)
    for k in list(inp):
        if isinstance(inp[k], torch.Tensor):
            inp[k] = inp[k].contiguous()
    Z = inp["Z_ext"][:, : w.K].contiguous()
    B, K, V, r = w.B, w.K, w.V, w.r
    zb = 2 if w.z_dtype == torch.bfloat16 else 4
    ub = 2 if w.uw_dtype == torch.bfloat16 else 4
    yb = 2 if w.y_dtype == torch.bfloat16 else 4

    # outputs and workspaces, allocated once
    toks = torch.empty(B, K, dtype=torch.int32, device=dev)
    q_tok = torch.empty(B, K, device=dev)
    q_lse = torch.empty(B, K, device=dev)
    vlen = torch.empty(B, dtype=torch.int32, device=dev)
    exp_tok = torch.empty(B, dtype=torch.float64, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    ws_d = torch.empty(D.dspark_draft_workspace_size(B, K, V, r), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(max(256, D.dspark_schedule_workspace_size(B, K)), dtype=torch.uint8, device=dev)
    ws_v = torch.empty(D.dspark_verify_workspace_size(B, K, V, r), dtype=torch.uint8, device=dev)
    gru = hs = None
    if args.head == "rnn":
        gru = tuple(t.contiguous() for t in synth.make_gru(r, seed=w.data_seed + 1000, device=dev))
        hs = torch.zeros(B, K, r, dtype=torch.bfloat16, device=dev)

    # one untimed draft gives the chain the target logits are built around
    corrected = torch.empty(B, K, V, device=dev)
    D.dspark_draft_block(Z, inp["U"], inp["W"], inp["prev_token"], inp["temperature"], inp["seed"],
                         toks, q_tok, q_lse, draft_len=inp["draft_len"], req_id=inp["req_id"],
                         corrected=corrected, workspace=ws_d, gru=gru, head_state=hs,
                         sampler=args.sampler)
    Y = build_targets_on_gpu(inp, toks, corrected, w, exact=args.targets == "exact")
    del corrected
    torch.cuda.empty_cache()

    def step(trace=None):
        D.dspark_draft_block(Z, inp["U"], inp["W"], inp["prev_token"], inp["temperature"],
                             inp["seed"], toks, q_tok, q_lse, draft_len=inp["draft_len"],
                             req_id=inp["req_id"], workspace=ws_d, trace=trace, gru=gru,
                             head_state=hs, sampler=args.sampler)
        D.dspark_schedule(inp["conf_logits"], vlen, inp["knot_tokens"], inp["knot_tps"],
                          w.schedule, draft_len=inp["draft_len"], expected_tokens=exp_tok,
                          workspace=ws_s, trace=trace)
        D.dspark_verify(Y, toks, q_tok, q_lse, Z, inp["U"], inp["W"], inp["prev_token"], vlen,
                        inp["temperature"], inp["seed"], acc, nxt, req_id=inp["req_id"],
                        workspace=ws_v, trace=trace, head_state=hs, sampler=args.sampler)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run = step
    launch = "kernel launches"
    graph = None
    if not args.eager:
        # the whole round as one HIP graph: every call enqueues kernels only (no allocation, no
        # memset, no host sync), so a capture records exactly the round's launches -- the way
        # a serving loop runs its rounds; a capture that fails leaves the launches timed
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
        except RuntimeError as e:
            print(f"graph capture failed ({e}); timing kernel launches", file=sys.stderr)
            graph = None
            launch = "kernel launches (graph capture failed)"
            torch.cuda.synchronize()
    if graph is not None:
        step()  # eager reference outputs
        torch.cuda.synchronize()
        ref = [t.clone() for t in (toks, q_tok, q_lse, vlen, acc, nxt)]
        for _ in range(max(3, args.warmup)):
            for t in (toks, q_tok, q_lse, vlen, acc, nxt):
                t.fill_(-3)
            graph.replay()
            torch.cuda.synchronize()
            assert all(torch.equal(a, b) for a, b in zip(ref, (toks, q_tok, q_lse, vlen, acc, nxt))), \
                "graph replay differs from the eager round"
            step()  # eager work between replays
            torch.cuda.synchronize()
        run = graph.replay
        launch = "one HIP graph per round"
    # timed region: the steps alone (no per-kernel events inside)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        run()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    if args.flush:
        # cold caches: each round timed alone after a 512 MB write (outside its events)
        junk = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        times = []
        for _ in range(args.steps):
            junk.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        del junk
        times.sort()
        ms_per_step = times[len(times) // 2]
        ms_total = ms_per_step * args.steps
    # the same steps again with HIP events around every kernel, on the stream the kernels
    # run on, for the per-kernel durations (the roofline's launch durations)
    trace = D.Trace(capacity=64 * (args.steps + 1) + 64)
    for _ in range(args.steps):
        step(trace)
    torch.cuda.synchronize()
    for bits_ws in (ws_d, ws_s, ws_v):
        bits = D.dspark_query_device_status(bits_ws)
        assert bits == 0, f"device status {bits:#x}"

    positions = int(inp["draft_len"].sum().item())
    value = positions * args.steps / (ms_total / 1e3)

    # per-kernel statistics from the HIP events of the timed region
    per = {}
    for name, ms in trace.records():
        s = per.setdefault(name, [0, 0.0])
        s[0] += 1
        s[1] += ms
    acc_host = acc.cpu().numpy()
    # requests whose round ended in a rejection at T > 0 (the residual pass's rows)
    n_resid = int(((acc < vlen) & (inp["temperature"] > 0)).sum().item())
    kernels = []
    for name, (cnt, tot) in sorted(per.items(), key=lambda kv: -kv[1][1]):
        avg_us = tot / cnt * 1e3
        nbytes = algorithmic_bytes(name, w, inp, acc_host, n_resid, zb, ub, yb)
        lps = cnt / args.steps
        per_launch = nbytes / lps if nbytes else None
        kernels.append({"kernel": name, "launches_per_step": lps,
                        "avg_us": round(avg_us, 2), "share": round(tot / max(1e-9, sum(v[1] for v in per.values())), 4),
                        "algorithmic_bytes_per_launch": (int(per_launch) if per_launch else per_launch),
                        "achieved_GBs": (round(per_launch / (avg_us * 1e-6) / 1e9, 1) if per_launch else None)})
    dom = next(k for k in kernels if k["algorithmic_bytes_per_launch"])
    # counters are kept per measured variant: the workload, plus the sampler, temperature,
    # target and head options that change the kernels' work
    variant = (args.workload + ("_block16" if args.sampler == "block16" else "")
               + (f"_t{args.temperature:g}" if args.temperature is not None else "")
               + ("_exact" if args.targets == "exact" else "")
               + ("_rnn" if args.head == "rnn" else ""))
    traffic = mfma_util = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            ent = tj.get(variant, {}).get(dom["kernel"])
            if ent and ent.get("source_hash") == _kernel_source_hash():
                traffic = ent["hbm_bytes_per_launch"]
                mfma_util = ent.get("mfma_util_pct")
        except Exception:
            traffic = mfma_util = None
    roofline = {"bound": "hbm", "kernel": dom["kernel"], "achieved": dom["achieved_GBs"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom["achieved_GBs"] / HBM_PEAK_GBS, 4), "traffic": traffic}
    # A drafting step whose per-token sampling takes longer at the vector-ALU issue peak than
    # its bytes take at the HBM peak is bound by the ALU: report it against that peak, keeping
    # its HBM figure alongside.
    if dom["kernel"] == "markov_head_step" and args.sampler == "token":
        T_h = inp["temperature"].float().cpu()
        L_h = inp["draft_len"].cpu().clamp(0, K)
        sampled = (T_h > 0).float()
        ops_step = float(V * sum(float(L_h[b]) * (ALU_OPS_SAMPLED * sampled[b] +
                                                   ALU_OPS_GREEDY * (1 - sampled[b]))
                                 for b in range(B))) / K
        if ops_step / (ALU_PEAK_TOPS * 1e12) > dom["algorithmic_bytes_per_launch"] / (HBM_PEAK_GBS * 1e9):
            tops = ops_step / (dom["avg_us"] * 1e-6) / 1e12
            hbm = {k: roofline[k] for k in ("achieved", "peak", "unit", "frac")}
            roofline.update({"bound": "alu", "achieved": round(tops, 2), "peak": round(ALU_PEAK_TOPS, 1),
                             "unit": "Tops/s", "frac": round(tops / ALU_PEAK_TOPS, 4),
                             "algorithmic_ops_per_launch": int(ops_step), "hbm": hbm})
            valu = None
            try:
                ent = json.load(open(args.traffic_json)).get(variant, {}).get(dom["kernel"])
                if ent and ent.get("source_hash") == _kernel_source_hash():
                    valu = ent.get("valu_busy_pct")
            except Exception:
                valu = None
            roofline["rocprof_valu_busy_pct"] = valu
    # the matrix cores' share of the dominant kernel when it is the bias contraction:
    # 2 B r V bf16 flops per drafting step over the same live launch duration
    if dom["kernel"] == "markov_head_step" and ub == 2 and r in (64, 128, 256):
        tflops = 2.0 * B * r * V / (dom["avg_us"] * 1e-6) / 1e12
        roofline["mfma"] = {"achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                            "rocprof_mfma_util_pct": mfma_util}
    step_bytes = sum((k["algorithmic_bytes_per_launch"] or 0) * k["launches_per_step"] for k in kernels)

    model = None
    if args.round_model:
        model = round_model_report(w, trace.records(), args.steps, inp, vlen, acc, ms_per_step)

    cpu = None
    if not args.no_cpu_baseline and args.head == "markov":
        cpu = cpu_baseline(inp, w, None, args.sampler)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded generator; random factors; no checkpoint)",
        "config": {"workload": f"{w.name}: B={B} K={K} V={V} r={r} base/factors "
                               f"{'bf16' if zb == 2 else 'fp32'}, target {'bf16' if yb == 2 else 'fp32'}, "
                               f"T={args.temperature if args.temperature is not None else ','.join(str(t) for t in w.temperature)}, "
                               f"schedule {'on' if w.schedule else 'off'}, "
                               f"{'per-token Gumbel-max' if args.sampler == 'token' else 'two-level block-race'} sampler"
                               + (", recurrent (GRU) head" if args.head == "rnn" else "")
                               + (", exact targets (every position accepted)" if args.targets == "exact" else ""),
                   "sampler": args.sampler,
                   "B": B, "K": K, "V": V, "r": r, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "caches": "flushed before every round (median round)" if args.flush else "warm",
        "launch": launch,
        "step_algorithmic_GBs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "wall_s": round(wall, 3),
        "mean_accept_len": round(float(acc.float().mean().item()), 3),
        "kernels": kernels,
    }
    if model is not None:
        out["round_model"] = model
    print(json.dumps(out), flush=True)


def _strip_comments(src: str) -> str:
    """The code of a C++ source without its comments and whitespace (string literals kept)."""
    import re
    token = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|\s+', re.S)
    return token.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", src).replace(" ", "")


def _kernel_source_hash() -> str:
    """Hash of the library's kernel code (comments and whitespace do not count)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "draft_head_verification_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            h.update(_strip_comments(open(os.path.join(csrc, f)).read()).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
