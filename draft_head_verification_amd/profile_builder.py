"""Throughput curve of this verification path, for the schedule.

The schedule weighs each extra verified token against the engine's throughput as a function
of the tokens in the verify batch, a curve measured beforehand per engine (QbitAI, "DSpark in
10 concepts", section "Variable-length drafts and hardware-aware scheduling"; 10100.com
commentary, section "letting the GPU decide how much to verify").  A serving engine would
measure its target model; this module measures the part that is built here -- dspark_verify
-- on the current GPU and returns the curve in the schedule's knot format.

Every verified position is accepted in the measured rounds (the proposal probability handed
in is tiny), so each round reads all of its target rows: the curve is the cost of verifying N
tokens, not of an early exit.
"""
from __future__ import annotations

import numpy as np
import torch

from . import dspark as D


def knots_from_timings(samples):
    """(N, seconds) pairs -> (knot_tokens, knot_tps): tokens/s = N / seconds, knots sorted by N,
    repeated N merged by their median time."""
    by_n = {}
    for n, t in samples:
        if not (n > 0 and t > 0):
            raise ValueError(f"invalid sample ({n}, {t})")
        by_n.setdefault(float(n), []).append(float(t))
    kt = np.array(sorted(by_n), dtype=np.float64)
    kp = np.array([n / float(np.median(by_n[n])) for n in kt], dtype=np.float64)
    return kt, kp


def measure_verify_curve(shapes, V=151936, r=256, K=16, y_dtype=torch.float32, reps=3,
                         warmup=1, seed=0, device="cuda"):
    """Time dspark_verify for each (B, L) in `shapes` (L <= K verified positions per request,
    N = B * (L + 1) target positions) and return (knot_tokens, knot_tps)."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    samples = []
    U = (0.05 * torch.randn(V, r, generator=gen)).to(torch.bfloat16).to(device)
    W = (0.05 * torch.randn(V, r, generator=gen)).to(torch.bfloat16).to(device)
    for B, L in shapes:
        if not (1 <= B and 0 <= L <= K):
            raise ValueError(f"invalid shape ({B}, {L})")
        Y = torch.randn(B, K + 1, V, generator=gen).to(y_dtype).to(device)
        Z = torch.randn(B, K, V, generator=gen).to(torch.bfloat16).to(device)
        toks = torch.randint(0, V, (B, K), generator=gen, dtype=torch.int32).to(device)
        q_tok = torch.full((B, K), 1e-30, device=device)  # every test passes
        q_lse = torch.zeros(B, K, device=device)
        prev = torch.randint(0, V, (B,), generator=gen, dtype=torch.int32).to(device)
        vlen = torch.full((B,), L, dtype=torch.int32, device=device)
        temp = torch.ones(B, device=device)
        acc = torch.empty(B, dtype=torch.int32, device=device)
        nxt = torch.empty(B, dtype=torch.int32, device=device)
        ws = torch.empty(D.dspark_verify_workspace_size(B, K, V, r), dtype=torch.uint8,
                         device=device)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for i in range(warmup + reps):
            ev[0].record()
            D.dspark_verify(Y, toks, q_tok, q_lse, Z, U, W, prev, vlen, temp, seed + i, acc, nxt,
                            workspace=ws)
            ev[1].record()
            torch.cuda.synchronize()
            if i >= warmup:
                samples.append((B * (L + 1), ev[0].elapsed_time(ev[1]) * 1e-3))
        if D.dspark_query_device_status(ws) != 0:
            raise RuntimeError("verify reported invalid device data")
        if not bool((acc == L).all()):
            raise RuntimeError("a measured round rejected a token")
        del Y, Z
        torch.cuda.empty_cache()
    return knots_from_timings(samples)
