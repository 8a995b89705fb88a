"""Helpers for the GPU-vs-oracle parity tests.

Rules these helpers keep:
  * Every input the oracle sees comes from the seeded generator (draft_head_verification_amd.
    synth) or from the oracle itself; nothing the HIP library produced is ever fed to the
    oracle.  Target logits of an oracle-checked request are built from the ORACLE's draft
    chain (oracle corrected rows + the generator's noise); the GPU verify receives those same
    rows, tokens and draft probabilities.
  * Requests that are not oracle-checked (full-size runs check a sample) get inputs built
    from the GPU's own draft -- they only exercise the launch at its real shape and are
    checked through properties that hold at any size.

Tolerances (floating point; integer results are compared exactly):
  corrected logits        |gpu - oracle| <= 2e-2 (stated bound); also checked at 1e-5 + 1e-6|c|
  q_tok, p_tok            absolute 1e-5 (probabilities)
  q_lse                   absolute 1e-4 (a log-normaliser of ~1.5e5 float32 terms)
  expected_tokens         relative 1e-12 (float64 on both sides)
  below T = 0.7 (the lowest sampling temperature of the stated workloads; the cases at T =
  0.05 go below it) the bounds on probabilities and log-normalisers are derived: an error e in
  the corrected logits moves ln q(x) by at most 2e/T and the log-normaliser by e/T, so with
  e = 3e-5 (the tight bound above at |c| <= 20) q_tok may move by 1e-5 + q * 6e-5 / T and q_lse
  by 1e-4 + 3e-5 / T (at T = 0.05: 1.2e-3 relative, 6e-4 absolute), and a sampled near-tie is a
  perturbed-score gap below 1e-4 + 6e-5 / T
Near-ties, where floating point may legitimately decide an integer differently:
  greedy draft            oracle top-two corrected-logit gap < 2e-5
  sampled draft / resample / bonus   oracle top-two perturbed-score gap < 1e-4
  accept test             |u - p/q| < 1e-5
A mismatch is accepted only at a near-tie; the count is reported.  After a draft-token
mismatch the request's chains differ, so later positions of that request are not compared.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
from draft_head_verification_amd import synth

TOL_C = 2e-2
TOL_C_TIGHT_ABS, TOL_C_TIGHT_REL = 1e-5, 1e-6
TOL_Q = 1e-5
TOL_LSE = 1e-4
TOL_EXP = 1e-12
T_STATED_MIN = 0.7   # lowest sampling temperature of the stated workloads
E_C = 3e-5           # corrected-logit error at |c| <= 20 under the tight bound


def tol_q(T, q):
    return TOL_Q + (q * 2 * E_C / T if 0 < T < T_STATED_MIN else 0.0)


def tol_lse(T):
    return TOL_LSE + (E_C / T if 0 < T < T_STATED_MIN else 0.0)


def tie_sample(T):
    """Near-tie width of a perturbed score c/T + G: 1e-4, plus the derived 2e/T below 0.7."""
    return TIE_SAMPLE + (2 * E_C / T if 0 < T < T_STATED_MIN else 0.0)


TIE_GREEDY = 2e-5
TIE_SAMPLE = 1e-4
TIE_ACCEPT = 1e-5


# every Tally.report of the session, written out at its end (conftest.py) when a directory
# for it is given in DSPARK_TALLY_DIR
REPORTS: list = []


@dataclass
class Tally:
    compared_positions: int = 0
    greedy_near_ties: int = 0
    sample_near_ties: int = 0
    accept_near_ties: int = 0
    schedule_near_ties: int = 0
    diverged_requests: int = 0
    notes: list = field(default_factory=list)

    def report(self, name):
        REPORTS.append(dict(case=name, positions=self.compared_positions,
                            greedy_near_ties=self.greedy_near_ties,
                            sample_near_ties=self.sample_near_ties,
                            accept_near_ties=self.accept_near_ties,
                            schedule_near_ties=self.schedule_near_ties,
                            diverged_requests=self.diverged_requests))
        print(f"[parity {name}] positions={self.compared_positions} "
              f"greedy_ties={self.greedy_near_ties} sample_ties={self.sample_near_ties} "
              f"accept_ties={self.accept_near_ties} schedule_ties={self.schedule_near_ties} "
              f"diverged={self.diverged_requests}", flush=True)


def to_device(inp: dict, device="cuda") -> dict:
    out = {}
    for k, v in inp.items():
        if isinstance(v, torch.Tensor):
            out[k] = v.to(device).contiguous()
        else:
            out[k] = v
    out["Z"] = out["Z_ext"][:, : inp["workload"].K].contiguous()
    return out


def compare_draft(g: dict, o: dict, rows, temps, tally: Tally, g_corr=None, o_corr=None,
                  Zrows=None):
    """g: GPU outputs (numpy, indexed by request); o: oracle outputs (indexed 0..len(rows))."""
    for i, b in enumerate(rows):
        T = float(temps[b])
        K = o["tokens"].shape[1]
        for k in range(K):
            ot, gt = int(o["tokens"][i, k]), int(g["tokens"][b, k])
            if ot == -1:
                assert gt == -1, (b, k, gt)
                assert g["q_tok"][b, k] == 0 and g["q_lse"][b, k] == 0
                continue
            tally.compared_positions += 1
            # q_lse does not depend on which token wins
            if T > 0:
                assert abs(g["q_lse"][b, k] - o["q_lse"][i, k]) <= tol_lse(T), (b, k, g["q_lse"][b, k], o["q_lse"][i, k])
            else:
                assert g["q_lse"][b, k] == 0 and g["q_tok"][b, k] == 1
            if g_corr is not None:
                gc, oc = g_corr[i][k], o_corr[i, k]
                # masked entries (-inf on both sides) agree exactly
                both = np.isneginf(gc) & np.isneginf(oc)
                err = np.where(both, 0.0, np.abs(gc.astype(np.float64) - np.where(both, 0.0, oc)))
                assert err.max() <= TOL_C, (b, k, err.max())
                assert np.all(err <= TOL_C_TIGHT_ABS + TOL_C_TIGHT_REL * np.abs(oc)), (b, k, err.max())
            if gt != ot:
                gap = o["gap"][i, k]
                limit = TIE_GREEDY if T == 0 else tie_sample(T)
                assert gap < limit, f"request {b} position {k}: gpu {gt} vs oracle {ot}, gap {gap}"
                if T == 0:
                    tally.greedy_near_ties += 1
                else:
                    tally.sample_near_ties += 1
                tally.diverged_requests += 1
                break
            if T > 0:
                assert abs(g["q_tok"][b, k] - o["q_tok"][i, k]) <= tol_q(T, o["q_tok"][i, k]), \
                    (b, k, g["q_tok"][b, k], o["q_tok"][i, k])


def oracle_targets(inp_cpu: dict, rows, tokens_rows, U_cpu, W_cpu) -> torch.Tensor:
    """Target logits [n, K+1, V] of the listed requests, built from the given draft chains
    with the oracle's corrected rows plus the generator's noise; rows past a request's draft
    length carry no bias."""
    w = inp_cpu["workload"]
    K = w.K
    Z_ext, noise = inp_cpu["Z_ext"], inp_cpu["noise"]
    out = []
    for i, b in enumerate(rows):
        kb = int(inp_cpu["draft_len"][b])
        corr = Z_ext[b].float().clone()
        for k in range(0, min(kb, K) + 1):
            prev = int(inp_cpu["prev_token"][b]) if k == 0 else int(tokens_rows[i, k - 1])
            corr[k] = torch.from_numpy(oracle.corrected_row(Z_ext[b, k], U_cpu, W_cpu, prev))
        out.append(synth.target_logits(corr[None], noise[b][None], w.y_dtype)[0])
    return torch.stack(out)


def compare_verify(g: dict, o: dict, rows, temps, tally: Tally):
    for i, b in enumerate(rows):
        T = float(temps[b])
        ga, oa = int(g["accept_len"][b]), int(o["accept_len"][i])
        gn, on = int(g["next_token"][b]), int(o["next_token"][i])
        if ga != oa:
            assert T > 0 and o["accept_margin"][i] < TIE_ACCEPT, (b, ga, oa, o["accept_margin"][i])
            tally.accept_near_ties += 1
            continue
        if gn != on:
            assert T > 0 and o["sample_margin"][i] < tie_sample(T), (b, gn, on, o["sample_margin"][i])
            tally.sample_near_ties += 1
        tested = min(oa + 1, o["p_tok"].shape[1])
        if g.get("p_tok") is not None:
            np.testing.assert_allclose(g["p_tok"][b, :tested], o["p_tok"][i, :tested], rtol=0,
                                       atol=TOL_Q)
            # positions after the deciding one were not tested: p is 0 there (the output is
            # allocated uninitialised, so a position left unwritten shows)
            assert np.all(g["p_tok"][b, tested:] == 0), (b, g["p_tok"][b, tested:])
        tally.compared_positions += tested
