"""Round cost model: time per emitted token of a draft / schedule / verify round.

The pages weigh speculative decoding by the time a round costs (drafting plus verification)
against the tokens it emits (Sina thread, section 4 "speculation is not free"; QbitAI "DSpark
in 10 concepts", section "Speculation is not free"; 10100.com commentary, section "speculative
decoding is block checking").  This module evaluates that trade-off for a batch of requests,
with

  * emitted tokens per request  E_b = 1 + sum_{k < L_b} P[b][k]
    (the accepted prefix plus the one correction or bonus token; P[b][k] is the
    probability that positions 0..k all pass, L_b the verified length);
  * verified tokens             N   = sum_b (L_b + 1)  (one target position per verified
    draft token plus the one that scores the correction / bonus);
  * round time                  t   = t_draft + N / T(N), with T the engine's throughput
    curve (tokens/s as a function of the tokens in the verify batch), piecewise linear
    between knots and clamped outside them -- the same curve the schedule uses;
  * t_draft                     drafting time of the round (for this path: the backbone's
    forward, which is not modelled here, plus K drafting steps of the Markov head, which are
    measured).

MeasuredRound builds the model from a measured run: the per-kernel times of a traced round
(drafting steps, their reductions, the fixed launches) and a measured verify throughput curve.

Everything is host-side float64 arithmetic on small arrays; it drives no GPU work.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def profile(knot_tokens, knot_tps, N):
    """Throughput T(N) of a piecewise-linear curve, clamped to the end knots."""
    kt = np.asarray(knot_tokens, dtype=np.float64)
    kp = np.asarray(knot_tps, dtype=np.float64)
    return np.interp(np.asarray(N, dtype=np.float64), kt, kp, left=kp[0], right=kp[-1])


def prefix_survival(survival):
    """P[b][k] = prod_{j <= k} s[b][j] from per-position (conditional) survival scores."""
    return np.cumprod(np.asarray(survival, dtype=np.float64), axis=1)


def round_cost(P, verify_len, knot_tokens, knot_tps, t_draft):
    """Cost of one round for a batch.

    P [B, K] prefix survival probabilities, verify_len [B] verified lengths (0..K),
    knot_tokens / knot_tps the throughput curve, t_draft the round's drafting time (s).
    Returns a dict: emitted [B] expected tokens per request, tokens (their sum), N verified
    tokens, t_verify, t_round (s), throughput (tokens/s), per_user (tokens/s of each request)
    and time_per_token (s per emitted token, batch average)."""
    P = np.asarray(P, dtype=np.float64)
    L = np.asarray(verify_len, dtype=np.int64)
    B, K = P.shape
    assert L.shape == (B,) and np.all((L >= 0) & (L <= K))
    mask = np.arange(K)[None, :] < L[:, None]
    emitted = 1.0 + np.sum(np.where(mask, P, 0.0), axis=1)
    N = float(np.sum(L + 1))
    t_verify = N / float(profile(knot_tokens, knot_tps, N))
    t_round = float(t_draft) + t_verify
    tokens = float(np.sum(emitted))
    return dict(emitted=emitted, tokens=tokens, N=N, t_verify=t_verify, t_round=t_round,
                throughput=tokens / t_round, per_user=emitted / t_round,
                time_per_token=t_round / (tokens / B))


def compare(P, verify_len, knot_tokens, knot_tps, t_draft, P1, t_draft1):
    """Per-user speed of a multi-token round against a one-token (MTP-1 style) round on the
    same requests: P1 [B] is each request's probability of passing its single draft token and
    t_draft1 that round's drafting time.  Returns (round, baseline, per-user speed ratio)."""
    r = round_cost(P, verify_len, knot_tokens, knot_tps, t_draft)
    P1 = np.asarray(P1, dtype=np.float64).reshape(-1, 1)
    base = round_cost(P1, np.ones(P1.shape[0], np.int64), knot_tokens, knot_tps, t_draft1)
    return r, base, float(np.mean(r["per_user"]) / np.mean(base["per_user"]))


# kernels of a drafting position, and the fixed launches of a round's draft and schedule
_PER_POSITION = ("markov_head_step", "draft_reduce", "rnn_step")
_FIXED = ("draft_prepare", "schedule", "schedule_prepare", "schedule_rank", "schedule_select")


@dataclass
class MeasuredRound:
    """Round costs taken from measurement.

    t_position  seconds per drafting position (head step + reduction, and the recurrent
                head's update when it runs), the mean over the traced positions;
    t_fixed     seconds of the launches a round pays once (draft set-up, schedule);
    knot_tokens, knot_tps  the measured verify throughput curve (tokens/s against the tokens
                in the verify batch), as profile_builder returns it."""
    t_position: float
    t_fixed: float
    knot_tokens: np.ndarray
    knot_tps: np.ndarray

    @classmethod
    def from_trace(cls, records, n_rounds, n_positions, knot_tokens, knot_tps):
        """records: (kernel name, milliseconds) of n_rounds traced rounds that drafted
        n_positions positions each (dspark Trace.records())."""
        per = sum(ms for name, ms in records if name in _PER_POSITION) * 1e-3
        fixed = sum(ms for name, ms in records if name in _FIXED) * 1e-3
        return cls(per / (n_rounds * n_positions), fixed / n_rounds,
                   np.asarray(knot_tokens, np.float64), np.asarray(knot_tps, np.float64))

    def draft_time(self, K):
        return self.t_fixed + K * self.t_position

    def round(self, P, verify_len, K):
        """round_cost of a round that drafts K positions and verifies verify_len of them."""
        return round_cost(P, verify_len, self.knot_tokens, self.knot_tps, self.draft_time(K))

    def against_one_token(self, P, verify_len, K):
        """Per-user speed of this round against a one-token round on the same requests (one
        drafting position, verified; its pass probability is each request's first survival
        probability).  Returns (round, one-token round, speed ratio)."""
        P = np.asarray(P, np.float64)
        return compare(P, verify_len, self.knot_tokens, self.knot_tps, self.draft_time(K),
                       P[:, 0], self.draft_time(1))
