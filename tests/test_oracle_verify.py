"""Pins for the oracle's lossless rejection-sampling verifier.

The rule is the one the pages attribute to Leviathan et al. (10100.com, "speculative
decoding" section; QbitAI, "Speculative decoding" section: the output distribution equals the
target's; wangjunjian.com tag page, post "Speculative Decoding", steps 3-4).  Checked here:
  * the first emitted token is distributed as the target p_1 (chi-squared, 200k request keys),
    and the second, given the first draft token was accepted, as p_2;
  * the acceptance probability at position 1 is sum_v min(p_v, q_v) (binomial test);
  * with a chain-independent drafter, the mean accepted length is
    sum_k prod_{j<=k} alpha_j, alpha_j = sum_v min(p_j, q_j) (Monte Carlo, 4 sigma);
  * special cases: T = 0 gives the exact-match prefix and an argmax correction; q = p always
    accepts and takes the bonus; a draft token with p = 0 is rejected at once;
  * where the random numbers come from: the per-token residual and bonus draws equal the argmax
    of log-weight + G with G from rocRAND's Philox on the residual / bonus stream.
Laws are checked for both samplers (per-token, and the optional two-level race).
"""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle


def _setup(n, V, r, K, T, seed=0, strong=0.7, noise=0.8, zero_head=False):
    """n requests sharing one set of logits but with different request keys."""
    g = torch.Generator().manual_seed(seed)
    U = strong * torch.randn(V, r, generator=g)
    if zero_head:
        U.zero_()
    W = strong * torch.randn(V, r, generator=g)
    zrow = torch.randn(K, V, generator=g)
    Z = zrow.expand(n, K, V).contiguous()
    Yrow = torch.randn(K + 1, V, generator=g) * noise + torch.cat([zrow, zrow[-1:]], 0)
    Y = Yrow.expand(n, K + 1, V).contiguous()
    prev = torch.full((n,), 2, dtype=torch.int32)
    temp = torch.full((n,), T)
    return Z, U, W, Y, prev, temp


def _run(Z, U, W, Y, prev, temp, L, seed=1234, sampler="token"):
    n, K, V = Z.shape
    d = oracle.draft_block(Z, U, W, prev, temp, seed, sampler=sampler)
    vl = torch.full((n,), L, dtype=torch.int32)
    v = oracle.verify(Y, d["tokens"], d["q_tok"].astype(np.float32), d["q_lse"].astype(np.float32),
                      Z, U, W, prev, vl, temp, seed, sampler=sampler)
    return d, v


def _emitted(d, v, i):
    """i-th emitted token (0-based) of each request, or -1 when the round emits fewer."""
    a = v["accept_len"]
    out = np.full(len(a), -1)
    take_draft = a > i
    out[take_draft] = d["tokens"][take_draft, i]
    take_next = a == i
    out[take_next] = v["next_token"][take_next]
    return out


@pytest.mark.parametrize("T,sampler", [(1.0, "token"), (0.7, "token"), (1.0, "block16"),
                                       (0.7, "block16")])
def test_output_distribution_equals_target(T, sampler):
    n, V, r, K = 200_000, 40, 4, 3  # three sampler blocks, the last one 8 tokens long
    Z, U, W, Y, prev, temp = _setup(n, V, r, K, T, seed=11)
    d, v = _run(Z, U, W, Y, prev, temp, L=K, sampler=sampler)
    T32 = float(np.float32(T))
    p1 = torch.softmax(Y[0, 0].double() / T32, 0).numpy()
    p2 = torch.softmax(Y[0, 1].double() / T32, 0).numpy()
    t1 = _emitted(d, v, 0)
    assert np.all(t1 >= 0)
    assert stats.chisquare(np.bincount(t1, minlength=V), p1 * n).pvalue > 1e-4
    t2 = _emitted(d, v, 1)
    sel = t2 >= 0
    assert sel.mean() > 0.2
    assert stats.chisquare(np.bincount(t2[sel], minlength=V), p2 * sel.sum()).pvalue > 1e-4
    # bonus draws (every draft accepted) follow the target of the extra row
    full = v["accept_len"] == K
    assert full.sum() > 2000
    pb = torch.softmax(Y[0, K].double() / T32, 0).numpy()
    assert stats.chisquare(np.bincount(v["next_token"][full], minlength=V),
                           pb * full.sum()).pvalue > 1e-4
    # the draft law alone differs from the target here, so the test has power
    q1 = np.bincount(d["tokens"][:, 0], minlength=V)
    assert stats.chisquare(q1, p1 * n).pvalue < 1e-6


def test_acceptance_rate_is_sum_of_min():
    n, V, r, K = 200_000, 16, 4, 1
    T = 1.0
    Z, U, W, Y, prev, temp = _setup(n, V, r, K, T, seed=12)
    d, v = _run(Z, U, W, Y, prev, temp, L=1)
    c1 = oracle.corrected_row(Z[0, 0], U, W, 2).astype(np.float64)
    q = torch.softmax(torch.from_numpy(c1), 0).numpy()
    p = torch.softmax(Y[0, 0].double(), 0).numpy()
    alpha = np.minimum(p, q).sum()
    k = int((v["accept_len"] >= 1).sum())
    assert stats.binomtest(k, n, alpha).pvalue > 1e-4


def test_mean_accepted_length_closed_form():
    n, V, r, K = 100_000, 16, 4, 4
    T = 1.0
    Z, U, W, Y, prev, temp = _setup(n, V, r, K, T, seed=13, zero_head=True, noise=0.6)
    d, v = _run(Z, U, W, Y, prev, temp, L=K)
    alphas = []
    for k in range(K):
        q = torch.softmax(Z[0, k].double(), 0)
        p = torch.softmax(Y[0, k].double(), 0)
        alphas.append(float(torch.minimum(p, q).sum()))
    expect = np.cumprod(alphas).sum()
    a = v["accept_len"].astype(np.float64)
    assert abs(a.mean() - expect) < 4 * a.std() / np.sqrt(n)


def test_greedy_exact_match_prefix():
    V, K = 50, 4
    g = torch.Generator().manual_seed(14)
    Y = torch.randn(1, K + 1, V, generator=g)
    am = Y[0].argmax(-1)
    Z = torch.randn(1, K, V, generator=g)
    U = torch.zeros(V, 2)
    W = torch.zeros(V, 2)
    tokens = am[:K].clone().to(torch.int32)[None]
    tokens[0, 2] = (am[2] + 1) % V
    ones = np.ones((1, K), np.float32)
    zeros = np.zeros((1, K), np.float32)
    prev = torch.zeros(1, dtype=torch.int32)
    temp = torch.zeros(1)
    v = oracle.verify(Y, tokens, ones, zeros, Z, U, W, prev, torch.tensor([K], dtype=torch.int32),
                      temp, 0)
    assert v["accept_len"][0] == 2 and v["next_token"][0] == int(am[2])
    tokens[0, 2] = am[2]
    tokens[0, 3] = am[3]
    v = oracle.verify(Y, tokens, ones, zeros, Z, U, W, prev, torch.tensor([K], dtype=torch.int32),
                      temp, 0)
    assert v["accept_len"][0] == K and v["next_token"][0] == int(am[K])
    # verify length 0: the round is one plain decoding step from row 0
    v = oracle.verify(Y, tokens, ones, zeros, Z, U, W, prev, torch.tensor([0], dtype=torch.int32),
                      temp, 0)
    assert v["accept_len"][0] == 0 and v["next_token"][0] == int(am[0])


def test_q_equal_p_always_accepts():
    n, V, r, K = 2000, 32, 4, 3
    g = torch.Generator().manual_seed(15)
    U = 0.5 * torch.randn(V, r, generator=g)
    W = 0.5 * torch.randn(V, r, generator=g)
    Z = torch.randn(K, V, generator=g).expand(n, K, V).contiguous()
    prev = torch.full((n,), 1, dtype=torch.int32)
    temp = torch.ones(n)
    d = oracle.draft_block(Z, U, W, prev, temp, 5, want_corrected=True)
    # target logits = the draft's own corrected logits (bonus row: any row)
    Y = torch.cat([torch.from_numpy(d["corrected"]), torch.from_numpy(d["corrected"][:, -1:])], 1)
    v = oracle.verify(Y, d["tokens"], d["q_tok"].astype(np.float32), d["q_lse"].astype(np.float32),
                      Z, U, W, prev, torch.full((n,), K, dtype=torch.int32), temp, 5)
    assert np.all(v["accept_len"] == K)


def test_zero_target_probability_rejects_immediately():
    n, V, r, K = 500, 16, 4, 2
    Z, U, W, Y, prev, temp = _setup(n, V, r, K, 1.0, seed=16)
    d = oracle.draft_block(Z, U, W, prev, temp, 9)
    Y = Y.clone()
    rows = np.arange(n)
    Y[rows, 0, d["tokens"][:, 0]] = -1e4  # p(x_1) underflows to exactly 0
    v = oracle.verify(Y, d["tokens"], d["q_tok"].astype(np.float32), d["q_lse"].astype(np.float32),
                      Z, U, W, prev, torch.full((n,), K, dtype=torch.int32), temp, 9)
    assert np.all(v["accept_len"] == 0)
    assert np.all(v["next_token"] != d["tokens"][:, 0])


@pytest.mark.parametrize("sampler", ["token", "block16"])
def test_bonus_draw_uses_extra_row_position_and_bonus_streams(sampler, rocrand_gumbel):
    """The bonus token is the draw from Y[L] / T at position L on the bonus stream(s) (a
    convention of where its random numbers come from: the law alone cannot tell).  Per-token
    mode: argmax(Y[L] / T + G) with G from rocRAND's Philox on stream 3."""
    n, V, r, K = 64, 40, 4, 3
    Z, U, W, Y, prev, temp = _setup(n, V, r, K, 1.0, seed=21, zero_head=True)
    Y = torch.cat([Z, Z[:, -1:]], 1).contiguous()  # q = p on the drafted rows: always accepted
    for L in (0, 2, 3):
        d, v = _run(Z, U, W, Y, prev, temp, L=L, seed=99, sampler=sampler)
        assert np.all(v["accept_len"] == L)
        for b in range(n):
            y = Y[b, L].double().numpy()
            if sampler == "token":
                want = int(np.argmax(y + rocrand_gumbel(99, b, L, V, 3)))
            else:
                want, _ = oracle.two_level_sample(y, 99, b, L, oracle.STREAM_BONUS,
                                                  oracle.STREAM_BONUS_WITHIN)
            assert v["next_token"][b] == want


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_residual_draw_is_keyed_per_token(T, rocrand_gumbel):
    """A rejected position j is resampled as argmax_v (log r_v + G_v), r = max(0, p - q_j),
    with G from rocRAND's Philox on stream 2 at position j; p from torch's softmax of Y / T and
    q_j from the corrected row (pinned to fp64 matmul) and the draft's own normaliser."""
    n, V, r, K = 48, 40, 4, 3
    Z, U, W, Y, prev, temp = _setup(n, V, r, K, T, seed=23, noise=1.5)
    d = oracle.draft_block(Z, U, W, prev, temp, 7, want_corrected=True)
    T32 = float(np.float32(T))
    vl = torch.full((n,), K, dtype=torch.int32)
    qt, ql = d["q_tok"].astype(np.float32), d["q_lse"].astype(np.float32)
    v = oracle.verify(Y, d["tokens"], qt, ql, Z, U, W, prev, vl, temp, 7)
    rejected = np.flatnonzero(v["accept_len"] < K)
    assert len(rejected) > 10
    for b in rejected:
        j = int(v["accept_len"][b])
        p = torch.softmax(Y[b, j].double() / T32, 0).numpy()
        q = np.exp(d["corrected"][b, j].astype(np.float64) / T32 - float(ql[b, j]))
        res = np.maximum(p - q, 0.0)
        with np.errstate(divide="ignore"):
            lw = np.where(res > 0, np.log(res), -np.inf)
        want = int(np.argmax(lw + rocrand_gumbel(7, b, j, V, 2)))
        assert v["next_token"][b] == want, (b, j)
