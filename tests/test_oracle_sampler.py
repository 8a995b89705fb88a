"""Pins for the oracle's samplers.

The default draw is the per-token Gumbel-max, x = argmax_v (a_v + G_v), keyed per token on
(seed, request, position, vocabulary index, stream).  Checked:
  * the token equals the argmax of a + G with G computed from rocRAND's Philox words under the
    documented keying (an independent generator and a library argmax), with zero-weight tokens;
  * the law: chi-squared against w / sum w over 150k request keys, with a power check.

The optional two-level sampler draws token v with probability w_v / sum w: a Gumbel race
between 16-token blocks weighted by their total weight, then a Gumbel-max inside the winning
block.  Checked:
  * the block uniforms are the documented words of Philox blocks (Philox itself is pinned to
    rocRAND in test_oracle_rng), and the block -> (counter, word) map is one-to-one;
  * with at most 16 tokens (one block) the draw is the textbook Gumbel-max argmax(a + G);
  * the law: chi-squared against w / sum w over 150k request keys, with a short last block,
    zero-weight tokens and a whole zero-weight block (never drawn);
  * a whole block whose weight dominates is chosen in proportion to its weight.
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle


@pytest.mark.parametrize("n", [1, 3, 16, 57, 1000])
def test_token_draw_is_argmax_over_rocrand_gumbels(n, rocrand_gumbel):
    rng = np.random.default_rng(100 + n)
    for trial in range(6):
        seed = int(rng.integers(0, 2**63))
        req, pos, stream = int(rng.integers(0, 5000)), int(rng.integers(0, 64)), trial % 4
        a = rng.normal(size=n) * 2.0
        if n > 3:
            a[rng.choice(n, size=n // 4, replace=False)] = -np.inf  # weight 0: never drawn
        g = rocrand_gumbel(seed, req, pos, n, stream)
        want = int(np.argmax(np.where(np.isfinite(a), a + g, -np.inf)))
        got, gap = oracle.token_sample(a, seed, req, pos, stream)
        assert got == want and np.isfinite(a[got]) and gap >= 0


def test_token_law_is_normalised_weights():
    n_draw, V = 150_000, 56
    rng = np.random.default_rng(6)
    logw = rng.normal(size=V) * 1.2
    logw[[3, 20, 21, 40]] = -np.inf
    w = np.exp(logw)
    p = w / w.sum()
    obs = np.zeros(V, np.int64)
    for req in range(n_draw):
        obs[oracle.token_sample(logw, 17, req, 2, oracle.STREAM_DRAFT)[0]] += 1
    assert obs[[3, 20, 21, 40]].sum() == 0
    live = p > 0
    assert stats.chisquare(obs[live], p[live] * n_draw).pvalue > 1e-4
    flat = live / live.sum()
    assert stats.chisquare(obs[live], flat[live] * n_draw).pvalue < 1e-6


def test_block_uniform_is_documented_philox_word():
    seed, req, pos, stream = 0x1234_5678_9ABC_DEF0, 77, 5, 2
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32)
    seen = set()
    for beta in range(0, 4096, 7):
        a, b, c = beta >> 4, (beta >> 2) & 3, beta & 3
        ctr = np.array([[4 * a + c, pos, req, stream]], np.uint32)
        word = int(oracle.philox(ctr, key)[0, b])
        assert oracle.block_uniform(seed, req, pos, beta, stream) == ((word >> 8) + 0.5) / 2**24
        assert (4 * a + c, b) not in seen
        seen.add((4 * a + c, b))


@pytest.mark.parametrize("n", [1, 5, 16])
def test_single_block_reduces_to_gumbel_max(n):
    rng = np.random.default_rng(n)
    for req in range(200):
        a = rng.normal(size=n) * 2
        u = oracle.uniform(9, req, 3, np.arange(n), oracle.STREAM_DRAFT_WITHIN)
        want = int(np.argmax(a - np.log(-np.log(u))))
        got, _ = oracle.two_level_sample(a, 9, req, 3, oracle.STREAM_DRAFT, oracle.STREAM_DRAFT_WITHIN)
        assert got == want


def test_law_is_normalised_weights():
    n_draw, V = 150_000, 56  # blocks of 16, 16, 16 and 8
    rng = np.random.default_rng(5)
    logw = rng.normal(size=V) * 1.2
    logw[[3, 20, 21]] = -np.inf        # zero-weight tokens
    logw[32:48] = -np.inf              # a whole zero-weight block
    w = np.exp(logw)
    p = w / w.sum()
    obs = np.zeros(V, np.int64)
    for req in range(n_draw):
        x, _ = oracle.two_level_sample(logw, 31, req, 0, oracle.STREAM_RESIDUAL,
                                       oracle.STREAM_RESIDUAL_WITHIN)
        obs[x] += 1
    assert obs[[3, 20, 21]].sum() == 0 and obs[32:48].sum() == 0
    live = p > 0
    assert stats.chisquare(obs[live], p[live] * n_draw).pvalue > 1e-4
    # a flat law over the same support is clearly rejected: the test has power
    flat = live / live.sum()
    assert stats.chisquare(obs[live], flat[live] * n_draw).pvalue < 1e-6


def test_block_chosen_in_proportion_to_its_weight():
    """Block 0 holds one heavy token and 15 light ones; block 1 sixteen equal tokens.  The
    block race must compare total weights (a max-based race would favour block 0)."""
    V, n_draw = 32, 60_000
    logw = np.full(V, 0.0)
    logw[0] = math.log(8.0)
    logw[1:16] = -30.0
    w = np.exp(logw)
    p_block0 = w[:16].sum() / w.sum()           # 8 / 24
    hits = sum(oracle.two_level_sample(logw, 3, req, 1, 0, 4)[0] < 16 for req in range(n_draw))
    assert abs(hits / n_draw - p_block0) < 4 * math.sqrt(p_block0 * (1 - p_block0) / n_draw)
