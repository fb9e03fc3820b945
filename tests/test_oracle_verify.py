"""Pins of the oracle's speculative-decoding verification (draft token x
accepted with probability min(1, p_t(x) / p_d(x)); the first rejection
replaced by a draw from max(p_t - p_d, 0) renormalised; a bonus draw from the
target's last row when every draft token is accepted), independent of the
oracle's own code:

* the emitted stream's law: the first emitted token follows the target
  softmax (chi-square) with a deliberately mismatched draft, and so does the
  second among rows that reach it; the acceptance rate equals the analytic
  sum_j min(p_t, p_d) and the acceptance length of K = 4 follows the product
  law; given a rejection at position 0 the token follows the normalised
  residual, given full acceptance the bonus token follows the target's last
  row (softmaxes and laws written out with scipy, draft tokens drawn from the
  draft softmax by numpy);
* a hand-worked row (p_t = 0.5/0.3/0.2 against p_d = 0.2/0.3/0.5);
* special cases that reduce to other pinned results: identical target and
  draft rows accept everything and their bonus draw is the standalone
  sampler's draw at offset + K; a masked draft token forces the residual
  fallback, the standalone draw at that position; greedy rows are numpy's
  argmax rule; tokens outside the vocabulary and masked target rows.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import stats


def _law_rows(seed, K, V):
    rng = np.random.default_rng(seed)
    tg = (rng.standard_normal((K + 1, V)) * 1.2).astype(np.float32)
    dr = (rng.standard_normal((K, V)) * 1.2).astype(np.float32)   # unrelated to the target
    return tg, dr


def _draft_tokens(dr, T, n, seed):
    """Draft tokens drawn from the draft softmax, position by position."""
    rng = np.random.default_rng(seed)
    K, V = dr.shape
    cols = [rng.choice(V, size=n, p=softmax(dr[i].astype(np.float64) / T)) for i in range(K)]
    return np.stack(cols, axis=1)


def _chi2_ok(counts, law):
    keep = law > 0
    assert counts[~keep].sum() == 0, "a token with zero probability was emitted"
    chi2 = stats.chi2_statistic(counts[keep], law[keep])
    thr = stats.chi2_quantile(int(keep.sum()) - 1, 1e-6)
    return chi2 < thr, (chi2, thr)


@pytest.mark.parametrize("fp64", [False, True])
def test_emitted_law_and_acceptance(fp64):
    K, V, T, n = 4, 6, 0.9, 200000
    tg, dr = _law_rows(21, K, V)
    tok = _draft_tokens(dr, T, n, seed=22)
    rid = np.arange(n, dtype=np.uint32)
    acc, out = oracle.verify_repeated(tg, dr, tok, T, seed=99, offset=40, row_ids=rid,
                                      fp64_noise=fp64)
    pt = [softmax(tg[i].astype(np.float64) / T) for i in range(K + 1)]
    pd = [softmax(dr[i].astype(np.float64) / T) for i in range(K)]
    alpha = [np.minimum(pt[i], pd[i]).sum() for i in range(K)]
    # emitted tokens: the accepted prefix is the draft's, then one more
    for q in range(0, n, 997):
        L = acc[q]
        assert (out[q, :L] == tok[q, :L]).all() and (out[q, L + 1:] == -1).all()
        assert 0 <= out[q, L] < V
    # the first emitted token follows p_t(row 0)
    ok, why = _chi2_ok(np.bincount(out[:, 0], minlength=V), pt[0])
    assert ok, why
    # the second, among rows that emit one, follows p_t(row 1)
    sel = acc >= 1
    ok, why = _chi2_ok(np.bincount(out[sel, 1], minlength=V), pt[1])
    assert ok, why
    # acceptance rate at position 0
    a0 = (acc >= 1).sum()
    sd = np.sqrt(n * alpha[0] * (1 - alpha[0]))
    assert abs(a0 - n * alpha[0]) < 5.5 * sd, (a0, n * alpha[0], sd)
    # acceptance length: P(L = m) = alpha_0 ... alpha_{m-1} (1 - alpha_m)
    law = np.array([np.prod(alpha[:m]) * (1 - alpha[m]) for m in range(K)] + [np.prod(alpha)])
    ok, why = _chi2_ok(np.bincount(acc, minlength=K + 1), law)
    assert ok, why
    # given a rejection at 0: the residual law; given full acceptance: p_t(row K)
    res = np.maximum(pt[0] - pd[0], 0)
    ok, why = _chi2_ok(np.bincount(out[acc == 0, 0], minlength=V), res / res.sum())
    assert ok, why
    ok, why = _chi2_ok(np.bincount(out[acc == K, K], minlength=V), pt[K])
    assert ok, why


def test_hand_worked_row():
    # p_t = 0.5 / 0.3 / 0.2 and p_d = 0.2 / 0.3 / 0.5 at temperature 1
    tg = np.log(np.array([[0.5, 0.3, 0.2], [0.1, 0.1, 0.8]])).astype(np.float32)
    dr = np.log(np.array([[0.2, 0.3, 0.5]])).astype(np.float32)
    n = 100000
    rid = np.arange(n, dtype=np.uint32)
    # token 2: accepted with probability 0.2 / 0.5; a rejection emits token 0,
    # the only token with p_t > p_d
    acc, out = oracle.verify_repeated(tg, dr, np.full((n, 1), 2), 1.0, seed=3, offset=0,
                                      row_ids=rid)
    assert abs((acc == 1).mean() - 0.4) < 5 * np.sqrt(0.24 / n)
    assert (out[acc == 0, 0] == 0).all() and (out[acc == 1, 0] == 2).all()
    # tokens 0 and 1 (p_t >= p_d) are always accepted
    for x in (0, 1):
        acc, out = oracle.verify_repeated(tg, dr, np.full((1000, 1), x), 1.0, seed=3, offset=0,
                                          row_ids=rid[:1000])
        assert (acc == 1).all() and (out[:, 0] == x).all()


def test_identical_rows_and_bonus_is_the_standalone_draw():
    rng = np.random.default_rng(31)
    B, K, V = 12, 3, 300
    tg = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    dr = tg[:, :K].copy()
    tok = rng.integers(0, V, (B, K))
    temp = rng.uniform(0.5, 1.2, B).astype(np.float32)
    rid = (rng.permutation(B) + 1000).astype(np.uint32)
    for fp64 in (False, True):
        acc, out, margin, gap = oracle.verify(tg, dr, tok, temp, seed=7, offset=50, row_ids=rid,
                                              fp64_noise=fp64)
        assert (acc == K).all()
        np.testing.assert_array_equal(out[:, :K], tok)
        ref, _, _ = oracle.sample_logits(tg[:, K], temp, seed=7, offset=50 + K, row_ids=rid,
                                         fp64_noise=fp64)
        np.testing.assert_array_equal(out[:, K], ref)


def test_masked_draft_token_takes_the_fallback_draw():
    """Identical rows except that the position-1 draft token is masked in
    both models: rejected there (p_t = 0), and the residual is zero, so the
    draw is the target's own: the standalone sampler's at offset + 1."""
    rng = np.random.default_rng(32)
    B, K, V = 10, 3, 200
    tg = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    tok = rng.integers(0, V, (B, K))
    tg[np.arange(B), 1, tok[:, 1]] = -np.inf
    dr = tg[:, :K].copy()
    temp = np.full(B, 0.8, dtype=np.float32)
    acc, out, _, _ = oracle.verify(tg, dr, tok, temp, seed=8, offset=5)
    assert (acc == 1).all()
    ref, _, _ = oracle.sample_logits(tg[:, 1], temp, seed=8, offset=6, row_ids=np.arange(B))
    np.testing.assert_array_equal(out[:, 1], ref)
    assert (out[:, 2:] == -1).all()


def test_greedy_rows():
    rng = np.random.default_rng(33)
    B, K, V = 40, 4, 30
    tg = np.round(rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)   # ties
    dr = rng.standard_normal((B, K, V)).astype(np.float32)
    am = np.argmax(tg, axis=2)                     # first occurrence
    tok = am[:, :K].copy()
    wrong = rng.random((B, K)) < 0.3
    tok[wrong] = (tok[wrong] + 1 + rng.integers(0, V - 1, wrong.sum())) % V
    for t in (0.0, -1.0, np.nan):
        acc, out, _, _ = oracle.verify(tg, dr, tok, np.full(B, t, dtype=np.float32), seed=1,
                                       offset=2)
        for b in range(B):
            bad = np.flatnonzero(tok[b] != am[b, :K])
            L = bad[0] if bad.size else K
            assert acc[b] == L
            np.testing.assert_array_equal(out[b, :L], tok[b, :L])
            assert out[b, L] == am[b, L]


def test_out_of_range_and_masked_tokens():
    rng = np.random.default_rng(34)
    B, K, V = 6, 2, 40
    tg = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    dr = rng.standard_normal((B, K, V)).astype(np.float32)
    tok = rng.integers(0, V, (B, K))
    tok[0, 0], tok[1, 0] = -1, V              # outside the vocabulary: rejected
    tg[2, 0, tok[2, 0]] = -np.inf             # masked in the target: rejected
    tg[3, 0, tok[3, 0]] = np.nan
    tg[4, 0, :] = -np.inf                     # nothing valid: rejected, no token
    tg[5, 0, ::2] = -np.inf                   # masked tokens never emitted
    for b in range(6):
        dr[b, 0, :] = 0.0
    temp = np.full(B, 1.0, dtype=np.float32)
    for offset in range(20):
        acc, out, _, _ = oracle.verify(tg, dr, tok, temp, seed=11, offset=offset)
        assert (acc[:5] == 0).all()
        assert (out[:4, 0] >= 0).all() and out[4, 0] == -1
        for b in (2, 3):
            assert out[b, 0] != tok[b, 0]
        assert out[5, 0] % 2 == 1 or (acc[5] >= 1 and out[5, 0] == tok[5, 0])


def test_acceptance_uniform_counter():
    """The acceptance uniform is the 52-bit midpoint value of words 0 and 1 of
    Philox counter (2^32 - 1, row id, position lo, position hi): no vocabulary
    word index reaches that counter value."""
    for seed, pos, r in ((0, 0, 0), (1234, 7, 3), (2**64 - 1, 2**40 + 5, 2**32 - 1)):
        ctr = [0xFFFFFFFF, r, pos & 0xFFFFFFFF, pos >> 32]
        x = oracle.philox_block(ctr, [seed & 0xFFFFFFFF, seed >> 32])
        k = ((int(x[0]) << 32) | int(x[1])) >> 12
        assert oracle.accept_uniform(seed, pos, r) == (k + 0.5) / 2**52
