"""GPU parity of speculative-decoding verification (fs_verify) against the
oracle, through the C ABI.

* Acceptance lengths and emitted tokens equal the oracle's on every row whose
  acceptance decisions are at least 1e-4 (relative) from their boundaries;
  the token at the first rejection (or the bonus token) equals the oracle's
  where its draw's margin exceeds 1e-3; every row has the emitted-prefix
  structure, and a floor on the number of compared draws keeps the token
  check from passing vacuously.  The draw's margin is the oracle's plain
  top-2 gap, except for residual draws, whose set-aside margin this file
  derives (draw_margin below) from the kernel's float32 probabilities.  Shapes: several chunks per row and a ragged tail, V % 4 != 0
  (scalar loads), K from 0 to 32, close and mismatched drafts, greedy rows,
  float32 and float64 noise.
* Reductions to the standalone sampler, bit for bit: identical target and
  draft rows accept every draft token and the bonus token is
  fs_sample_logits on target row K at offset + K; a draft token masked in
  both models takes the residual fallback, fs_sample_logits on that row at
  its position.
* Edge rows: tokens outside the vocabulary, masked tokens, a target row with
  no valid logit, +inf and NaN logits, V = 1, K = 0, B = 0; determinism and
  batch-permutation invariance with row ids.
* The emitted law on the GPU: the first emitted token follows the target
  softmax and the acceptance length the product law, over 2^16 logical rows.
* Full size: the Qwen3-8B-shaped vocabulary (V = 151936), K = 4, B in
  {1, 8, 64}, every row against the oracle.
"""
import numpy as np
import pytest
import torch
from scipy.special import softmax

import decode_exact_categorical_amd as fs
import oracle
import synthetic
from gpu_common import GAP, need_gpu, say
from oracle import stats

pytestmark = pytest.mark.gpu

DECISION_MARGIN = 1e-4


def prob_tol(z):
    """Relative error bound of the kernel's float32 probability of a token whose
    scaled logit is z = (y - M) / t: three roundings in the exponent's argument
    ((y - M), the product with 1/t) grow with |z|, plus an ulp or two of exp2
    and of the normaliser's sum; 4e-7 (4 + |z|) covers them."""
    return 4e-7 * (4.0 + np.abs(z))


def _probs(y, t):
    """(z, p) of one row's temperature softmax over its valid logits, float64
    (the verification semantics: a +inf maximum shares the mass among the +inf
    logits; z is 0 where p does not go through exp)."""
    y = np.asarray(y, dtype=np.float64)
    valid = ~np.isnan(y) & (y != -np.inf)
    z = np.zeros_like(y)
    p = np.zeros_like(y)
    if not valid.any():
        return z, p
    M = y[valid].max()
    if M == np.inf:
        p[valid & (y == np.inf)] = 1.0
    else:
        z[valid] = (y[valid] - M) / t
        p[valid] = np.exp(z[valid])
    return z, p / p.sum()


def draw_margin(target, draft, temp, ref, *, seed, offset, row_ids=None, fp64=False):
    """Per row, the margin of the draw at the oracle's accept_len.  Bonus,
    fallback and greedy draws: the oracle's plain top-2 gap.  Residual draws
    (a sampled rejection with a nonzero residual): the kernel forms each
    probability in float32, so its residual r_j = max(p_t - p_d, 0) may move by
    prob_tol(z) (p_t + p_d); the margin is the winner's score log r_j + g_j with
    its residual lowered by that bound, minus the best other score with its
    residual raised by its own (negative when the draw rests on a residual of
    rounding size)."""
    r_acc, r_out, _, gap = ref
    target = np.asarray(target, dtype=np.float32)
    draft = np.asarray(draft, dtype=np.float32)
    temp = np.asarray(temp, dtype=np.float64)
    B, K1, V = target.shape
    K = K1 - 1
    gap = gap.copy()
    for b in range(B):
        L, t = int(r_acc[b]), float(temp[b])
        if L == K or not (t > 0.0):
            continue
        zt, pt = _probs(target[b, L], t)
        zd, pd = _probs(draft[b, L], t)
        rr = np.maximum(pt - pd, 0.0)
        if not (rr > 0.0).any():
            continue                        # the fallback draw: its plain gap stands
        rid = b if row_ids is None else int(row_ids[b])
        g = oracle.noise_row(seed, offset + L, rid, V, fp64)
        mass = pt + pd
        tol = np.maximum(prob_tol(zt), prob_tol(zd)) * mass
        win = int(r_out[b, L])
        lo = np.log(rr[win] - tol[win]) + g[win] if rr[win] - tol[win] > 0.0 else -np.inf
        other = mass > 0.0
        other[win] = False
        up = rr + tol
        other &= up > 0.0
        hi = (np.log(up[other]) + g[other]).max() if other.any() else -np.inf
        gap[b] = np.inf if hi == -np.inf else lo - hi
    return gap


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def _run(dev, target, draft, tokens, temp, *, seed, offset, row_ids=None, fp64=False):
    rid = None if row_ids is None else torch.as_tensor(row_ids, dtype=torch.int32).to(dev)
    acc, out = fs.verify(target.to(dev), draft.to(dev), tokens.to(dev), temp.to(dev), seed=seed,
                         offset=offset, row_ids=rid, fp64_noise=fp64)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy()


def _check(acc, out, tokens, ref, what, gap, min_decided=0.75, min_drawn=0.9):
    """The parity rule, with `gap` the draws' margins (draw_margin); returns
    (rows compared, tokens compared)."""
    r_acc, r_out, margin, _ = ref
    tokens = np.asarray(tokens)
    B, K1 = out.shape
    K = K1 - 1
    for b in range(B):                     # structure of every row
        L = acc[b]
        assert 0 <= L <= K, (what, b, L)
        assert (out[b, :L] == tokens[b, :L]).all(), (what, b)
        assert (out[b, L + 1:] == -1).all(), (what, b)
    decided = margin > DECISION_MARGIN
    assert decided.mean() >= min_decided, (what, decided.mean())
    bad = np.flatnonzero(decided & (acc != r_acc))
    assert bad.size == 0, (f"{what}: acceptance lengths differ on rows {bad[:5]}: got {acc[bad[:5]]} "
                           f"oracle {r_acc[bad[:5]]} margin {margin[bad[:5]]}")
    rows = np.flatnonzero(decided & (gap > GAP))
    tok = out[rows, acc[rows]]
    r_tok = r_out[rows, r_acc[rows]]
    bad = rows[tok != r_tok]
    assert bad.size == 0, (f"{what}: emitted tokens differ on rows {bad[:5]}: got "
                           f"{out[bad[:5], acc[bad[:5]]]} oracle {r_out[bad[:5], r_acc[bad[:5]]]} "
                           f"gap {gap[bad[:5]]}")
    assert rows.size >= min_drawn * B, (f"{what}: only {rows.size} of {B} drawn tokens compared")
    return decided.sum(), rows.size


CASES = [
    dict(B=4, K=4, V=1000),
    dict(B=37, K=3, V=5003),                      # V % 4 != 0: scalar loads
    dict(B=64, K=4, V=32768),
    dict(B=8, K=1, V=151936),
    dict(B=3, K=0, V=777),                        # a plain draw from target row 0
    dict(B=16, K=8, V=4099),
    dict(B=5, K=32, V=300),
    dict(B=24, K=2, V=70001, draft_noise=3.0),    # a mismatched draft: rejections
    dict(B=50, K=5, V=2000, draft_noise=0.1),     # a close draft: mostly accepted
]


@pytest.mark.parametrize("fp64", [False, True])
@pytest.mark.parametrize("case", CASES)
def test_verify_parity(dev, case, fp64):
    case = dict(case)
    B, K, V = case.pop("B"), case.pop("K"), case.pop("V")
    say(f"verify B={B} K={K} V={V} fp64={fp64} {case}")
    target, draft, tokens = synthetic.spec_decode(B, K, V, seed=60 + B + K, **case)
    temp = synthetic.temperatures(B, seed=61 + B)
    if B >= 3:
        temp[1], temp[2] = 0.0, float("nan")     # greedy rows
    rid = (np.arange(B) * 7 + 3).astype(np.uint32)
    acc, out = _run(dev, target, draft, tokens, temp, seed=4321, offset=1000, row_ids=rid,
                    fp64=fp64)
    ref = oracle.verify(target.numpy(), draft.numpy(), tokens.numpy(), temp.numpy(), seed=4321,
                        offset=1000, row_ids=rid, fp64_noise=fp64)
    gap = draw_margin(target.numpy(), draft.numpy(), temp.numpy(), ref, seed=4321, offset=1000,
                      row_ids=rid, fp64=fp64)
    n_rows, n_tok = _check(acc, out, tokens.numpy(), ref, f"B={B} K={K} V={V}", gap)
    say(f"  compared {n_rows} rows, {n_tok} drawn tokens; mean accept {acc.mean():.2f}")


def test_identical_rows_bonus_is_the_standalone_draw(dev):
    B, K, V = 20, 3, 9001
    say("verify identical rows")
    target, _, tokens = synthetic.spec_decode(B, K, V, seed=70)
    draft = target[:, :K].contiguous()
    temp = synthetic.temperatures(B, seed=71)
    for fp64 in (False, True):
        acc, out = _run(dev, target, draft, tokens, temp, seed=5, offset=77, fp64=fp64)
        assert (acc == K).all()
        assert (out[:, :K] == tokens.numpy()).all()
        ref = fs.sample_logits(target[:, K].contiguous().to(dev), temp.to(dev), seed=5,
                               offset=77 + K, fp64_noise=fp64)
        assert (out[:, K] == ref.cpu().numpy()).all()


def test_masked_draft_token_takes_the_fallback(dev):
    B, K, V = 12, 3, 5000
    say("verify residual fallback")
    target, _, tokens = synthetic.spec_decode(B, K, V, seed=72)
    target[torch.arange(B), 1, tokens[:, 1]] = -float("inf")
    draft = target[:, :K].contiguous()
    temp = torch.full((B,), 0.9)
    acc, out = _run(dev, target, draft, tokens, temp, seed=6, offset=10)
    assert (acc == 1).all()
    ref = fs.sample_logits(target[:, 1].contiguous().to(dev), temp.to(dev), seed=6, offset=11)
    assert (out[:, 1] == ref.cpu().numpy()).all()
    assert (out[:, 2:] == -1).all()


def test_edge_rows(dev):
    B, K, V = 8, 2, 3001
    say("verify edge rows")
    target, draft, tokens = synthetic.spec_decode(B, K, V, seed=73)
    tokens[0, 0], tokens[1, 0] = -1, V              # outside the vocabulary
    target[2, 0, tokens[2, 0]] = -float("inf")      # masked in the target
    target[3, 0, tokens[3, 0]] = float("nan")
    target[4, 0, :] = -float("inf")                 # no valid target logit
    target[5, 0, 17] = target[5, 0, 900] = float("inf")   # +inf logits share the mass
    draft[5, 0, :] = 0.0
    tokens[5, 0] = 5
    draft[6, 1, :] = -float("inf")                  # draft row with no valid logit
    temp = torch.full((B,), 1.0)
    acc, out = _run(dev, target, draft, tokens, temp, seed=9, offset=3)
    ref = oracle.verify(target.numpy(), draft.numpy(), tokens.numpy(), temp.numpy(), seed=9,
                        offset=3)
    gap = draw_margin(target.numpy(), draft.numpy(), temp.numpy(), ref, seed=9, offset=3)
    assert (acc[:6] == 0).all() and (ref[0][:6] == 0).all()
    assert out[4, 0] == -1 and ref[1][4, 0] == -1
    assert out[5, 0] in (17, 900)
    for b in (0, 1, 2, 3):
        assert out[b, 0] != tokens[b, 0]
    _check(acc, out, tokens.numpy(), ref, "edge rows", gap, min_decided=0.5, min_drawn=0.5)
    # V = 1 and K = 0
    t1 = torch.zeros((3, 3, 1))
    d1 = torch.zeros((3, 2, 1))
    tk = torch.zeros((3, 2), dtype=torch.int64)
    acc, out = _run(dev, t1, d1, tk, torch.full((3,), 0.7), seed=1, offset=0)
    assert (acc == 2).all() and (out == 0).all()
    target, _, _ = synthetic.spec_decode(6, 0, 4000, seed=74)
    temp = synthetic.temperatures(6, seed=75)
    acc, out = _run(dev, target, torch.zeros((6, 0, 4000)), torch.zeros((6, 0), dtype=torch.int64),
                    temp, seed=2, offset=8)
    ref = fs.sample_logits(target[:, 0].contiguous().to(dev), temp.to(dev), seed=2, offset=8)
    assert (acc == 0).all() and (out[:, 0] == ref.cpu().numpy()).all()
    # B = 0
    acc, out = _run(dev, torch.zeros((0, 3, 10)), torch.zeros((0, 2, 10)),
                    torch.zeros((0, 2), dtype=torch.int64), torch.zeros(0), seed=1, offset=0)
    assert acc.shape == (0,) and out.shape == (0, 3)


def test_determinism_and_permutation(dev):
    B, K, V = 32, 4, 20000
    say("verify determinism and batch permutation")
    target, draft, tokens = synthetic.spec_decode(B, K, V, seed=76, draft_noise=1.5)
    temp = synthetic.temperatures(B, seed=77)
    rid = np.arange(B, dtype=np.uint32) + 50
    a1, o1 = _run(dev, target, draft, tokens, temp, seed=3, offset=5, row_ids=rid)
    a2, o2 = _run(dev, target, draft, tokens, temp, seed=3, offset=5, row_ids=rid)
    assert (a1 == a2).all() and (o1 == o2).all()
    perm = np.random.default_rng(0).permutation(B)
    pp = torch.from_numpy(perm)
    a3, o3 = _run(dev, target[pp].contiguous(), draft[pp].contiguous(), tokens[pp].contiguous(),
                  temp[pp].contiguous(), seed=3, offset=5, row_ids=rid[perm])
    assert (a3 == a1[perm]).all() and (o3 == o1[perm]).all()
    _, o4 = _run(dev, target, draft, tokens, temp, seed=3, offset=6, row_ids=rid)
    assert not (o4 == o1).all()           # another offset draws other uniforms and noise


def test_emitted_law_on_gpu(dev):
    K, V, T, n = 2, 6, 0.9, 1 << 16
    say(f"verify law over {n} logical rows")
    rng = np.random.default_rng(80)
    tg = (rng.standard_normal((K + 1, V)) * 1.2).astype(np.float32)
    dr = (rng.standard_normal((K, V)) * 1.2).astype(np.float32)
    pt = [softmax(tg[i].astype(np.float64) / T) for i in range(K + 1)]
    pd = [softmax(dr[i].astype(np.float64) / T) for i in range(K)]
    tok = np.stack([rng.choice(V, size=n, p=pd[i]) for i in range(K)], axis=1)
    target = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(tg, (n, K + 1, V))))
    draft = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(dr, (n, K, V))))
    rid = np.arange(n, dtype=np.uint32) * 3 + 1
    acc, out = _run(dev, target, draft, torch.from_numpy(tok), torch.full((n,), T), seed=31,
                    offset=2, row_ids=rid)
    alpha = [np.minimum(pt[i], pd[i]).sum() for i in range(K)]
    law_len = np.array([np.prod(alpha[:m]) * (1 - alpha[m]) for m in range(K)] + [np.prod(alpha)])
    for counts, law in ((np.bincount(out[:, 0], minlength=V), pt[0]),
                        (np.bincount(acc, minlength=K + 1), law_len)):
        chi2 = stats.chi2_statistic(counts, law)
        assert chi2 < stats.chi2_quantile(len(law) - 1, 1e-6), chi2
    # the same rows through the oracle, every 64th
    sel = np.arange(0, n, 64)
    r_acc, r_out = oracle.verify_repeated(tg, dr, tok[sel], T, seed=31, offset=2, row_ids=rid[sel])
    assert (acc[sel] == r_acc).mean() > 0.999
    same = acc[sel] == r_acc
    assert (out[sel][same] == r_out[same]).mean() > 0.999


@pytest.mark.parametrize("B", [1, 8, 64])
def test_verify_qwen_vocabulary(dev, B):
    K, V = 4, 151936
    say(f"verify full size B={B} K={K} V={V}")
    target, draft, tokens = synthetic.spec_decode(B, K, V, seed=90 + B)
    temp = synthetic.temperatures(B, seed=91)
    acc, out = _run(dev, target, draft, tokens, temp, seed=1234, offset=17)
    say("  oracle")
    ref = oracle.verify(target.numpy(), draft.numpy(), tokens.numpy(), temp.numpy(), seed=1234,
                        offset=17)
    gap = draw_margin(target.numpy(), draft.numpy(), temp.numpy(), ref, seed=1234, offset=17)
    n_rows, n_tok = _check(acc, out, tokens.numpy(), ref, f"qwen B={B}", gap, min_decided=0.7)
    say(f"  compared {n_rows} rows, {n_tok} drawn tokens; mean accept {acc.mean():.2f}")
