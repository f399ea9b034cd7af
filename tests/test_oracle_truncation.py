"""Pins for the oracle's top-k / top-p truncation of the target distribution
([P3] gogongxt notes "SGLang 的实现": target probabilities renormalised by
top-k, then top-p, one value per request, before verification).

Readings under test: top-k keeps every token whose logit is at least the k-th
largest (ties with it kept); top-p, on what top-k kept, keeps whole groups of
equal logits from the top until the kept share first reaches top_p; then p is
renormalised. Checked against hand cases, numpy's partition, the invariants the
definition fixes (an upper set of logits, minimality of the top-p set), and
chi-square losslessness with respect to the truncated target."""
import numpy as np
import pytest
from scipy import special, stats

import oracle


def _one(logits_row, x, top_k=None, top_p=None, T=1.0, u=(0.0, 0.5)):
    """K = 1, one draft x: returns (VerifyResult, p_draft of x)."""
    lg = np.asarray(logits_row, np.float32)[None, None, :].repeat(2, axis=1)
    r = oracle.verify(lg, np.array([[x]]), np.array([1]),
                      np.array([T], np.float32), np.array([u], np.float32),
                      top_k=None if top_k is None else np.array([top_k]),
                      top_p=None if top_p is None else np.array([top_p], np.float32))
    return r, r.p_draft[0, 0]


def test_hand_cases_top_p():
    # p = [.5, .3, .15, .05]: top_p = .79 keeps {0, 1} (.5 < .79 <= .8),
    # renormalised to [.625, .375]; top_p = .81 keeps {0, 1, 2}.
    lg = np.log([0.5, 0.3, 0.15, 0.05])
    for x, want in [(0, 0.625), (1, 0.375), (2, 0.0), (3, 0.0)]:
        r, pd = _one(lg, x, top_p=0.79)
        assert pd == pytest.approx(want, abs=1e-7)
        assert r.trunc_thr[0, 0] == pytest.approx(np.float32(np.log(0.3)))
    for x, want in [(0, 0.5 / 0.95), (2, 0.15 / 0.95), (3, 0.0)]:
        _, pd = _one(lg, x, top_p=0.81)
        assert pd == pytest.approx(want, rel=1e-6, abs=1e-7)
    # top_p below the largest probability keeps the argmax alone
    _, pd = _one(lg, 0, top_p=0.2)
    assert pd == pytest.approx(1.0)


def test_hand_cases_top_k_with_ties():
    # logits [3, 2, 2, 2, 1]: k = 2 keeps the 3 and every 2 (tied with the
    # 2nd largest); k = 1 keeps only the 3; k = 4 keeps 4 tokens.
    lg = np.array([3.0, 2.0, 2.0, 2.0, 1.0])
    e = np.exp(lg)
    for k, kept in [(1, [0]), (2, [0, 1, 2, 3]), (4, [0, 1, 2, 3]), (5, [0, 1, 2, 3, 4])]:
        Z = e[kept].sum()
        for x in range(5):
            _, pd = _one(lg, x, top_k=k)
            want = e[x] / Z if x in kept else 0.0
            assert pd == pytest.approx(want, rel=1e-6, abs=1e-12), (k, x)
    # top-p after top-k: k = 4 keeps [3, 2, 2, 2]; shares .4046, .1488 x 3.
    # top_p = .5 takes the 3 (.40 < .5), then the whole tied group of 2s.
    Z = e[:4].sum()
    _, pd = _one(lg, 1, top_k=4, top_p=0.5)
    assert pd == pytest.approx(e[1] / Z, rel=1e-6)
    _, pd = _one(lg, 0, top_k=4, top_p=0.4)  # .4046 >= .4: the 3 alone
    assert pd == pytest.approx(1.0)


@pytest.mark.parametrize("T", [0.5, 1.0, 1.7])
def test_top_k_keeps_the_k_largest(T):
    """Distinct logits: the kept set is numpy's k largest, and kept tokens
    keep their relative probabilities (scipy's softmax)."""
    rng = np.random.default_rng(int(T * 10))
    V = 40
    for trial in range(5):
        lg = rng.standard_normal(V).astype(np.float32) * 2
        k = int(rng.integers(1, V))
        top = set(np.argpartition(-lg.astype(np.float64), k - 1)[:k].tolist())
        p = special.softmax(lg.astype(np.float64) / float(np.float32(T)))
        Z = p[list(top)].sum()
        for x in range(V):
            r, pd = _one(lg, x, top_k=k, T=T)
            want = p[x] / Z if x in top else 0.0
            assert pd == pytest.approx(want, rel=1e-9, abs=1e-15)
        assert (lg >= r.trunc_thr[0, 0]).sum() == k


@pytest.mark.parametrize("seed", range(6))
def test_top_p_set_is_minimal_upper_set(seed):
    """For random rows, top-k and top-p: the kept set is an upper set of the
    logits; its share of what top-k kept is at least top_p; without its
    lowest group of tied logits it would fall below top_p."""
    rng = np.random.default_rng(100 + seed)
    V = 64
    lg = np.round(rng.standard_normal(V) * 2, 1).astype(np.float32)  # ties
    T = float(np.float32(rng.uniform(0.5, 1.5)))
    k = int(rng.integers(1, V + 5))
    tp = float(np.float32(rng.uniform(0.05, 0.99)))
    r, _ = _one(lg, 0, top_k=k, top_p=tp, T=T)
    thr = r.trunc_thr[0, 0]
    kept = lg >= thr
    p = special.softmax(lg.astype(np.float64) / T)
    kth = np.sort(lg)[::-1][k - 1] if k < V else -np.inf
    after_k = lg >= kth
    share = p[kept].sum() / p[after_k].sum()
    assert share >= tp - 1e-12
    lowest = lg == lg[kept].min()
    if kept.sum() > lowest.sum():
        assert (p[kept & ~lowest].sum() / p[after_k].sum()) < tp
    # every kept token is at least every dropped token
    if (~kept).any():
        assert lg[kept].min() > lg[~kept].max()
    # p_draft of each token follows the kept set
    for x in range(0, V, 7):
        _, pd = _one(lg, x, top_k=k, top_p=tp, T=T)
        want = p[x] / p[kept].sum() if kept[x] else 0.0
        assert pd == pytest.approx(want, rel=1e-9, abs=1e-15)


def test_no_truncation_is_unchanged():
    rng = np.random.default_rng(7)
    B, K, V = 50, 3, 30
    lg = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    d = rng.integers(0, V, (B, K)).astype(np.int32)
    dl = rng.integers(0, K + 1, B).astype(np.int32)
    T = rng.uniform(0.3, 2, B).astype(np.float32)
    u = rng.random((B, K + 1)).astype(np.float32)
    a = oracle.verify(lg, d, dl, T, u)
    for tk in (0, -1, V, V + 3):
        b = oracle.verify(lg, d, dl, T, u, top_k=np.full(B, tk, np.int32),
                          top_p=np.ones(B, np.float32))
        np.testing.assert_array_equal(a.out_tokens, b.out_tokens)
        np.testing.assert_array_equal(a.p_draft, b.p_draft)
        assert np.isinf(b.trunc_thr[~np.isnan(b.trunc_thr)]).all()


def test_greedy_ignores_truncation_and_invalid_top_p_is_flagged():
    rng = np.random.default_rng(8)
    B, K, V = 20, 2, 16
    lg = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    d = lg[:, :K].argmax(-1).astype(np.int32)
    dl = np.full(B, K, np.int32)
    T = np.zeros(B, np.float32)
    a = oracle.verify(lg, d, dl, T)
    b = oracle.verify(lg, d, dl, T, top_k=np.full(B, 1, np.int32),
                      top_p=np.full(B, 0.01, np.float32))
    np.testing.assert_array_equal(a.out_tokens, b.out_tokens)
    bad = np.array([0.0, -0.5, 1.5, np.nan], np.float32)
    r = oracle.verify(lg[:4], d[:4], dl[:4], T[:4], top_p=bad)
    assert (r.status == oracle.ST_TOP_P).all()


def test_argmax_only():
    """top_k = 1, or a tiny top_p, leaves the argmax alone: it is always
    accepted as a draft and always drawn."""
    rng = np.random.default_rng(9)
    B, V = 400, 50
    lg = rng.standard_normal((B, 2, V)).astype(np.float32)
    am = lg.argmax(-1).astype(np.int32)
    T = np.ones(B, np.float32)
    u = rng.random((B, 2)).astype(np.float32)
    for kw in ({"top_k": np.ones(B, np.int32)},
               {"top_p": np.full(B, 1e-4, np.float32)}):
        r = oracle.verify(lg, am[:, :1], np.ones(B, np.int32), T, u, **kw)
        assert (r.num_emitted == 2).all()
        np.testing.assert_array_equal(r.out_tokens, am)
        other = (am[:, :1] + 1) % V
        r = oracle.verify(lg, other, np.ones(B, np.int32), T, u, **kw)
        assert (r.num_emitted == 1).all() and (r.out_tokens[:, 0] == am[:, 0]).all()


def _truncated(lp, T, k, tp):
    """The truncated target for distinct logits, by numpy sorting."""
    p = special.softmax(lp / T)
    order = np.argsort(-lp)
    keep = np.zeros(len(lp), bool)
    keep[order[:k]] = True
    pk = np.where(keep, p, 0.0)
    pk /= pk.sum()
    cum = np.cumsum(pk[order])
    n = int(np.searchsorted(cum, tp)) + 1
    keep2 = np.zeros(len(lp), bool)
    keep2[order[:n]] = True
    out = np.where(keep2, pk, 0.0)
    return out / out.sum()


@pytest.mark.parametrize("mode", ["onehot", "given_q", "bonus"])
def test_chi_square_follows_the_truncated_target(mode):
    """Lossless with respect to the truncated target: the first emitted token
    is distributed as p' (V = 8, top_k = 6, top_p = 0.85, 10^6 draws)."""
    rng = np.random.default_rng({"onehot": 11, "given_q": 12, "bonus": 13}[mode])
    V, N, T, k, tp = 8, 1_000_000, float(np.float32(0.9)), 6, np.float32(0.85)
    lp = rng.standard_normal(V) * 1.2
    want = _truncated(lp.astype(np.float32).astype(np.float64), T, k, float(tp))
    assert (want == 0).sum() >= 3  # both truncations bite
    u = rng.random((N, 2)).astype(np.float32)
    kw = dict(top_k=np.full(N, k, np.int32), top_p=np.full(N, tp, np.float32),
              nthreads=8)
    Tn = np.full(N, T, np.float32)
    if mode == "bonus":
        logits = np.broadcast_to(lp.astype(np.float32), (N, 1, V)).copy()
        r = oracle.verify(logits, np.zeros((N, 0), np.int32), np.zeros(N, np.int32),
                          Tn, u[:, :1], **kw)
    else:
        logits = np.broadcast_to(lp.astype(np.float32), (N, 2, V)).copy()
        if mode == "onehot":
            draft = rng.integers(0, V, (N, 1)).astype(np.int32)
            q = None
        else:
            qv = special.softmax(rng.standard_normal(V) * 1.5)
            draft = rng.choice(V, size=(N, 1), p=qv).astype(np.int32)
            q = np.broadcast_to(qv.astype(np.float32), (N, 1, V)).copy()
        r = oracle.verify(logits, draft, np.ones(N, np.int32), Tn, u, q=q, **kw)
    counts = np.bincount(r.out_tokens[:, 0], minlength=V)
    assert counts[want == 0].sum() == 0
    m = want > 0
    pv = stats.chisquare(counts[m], want[m] * N).pvalue
    assert pv > 1e-3, (counts, want * N, pv)
