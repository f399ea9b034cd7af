"""Pins for the oracle's verification (CPU only).

Greedy verification reduces to a first-occurrence argmax; probabilities are
checked against scipy's softmax and closed forms; the sampling path is checked
for losslessness with chi-square tests (the output follows the target p for
any draft q), for the rejection rate 1 - sum(min(p, q)), and for the mean
number of tokens per step (1 - a^(K+1)) / (1 - a).
"""
import math

import numpy as np
import pytest
from scipy import special, stats

import oracle


def _rng(s):
    return np.random.default_rng(s)


# ----------------------------------------------------------------- greedy ---
def test_greedy_matches_first_occurrence_argmax():
    rng = _rng(1)
    B, K, V = 200, 4, 37
    # small integer logits make ties common
    logits = rng.integers(-3, 4, (B, K + 1, V)).astype(np.float32)
    am = logits.argmax(-1)  # numpy returns the first occurrence
    draft = am[:, :K].copy().astype(np.int32)
    dl = rng.integers(0, K + 1, B).astype(np.int32)
    # corrupt one position per sequence at random
    bad = rng.integers(0, K, B)
    flip = rng.random(B) < 0.6
    draft[flip, bad[flip]] = (draft[flip, bad[flip]] + 1) % V
    r = oracle.verify(logits, draft, dl, np.zeros(B, np.float32))
    for b in range(B):
        a = 0
        while a < dl[b] and draft[b, a] == am[b, a]:
            a += 1
        want = list(draft[b, :a]) + [am[b, a]]
        assert r.num_emitted[b] == a + 1
        assert r.out_tokens[b, :a + 1].tolist() == want
        assert (r.out_tokens[b, a + 1:] == -1).all()
    assert (r.status == 0).all()


def test_greedy_special_cases():
    V = 10
    logits = np.zeros((1, 3, V), np.float32)
    logits[0, 0, 4] = 1.0
    logits[0, 1, 7] = 2.0
    logits[0, 2, 3] = 5.0
    # d = 0: emit argmax of row 0
    r = oracle.verify(logits, np.array([[4, 7]]), np.array([0]), np.zeros(1))
    assert r.out_tokens.tolist() == [[4, -1, -1]] and r.num_emitted[0] == 1
    # all accepted: bonus is argmax of row d
    r = oracle.verify(logits, np.array([[4, 7]]), np.array([2]), np.zeros(1))
    assert r.out_tokens.tolist() == [[4, 7, 3]] and r.num_emitted[0] == 3
    # all-equal row: the lowest index wins
    z = np.zeros((1, 2, V), np.float32)
    r = oracle.verify(z, np.array([[0]]), np.array([0]), np.zeros(1))
    assert r.out_tokens[0, 0] == 0


# ------------------------------------------------------------ probabilities -
def test_p_draft_matches_scipy_softmax_and_is_shift_invariant():
    rng = _rng(2)
    B, K, V = 16, 3, 1000
    logits = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    T = rng.uniform(0.3, 2.0, B).astype(np.float32)
    draft = rng.integers(0, V, (B, K)).astype(np.int32)
    dl = np.full(B, K, np.int32)
    u = np.zeros((B, K + 1), np.float32)  # accept every draft: all p_draft set
    r = oracle.verify(logits, draft, dl, T, u)
    ref = special.softmax(logits[:, :K].astype(np.float64) / T[:, None, None]
                          .astype(np.float64), axis=-1)
    want = np.take_along_axis(ref, draft[..., None].astype(np.int64), -1)[..., 0]
    np.testing.assert_allclose(r.p_draft, want, rtol=1e-12)
    r2 = oracle.verify(logits + np.float32(37.0), draft, dl, T, u)
    np.testing.assert_allclose(r2.p_draft, r.p_draft, rtol=1e-5)


def test_uniform_logits_give_one_over_v():
    V = 151936
    logits = np.full((1, 2, V), 3.25, np.float32)
    r = oracle.verify(logits, np.array([[123]]), np.array([1]),
                      np.array([0.7], np.float32),
                      np.array([[0.0, 0.5]], np.float32))
    assert r.p_draft[0, 0] == pytest.approx(1.0 / V, rel=1e-12)


def test_bf16_rows_decode_like_torch():
    import torch
    rng = _rng(3)
    B, K, V = 8, 2, 513
    x = torch.from_numpy((rng.standard_normal((B, K + 1, V)) * 3)
                         .astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    f32 = x.to(torch.float32).numpy()
    draft = rng.integers(0, V, (B, K)).astype(np.int32)
    dl = np.full(B, K, np.int32)
    T = np.full(B, 0.7, np.float32)
    u = rng.random((B, K + 1)).astype(np.float32)
    a = oracle.verify(bits, draft, dl, T, u)
    b = oracle.verify(f32, draft, dl, T, u)
    assert (a.out_tokens == b.out_tokens).all()
    np.testing.assert_array_equal(a.p_draft, b.p_draft)


# -------------------------------------------------------------- inverse CDF -
def _logits_for_weights(w):
    """Logits whose softmax at T=1 is proportional to w (w = 0 -> -inf)."""
    w = np.asarray(w, np.float64)
    with np.errstate(divide="ignore"):
        return np.log(w).astype(np.float32)


@pytest.mark.parametrize("w,u,want", [
    # smallest i with cumsum(w)[i] > u * sum(w)
    ([1, 1, 1, 1], 0.0, 0),
    ([1, 1, 1, 1], 0.2499, 0),
    ([1, 1, 1, 1], 0.25, 1),     # cumsum 1 is not > 1: strict test
    ([1, 1, 1, 1], 0.9999, 3),
    ([0, 1, 0, 3], 0.25, 3),     # zero weights are never chosen
    ([0, 1, 0, 3], 0.0, 1),
    ([2, 0, 0, 0], 0.9, 0),
])
def test_bonus_draw_inverse_cdf_hand_cases(w, u, want):
    # d = 0 and T = 1: the single emitted token is the bonus draw from p_0.
    lg = _logits_for_weights(w)[None, None, :].repeat(2, axis=1)
    r = oracle.verify(lg, np.array([[0]]), np.array([0]),
                      np.array([1.0], np.float32),
                      np.array([[0.5, u]], np.float32))
    assert r.out_tokens[0, 0] == want
    c = np.cumsum(np.asarray(w, np.float64)) / np.sum(w)
    assert r.cdf_hi[0] == pytest.approx(c[want])


def test_one_hot_residual_excludes_the_rejected_token():
    # p = [0.5, 0.25, 0.25]; draft x = 0 rejected (u = 0.9 > 0.5); residual is
    # p with x zeroed: [0, .25, .25] -> final coin 0.4 picks token 1, 0.6 -> 2.
    lg = _logits_for_weights([2, 1, 1])[None, None, :].repeat(2, axis=1)
    for fc, want in [(0.4, 1), (0.6, 2), (0.0, 1)]:
        r = oracle.verify(lg, np.array([[0]]), np.array([1]),
                          np.array([1.0], np.float32),
                          np.array([[0.9, fc]], np.float32))
        assert r.num_emitted[0] == 1 and r.out_tokens[0, 0] == want
        assert r.alpha[0, 0] == pytest.approx(0.5)


def test_given_q_residual_is_positive_part_of_p_minus_q():
    # p = [.5, .3, .2], q = [.1, .6, .3]: draft x = 1 has alpha = .3/.6 = .5.
    # residual max(0, p - q) = [.4, 0, 0] -> always token 0.
    p = np.array([0.5, 0.3, 0.2])
    lg = np.log(p).astype(np.float32)[None, None, :].repeat(2, axis=1)
    q = np.array([[[0.1, 0.6, 0.3]]], np.float32)
    for fc in (0.0, 0.5, 0.99):
        r = oracle.verify(lg, np.array([[1]]), np.array([1]),
                          np.array([1.0], np.float32),
                          np.array([[0.75, fc]], np.float32), q=q)
        assert r.out_tokens[0, 0] == 0 and r.num_emitted[0] == 1
        assert r.alpha[0, 0] == pytest.approx(0.5, rel=1e-6)
    # u <= alpha accepts; the bonus then comes from row 1
    r = oracle.verify(lg, np.array([[1]]), np.array([1]),
                      np.array([1.0], np.float32),
                      np.array([[0.4, 0.0]], np.float32), q=q)
    assert r.num_emitted[0] == 2 and r.out_tokens[0, :2].tolist() == [1, 0]


# ----------------------------------------------------------- losslessness ---
def _chi2_pvalue(counts, p):
    exp = p * counts.sum()
    return stats.chisquare(counts, exp).pvalue


@pytest.mark.parametrize("mode", ["onehot", "given_q"])
def test_chi_square_first_token_follows_target(mode):
    """Lossless rejection sampling: whatever q the draft came from, the first
    emitted token is distributed as the target p (V = 8, 10^6 draws)."""
    rng = _rng(4 if mode == "onehot" else 5)
    V, N = 8, 1_000_000
    lp = rng.standard_normal(V) * 1.2
    p = special.softmax(lp)
    logits = np.broadcast_to(lp.astype(np.float32), (N, 2, V)).copy()
    u = rng.random((N, 2)).astype(np.float32)
    if mode == "onehot":
        draft = rng.integers(0, V, (N, 1)).astype(np.int32)
        q = None
    else:
        qv = special.softmax(rng.standard_normal(V) * 1.5)
        draft = rng.choice(V, size=(N, 1), p=qv).astype(np.int32)
        q = np.broadcast_to(qv.astype(np.float32), (N, 1, V)).copy()
    r = oracle.verify(logits, draft, np.ones(N, np.int32),
                      np.ones(N, np.float32), u, q=q, nthreads=8)
    counts = np.bincount(r.out_tokens[:, 0], minlength=V)
    pv = _chi2_pvalue(counts, p)
    assert pv > 1e-3, (counts, p * N, pv)
    if mode == "given_q":
        # rejection probability = 1 - sum(min(p, q))
        rej = np.mean(r.num_emitted == 1)
        want = 1.0 - np.minimum(p, qv.astype(np.float32)).sum()
        se = math.sqrt(want * (1 - want) / N)
        assert abs(rej - want) < 5 * se


def test_chi_square_bonus_token_follows_target():
    rng = _rng(6)
    V, N = 8, 1_000_000
    lp = rng.standard_normal(V)
    logits = np.broadcast_to(lp.astype(np.float32), (N, 1, V)).copy()
    u = rng.random((N, 1)).astype(np.float32)
    r = oracle.verify(logits, np.zeros((N, 0), np.int32), np.zeros(N, np.int32),
                      np.full(N, 0.8, np.float32), u, nthreads=8)
    counts = np.bincount(r.out_tokens[:, 0], minlength=V)
    assert _chi2_pvalue(counts, special.softmax(lp / 0.8)) > 1e-3


def test_q_equal_p_never_rejects_and_certain_token_always_accepts():
    rng = _rng(7)
    V, N, K = 8, 200, 3
    lp = rng.standard_normal((N, K + 1, V)).astype(np.float32)
    p = special.softmax(lp[:, :K].astype(np.float64), axis=-1)
    draft = np.array([[rng.choice(V, p=p[n, j]) for j in range(K)]
                      for n in range(N)], np.int32)
    r = oracle.verify(lp, draft, np.full(N, K, np.int32), np.ones(N, np.float32),
                      rng.random((N, K + 1)).astype(np.float32),
                      q=p.astype(np.float32))
    # alpha = min(1, p/q) = 1 up to the float32 rounding of q
    assert np.nanmin(r.alpha) > 1 - 1e-6
    assert (r.num_emitted == K + 1).mean() > 0.99
    # p(x) = 1 exactly (all other logits -inf): one-hot drafts always accepted
    lg = np.full((50, K + 1, V), -np.inf, np.float32)
    lg[:, :, 3] = 0.0
    r = oracle.verify(lg, np.full((50, K), 3, np.int32), np.full(50, K, np.int32),
                      np.ones(50, np.float32),
                      np.full((50, K + 1), np.nextafter(np.float32(1),
                                                        np.float32(0))))
    assert (r.num_emitted == K + 1).all() and (r.out_tokens == 3).all()


@pytest.mark.parametrize("alpha", [0.2, 0.5, 0.8])
def test_mean_tokens_per_step_closed_form(alpha):
    """With every draft accepted independently with probability a, the mean
    number of tokens per step is (1 - a^(K+1)) / (1 - a) (numerator of the
    speed-up formula on the m.nxbn.cn guide, section 2.3)."""
    rng = _rng(int(alpha * 100))
    K, N = 3, 200_000
    lg = np.log(np.array([alpha, 1 - alpha]))[None, None, :].astype(np.float32)
    logits = np.broadcast_to(lg, (N, K + 1, 2)).copy()
    u = rng.random((N, K + 1)).astype(np.float32)
    r = oracle.verify(logits, np.zeros((N, K), np.int32), np.full(N, K, np.int32),
                      np.ones(N, np.float32), u, nthreads=8)
    want = (1 - alpha ** (K + 1)) / (1 - alpha)
    var = np.var(r.num_emitted)
    assert abs(r.num_emitted.mean() - want) < 5 * math.sqrt(var / N)


# ----------------------------------------------------------------- status ---
def test_status_bits():
    V, K = 16, 2
    lg = np.zeros((6, K + 1, V), np.float32)
    draft = np.zeros((6, K), np.int32)
    dl = np.full(6, K, np.int32)
    T = np.zeros(6, np.float32)
    dl[0] = K + 1                  # draft_len > K
    draft[1, 1] = V                # token out of range
    lg[2, 1, 5] = np.nan           # non-finite row
    T[3] = -1.0                    # bad temperature
    lg[4, 0, :] = -np.inf          # no finite entry
    r = oracle.verify(lg, draft, dl, T)
    assert r.status.tolist() == [oracle.ST_DRAFT_LEN, oracle.ST_TOKEN_RANGE,
                                 oracle.ST_NONFINITE, oracle.ST_TEMPERATURE,
                                 oracle.ST_NONFINITE, 0]
    assert (r.out_tokens[:5] == -1).all() and r.num_emitted[5] == K + 1
    r = oracle.verify(lg[5:], draft[5:], dl[5:], np.ones(1, np.float32), None)
    assert r.status.tolist() == [oracle.ST_NO_UNIFORMS]
    # positive temperatures below the smallest normal float are rejected
    tiny = np.array([1e-40, np.finfo(np.float32).tiny, np.inf], np.float32)
    u = np.zeros((3, K + 1), np.float32)
    r = oracle.verify(lg[:3] * 0, np.zeros((3, K), np.int32),
                      np.zeros(3, np.int32), tiny, u)
    assert r.status.tolist() == [oracle.ST_TEMPERATURE, 0, oracle.ST_TEMPERATURE]


# ------------------------------------------------------- whole-step greedy ---
def _toy_target(ctx, V, seed, w=2):
    """Context-deterministic toy target: logits depend only on the last w
    tokens (hash-seeded noise plus a boost that makes the text repetitive)."""
    key = (seed, *[int(t) for t in ctx[-w:]])
    r = np.random.default_rng(abs(hash(key)) % (2 ** 63))
    lg = r.standard_normal(V).astype(np.float32)
    lg[(sum(int(t) for t in ctx[-w:]) * 7 + 3) % V] += 2.5
    return lg


def test_speculative_greedy_equals_plain_greedy():
    """The m.nxbn.cn guide's check (section 5.4): decode once without
    speculation and once with it; greedy outputs must agree token for token."""
    V, K, steps = 32, 4, 120
    prompt = [1, 2, 3, 4, 5, 1, 2, 3]
    plain = list(prompt)
    while len(plain) < len(prompt) + steps + K + 2:
        plain.append(int(np.argmax(_toy_target(plain, V, 11))))
    sam = oracle.SAM(prompt)
    text = list(prompt)
    accepted = 0
    while len(text) < len(prompt) + steps:
        d, dl, _ = sam.draft(K)
        rows = np.stack([_toy_target(text + d[:j].tolist(), V, 11)
                         for j in range(K + 1)])[None]
        r = oracle.verify(rows, d[None], np.array([dl]), np.zeros(1, np.float32))
        em = r.out_tokens[0, :r.num_emitted[0]].tolist()
        accepted += r.num_emitted[0] - 1
        sam.extend(em)
        text += em
    assert text == plain[:len(text)]
    assert accepted > steps // 4  # the drafts were actually exercised


def test_acceptance_boundary_is_inclusive():
    """Accept iff eps <= alpha(x) (the cann-recipes-train article, section
    1.1). Two equal logits give p = 1/2 exactly, so u = 0.5 must accept."""
    lg = np.zeros((1, 2, 2), np.float32)
    r = oracle.verify(lg, np.array([[0]]), np.array([1]),
                      np.array([1.0], np.float32),
                      np.array([[0.5, 0.1]], np.float32))
    assert r.num_emitted[0] == 2 and r.out_tokens[0, 0] == 0
    r = oracle.verify(lg, np.array([[0]]), np.array([1]),
                      np.array([1.0], np.float32),
                      np.array([[np.nextafter(np.float32(0.5), np.float32(1)),
                                 0.1]], np.float32))
    assert r.num_emitted[0] == 1 and r.out_tokens[0, 0] == 1


def test_bonus_comes_from_row_draft_len():
    """All d drafts accepted: the bonus is drawn from the target at row d (the
    extra position after the last draft, m.nxbn.cn guide section 2.2)."""
    V, K = 8, 3
    lg = np.full((2, K + 1, V), -np.inf, np.float32)
    # rows 0..2 certain of tokens 1, 2, 3; row 3 certain of token 6
    for j, t in enumerate([1, 2, 3, 6]):
        lg[:, j, t] = 0.0
    draft = np.array([[1, 2, 3], [1, 2, 3]], np.int32)
    dl = np.array([3, 2], np.int32)
    u = np.full((2, K + 1), 0.3, np.float32)
    r = oracle.verify(lg, draft, dl, np.ones(2, np.float32), u)
    assert r.out_tokens[0].tolist() == [1, 2, 3, 6] and r.num_emitted[0] == 4
    assert r.out_tokens[1].tolist() == [1, 2, 3, -1] and r.num_emitted[1] == 3
    g = oracle.verify(lg, draft, dl, np.zeros(2, np.float32))
    assert g.out_tokens[0].tolist() == [1, 2, 3, 6]
    assert g.out_tokens[1].tolist() == [1, 2, 3, -1]


def test_empty_residual_falls_back_to_target():
    """If max(0, p - q) is zero everywhere (q >= p elementwise, as float32 q
    that sums above 1 can be), the draw falls back to p."""
    lg = np.zeros((1, 2, 2), np.float32)          # p = [.5, .5]
    q = np.array([[[0.55, 0.55]]], np.float32)    # alpha(0) = .5/.55
    for fc, want in [(0.3, 0), (0.7, 1)]:
        r = oracle.verify(lg, np.array([[0]]), np.array([1]),
                          np.array([1.0], np.float32),
                          np.array([[0.95, fc]], np.float32), q=q)
        assert r.num_emitted[0] == 1 and r.out_tokens[0, 0] == want
