"""Pins for the oracle's log-probabilities of emitted tokens: log softmax of
the row at the sequence's temperature (1 for greedy sequences), checked
against scipy's log_softmax and against properties the definition fixes."""
import numpy as np
import pytest
from scipy import special

import oracle


def _case(B=6, K=3, V=257, seed=0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((B, K + 1, V)) * 2.0).astype(np.float32)
    out = rng.integers(0, V, (B, K + 1)).astype(np.int32)
    nem = rng.integers(1, K + 2, B).astype(np.int32)
    T = np.array([0.0, 1.0, 0.7, 2.5, 0.0, 1e-3][:B], np.float32)
    return x, out, nem, T


def test_against_scipy_log_softmax():
    x, out, nem, T = _case()
    lp = oracle.logprobs(x, out, nem, T)
    for b in range(x.shape[0]):
        t = float(T[b]) if T[b] > 0 else 1.0
        for j in range(x.shape[1]):
            if j < nem[b]:
                want = special.log_softmax(x[b, j].astype(np.float64) / t)[out[b, j]]
                assert lp[b, j] == pytest.approx(want, abs=1e-9)
            else:
                assert np.isnan(lp[b, j])


def test_properties():
    x, out, nem, T = _case(seed=3)
    B, R, V = x.shape
    full = np.full(B, R, np.int32)
    # every token of a row: the probabilities sum to one
    for b in range(B):
        lps = [oracle.logprobs(x[b:b + 1], np.full((1, R), v, np.int32),
                               full[b:b + 1], T[b:b + 1])[0, 0] for v in range(V)]
        assert np.exp(lps).sum() == pytest.approx(1.0, abs=1e-9)
    # the row's argmax has the largest logprob, and a uniform row gives -log V
    am = x.argmax(axis=2).astype(np.int32)
    lp_am = oracle.logprobs(x, am, full, T)
    lp_any = oracle.logprobs(x, out, full, T)
    assert (lp_am >= lp_any - 1e-12).all()
    u = np.zeros((1, R, V), np.float32)
    lp_u = oracle.logprobs(u, out[:1], full[:1], np.array([0.9], np.float32))
    np.testing.assert_allclose(lp_u, -np.log(V), atol=1e-12)
    # a shift of the whole row changes nothing
    lp_s = oracle.logprobs(x + 5.0, out, full, T)
    np.testing.assert_allclose(lp_s, lp_any, atol=1e-5)


def test_bf16_rows_use_the_widened_values():
    x, out, nem, T = _case(seed=5)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    widened = (bits.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(oracle.logprobs(bits, out, nem, T),
                                  oracle.logprobs(widened, out, nem, T))
