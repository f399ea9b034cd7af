"""Log-probabilities of the emitted tokens ([P1] cann-recipes-train article
§2.1, which compares draft-token logprobs between decoding paths), on the GPU
through the C ABI, against the oracle.

For every sequence the oracle judges the same way (same emitted tokens; tied
decisions are counted and skipped), logprobs[b, j] for j < num_emitted is
log softmax(l_j / T)[token] (T = 1 for greedy sequences) and NaN after it.
The oracle computes the expected values from its own emitted tokens, never
from the device's.

Tolerance: the device computes (l - m) / T - ln S in float32, with S a sum of
V exponentials taken in chunks (each term within a few ulp, partial sums of 32
terms per lane and tree sums above). The sum's relative error stays below
~4e-6, i.e. an absolute error below ~4e-6 in ln S; the scaled difference
(l - m) * log2(e) / T and the final * ln 2 are rounded a few times (relative
~2e-7 of the result). The bar is |gpu - oracle| <= LP_ATOL + LP_RTOL * |oracle|.
"""
import numpy as np
import pytest
import torch
from scipy import special

import oracle
import sam_drafting_lossless_amd as ssl
from _parity import Tally, compare_verify, dev, say, to_host_logits

pytestmark = pytest.mark.gpu

LP_ATOL = 2e-5
LP_RTOL = 2e-6
SENTINEL = 12345.0


def _check_logprobs(g_lp, tied, r, x_host, T, what):
    g_lp = np.asarray(g_lp, np.float64)
    want = oracle.logprobs(x_host, r.out_tokens, r.num_emitted, T)
    n = 0
    for b in range(g_lp.shape[0]):
        if r.status[b] or tied[b]:
            continue
        e = int(r.num_emitted[b])
        assert np.isnan(g_lp[b, e:]).all(), f"{what} b={b}: {g_lp[b]} past {e}"
        assert np.isfinite(want[b, :e]).all()
        err = np.abs(g_lp[b, :e] - want[b, :e])
        bar = LP_ATOL + LP_RTOL * np.abs(want[b, :e])
        assert (err <= bar).all(), (f"{what} b={b}: gpu {g_lp[b, :e]} oracle "
                                    f"{want[b, :e]}")
        n += e
    return n


def _inputs(rng, B, K, V, greedy_share=0.3, scale=1.5):
    x = (rng.standard_normal((B, K + 1, V)) * scale).astype(np.float32)
    dl = rng.integers(0, K + 1, B).astype(np.int32)
    draft = x[:, :K].argmax(-1).astype(np.int32)
    flip = rng.random((B, K)) < 0.3
    draft[flip] = rng.integers(0, V, int(flip.sum()))
    for b in range(B):
        for j in range(K):
            x[b, j, draft[b, j]] += rng.uniform(0, 6)
    T = rng.uniform(0.4, 1.6, B).astype(np.float32)
    T[rng.random(B) < greedy_share] = 0.0
    u = rng.random((B, K + 1)).astype(np.float32)
    return x, draft, dl, T, u


def _verify(t, draft, dl, T, u, q=None):
    B, R = t.shape[0], t.shape[1]
    lp = torch.full((B, R), SENTINEL, dtype=torch.float32, device="cuda")
    g = ssl.spec_verify(t, dev(draft, torch.int32), dev(dl, torch.int32),
                        dev(T, torch.float32), dev(u, torch.float32), q,
                        logprobs=lp)
    torch.cuda.synchronize()
    return tuple(a.cpu().numpy() for a in g), lp.cpu().numpy()


@pytest.mark.parametrize("B,K,V", [(6, 3, 32), (5, 4, 8193), (4, 2, 3 * 8192 + 4),
                                   (3, 16, 4099), (8, 3, 151936)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_logprobs_one_hot_and_greedy(B, K, V, dtype):
    say(f"[gpu] logprobs one-hot/greedy {dtype} B={B} K={K} V={V}")
    rng = np.random.default_rng(B * 31 + V + (dtype == "bf16"))
    x, draft, dl, T, u = _inputs(rng, B, K, V)
    t = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    xh = to_host_logits(t)
    g, lp = _verify(t, draft, dl, T, u)
    r = oracle.verify(xh, draft, dl, T, u, nthreads=8)
    tally = Tally()
    tied = compare_verify(*g, r, T, u, tally, what=f"logprobs {dtype}")
    n = _check_logprobs(lp, tied, r, xh, T, f"logprobs {dtype}")
    assert n > 0
    say(f"    {n} logprobs")
    tally.check()


@pytest.mark.parametrize("B,K,V", [(4, 3, 32), (3, 5, 30011), (2, 4, 151936)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_logprobs_given_q(B, K, V, dtype):
    """The residual draw (max(0, p - q) normalised) writes the target's own
    log-probability of the token it draws."""
    say(f"[gpu] logprobs given q {dtype} B={B} K={K} V={V}")
    rng = np.random.default_rng(V * 7 + B + (dtype == "bf16"))
    x = (rng.standard_normal((B, K + 1, V)) * 1.4).astype(np.float32)
    T = rng.uniform(0.5, 1.2, B).astype(np.float32)
    ql = x[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32) * 0.9
    q = special.softmax(ql.astype(np.float64) / T[:, None, None], axis=-1)
    draft = np.array([[rng.choice(V, p=q[b, j]) for j in range(K)]
                      for b in range(B)], np.int32)
    dl = rng.integers(0, K + 1, B).astype(np.int32)
    u = rng.random((B, K + 1)).astype(np.float32)
    t = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    xh = to_host_logits(t)
    q32 = q.astype(np.float32)
    g, lp = _verify(t, draft, dl, T, u, torch.from_numpy(q32).cuda())
    r = oracle.verify(xh, draft, dl, T, u, q32, nthreads=8)
    tied = compare_verify(*g, r, T, u, None, what=f"given-q {dtype}")
    assert _check_logprobs(lp, tied, r, xh, T, f"given-q {dtype}") > 0


def test_logprobs_masked_tokens_and_flagged_rows():
    """-inf entries; a row with NaN flags its sequence (its logprobs are not
    written, like its other outputs)."""
    say("[gpu] logprobs with -inf entries and a flagged sequence")
    rng = np.random.default_rng(5)
    B, K, V = 12, 3, 20000
    x, draft, dl, T, u = _inputs(rng, B, K, V, greedy_share=0.5)
    x[:, :, rng.choice(V, 6000, replace=False)] = -np.inf
    draft = np.nan_to_num(x[:, :K], neginf=-1e30).argmax(-1).astype(np.int32)
    dl[3] = K
    x[3, 1, 7] = np.nan
    g, lp = _verify(torch.from_numpy(x).cuda(), draft, dl, T, u)
    r = oracle.verify(x, draft, dl, T, u, nthreads=8)
    tied = compare_verify(*g, r, T, u, None, what="masked")
    assert r.status[3] == ssl.ST_NONFINITE
    assert (lp[3] == SENTINEL).all()
    assert _check_logprobs(lp, tied, r, x, T, "masked") > 0


def test_logprobs_of_the_fused_step_and_the_two_calls():
    """spec_step and spec_stream + spec_finish write the same logprobs as
    spec_verify on the same inputs (the automaton does not change them)."""
    say("[gpu] logprobs: fused step and two-call form")
    rng = np.random.default_rng(17)
    B, K, V = 16, 3, 151936
    x, draft, dl, T, u = _inputs(rng, B, K, V)
    t = torch.from_numpy(x).cuda()
    g, lp = _verify(t, draft, dl, T, u)
    hist = rng.integers(0, V, (B, 40)).astype(np.int32)
    outs = []
    for two in (False, True):
        st = ssl.SamState(B, 100, V, "cuda")
        st.extend(dev(hist), dev(np.full(B, 40, np.int32)))
        lp2 = torch.full((B, K + 1), SENTINEL, dtype=torch.float32, device="cuda")
        args = (t, dev(draft), dev(dl), dev(T), dev(u))
        if two:
            ws = ssl.verify_workspace(B, K, V)
            ssl.spec_stream(*args, ws)
            ssl.spec_finish(*args, ws, state=st, logprobs=lp2)
        else:
            ssl.spec_step(*args, st, logprobs=lp2)
        torch.cuda.synchronize()
        outs.append(lp2.cpu().numpy())
    for o in outs:
        np.testing.assert_array_equal(o, lp)
    r = oracle.verify(x, draft, dl, T, u, nthreads=8)
    tied = compare_verify(*g, r, T, u, None, what="fused")
    assert _check_logprobs(lp, tied, r, x, T, "fused") > 0
