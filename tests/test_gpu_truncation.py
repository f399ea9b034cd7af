"""Top-k / top-p truncation of the target before verification ([P3] gogongxt
notes "SGLang 的实现"), on the GPU through the C ABI, against the oracle.

Bars: as for untruncated verification (greedy bit-exact; T > 0 decisions equal
except coin ties; p_draft within 1e-5 relative). In addition, a sequence
whose top-p decision the oracle found within TRUNC_TIE (relative to the mass
top-k kept) of flipping, at any row it judged, may keep a different set on
the device (the device sums in float): such a sequence, when the device's
outputs differ from the oracle's, is set aside, counted and bounded
(``_parity.Tally``)."""
import numpy as np
import pytest
import torch
from scipy import special, stats

import oracle
import sam_drafting_lossless_amd as ssl
from _parity import P_ATOL, P_RTOL, Tally, compare_verify, dev, say, to_host_logits

pytestmark = pytest.mark.gpu

TRUNC_TIE = 1e-5


def _params(rng, B, V):
    """Per-sequence top_k / top_p: off, top-k only, top-p only, both."""
    kind = rng.integers(0, 4, B)
    top_k = np.where(kind % 2 == 1, rng.integers(1, min(V, 300) + 1, B), 0)
    top_p = np.where(kind >= 2, rng.uniform(0.2, 0.98, B), 1.0)
    return top_k.astype(np.int32), top_p.astype(np.float32)


def _inputs(rng, B, K, V, scale=1.5, greedy_share=0.15):
    x = (rng.standard_normal((B, K + 1, V)) * scale).astype(np.float32)
    dl = rng.integers(0, K + 1, B).astype(np.int32)
    draft = x[:, :K].argmax(-1).astype(np.int32)
    flip = rng.random((B, K)) < 0.35
    draft[flip] = rng.integers(0, V, int(flip.sum()))
    for b in range(B):
        for j in range(K):
            x[b, j, draft[b, j]] += rng.uniform(0, 5)
    T = rng.uniform(0.4, 1.6, B).astype(np.float32)
    T[rng.random(B) < greedy_share] = 0.0
    u = rng.random((B, K + 1)).astype(np.float32)
    return x, draft, dl, T, u


def _run(t, draft, dl, T, u, top_k, top_p, q=None):
    g = ssl.spec_verify(t, dev(draft, torch.int32), dev(dl, torch.int32),
                        dev(T, torch.float32), dev(u, torch.float32), q,
                        top_k=None if top_k is None else dev(top_k, torch.int32),
                        top_p=None if top_p is None else dev(top_p, torch.float32))
    torch.cuda.synchronize()
    return tuple(a.cpu().numpy() for a in g)


def _compare(g, r, T, u, what, tally):
    """Sets aside a sequence only if the device disagrees with the oracle on
    it and the oracle found its top-p decision within TRUNC_TIE of flipping;
    every other sequence is compared at the usual bar."""
    mg = np.where(np.isnan(r.trunc_margin), np.inf, r.trunc_margin).min(axis=1)
    out, nem, pd, st = (np.asarray(a) for a in g)
    pd_ok = np.isclose(pd, r.p_draft, rtol=P_RTOL, atol=P_ATOL) | (
        (pd < 0) & (r.p_draft < 0))
    agree = ((nem == r.num_emitted) & (out == r.out_tokens).all(axis=1)
             & pd_ok.all(axis=1) & (st == r.status))
    near = (mg <= TRUNC_TIE) & ~agree
    keep = ~near
    sub = oracle.VerifyResult(r.out_tokens[keep], r.num_emitted[keep], r.p_draft[keep],
                              r.alpha[keep], r.cdf_lo[keep], r.cdf_hi[keep],
                              r.status[keep])
    compare_verify(*(a[keep] for a in g), sub, np.asarray(T)[keep],
                   None if u is None else np.asarray(u)[keep], tally, what=what)
    tally.set_aside += int(near.sum())
    tally.sequences += len(near)
    return int(near.sum())


@pytest.mark.parametrize("B,K,V", [(8, 3, 32), (6, 4, 8193), (5, 2, 3 * 8192 + 4),
                                   (4, 16, 4099), (8, 3, 151936)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_truncated_sampling_matches_oracle(B, K, V, dtype):
    say(f"[gpu] truncation {dtype} B={B} K={K} V={V}")
    rng = np.random.default_rng(B * 131 + V + (dtype == "bf16"))
    x, draft, dl, T, u = _inputs(rng, B, K, V)
    top_k, top_p = _params(rng, B, V)
    t = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    xh = to_host_logits(t)
    g = _run(t, draft, dl, T, u, top_k, top_p)
    r = oracle.verify(xh, draft, dl, T, u, nthreads=8, top_k=top_k, top_p=top_p)
    tally = Tally()
    near = _compare(g, r, T, u, f"trunc {dtype}", tally)
    assert near <= max(1, B // 10)
    tally.check()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_chunks_per_wavefront(dtype):
    """V = 1,000,000 (123 fp32 chunks, 62 bf16): the select kernel's
    wavefronts each take several chunks' segments in turn (the next one
    requested while the current one is worked), with top-k, top-p and both."""
    say(f"[gpu] truncation: V = 1,000,000 {dtype}")
    rng = np.random.default_rng(91 + (dtype == "bf16"))
    B, K, V = 6, 1, 1_000_000
    x, draft, dl, T, u = _inputs(rng, B, K, V, greedy_share=0.0)
    top_k = np.array([0, 40, 0, 2000, 0, 7], np.int32)
    top_p = np.array([0.9, 1.0, 0.5, 0.95, 0.99, 0.8], np.float32)
    t = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    xh = to_host_logits(t)
    g = _run(t, draft, dl, T, u, top_k, top_p)
    r = oracle.verify(xh, draft, dl, T, u, nthreads=8, top_k=top_k, top_p=top_p)
    tally = Tally()
    near = _compare(g, r, T, u, f"many chunks {dtype}", tally)
    assert near <= 1
    tally.check()


def test_boundary_tokens():
    """K = 1 drafts at the k-th and (k+1)-th largest logits and at the tokens
    around the top-p cut: p_draft (p'(x), 0 when x is dropped) follows the
    oracle token by token."""
    say("[gpu] truncation: boundary tokens")
    rng = np.random.default_rng(77)
    B, V = 64, 30011
    x = (rng.standard_normal((B, 2, V)) * 2).astype(np.float32)
    T = rng.uniform(0.5, 1.5, B).astype(np.float32)
    top_k = np.where(np.arange(B) % 2 == 0, rng.integers(2, 500, B), 0).astype(np.int32)
    top_p = np.where(np.arange(B) % 4 >= 2, rng.uniform(0.3, 0.95, B), 1.0).astype(np.float32)
    order = np.argsort(-x[:, 0], axis=1, kind="stable")
    draft = np.empty((B, 1), np.int32)
    for b in range(B):
        k = top_k[b] if top_k[b] > 0 else int(rng.integers(2, 3000))
        draft[b, 0] = order[b, k - 1 + (b // 2) % 2]  # k-th or (k+1)-th largest
    u = np.full((B, 2), 0.5, np.float32)
    dl = np.ones(B, np.int32)
    g = _run(torch.from_numpy(x).cuda(), draft, dl, T, u, top_k, top_p)
    r = oracle.verify(x, draft, dl, T, u, nthreads=8, top_k=top_k, top_p=top_p)
    tally = Tally()
    _compare(g, r, T, u, "boundary", tally)
    zero = (r.p_draft[:, 0] == 0).sum()
    assert 8 <= zero <= B - 8, zero  # both kept and dropped drafts were judged
    say(f"    dropped drafts {zero}")
    tally.check()


@pytest.mark.parametrize("mode", ["onehot", "bonus"])
def test_chi_square_follows_truncated_target(mode):
    """Lossless with respect to the truncated target, on the device: V = 8,
    top_k = 6, top_p = 0.85, 400k sequences in one call."""
    say(f"[gpu] truncation chi-square {mode}")
    rng = np.random.default_rng(21 if mode == "onehot" else 22)
    V, N, T, k, tp = 8, 400_000, np.float32(0.9), 6, np.float32(0.85)
    lp = (rng.standard_normal(V) * 1.2).astype(np.float32)
    # p' by sorting (distinct logits): top-k, then the smallest top set whose
    # share reaches top_p.
    p = special.softmax(lp.astype(np.float64) / float(T))
    order = np.argsort(-lp)
    pk = np.zeros(V)
    pk[order[:k]] = p[order[:k]]
    pk /= pk.sum()
    n = int(np.searchsorted(np.cumsum(pk[order]), float(tp))) + 1
    want = np.zeros(V)
    want[order[:n]] = pk[order[:n]]
    want /= want.sum()
    assert (want == 0).sum() >= 3
    R = 1 if mode == "bonus" else 2
    x = torch.from_numpy(lp).cuda().expand(N, R, V).contiguous()
    u = rng.random((N, R)).astype(np.float32)
    if mode == "bonus":
        draft = np.zeros((N, 1), np.int32)
        dl = np.zeros(N, np.int32)
        x = torch.cat([x, x], dim=1)
        u = np.concatenate([np.zeros((N, 1), np.float32), u], axis=1)
    else:
        draft = rng.integers(0, V, (N, 1)).astype(np.int32)
        dl = np.ones(N, np.int32)
    g = _run(x, draft, dl, np.full(N, T, np.float32), u,
             np.full(N, k, np.int32), np.full(N, tp, np.float32))
    assert (g[3] == 0).all()
    counts = np.bincount(g[0][:, 0], minlength=V)
    assert counts[want == 0].sum() == 0
    m = want > 0
    pv = stats.chisquare(counts[m], want[m] * N).pvalue
    say(f"    p-value {pv:.3g}")
    assert pv > 1e-3, (counts, want * N)


@pytest.mark.parametrize("case", ["crowded_top_p", "crowded_top_k", "beyond_window"])
def test_rows_beyond_the_candidate_list(case):
    """Rows whose threshold bin range holds more than 8,192 tokens (logits
    crowded into one or two bins: no band fits a segment, every chunk is
    re-read, and the candidates are walked again in each selection round),
    or lies past the 32-octave window (low T, large k)."""
    say(f"[gpu] truncation: {case}")
    rng = np.random.default_rng({"crowded_top_p": 61, "crowded_top_k": 62,
                                 "beyond_window": 63}[case])
    B, K, V = 12, 2, 20000
    if case == "beyond_window":
        x = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
        T = np.full(B, 0.05, np.float32)
        top_k = np.full(B, 5000, np.int32)
        top_p = None
    else:
        # 9,000 tokens within 0.02 of each other (one or two bins), the rest
        # far below: each crowded token carries ~1/9000 of the mass, so a
        # top-p decision rarely lands within 1e-5 of flipping.
        x = np.full((B, K + 1, V), -30.0, np.float32)
        x[:, :, :9000] = rng.uniform(0.0, 0.02, (B, K + 1, 9000))
        x = np.ascontiguousarray(np.take_along_axis(
            x, rng.permuted(np.tile(np.arange(V), (B, K + 1, 1)), axis=2), axis=2))
        T = np.full(B, 1.0, np.float32)
        if case == "crowded_top_p":
            top_k, top_p = None, np.full(B, 0.5, np.float32)
        else:
            top_k, top_p = np.full(B, 4500, np.int32), None
    draft = rng.integers(0, V, (B, K)).astype(np.int32)
    dl = np.full(B, K, np.int32)
    u = rng.random((B, K + 1)).astype(np.float32)
    g = _run(torch.from_numpy(x).cuda(), draft, dl, T, u, top_k, top_p)
    r = oracle.verify(x, draft, dl, T, u, nthreads=8, top_k=top_k, top_p=top_p)
    tally = Tally()
    near = _compare(g, r, T, u, case, tally)
    assert near <= B // 3
    tally.check()


@pytest.mark.parametrize("case,n_tied", [("spread", 1024), ("one_wavefront", 1024),
                                         ("one_wavefront", 1025)])
def test_chunk_segment_capacity(case, n_tied):
    """A chunk's band fills its 1,024-logit segment exactly (the selection
    takes its candidates from the segment) or would overflow it by one (the
    chunk keeps no band and the selection re-reads it): n_tied tokens share
    the top-k cut's logit in the first fp32 chunk (8,192 tokens), either
    spread over it or all in the part one wavefront reads (thread (e // 4) %
    256 holds element e), ten tokens lie above the cut in the second chunk
    and the rest far below. Ties at the cut are kept, so the oracle's set is
    unique."""
    say(f"[gpu] truncation: segment capacity {case} {n_tied}")
    rng = np.random.default_rng(71 + n_tied + (case == "spread"))
    B, K, V = 8, 2, 20000
    R = K + 1
    x = np.full((B, R, V), -30.0, np.float32)
    e = np.arange(8192)
    pool = e if case == "spread" else e[((e // 4) % 256) // 64 == 2]
    tied = np.zeros((B, R, n_tied), np.int64)
    for b in range(B):
        for j in range(R):
            tied[b, j] = rng.choice(pool, n_tied, replace=False)
            x[b, j, tied[b, j]] = 1.0
            x[b, j, 8192 + rng.choice(8192, 10, replace=False)] = 5.0
    # drafts: a token raised to 10 above the cut (p ~ 0.9, mostly
    # accepted) or a token far below it (dropped, so rejected)
    draft = rng.integers(16384, V, (B, K)).astype(np.int32)
    for b in range(B):
        for j in range(K):
            if rng.random() < 0.6:
                draft[b, j] = 8192 + int(rng.integers(8192))
                x[b, j, draft[b, j]] = 10.0
    dl = np.full(B, K, np.int32)
    T = np.full(B, 1.0, np.float32)
    u = rng.random((B, R)).astype(np.float32)
    top_k = np.full(B, 100, np.int32)
    g = _run(torch.from_numpy(x).cuda(), draft, dl, T, u, top_k, None)
    r = oracle.verify(x, draft, dl, T, u, nthreads=8, top_k=top_k)
    tally = Tally()
    assert _compare(g, r, T, u, f"segment {case} {n_tied}", tally) == 0
    tally.check()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_band_missing_the_row_range(dtype):
    """Chunks whose own top_p point lies far from the row's threshold: the
    first chunk holds N(0, 1.5^2) logits, the second 4,000 tokens in [3, 3.5]
    that carry most of the row's probability (the rest far below), so the
    row's top-p threshold (top_p = 0.9) falls near the first chunk's median
    of probability, some 20 bins above the band that chunk chose around its
    own 0.9 point, and below every token of the second chunk's band. The
    selection re-reads both chunks."""
    say(f"[gpu] truncation: band missing the range {dtype}")
    rng = np.random.default_rng(81 + (dtype == "bf16"))
    B, K = 8, 2
    R, V = K + 1, 3 * 16384
    x = np.full((B, R, V), -30.0, np.float32)
    c0 = 16384 if dtype == "bf16" else 8192  # tokens per chunk
    x[:, :, :c0] = rng.standard_normal((B, R, c0)) * 1.5
    for b in range(B):
        for j in range(R):
            x[b, j, c0 + rng.choice(c0, 4000, replace=False)] = rng.uniform(3.0, 3.5, 4000)
    draft = rng.integers(0, V, (B, K)).astype(np.int32)
    for b in range(B):
        for j in range(K):
            if rng.random() < 0.6:
                draft[b, j] = int(np.argmax(x[b, j]))
    dl = rng.integers(0, K + 1, B).astype(np.int32)
    T = np.full(B, 1.0, np.float32)
    u = rng.random((B, R)).astype(np.float32)
    top_p = np.full(B, 0.9, np.float32)
    t = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    xh = to_host_logits(t)
    g = _run(t, draft, dl, T, u, None, top_p)
    r = oracle.verify(xh, draft, dl, T, u, nthreads=8, top_p=top_p)
    tally = Tally()
    _compare(g, r, T, u, f"band miss {dtype}", tally)
    tally.check()


@pytest.mark.parametrize("octaves", [9.5, 10.5, 11.5, 13.0])
def test_weight_above_band_near_and_deep(octaves):
    """The weight above a top-p band is taken from the histogram's
    fixed-point masses when the band starts within 12 octaves (96 bins) of
    its chunk's max, and summed from the tokens' weights when it starts
    deeper. Rows built to put the bands at a chosen depth: per 8,192-token
    chunk one token at the top, 20 tokens spread over the octaves between,
    and the rest spread over the 6 octaves from `octaves` below the top
    down; top_p is about the row's share above `octaves` + 1, so each chunk's band
    (it fits its segment) starts about 8 * octaves bins down: bins 79-83,
    87-91, 95-101 (both ways within one row) and 105-114 for the four cases
    (found by replaying the chunks' band choice on the CPU). Everything
    above the band is kept, so p_draft and the draws depend on its weight,
    at the usual bar."""
    say(f"[gpu] truncation: weight above a band {octaves} octaves down")
    rng = np.random.default_rng(int(octaves * 10))
    B, K, C = 4, 2, 8192
    R, V = K + 1, 16 * C
    ln2 = float(np.log(2.0))
    x = np.empty((B, R, V), np.float32)
    draft = np.zeros((B, K), np.int32)
    for b in range(B):
        for j in range(R):
            row = -(octaves + rng.uniform(0.0, 6.0, V)) * ln2
            mids = []
            for c in range(V // C):
                row[c * C + rng.integers(C)] = rng.uniform(-0.1, 0.0)
                mid = c * C + rng.choice(C, 20, replace=False)
                row[mid] = -rng.uniform(1.0, octaves - 1.0, 20) * ln2
                mids.extend(mid.tolist())
            x[b, j] = row
            if j < K:
                draft[b, j] = int(np.argmax(row)) if rng.random() < 0.5 else int(rng.choice(mids))
    x64 = x[:, 0].astype(np.float64)
    w = np.exp(x64 - x64.max(-1, keepdims=True))
    # (0.1 % past that share, so that no row's decision sits on a tie)
    top_p = (1.001 * (w * (w > 2.0 ** -(octaves + 1))).sum(-1) / w.sum(-1)).astype(np.float32)
    dl = np.full(B, K, np.int32)
    T = np.ones(B, np.float32)
    u = rng.random((B, R)).astype(np.float32)
    t = torch.from_numpy(x).cuda()
    g = _run(t, draft, dl, T, u, None, top_p)
    r = oracle.verify(to_host_logits(t), draft, dl, T, u, nthreads=8, top_p=top_p)
    tally = Tally()
    _compare(g, r, T, u, f"above band {octaves}", tally)
    tally.check()
    assert (np.asarray(g[2]) >= 0).any()  # some draft probability was compared


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_truncation_with_given_q(dtype):
    say(f"[gpu] truncation with given q {dtype}")
    rng = np.random.default_rng(55 + (dtype == "bf16"))
    B, K, V = 5, 3, 30011
    x = (rng.standard_normal((B, K + 1, V)) * 1.4).astype(np.float32)
    T = rng.uniform(0.5, 1.2, B).astype(np.float32)
    ql = x[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32) * 0.9
    q = special.softmax(ql.astype(np.float64) / T[:, None, None], axis=-1)
    draft = np.array([[rng.choice(V, p=q[b, j]) for j in range(K)]
                      for b in range(B)], np.int32)
    dl = np.full(B, K, np.int32)
    u = rng.random((B, K + 1)).astype(np.float32)
    top_k = np.array([0, 50, 0, 400, 2000], np.int32)
    top_p = np.array([0.9, 1.0, 0.6, 0.95, 1.0], np.float32)
    t = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    xh = to_host_logits(t)
    q32 = q.astype(np.float32)
    g = _run(t, draft, dl, T, u, top_k, top_p, torch.from_numpy(q32).cuda())
    r = oracle.verify(xh, draft, dl, T, u, q32, nthreads=8, top_k=top_k, top_p=top_p)
    tally = Tally()
    _compare(g, r, T, u, f"given-q {dtype}", tally)
    tally.check()


def test_fused_step_and_two_calls_equal_verify():
    say("[gpu] truncation: spec_step and spec_stream + spec_finish")
    rng = np.random.default_rng(31)
    B, K, V = 16, 3, 151936
    x, draft, dl, T, u = _inputs(rng, B, K, V)
    top_k, top_p = _params(rng, B, V)
    t = torch.from_numpy(x).cuda()
    ref = _run(t, draft, dl, T, u, top_k, top_p)
    hist = rng.integers(0, V, (B, 40)).astype(np.int32)
    tk, tp = dev(top_k), dev(top_p)
    for two in (False, True):
        st = ssl.SamState(B, 100, V, "cuda")
        st.extend(dev(hist), dev(np.full(B, 40, np.int32)))
        args = (t, dev(draft), dev(dl), dev(T), dev(u))
        if two:
            ws = ssl.verify_workspace(B, K, V, truncation=True)
            ssl.spec_stream(*args, ws, top_k=tk, top_p=tp)
            got = ssl.spec_finish(*args, ws, state=st, top_k=tk, top_p=tp)[:4]
        else:
            got = ssl.spec_step(*args, st, top_k=tk, top_p=tp)[:4]
        torch.cuda.synchronize()
        for a_, b_ in zip(got, ref):
            np.testing.assert_array_equal(a_.cpu().numpy(), b_)


def test_no_op_truncation_is_bit_identical():
    say("[gpu] truncation: k >= V, k <= 0 and top_p = 1 change nothing")
    rng = np.random.default_rng(41)
    B, K, V = 12, 3, 8193
    x, draft, dl, T, u = _inputs(rng, B, K, V)
    t = torch.from_numpy(x).cuda()
    ref = _run(t, draft, dl, T, u, None, None)
    top_k = np.array([0, -1, V, V + 7] * 3, np.int32)
    got = _run(t, draft, dl, T, u, top_k, np.ones(B, np.float32))
    for a_, b_ in zip(got, ref):
        np.testing.assert_array_equal(a_, b_)


def test_top_p_status_and_workspace_errors():
    say("[gpu] truncation: invalid top_p, small workspace")
    B, K, V = 4, 2, 100
    x = torch.zeros((B, K + 1, V), device="cuda")
    d = dev(np.zeros((B, K), np.int32))
    dl = dev(np.zeros(B, np.int32))
    T = dev(np.full(B, 0.8, np.float32))
    u = dev(np.zeros((B, K + 1), np.float32))
    tp = dev(np.array([0.0, 1.5, np.nan, 0.5], np.float32))
    _, _, _, st = ssl.spec_verify(x, d, dl, T, u, top_p=tp)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [ssl.ST_TOP_P] * 3 + [0]
    small = ssl.verify_workspace(B, K, V)
    with pytest.raises(ssl.SpecSamError, match="SS_WS_TRUNCATION"):
        ssl.spec_verify(x, d, dl, T, u, top_p=tp, workspace=small)
