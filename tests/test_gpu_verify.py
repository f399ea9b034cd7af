"""GPU parity of spec_verify against the oracle (through the C ABI)."""
import math

import numpy as np
import pytest
import torch
from scipy import special, stats

import oracle
import sam_drafting_lossless_amd as ssl
import synth
from _parity import Tally, compare_verify, dev, say, to_host_logits

pytestmark = pytest.mark.gpu


def _run(logits, draft, dl, T, u=None, q=None, status0=None):
    """Runs GPU and oracle on identical inputs; returns (gpu tuple, oracle)."""
    B = logits.shape[0]
    st = dev(np.zeros(B, np.int32) if status0 is None else status0)
    g = ssl.spec_verify(logits, dev(draft, torch.int32), dev(dl, torch.int32),
                        dev(T, torch.float32),
                        None if u is None else dev(u, torch.float32),
                        q, status=st)
    torch.cuda.synchronize()
    g = tuple(t.cpu().numpy() for t in g)
    r = oracle.verify(to_host_logits(logits), draft, dl, T, u,
                      None if q is None else q.cpu().numpy(), nthreads=8)
    return g, r


def _drafts_near_argmax(rng, logits_np, K, dl, flip=0.4):
    am = logits_np[:, :K].argmax(-1).astype(np.int32)
    B, V = logits_np.shape[0], logits_np.shape[2]
    bad = rng.random((B, K)) < flip
    am[bad] = rng.integers(0, V, int(bad.sum()))
    return am


SHAPES = [  # (B, K, V): tiny, one chunk, ragged chunks, scalar path, Qwen
    (1, 3, 32), (3, 1, 1), (5, 4, 7), (7, 2, 8192), (6, 3, 8193),
    (4, 5, 3 * 8192 + 4), (3, 16, 4099), (2, 3, 151936), (33, 2, 1000),
]


@pytest.mark.parametrize("B,K,V", SHAPES)
def test_greedy_bit_exact(B, K, V):
    say(f"[gpu] greedy B={B} K={K} V={V}")
    rng = np.random.default_rng(B * 1000 + V)
    x = rng.integers(-4, 5, (B, K + 1, V)).astype(np.float32)  # many ties
    dl = rng.integers(0, K + 1, B).astype(np.int32)
    draft = _drafts_near_argmax(rng, x, K, dl)
    g, r = _run(torch.from_numpy(x).cuda(), draft, dl, np.zeros(B, np.float32))
    compare_verify(*g, r, np.zeros(B), None, what="greedy")


@pytest.mark.parametrize("B,K,V", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sampling_one_hot(B, K, V, dtype):
    say(f"[gpu] one-hot sampling {dtype} B={B} K={K} V={V}")
    rng = np.random.default_rng(B * 77 + V + (dtype == "bf16"))
    x = (rng.standard_normal((B, K + 1, V)) * 1.5).astype(np.float32)
    dl = rng.integers(0, K + 1, B).astype(np.int32)
    draft = _drafts_near_argmax(rng, x, K, dl, flip=0.3)
    # make drafts plausible so both accepts and rejects happen
    for b in range(B):
        for j in range(K):
            x[b, j, draft[b, j]] += rng.uniform(0, 6)
    T = rng.uniform(0.4, 1.6, B).astype(np.float32)
    u = rng.random((B, K + 1)).astype(np.float32)
    t = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    g, r = _run(t, draft, dl, T, u)
    tally = Tally()
    compare_verify(*g, r, T, u, tally, what=f"one-hot {dtype}")
    tally.check()


@pytest.mark.parametrize("B,K,V", [(4, 3, 32), (5, 2, 8193), (3, 5, 30011),
                                   (2, 4, 151936)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sampling_given_q(B, K, V, dtype):
    say(f"[gpu] given-q sampling {dtype} B={B} K={K} V={V}")
    rng = np.random.default_rng(V + B + (dtype == "bf16"))
    x = (rng.standard_normal((B, K + 1, V)) * 1.4).astype(np.float32)
    T = rng.uniform(0.5, 1.2, B).astype(np.float32)
    ql = x[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32) * 0.7
    q = special.softmax(ql.astype(np.float64) / T[:, None, None], axis=-1)
    draft = np.array([[rng.choice(V, p=q[b, j]) for j in range(K)]
                      for b in range(B)], np.int32)
    dl = rng.integers(0, K + 1, B).astype(np.int32)
    u = rng.random((B, K + 1)).astype(np.float32)
    t = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    g, r = _run(t, draft, dl, T, u, q=torch.from_numpy(q.astype(np.float32)).cuda())
    tally = Tally()
    compare_verify(*g, r, T, u, tally, what=f"given-q {dtype}")
    tally.check()


def test_mixed_greedy_and_sampling_batch_with_masked_tokens():
    say("[gpu] mixed T, -inf entries")
    rng = np.random.default_rng(9)
    B, K, V = 24, 4, 20000
    x = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    x[:, :, rng.choice(V, 5000, replace=False)] = -np.inf
    T = np.where(rng.random(B) < 0.5, 0.0, 0.9).astype(np.float32)
    dl = rng.integers(0, K + 1, B).astype(np.int32)
    draft = _drafts_near_argmax(rng, np.nan_to_num(x, neginf=-1e9), K, dl)
    u = rng.random((B, K + 1)).astype(np.float32)
    g, r = _run(torch.from_numpy(x).cuda(), draft, dl, T, u)
    compare_verify(*g, r, T, u, None, what="mixed")


def test_status_words_match_oracle():
    say("[gpu] status words")
    V, K = 16, 2
    x = np.zeros((7, K + 1, V), np.float32)
    draft = np.zeros((7, K), np.int32)
    dl = np.full(7, K, np.int32)
    T = np.zeros(7, np.float32)
    dl[0] = K + 1
    draft[1, 1] = V
    x[2, 1, 5] = np.nan
    T[3] = -1.0
    x[4, 0, :] = -np.inf
    x[5, 2, 3] = np.inf
    g, r = _run(torch.from_numpy(x).cuda(), draft, dl, T)
    compare_verify(*g, r, T, None, what="status")
    assert g[3][6] == 0 and g[1][6] == K + 1
    # temperatures: denormal, smallest normal, inf, NaN
    Tt = np.array([1e-40, np.finfo(np.float32).tiny, np.inf, np.nan], np.float32)
    g, r = _run(torch.zeros((4, K + 1, V), device="cuda"),
                np.zeros((4, K), np.int32), np.zeros(4, np.int32), Tt,
                np.zeros((4, K + 1), np.float32))
    assert g[3].tolist() == r.status.tolist() == [
        ssl.ST_TEMPERATURE, 0, ssl.ST_TEMPERATURE, ssl.ST_TEMPERATURE]
    # T > 0 without uniforms
    g, r = _run(torch.from_numpy(x[6:]).cuda(), draft[6:], dl[6:],
                np.ones(1, np.float32), None)
    assert g[3].tolist() == [ssl.ST_NO_UNIFORMS] == r.status.tolist()


def test_sticky_status_is_ored_and_untouched_outputs():
    say("[gpu] sticky status")
    x = torch.zeros((2, 2, 8), device="cuda")
    st0 = np.array([ssl.ST_SAM_CAPACITY, 0], np.int32)
    out = torch.full((2, 2), 77, dtype=torch.int32, device="cuda")
    g = ssl.spec_verify(x, dev(np.array([[0], [0]]), torch.int32),
                        dev(np.array([5, 1]), torch.int32),
                        dev(np.zeros(2), torch.float32), status=dev(st0),
                        out_tokens=out)
    torch.cuda.synchronize()
    assert g[3].cpu().tolist() == [ssl.ST_SAM_CAPACITY | ssl.ST_DRAFT_LEN, 0]
    assert g[0][0].cpu().tolist() == [77, 77]
    assert g[0][1].cpu().tolist() == [0, 0]


def test_host_argument_errors():
    x = torch.zeros((2, 4, 8), device="cuda")
    i = torch.zeros((2, 3), dtype=torch.int32, device="cuda")
    d = torch.zeros(2, dtype=torch.int32, device="cuda")
    T = torch.zeros(2, device="cuda")
    with pytest.raises(ssl.SpecSamError):
        ssl.spec_verify(x.double(), i, d, T)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ssl.SpecSamError, match="workspace"):
        ssl.spec_verify(x, i, d, T, workspace=ws)
    with pytest.raises(ssl.SpecSamError, match="workspace"):
        ssl.spec_stream(x, i, d, T, None, ws)
    st = ssl.SamState(2, 16, 8, "cuda")
    q = torch.full((2, 3, 8), 0.125, device="cuda")
    w = ssl.verify_workspace(2, 3, 8)
    with pytest.raises(ssl.SpecSamError, match="one-hot"):
        ssl.spec_finish(x, i, d, T, None, w, q, st)


@pytest.mark.parametrize("mode", ["onehot", "given_q"])
def test_gpu_chi_square_first_token(mode):
    """Losslessness on the GPU: 10^6 sequences in one launch, V = 8."""
    say(f"[gpu] chi-square {mode}")
    rng = np.random.default_rng(21 if mode == "onehot" else 22)
    V, N = 8, 1_000_000
    lp = rng.standard_normal(V) * 1.2
    p = special.softmax(lp)
    x = torch.from_numpy(lp.astype(np.float32)).cuda().expand(N, 2, V).contiguous()
    u = rng.random((N, 2)).astype(np.float32)
    if mode == "onehot":
        draft = rng.integers(0, V, (N, 1)).astype(np.int32)
        q = None
    else:
        qv = special.softmax(rng.standard_normal(V) * 1.5)
        draft = rng.choice(V, size=(N, 1), p=qv).astype(np.int32)
        q = torch.from_numpy(qv.astype(np.float32)).cuda().expand(N, 1, V).contiguous()
    out, nem, _, st = ssl.spec_verify(x, dev(draft), dev(np.ones(N, np.int32)),
                                      dev(np.ones(N, np.float32)), dev(u), q)
    first = out[:, 0].cpu().numpy()
    assert (st.cpu().numpy() == 0).all()
    counts = np.bincount(first, minlength=V)
    pv = stats.chisquare(counts, p * N).pvalue
    assert pv > 1e-3, (counts, p * N, pv)


@pytest.mark.parametrize("alpha", [0.2, 0.5, 0.8])
def test_gpu_mean_tokens_closed_form(alpha):
    K, N = 3, 500_000
    lg = np.log(np.array([alpha, 1 - alpha])).astype(np.float32)
    x = torch.from_numpy(lg).cuda().expand(N, K + 1, 2).contiguous()
    u = np.random.default_rng(5).random((N, K + 1)).astype(np.float32)
    _, nem, _, _ = ssl.spec_verify(x, dev(np.zeros((N, K), np.int32)),
                                   dev(np.full(N, K, np.int32)),
                                   dev(np.ones(N, np.float32)), dev(u))
    m = nem.double().mean().item()
    want = (1 - alpha ** (K + 1)) / (1 - alpha)
    sd = nem.double().std().item()
    assert abs(m - want) < 5 * sd / math.sqrt(N)


# ----------------------------------------------------- full-size workloads ---
def _full_step(cfg, step=0):
    gt = synth.token_streams(cfg, steps=2)
    n = np.full(cfg.B, cfg.hist_len, np.int32)
    x = synth.target_logits(cfg, step, gt, n, device="cuda")
    return gt, n, x


@pytest.mark.parametrize("c", [2, 3, 4])
def test_full_size_sam_draft_shapes(c):
    """One verify at the workload's full size, drafts taken from gt so that a
    realistic share is accepted; every output compared."""
    cfg = synth.config(c)
    say(f"[gpu] full-size verify {cfg.name}")
    rng = np.random.default_rng(c)
    gt, n, x = _full_step(cfg)
    draft = np.stack([gt[b, n[b]:n[b] + cfg.K] for b in range(cfg.B)]).astype(np.int32)
    wrong = rng.random(draft.shape) < 0.3
    draft[wrong] = rng.integers(0, cfg.V, int(wrong.sum()))
    dl = rng.integers(0, cfg.K + 1, cfg.B).astype(np.int32)
    T = np.full(cfg.B, cfg.T, np.float32)
    u = synth.uniforms(cfg, 0)
    g, r = _run(x, draft, dl, T, u)
    tally = Tally()
    compare_verify(*g, r, T, u, tally, what=cfg.name)
    tally.check()


def test_full_size_draft_model_q():
    cfg = synth.config(5)
    say(f"[gpu] full-size verify {cfg.name}")
    x = synth.noise(cfg, 0, "cuda")
    q, draft = synth.draft_model_inputs(cfg, 0, x, "cuda")
    T = np.full(cfg.B, cfg.T, np.float32)
    u = synth.uniforms(cfg, 0)
    dl = np.full(cfg.B, cfg.K, np.int32)
    g, r = _run(x, draft, dl, T, u, q=q)
    tally = Tally()
    compare_verify(*g, r, T, u, tally, what=cfg.name)
    say(f"    mean tokens/step {g[1].mean():.3f}")
    tally.check()


def test_one_workspace_serves_every_shape_that_fits():
    """The workspace is scratch: one buffer, with whatever the previous call
    left in it, serves calls of any shape whose size fits."""
    say("[gpu] workspace reuse across shapes")
    ws = ssl.verify_workspace(40, 6, 40000)
    ws.fill_(0xA5)
    rng = np.random.default_rng(3)
    for (B, K, V, T) in [(40, 6, 40000, 1.0), (40, 6, 40000, 0.0),
                         (7, 2, 9000, 0.0), (33, 5, 12345, 0.8),
                         (40, 6, 40000, 0.5), (1, 1, 17, 1.3), (1, 1, 17, 0.0)]:
        x = (rng.standard_normal((B, K + 1, V)) * 1.5).astype(np.float32)
        dl = rng.integers(0, K + 1, B).astype(np.int32)
        draft = _drafts_near_argmax(rng, x, K, dl, flip=0.5)
        Ta = np.full(B, T, np.float32)
        u = rng.random((B, K + 1)).astype(np.float32)
        st = dev(np.zeros(B, np.int32))
        g = ssl.spec_verify(torch.from_numpy(x).cuda(), dev(draft), dev(dl),
                            dev(Ta), dev(u), workspace=ws, status=st)
        torch.cuda.synchronize()
        g = tuple(t.cpu().numpy() for t in g)
        r = oracle.verify(x, draft, dl, Ta, u, nthreads=8)
        compare_verify(*g, r, Ta, u, None, what=f"reuse B={B} K={K} V={V}")


@pytest.mark.parametrize("B,K", [(64, 3), (2048, 3), (2049, 6)])
@pytest.mark.parametrize("lengths", ["empty", "full", "mixed"])
def test_row_lanes_across_batch_sizes(B, K, lengths):
    """The stream grid is (sequence, row lane, chunk), lane q streaming rows
    q, q + G, ...: G = K + 1 (a workgroup per row) when B x nchunks < 4096
    (B = 64 here, V = 9000 gives two chunks), G = 2 for K <= 3 above it (B =
    2048), G = 4 for larger K (B = 2049, K = 6: lanes take rows {0, 4},
    {1, 5}, {2, 6}, {3}); all give the oracle's results for all-empty,
    all-full and mixed draft lengths (with invalid lengths mixed in, which
    are reported and need no rows)."""
    say(f"[gpu] row lanes B={B} K={K} {lengths}")
    rng = np.random.default_rng(B + K + len(lengths))
    V = 9000  # two chunks, the second ragged
    x = (rng.standard_normal((B, K + 1, V)) * 1.5).astype(np.float32)
    if lengths == "empty":
        dl = np.zeros(B, np.int32)
    elif lengths == "full":
        dl = np.full(B, K, np.int32)
    else:
        dl = rng.choice([0, 0, 0, 1, 2, K - 1, K, -1, K + 1], B).astype(np.int32)
    draft = _drafts_near_argmax(rng, x, K, np.clip(dl, 0, K), flip=0.5)
    T = np.where(rng.random(B) < 0.5, 0.0, 0.9).astype(np.float32)
    u = rng.random((B, K + 1)).astype(np.float32)
    g, r = _run(torch.from_numpy(x).cuda(), draft, dl, T, u)
    compare_verify(*g, r, T, u, None, what=f"lanes B={B} K={K} {lengths}")


# ------------------------------------------- finalize: how partials arrive ---
# The finalize kernel takes each row's chunk partials one per thread when
# (K+1) x nchunks <= 256, through an LDS loop up to 1024, and from global
# memory above that. fp32 chunks hold 8192 logits: K = 16 at V = 151936 gives
# 17 x 19 = 323 (the LDS loop), K = 16 at V = 524288 gives 17 x 64 = 1088
# (global partials).
@pytest.mark.parametrize("V", [151936, 524288])
@pytest.mark.parametrize("mode", ["greedy", "onehot", "given_q"])
def test_finalize_partial_paths_at_k16(V, mode):
    K = 16
    B = 6 if V == 151936 else 4
    say(f"[gpu] finalize partials K={K} V={V} {mode} ({(K + 1) * -(-V // 8192)} per row set)")
    rng = np.random.default_rng(V + len(mode))
    x = (rng.standard_normal((B, K + 1, V)) * 1.5).astype(np.float32)
    dl = np.array([K, K, K - 1, 7, 0, K][:B], np.int32)
    q = None
    if mode == "greedy":
        draft = _drafts_near_argmax(rng, x, K, dl, flip=0.08)
        T = np.zeros(B, np.float32)
        u = None
    else:
        T = rng.uniform(0.7, 1.2, B).astype(np.float32)
        u = rng.random((B, K + 1)).astype(np.float32)
        if mode == "onehot":
            draft = rng.integers(0, V, (B, K)).astype(np.int32)
            # strong boosts, so that acceptance runs deep into the rows
            for b in range(B):
                for j in range(K):
                    x[b, j, draft[b, j]] += rng.uniform(16, 24)
        else:
            ql = x[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32) * 0.3
            qd = special.softmax(ql.astype(np.float64) / T[:, None, None], axis=-1)
            draft = np.array([[rng.choice(V, p=qd[b, j]) for j in range(K)]
                              for b in range(B)], np.int32)
            q = torch.from_numpy(qd.astype(np.float32)).cuda()
            del qd
    g, r = _run(torch.from_numpy(x).cuda(), draft, dl, T, u, q=q)
    compare_verify(*g, r, T, u, None, what=f"K=16 V={V} {mode}")
    if mode != "given_q":
        assert g[1].max() >= 8, g[1]  # deep acceptance: many rows combined
    say(f"    emitted {g[1].tolist()}")


# --------------------------------------- draw: a target on a chunk boundary --
def test_draw_target_on_a_chunk_boundary():
    """The draw picks the chunk from the running sum of chunk weights, then
    the token inside it by the target left over. When the target falls
    between the first chunk's total and the float sum that precedes the
    second chunk (which rounding can leave above the first chunk's total),
    the token is the first positive one of the second chunk, not its last.

    Row: V = 3 x 8192 fp32 at T = 1; token 100 has logit -15.6 (weight
    2^-22.5 relative to the max, in (2^-23, 2^-22)); tokens 8202, 8212 and
    8222 have logit 0 (weight 1); all else -inf. Chunk sums W0 ~ 1.68e-7 and
    W1 = 3, so W0 + W1 rounds up to 3 + 2^-22 and the sum before chunk 1
    reads 2^-22 > W0. The final coin puts the target midway between W0 and
    2^-22: the oracle (double precision) and the inverse CDF's definition
    give token 8202. Case 2 rejects draft 8222 first, so the residual has
    chunk weights W0 and 2 (2 + W0 also rounds up). The margins are 20 % of
    the interval, far beyond rounding, so the token must match exactly."""
    say("[gpu] draw: target on a chunk boundary")
    V = 3 * 8192
    x = np.full((2, 2, V), -np.inf, np.float32)
    x[:, :, 100] = -15.6
    x[:, :, [8202, 8212, 8222]] = 0.0
    w0 = float(np.exp2(np.float32(-15.6) * np.float32(1.4426950408889634)))
    assert 2.0 ** -23 < w0 < 2.0 ** -22
    t = 0.5 * (w0 + 2.0 ** -22)
    draft = np.array([[0], [8222]], np.int32)
    dl = np.array([0, 1], np.int32)
    T = np.ones(2, np.float32)
    u = np.array([[0.5, t / 3.0], [0.999, t / 2.0]], np.float32)
    g, r = _run(torch.from_numpy(x).cuda(), draft, dl, T, u)
    assert r.out_tokens.tolist() == [[8202, -1], [8202, -1]], r.out_tokens
    np.testing.assert_array_equal(g[0], r.out_tokens)
    np.testing.assert_array_equal(g[1], [1, 1])


# ------------------------- draw: quarters of a chunk, the top coin, gaps ---
# Token positions on both sides of every quarter boundary (2048 fp32 tokens,
# 4096 bf16) and chunk boundary (8192 / 16384) of the first two chunks, and
# in a ragged last chunk.
def _boundary_tokens(V, per_chunk):
    q = per_chunk // 4
    pos = [5]
    for c in range(2):
        for i in range(1, 5):
            e = c * per_chunk + i * q
            pos += [e - 1, e]
    pos += [V - 3, V - 1]
    return sorted(p for p in set(pos) if p < V)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_draw_every_quarter_and_chunk_boundary(dtype):
    """Equal logits on tokens placed on both sides of each quarter and chunk
    boundary (all others -inf), and one coin per CDF interval, at its middle:
    the inverse CDF in token order must give exactly the k-th token for the
    k-th interval. Rows without drafts draw from the row (n tokens); rows whose
    single draft (one of the tokens) is rejected (its coin 1, p(x) = 1/n < 1)
    draw from the rest (n - 1 tokens, the draft left out). A draw that took
    quarters, chunks or their sums out of token order, or lost a boundary
    token, fails here."""
    say(f"[gpu] draw: quarter and chunk boundaries {dtype}")
    per_chunk = 8192 if dtype == "f32" else 16384
    V = 2 * per_chunk + 3 * 1024 + 8
    pos = _boundary_tokens(V, per_chunk)
    n = len(pos)
    rows = []  # (draft token or -1, coin)
    for k in range(n):
        rows.append((-1, (k + 0.5) / n))
    for xi in (0, n // 2, n - 1):
        for k in range(n - 1):
            rows.append((pos[xi], (k + 0.5) / (n - 1)))
    B, K = len(rows), 1
    x = np.full((B, K + 1, V), -np.inf, np.float32)
    x[:, :, pos] = 0.0
    draft = np.array([[max(t, 0)] for t, _ in rows], np.int32)
    dl = np.array([0 if t < 0 else 1 for t, _ in rows], np.int32)
    u = np.array([[1.0 if t >= 0 else 0.5, c] for t, c in rows], np.float32)
    T = np.ones(B, np.float32)
    t = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    g, r = _run(t, draft, dl, T, u)
    for b, (tx, c) in enumerate(rows):
        rest = [p for p in pos if p != tx]
        want = rest[int(c * len(rest))]
        assert r.out_tokens[b].tolist() == [want, -1], (b, r.out_tokens[b], want)
    np.testing.assert_array_equal(g[0], r.out_tokens)
    np.testing.assert_array_equal(g[1], r.num_emitted)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_top_coin_takes_the_last_positive_token(dtype):
    """A final coin of 1 (the top of its range) puts the draw's target at the
    total weight, which no running sum exceeds: the inverse CDF's definition
    then takes the last token of positive weight. Rows: random logits in
    [-3, 0] up to a per-row cut, -inf from there on, except (half the rows)
    the draft token x at logit 2.5, alone past the cut in its own chunk, and
    one token before the cut at logit 3 (the row max, so that x's weight is
    not the row's reference). x's coin is 1, so x is rejected (p(x) < 1) and
    the draw is from the row without x: its last positive token is the one
    just before the cut. x's quarter, and its chunk, must then weigh exactly
    nothing: a rounding residue left by taking x's weight out would send the
    top coin past every token the draw can still take. The other rows have
    no drafts: their draw is the token just before the cut."""
    say(f"[gpu] draw: top coin {dtype}")
    per_chunk = 8192 if dtype == "f32" else 16384
    V = 4 * per_chunk + 512
    rng = np.random.default_rng(77 + (dtype == "bf16"))
    B, K = 24, 1
    x = np.full((B, K + 1, V), -np.inf, np.float32)
    draft = np.zeros((B, K), np.int32)
    dl = np.zeros(B, np.int32)
    want = np.zeros(B, np.int64)
    for b in range(B):
        cut = int(rng.integers(per_chunk // 2, 3 * per_chunk))
        x[b, :, :cut] = rng.uniform(-3.0, 0.0, (K + 1, cut)).astype(np.float32)
        x[b, :, int(rng.integers(0, cut - 1))] = 3.0
        want[b] = cut - 1
        if b % 2 == 0:
            xc = (cut // per_chunk + 1) * per_chunk + int(rng.integers(0, per_chunk))
            xc = min(xc, V - 1)
            x[b, 0, xc] = 2.5
            draft[b, 0] = xc
            dl[b] = 1
    u = np.ones((B, K + 1), np.float32)
    T = np.ones(B, np.float32)
    t = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    g, r = _run(t, draft, dl, T, u)
    np.testing.assert_array_equal(r.out_tokens[:, 0], want)
    np.testing.assert_array_equal(g[0], r.out_tokens)
    np.testing.assert_array_equal(g[1], r.num_emitted)


# ------------------------------------------------------------- alignment ---
def test_misaligned_logits_or_q_are_rejected():
    """Logits and q must start on a 16-byte boundary (the stream pass reads
    them 16 bytes at a time); a contiguous view that starts elsewhere is an
    invalid argument, while a row length that is not a multiple of the
    vector width (aligned base) takes the element-wise loads."""
    say("[gpu] misaligned views")
    B, K, V = 2, 2, 64
    base = torch.zeros(B * (K + 1) * V + 4, device="cuda")
    x = base[1:1 + B * (K + 1) * V].view(B, K + 1, V)
    assert x.is_contiguous() and x.data_ptr() % 16 == 4
    d = torch.zeros((B, K), dtype=torch.int32, device="cuda")
    dl = torch.zeros(B, dtype=torch.int32, device="cuda")
    T = torch.zeros(B, device="cuda")
    with pytest.raises(ssl.SpecSamError, match="16-byte"):
        ssl.spec_verify(x, d, dl, T)
    xb = torch.zeros(B * (K + 1) * V + 8, dtype=torch.bfloat16, device="cuda")
    xb = xb[1:1 + B * (K + 1) * V].view(B, K + 1, V)
    assert xb.data_ptr() % 16 == 2
    with pytest.raises(ssl.SpecSamError, match="16-byte"):
        ssl.spec_verify(xb, d, dl, T)
    qb = torch.full((B * K * V + 4,), 1.0 / V, device="cuda")
    q = qb[2:2 + B * K * V].view(B, K, V)
    xa = torch.zeros((B, K + 1, V), device="cuda")
    with pytest.raises(ssl.SpecSamError, match="16-byte"):
        ssl.spec_verify(xa, d, dl, torch.ones(B, device="cuda"),
                        torch.full((B, K + 1), 0.5, device="cuda"), q)
    tree_x = base[1:1 + B * 3 * V].view(B, 3, V)
    with pytest.raises(ssl.SpecSamError, match="16-byte"):
        ssl.spec_verify_tree(tree_x, torch.zeros((B, 3), dtype=torch.int32, device="cuda"),
                             torch.tensor([[-1, 0, 0]] * B, dtype=torch.int32, device="cuda"),
                             torch.ones(B, dtype=torch.int32, device="cuda"), T)
    # an aligned base with V not a multiple of the vector width still works
    x7 = torch.from_numpy(np.arange(B * (K + 1) * 7, dtype=np.float32).reshape(B, K + 1, 7)).cuda()
    g, r = _run(x7, np.zeros((B, K), np.int32), np.zeros(B, np.int32), np.zeros(B, np.float32))
    compare_verify(*g, r, np.zeros(B), None, what="V=7")
