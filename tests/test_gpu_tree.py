"""Draft-tree verification ([P3] gogongxt notes "SGLang 的实现", the
target-only tree walk with both thresholds at 1) on the GPU through the C
ABI, against the oracle.

Bars: greedy trees bit-exact (tokens, nodes, counts); T > 0 equal except
where, at the depth where the device's and the oracle's paths part, the
coin lies within TIE of one of the oracle's running sums, or (both ending
with the final draw from the same node) the final coin within TIE of a CDF
breakpoint; such cases are counted and bounded (``_parity.Tally``); status
words equal."""
import numpy as np
import pytest
import torch
from scipy import special, stats

import oracle
import sam_drafting_lossless_amd as ssl
from _parity import compare_tree, dev, say, to_host_logits

pytestmark = pytest.mark.gpu


def _trees(rng, B, N, V, x):
    """Random trees with distinct sibling tokens; children are often the
    parent row's top tokens, and their logits are raised in the parent's row
    so that acceptances happen."""
    tok = np.zeros((B, N), np.int32)
    par = np.full((B, N), -1, np.int32)
    for b in range(B):
        for i in range(1, N):
            p = int(rng.integers(max(0, i - 4), i)) if rng.random() < 0.7 else int(rng.integers(0, i))
            used = {int(tok[b, c]) for c in range(1, i) if par[b, c] == p}
            top = np.argsort(-x[b, p])[:4]
            t = int(top[rng.integers(0, 4)]) if rng.random() < 0.6 else int(rng.integers(0, V))
            while t in used:
                t = (t + 1) % V
            par[b, i], tok[b, i] = p, t
            x[b, p, t] += rng.uniform(0, 3)
    return tok, par


def _run(t, tok, par, n, T, u):
    g = ssl.spec_verify_tree(t, dev(tok), dev(par), dev(n), dev(T, torch.float32),
                             None if u is None else dev(u, torch.float32))
    torch.cuda.synchronize()
    return tuple(a.cpu().numpy() for a in g)


@pytest.mark.parametrize("B,N,V", [(16, 8, 32), (12, 16, 8193), (8, 32, 30011),
                                   (6, 64, 151936), (5, 1, 100), (9, 5, 3 * 8192 + 4)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tree_matches_oracle(B, N, V, dtype):
    say(f"[gpu] tree {dtype} B={B} N={N} V={V}")
    rng = np.random.default_rng(B * 7 + N * 131 + V + (dtype == "bf16"))
    x = (rng.standard_normal((B, N, V)) * 1.5).astype(np.float32)
    tok, par = _trees(rng, B, N, V, x)
    n = rng.integers(1, N + 1, B).astype(np.int32)
    T = rng.uniform(0.4, 1.5, B).astype(np.float32)
    T[rng.random(B) < 0.3] = 0.0
    u = rng.random((B, N)).astype(np.float32)
    t = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    xh = to_host_logits(t)
    g = _run(t, tok, par, n, T, u)
    r = oracle.verify_tree(xh, tok, par, n, T, u, nthreads=8)
    compare_tree(g, r, T, u, what=f"tree {dtype}")
    assert (g[2] > 1).any() or N == 1  # some drafts were accepted
    say(f"    emitted={int(g[2][r.status == 0].sum())}")


def test_chain_tree_equals_linear_verification():
    """A chain is the linear case: the tree entry point and spec_verify agree
    on the same rows, drafts and coins."""
    say("[gpu] tree: chains against spec_verify")
    rng = np.random.default_rng(5)
    B, N, V = 64, 5, 8193
    x = (rng.standard_normal((B, N, V)) * 1.5).astype(np.float32)
    tok = np.zeros((B, N), np.int32)
    for b in range(B):
        for i in range(1, N):
            tok[b, i] = x[b, i - 1].argmax() if rng.random() < 0.6 else rng.integers(0, V)
            x[b, i - 1, tok[b, i]] += rng.uniform(0, 3)
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    n = rng.integers(1, N + 1, B).astype(np.int32)
    T = np.where(rng.random(B) < 0.4, 0.0, 0.9).astype(np.float32)
    u = rng.random((B, N)).astype(np.float32)
    t = torch.from_numpy(x).cuda()
    g = _run(t, tok, par, n, T, u)
    lin = ssl.spec_verify(t, dev(tok[:, 1:]), dev(n - 1), dev(T), dev(u))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(g[0], lin[0].cpu().numpy())
    np.testing.assert_array_equal(g[2], lin[1].cpu().numpy())


def test_chi_square_on_device():
    """The first emitted token follows p_root; after node 1 is accepted the
    second follows p_1; after the leaf node 2, p_2 (V = 8, 400k sequences)."""
    say("[gpu] tree chi-square")
    rng = np.random.default_rng(6)
    V, N, M = 8, 6, 400_000
    rows = (rng.standard_normal((N, V)) * 1.2).astype(np.float32)
    tok = np.array([0, 3, 5, 1, 2, 3], np.int32)
    par = np.array([-1, 0, 0, 0, 1, 1], np.int32)
    T = np.float32(0.9)
    x = torch.from_numpy(rows).cuda().expand(M, N, V).contiguous()
    u = rng.random((M, N)).astype(np.float32)
    out, nodes, nem, st = _run(x, np.tile(tok, (M, 1)), np.tile(par, (M, 1)),
                               np.full(M, N, np.int32), np.full(M, T, np.float32), u)
    assert (st == 0).all()
    p = special.softmax(rows.astype(np.float64) / float(T), axis=1)
    pv = [stats.chisquare(np.bincount(out[:, 0], minlength=V), p[0] * M).pvalue]
    for node in (1, 2):
        sel = nodes[:, 0] == node
        pv.append(stats.chisquare(np.bincount(out[sel, 1], minlength=V),
                                  p[node] * sel.sum()).pvalue)
    say(f"    p-values {pv}")
    assert min(pv) > 1e-3


def test_tree_status_and_errors():
    say("[gpu] tree: status words and host errors")
    V, N = 10, 4
    x = np.zeros((7, N, V), np.float32)
    tok = np.array([[0, 1, 2, 3]] * 7, np.int32)
    par = np.array([[-1, 0, 0, 1]] * 7, np.int32)
    n = np.full(7, N, np.int32)
    tok[0, 2] = 1          # duplicate sibling token
    par[1, 2] = 2          # parent not before the node
    tok[2, 3] = V          # token out of range
    n[3] = 0               # no root
    par[4, 0] = 0          # root with a parent
    x[5, 1, 3] = np.nan    # a row with NaN
    n[6] = N + 1           # more nodes than rows
    T = np.zeros(7, np.float32)
    g = _run(torch.from_numpy(x).cuda(), tok, par, n, T, None)
    r = oracle.verify_tree(x, tok, par, np.minimum(n, N + 1), T)
    want = [ssl.ST_TREE] * 5 + [ssl.ST_NONFINITE, ssl.ST_TREE]
    assert g[3].tolist() == want
    assert r.status.tolist() == want
    with pytest.raises(ssl.SpecSamError, match="N=65"):
        ssl.spec_verify_tree(torch.zeros((1, 65, 8), device="cuda"),
                             *(dev(np.zeros((1, 65), np.int32)) for _ in range(2)),
                             dev(np.ones(1, np.int32)), dev(np.zeros(1, np.float32)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_top_coin_leaves_the_children_out(dtype):
    """Every coin 1 (the top of its range): no child's running sum reaches it
    (their probabilities sum below 1), so the final token is drawn at the
    root with the children left out, and the top coin takes the last token of
    positive weight among the rest. Rows: random logits in [-3, 0] up to a
    per-row cut, -inf after it, one token before the cut at 3 (the row max);
    three children past the cut at logit 2.5, two of them in one quarter of
    one chunk and the third alone in a later chunk, so that nothing else
    weighs anything in their quarters. Taken out of the quarter sums, they
    must leave those quarters empty: a rounding residue would send the top
    coin past every token the draw can take. The draw must give the token
    just before the cut, as the oracle does."""
    say(f"[gpu] tree: top coin {dtype}")
    per_chunk = 8192 if dtype == "f32" else 16384
    q = per_chunk // 4
    V = 5 * per_chunk + 256
    rng = np.random.default_rng(91 + (dtype == "bf16"))
    B, N = 12, 4
    x = np.full((B, N, V), -np.inf, np.float32)
    tok = np.zeros((B, N), np.int32)
    par = np.array([[-1, 0, 0, 0]] * B, np.int32)
    want = np.zeros(B, np.int64)
    for b in range(B):
        cut = int(rng.integers(per_chunk // 2, 2 * per_chunk))
        x[b, :, :cut] = rng.uniform(-3.0, 0.0, (N, cut)).astype(np.float32)
        x[b, :, int(rng.integers(0, cut - 1))] = 3.0
        c0 = cut // per_chunk + 1
        qq = int(rng.integers(0, 4))
        t1 = c0 * per_chunk + qq * q + int(rng.integers(0, q // 2))
        t2 = t1 + 1 + int(rng.integers(0, q // 2 - 1))
        t3 = (c0 + 2) * per_chunk + int(rng.integers(0, per_chunk))
        tok[b, 1:] = [t1, t2, t3]
        x[b, 0, [t1, t2, t3]] = 2.5
        want[b] = cut - 1
    n = np.full(B, N, np.int32)
    T = np.ones(B, np.float32)
    u = np.ones((B, N), np.float32)
    t = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    g = _run(t, tok, par, n, T, u)
    r = oracle.verify_tree(to_host_logits(t), tok, par, n, T, u, nthreads=8)
    np.testing.assert_array_equal(r.out_tokens[:, 0], want)
    np.testing.assert_array_equal(g[0], r.out_tokens)
    np.testing.assert_array_equal(g[1], r.out_nodes)
    np.testing.assert_array_equal(g[2], r.num_emitted)
