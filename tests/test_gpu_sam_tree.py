"""Draft trees from the automaton (several candidates: the draft state and
its suffix-link ancestors, merged into a trie) on the GPU through the C ABI,
bit-exact against the oracle; then drafted trees verified by
spec_verify_tree against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import sam_drafting_lossless_amd as ssl
import synth
from _parity import compare_tree, dev, say, to_host_logits

pytestmark = pytest.mark.gpu


def _streams(B, n, V, seed):
    cfg = synth.config(3, B=B, V=V, hist_len=n, steps=0, warmup=0, seed=seed)
    return synth.token_streams(cfg, 0)[:, :n]


@pytest.mark.parametrize("V", [4, 50, 151936])
def test_draft_tree_matches_oracle(V):
    say(f"[gpu] automaton draft trees V={V}")
    B, n = 24, 600
    gt = _streams(B, n, V, 7 + V)
    st = ssl.SamState(B, n + 200, V, "cuda")
    sams = [oracle.SAM(np.zeros(0, np.int32)) for _ in range(B)]
    rng = np.random.default_rng(V)
    pos = np.zeros(B, np.int64)
    for step in range(6):
        # extend by a different count per sequence (a long prefill first)
        cnt = rng.integers(50, 200, B) if step == 0 else rng.integers(0, 6, B)
        cnt = np.minimum(cnt, n - pos).astype(np.int32)
        L = max(1, int(cnt.max()))
        toks = np.full((B, L), -1, np.int32)
        for b in range(B):
            toks[b, :cnt[b]] = gt[b, pos[b]:pos[b] + cnt[b]]
            sams[b].extend(toks[b, :cnt[b]])
        st.extend(dev(toks), dev(cnt))
        pos += cnt
        for K, M in [(3, 1), (4, 4), (2, 10), (5, 12), (1, 63)]:
            tok, par, nn, ml = (t.cpu().numpy() for t in st.draft_tree(K, M))
            for b in range(B):
                wt, wp, wn, wml = sams[b].draft_tree(K, M)
                assert nn[b] == wn and ml[b] == wml, (step, K, M, b)
                np.testing.assert_array_equal(tok[b], wt)
                np.testing.assert_array_equal(par[b], wp)
    assert (st.status().cpu().numpy() == 0).all()


def test_drafted_trees_verify_like_the_oracle():
    """Trees drafted on the device go straight into spec_verify_tree, with
    target logits that raise the tree's tokens in their parents' rows; the
    oracle verifies its own trees (equal to the device's by the test above)
    on the same logits and coins."""
    say("[gpu] automaton trees into spec_verify_tree")
    B, n, V, K, M = 32, 800, 151936, 3, 5
    N = 1 + K * M
    gt = _streams(B, n, V, 99)
    st = ssl.SamState(B, n, V, "cuda")
    st.extend(dev(gt), dev(np.full(B, n, np.int32)))
    tok, par, nn, _ = st.draft_tree(K, M)
    sams = [oracle.SAM(gt[b]) for b in range(B)]
    ot = np.stack([s.draft_tree(K, M)[0] for s in sams])
    op = np.stack([s.draft_tree(K, M)[1] for s in sams])
    on = np.array([s.draft_tree(K, M)[2] for s in sams], np.int32)
    np.testing.assert_array_equal(tok.cpu().numpy(), ot)
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((B, N, V)) * 1.5).astype(np.float32)
    for b in range(B):
        for i in range(1, on[b]):
            if rng.random() < 0.7:
                x[b, op[b, i], ot[b, i]] += rng.uniform(4, 12)
    T = np.where(rng.random(B) < 0.3, 0.0, 0.9).astype(np.float32)
    u = rng.random((B, N)).astype(np.float32)
    t = torch.from_numpy(x).cuda()
    g = ssl.spec_verify_tree(t, tok, par, nn, dev(T), dev(u))
    torch.cuda.synchronize()
    out, nodes, nem, status = (a.cpu().numpy() for a in g)
    r = oracle.verify_tree(to_host_logits(t), ot, op, on, T, u, nthreads=8)
    compare_tree((out, nodes, nem, status), r, T, u, what="drafted trees")
    assert nem.max() > 1
    say(f"    tokens={int(nem.sum())}")


def test_host_errors():
    st = ssl.SamState(2, 100, 10, "cuda")
    with pytest.raises(ssl.SpecSamError, match="1 \\+ M\\*K"):
        st.draft_tree(8, 8)  # 65 nodes
    with pytest.raises(ssl.SpecSamError, match="1 \\+ M\\*K"):
        st.draft_tree(3, 4, N=12)
