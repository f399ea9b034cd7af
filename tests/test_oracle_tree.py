"""Pins for the oracle's draft-tree verification ([P3] gogongxt notes "SGLang
的实现": the target-only tree walk, with both of its thresholds at 1).

Checked against: the linear verifier on chain-shaped trees (a chain is the
linear case, and the linear verifier has its own pins), hand cases of the
running-sum rule over siblings, greedy trees by enumerating every node's path,
and chi-square of the first two emitted tokens against the target."""
import numpy as np
import pytest
from scipy import special, stats

import oracle


def _chain(B, n, V, rng, T, scale=1.5):
    N = n
    x = (rng.standard_normal((B, N, V)) * scale).astype(np.float32)
    tok = np.zeros((B, N), np.int32)
    tok[:, 1:] = rng.integers(0, V, (B, N - 1))
    for b in range(B):  # drafts often right
        for i in range(1, N):
            if rng.random() < 0.6:
                tok[b, i] = x[b, i - 1].argmax()
            x[b, i - 1, tok[b, i]] += rng.uniform(0, 3)
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    return x, tok, par


@pytest.mark.parametrize("T", [0.0, 0.8])
def test_chain_tree_is_the_linear_verifier(T):
    rng = np.random.default_rng(int(T * 10) + 1)
    B, N, V = 300, 5, 40
    x, tok, par = _chain(B, N, V, rng, T)
    n_nodes = rng.integers(1, N + 1, B).astype(np.int32)
    u = rng.random((B, N)).astype(np.float32)
    Tb = np.full(B, T, np.float32)
    r = oracle.verify_tree(x, tok, par, n_nodes, Tb, u)
    lin = oracle.verify(x, tok[:, 1:], n_nodes - 1, Tb, u)
    np.testing.assert_array_equal(r.status, 0)
    np.testing.assert_array_equal(r.num_emitted, lin.num_emitted)
    np.testing.assert_array_equal(r.out_tokens, lin.out_tokens)
    # nodes: the accepted drafts are nodes 1..a, the last token came from row a
    for b in range(B):
        a = r.num_emitted[b] - 1
        assert r.out_nodes[b, :a + 1].tolist() == list(range(1, a + 1)) + [a]


def test_running_sum_over_siblings_hand_cases():
    # p(root row) = [.5, .3, .2]; the root's children carry tokens 2 then 0.
    # Running sums .2, .7: u = .15 takes token 2, u = .6 token 0, u = .8
    # rejects both and the final draw from p without {2, 0} is token 1.
    lg = np.log(np.array([0.5, 0.3, 0.2]))
    N = 3
    x = np.tile(lg.astype(np.float32), (1, N, 1))
    tok = np.array([[0, 2, 0]], np.int32)
    par = np.array([[-1, 0, 0]], np.int32)
    for ut, want, node in [(0.15, 2, 1), (0.19, 2, 1), (0.6, 0, 2), (0.69, 0, 2),
                           (0.71, 1, 0), (0.99, 1, 0)]:
        for fc in (0.0, 0.5, 0.99):
            u = np.array([[ut, 0.5, fc]], np.float32)
            r = oracle.verify_tree(x, tok, par, [3], [1.0], u)
            assert r.out_tokens[0, 0] == want, (ut, fc)
            assert r.out_nodes[0, 0] == node
            if node == 0:
                assert r.num_emitted[0] == 1
            else:
                assert r.num_emitted[0] == 2  # leaf: bonus from its row


def _greedy_by_paths(x, tok, par, n):
    """Deepest node whose whole path is the greedy continuation (every token
    on it is the argmax of its parent's row), then the argmax of that node's
    row; by enumerating nodes. With distinct sibling tokens such nodes form
    one chain, so the deepest is unique."""
    best, best_depth = 0, 0
    for i in range(1, n):
        path, v = [], i
        while v > 0:
            path.append(v)
            v = par[v]
        if all(tok[c] == np.argmax(x[par[c]]) for c in path) and len(path) > best_depth:
            best, best_depth = i, len(path)
    nodes = []
    v = best
    while v > 0:
        nodes.append(v)
        v = par[v]
    nodes = nodes[::-1]
    return [int(tok[c]) for c in nodes] + [int(np.argmax(x[best]))], nodes + [best]


def _random_tree(rng, N, V, x):
    par = np.full(N, -1, np.int32)
    tok = np.zeros(N, np.int32)
    for i in range(1, N):
        p = int(rng.integers(0, i))
        used = {int(tok[c]) for c in range(1, i) if par[c] == p}
        am = int(np.argmax(x[p]))
        t = am if (rng.random() < 0.5 and am not in used) else int(rng.integers(0, V))
        while t in used:
            t = (t + 1) % V
        par[i], tok[i] = p, t
    return tok, par


def test_greedy_tree_is_the_deepest_greedy_path():
    rng = np.random.default_rng(3)
    B, N, V = 200, 8, 6
    x = rng.integers(-3, 4, (B, N, V)).astype(np.float32)  # ties
    tok = np.zeros((B, N), np.int32)
    par = np.zeros((B, N), np.int32)
    for b in range(B):
        tok[b], par[b] = _random_tree(rng, N, V, x[b])
    n_nodes = rng.integers(1, N + 1, B).astype(np.int32)
    r = oracle.verify_tree(x, tok, par, n_nodes, np.zeros(B, np.float32))
    for b in range(B):
        want, nodes = _greedy_by_paths(x[b], tok[b], par[b], n_nodes[b])
        e = r.num_emitted[b]
        assert r.out_tokens[b, :e].tolist() == want, b
        assert r.out_nodes[b, :e].tolist() == nodes, b


def test_chi_square_first_two_tokens_follow_the_target():
    """Root with three children (one of them with two children of its own):
    the first emitted token is distributed as p_root, and the second, given
    the first was a child c, as p_c (V = 8, 10^6 draws)."""
    rng = np.random.default_rng(4)
    V, N, M = 8, 6, 1_000_000
    rows = (rng.standard_normal((N, V)) * 1.2).astype(np.float32)
    tok = np.array([0, 3, 5, 1, 2, 3], np.int32)
    par = np.array([-1, 0, 0, 0, 1, 1], np.int32)
    x = np.broadcast_to(rows, (M, N, V)).copy()
    u = rng.random((M, N)).astype(np.float32)
    T = np.float32(0.9)
    r = oracle.verify_tree(x, np.tile(tok, (M, 1)), np.tile(par, (M, 1)),
                           np.full(M, N, np.int32), np.full(M, T, np.float32), u,
                           nthreads=8)
    assert (r.status == 0).all()
    p = special.softmax(rows.astype(np.float64) / float(T), axis=1)
    c1 = np.bincount(r.out_tokens[:, 0], minlength=V)
    assert stats.chisquare(c1, p[0] * M).pvalue > 1e-3
    # second token after the first child (node 1, token 3) was accepted
    sel = r.out_nodes[:, 0] == 1
    c2 = np.bincount(r.out_tokens[sel, 1], minlength=V)
    assert stats.chisquare(c2, p[1] * sel.sum()).pvalue > 1e-3
    # and after node 2 (token 5), a leaf: the bonus from its row
    sel = r.out_nodes[:, 0] == 2
    c2 = np.bincount(r.out_tokens[sel, 1], minlength=V)
    assert stats.chisquare(c2, p[2] * sel.sum()).pvalue > 1e-3


def test_tree_status():
    V, N = 10, 4
    x = np.zeros((5, N, V), np.float32)
    tok = np.array([[0, 1, 2, 3]] * 5, np.int32)
    par = np.array([[-1, 0, 0, 1]] * 5, np.int32)
    n = np.full(5, N, np.int32)
    tok[0, 2] = 1          # duplicate sibling token
    par[1, 2] = 2          # parent not before the node
    tok[2, 3] = V          # token out of range
    n[3] = 0               # no root
    par[4, 0] = 0          # root with a parent
    r = oracle.verify_tree(x, tok, par, n, np.zeros(5, np.float32))
    assert (r.status == oracle.ST_TREE).all()
    # unused nodes past n_nodes are ignored
    tok2, par2 = tok[:1].copy(), par[:1].copy()
    r = oracle.verify_tree(x[:1], tok2, par2, [2], [0.0])
    assert r.status[0] == 0
