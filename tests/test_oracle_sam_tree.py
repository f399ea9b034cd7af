"""Pins for the oracle's draft tree from several automaton candidates (the
tree the draft-tree verifier takes; its candidates are the continuations
after the first occurrences of the text's longest repeated suffix and of each
shorter suffix class along the suffix links, [P1] §1.1 and [P4] "Drafting
with Suffix Automaton" for the single candidate).

Checked by direct search: for each suffix length L of the text, the set of
positions where that suffix ends; lengths with equal sets form one class
(one automaton state), classes ordered from the longest suffix that also
occurs earlier; each class gives the tokens after its first end. The first M
classes' continuations, merged into a trie in order, must be the oracle's
tree node for node; candidate 0 is the single draft."""
import numpy as np
import pytest

import oracle


def _brute_tree(S, K, M):
    n = len(S)
    classes = []
    prev = None
    for L in range(n - 1, 0, -1):
        suf = S[n - L:]
        ends = tuple(e for e in range(L - 1, n) if S[e - L + 1:e + 1] == suf)
        if len(ends) < 2:
            continue  # occurs only at the end: not a match yet
        if ends != prev:
            classes.append((L, ends))
            prev = ends
    tok, par = [-1], [-1]
    for L, ends in classes[:M]:
        p = ends[0]
        cont = S[p + 1:p + 1 + K]
        cur = 0
        for t in cont:
            nxt = [v for v in range(1, len(tok)) if par[v] == cur and tok[v] == t]
            if nxt:
                cur = nxt[0]
            else:
                tok.append(t)
                par.append(cur)
                cur = len(tok) - 1
    ml = classes[0][0] if classes else 0
    return tok, par, ml


@pytest.mark.parametrize("alpha", [2, 3, 5, 50])
def test_tree_by_direct_search(alpha):
    rng = np.random.default_rng(alpha)
    for trial in range(25):
        n = int(rng.integers(1, 120))
        if rng.random() < 0.5:  # copy spans, so long repeats occur
            S = []
            while len(S) < n:
                if S and rng.random() < 0.6:
                    a = int(rng.integers(0, len(S)))
                    S += S[a:a + int(rng.integers(1, 10))]
                else:
                    S.append(int(rng.integers(0, alpha)))
            S = S[:n]
        else:
            S = rng.integers(0, alpha, n).tolist()
        sam = oracle.SAM(np.array(S, np.int32))
        for K, M in [(3, 1), (4, 3), (2, 8), (5, 12)]:
            tok, par, nn, ml = sam.draft_tree(K, M)
            wt, wp, wml = _brute_tree(S, K, M)
            assert nn == len(wt), (trial, K, M)
            assert tok[:nn].tolist() == wt and par[:nn].tolist() == wp, (trial, K, M)
            assert ml == wml
            assert (tok[nn:] == -1).all() and (par[nn:] == -1).all()
            # candidate 0 is the single draft
            d, dl, dml = sam.draft(K)
            assert dml == ml
            chain = [v for v in range(1, 1 + dl)]
            assert tok[chain].tolist() == d[:dl].tolist()
            assert par[chain].tolist() == [0] + chain[:-1] if dl else True


def test_abcbc_tree():
    """ABCBC: BC and C both end at {2, 4}, so they are one state, whose
    first end 2 gives the draft 'BC' (the tokens after position 2, cut at the
    end); its link is the root, so M = 4 still gives one candidate."""
    A, B, C = 0, 1, 2
    sam = oracle.SAM(np.array([A, B, C, B, C], np.int32))
    tok, par, nn, ml = sam.draft_tree(3, 4)
    assert ml == 2 and nn == 3
    assert tok[:3].tolist() == [-1, B, C] and par[:3].tolist() == [-1, 0, 1]


def test_empty_and_unmatched():
    sam = oracle.SAM(np.array([], np.int32))
    tok, par, nn, ml = sam.draft_tree(3, 4)
    assert nn == 1 and ml == 0
    sam = oracle.SAM(np.array([4, 5, 6], np.int32))
    tok, par, nn, ml = sam.draft_tree(3, 4)
    assert nn == 1 and ml == 0
