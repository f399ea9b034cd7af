"""Pins for the oracle's static-automaton matching ([P4] SAM-Decoding summary
§3: "Drafting with Suffix Automaton", "Update of Suffix Automaton", and the
choice between the static and the dynamic automaton).

The match state of a generated text G in an automaton over a reference text
R must describe the longest suffix of G that occurs somewhere in R; its
min_endpos must be the first end position of that suffix in R, and the static
draft the tokens after it. These are checked by direct search."""
import numpy as np
import pytest

import oracle


def _longest_suffix_in(R, G):
    """(L, first end position in R) of the longest suffix of G occurring in R."""
    n = len(G)
    for L in range(n, 0, -1):
        w = G[n - L:]
        for e in range(L - 1, len(R)):
            if R[e - L + 1:e + 1] == w:
                return L, e
    return 0, -1


@pytest.mark.parametrize("alpha", [2, 3, 4, 8, 151936])
def test_matching_statistics_by_direct_search(alpha):
    rng = np.random.default_rng(alpha)
    K = 4
    for trial in range(6):
        R = rng.integers(0, alpha, rng.integers(1, 90)).tolist()
        # G mixes spans copied from R with fresh tokens, so matches of every
        # length occur.
        G = []
        while len(G) < 60:
            if rng.random() < 0.6 and len(R) > 1:
                a = int(rng.integers(0, len(R)))
                G += R[a:a + int(rng.integers(1, 12))]
            else:
                G.append(int(rng.integers(0, alpha)))
        G = G[:60]
        sam = oracle.SAM(np.array(R, np.int32))
        ex = sam.export()
        st = np.zeros(1, np.int32)
        ml = np.zeros(1, np.int32)
        for i, t in enumerate(G):
            sam.match(st, ml, np.array([[t]], np.int32))
            L, e = _longest_suffix_in(R, G[:i + 1])
            assert ml[0] == L, (trial, i)
            s = st[0]
            if L > 0:
                # the matched suffix is one of the strings of state s
                assert ex["len"][ex["link"][s]] < L <= ex["len"][s]
                assert ex["min_endpos"][s] == e
            else:
                assert s == 0
            d, dl = sam.static_draft(st, ml, K)
            want = [] if L == 0 else R[e + 1:e + 1 + K]
            assert dl[0] == len(want)
            assert d[0, :dl[0]].tolist() == want
            assert (d[0, dl[0]:] == -1).all()


def test_abcbc_example():
    """The ABCBC example: endpos(BC) = {2, 4}, so a generated text ending in
    BC matches the state of BC, first ending at position 2, and drafts the
    tokens after it (cut at the end of the reference text)."""
    A, B, C, X = 0, 1, 2, 3
    sam = oracle.SAM(np.array([A, B, C, B, C], np.int32))
    st = np.zeros(1, np.int32)
    ml = np.zeros(1, np.int32)
    sam.match(st, ml, np.array([[X]], np.int32))
    assert (st[0], ml[0]) == (0, 0)
    sam.match(st, ml, np.array([[B, C]], np.int32))
    assert ml[0] == 2
    ex = sam.export()
    assert ex["min_endpos"][st[0]] == 2
    d, dl = sam.static_draft(st, ml, 3)
    assert dl[0] == 2 and d[0].tolist() == [B, C, -1]
    # one more C: "BCC" does not occur; the longest suffix that does is "C"
    sam.match(st, ml, np.array([[C]], np.int32))
    assert ml[0] == 1 and ex["min_endpos"][st[0]] == 2


def test_counts_limit_the_tokens_consumed():
    sam = oracle.SAM(np.array([5, 6, 7, 5, 6, 8], np.int32))
    st = np.zeros(2, np.int32)
    ml = np.zeros(2, np.int32)
    toks = np.array([[5, 6, 7], [5, 6, 8]], np.int32)
    sam.match(st, ml, toks, counts=np.array([2, 3], np.int32))
    assert ml.tolist() == [2, 3]


def test_selection_prefers_the_dynamic_draft():
    """The static draft is taken only when its match is longer than the
    dynamic one's by more than delta."""
    sd = np.array([[1, 1], [2, 2], [3, 3], [4, 4]], np.int32)
    dd = np.array([[9, 9], [8, 8], [7, 7], [6, 6]], np.int32)
    sl = np.array([2, 2, 2, 0], np.int32)
    dl = np.array([1, 2, 0, 2], np.int32)
    sm = np.array([5, 4, 10, 0], np.int32)
    dm = np.array([2, 2, 0, 3], np.int32)
    d, l, src = oracle.select_drafts(sd, sl, sm, dd, dl, dm, delta=2)
    # 5 > 2+2 static; 4 > 4 no; 10 > 2 static; 0 > 5 no
    assert src.tolist() == [1, 0, 1, 0]
    assert d.tolist() == [[1, 1], [8, 8], [3, 3], [6, 6]]
    assert l.tolist() == [2, 2, 2, 2]
