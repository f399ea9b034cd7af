"""Pins for the oracle's suffix automaton (CPU only).

Each test checks the std::map automaton against something other than itself:
the ABCBC worked example, brute-force string search, the endpos definition,
and the textbook size bounds.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "abcbc.json")


def _walk(sam_export, string):
    """State reached by reading `string` from the root, or None."""
    edges = {(int(s), int(t)): int(d) for s, t, d in sam_export["edges"]}
    s = 0
    for c in string:
        s = edges.get((s, int(c)))
        if s is None:
            return None
    return s


def _prefix_states(exp, n):
    """The state created for each prefix S[0..i] is the one whose min_endpos
    is i and whose len is i + 1 (the 'cur' of that extension)."""
    out = {}
    for s in range(len(exp["len"])):
        if exp["len"][s] == exp["min_endpos"][s] + 1 and exp["min_endpos"][s] >= 0:
            out[int(exp["min_endpos"][s])] = s
    assert sorted(out) == list(range(n))
    return out


def _endpos_from_links(exp, n):
    """endpos(v) = positions i whose prefix state has v on its link chain."""
    pre = _prefix_states(exp, n)
    ep = {s: set() for s in range(len(exp["len"]))}
    for i, s in pre.items():
        while s != -1:
            ep[s].add(i)
            s = int(exp["link"][s])
    return ep


def _brute_endpos(text, sub):
    L = len(sub)
    return {e for e in range(L - 1, len(text))
            if list(text[e - L + 1:e + 1]) == list(sub)}


def test_abcbc_worked_example():
    g = json.load(open(GOLDEN))
    text = g["text"]
    sam = oracle.SAM(text)
    exp = sam.export()
    hd = g["hand_derived"]
    assert exp["len"].tolist() == hd["len"]
    assert exp["link"].tolist() == hd["link"]
    assert exp["min_endpos"].tolist() == hd["min_endpos"]
    assert exp["edges"].tolist() == hd["edges"]
    assert exp["last"] == hd["last"]
    # The page's printed facts.
    bc = g["page_printed"]["endpos_BC"]
    s_bc = _walk(exp, [1, 2])
    ep = _endpos_from_links(exp, len(text))
    assert sorted(ep[s_bc]) == bc
    assert exp["min_endpos"][s_bc] == min(bc)
    d, dl, ml = sam.draft(3)
    assert d.tolist() == hd["draft_K3"]["draft"]
    assert dl == hd["draft_K3"]["draft_len"] and ml == hd["draft_K3"]["match_len"]
    assert d[:dl].tolist() == g["page_printed"]["draft_after_ABCBC"]
    # last walks one suffix link to the node "BC".
    assert sam.last_walk_hops == 1
    assert int(exp["link"][exp["last"]]) == _walk(
        exp, g["page_printed"]["walk_from_last_reaches_state_of"])


def _brute_match(text, K):
    """Plain definition: L* = largest L >= 1 such that the suffix of length L
    also ends at some e < n-1; p* = smallest such e; draft = text[p*+1 ...]
    cut to K tokens and to the end of the text."""
    n = len(text)
    best_L, best_e = 0, -1
    for L in range(1, n):
        suf = text[n - L:]
        ends = [e for e in range(L - 1, n - 1)
                if np.array_equal(text[e - L + 1:e + 1], suf)]
        if not ends:
            break  # a longer suffix cannot occur if this one does not
        best_L, best_e = L, min(ends)
    if best_L == 0:
        return [], 0
    d = min(K, n - 1 - best_e)
    return text[best_e + 1:best_e + 1 + d].tolist(), best_L


@pytest.mark.parametrize("alphabet", [2, 3, 4, 8, 151936])
def test_longest_suffix_and_draft_brute_force(alphabet):
    rng = np.random.default_rng(alphabet)
    for trial in range(6):
        n = int(rng.integers(1, 201))
        if alphabet > 100:
            # large vocabulary: draw from a small pool so that repeats occur
            pool = rng.choice(alphabet, size=12, replace=False)
            text = pool[rng.integers(0, 12, n)].astype(np.int32)
        else:
            text = rng.integers(0, alphabet, n).astype(np.int32)
        sam = oracle.SAM()
        for i in range(n):
            sam.extend(text[i:i + 1])
            for K in (1, 3, 5):
                d, dl, ml = sam.draft(K)
                want, wl = _brute_match(text[:i + 1], K)
                assert ml == wl, (alphabet, trial, i, K)
                assert d[:dl].tolist() == want, (alphabet, trial, i, K)
                assert (d[dl:] == -1).all()
            assert sam.last_walk_hops == 1


@pytest.mark.parametrize("seed", range(8))
def test_recognition_and_endpos(seed):
    """For small texts: the automaton accepts exactly the substrings; every
    string of a state (lengths len[link]+1 .. len) has the state's endpos, as
    computed from the link tree; min_endpos is the first end position."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 13))
    text = rng.integers(0, 3, n).astype(np.int32)
    sam = oracle.SAM(text)
    exp = sam.export()
    ep = _endpos_from_links(exp, n)
    subs = {tuple(text[a:b]) for a in range(n) for b in range(a + 1, n + 1)}
    # every substring is accepted, in the state whose endpos matches
    for sub in subs:
        s = _walk(exp, sub)
        assert s is not None
        want = _brute_endpos(text, sub)
        assert ep[s] == want
        assert exp["min_endpos"][s] == min(want)
        assert exp["len"][exp["link"][s]] < len(sub) <= exp["len"][s]
    # nothing else is accepted: all strings over {0,1,2} up to length n+1
    import itertools
    for L in range(1, min(n + 1, 6) + 1):
        for cand in itertools.product(range(3), repeat=L):
            assert (_walk(exp, cand) is not None) == (cand in subs)


@pytest.mark.parametrize("alphabet", [1, 2, 3, 26, 151936])
def test_size_bounds_and_link_invariants(alphabet):
    rng = np.random.default_rng(7 + alphabet)
    for n in [1, 2, 3, 4, 17, 300, 2000]:
        text = rng.integers(0, alphabet, n).astype(np.int32)
        sam = oracle.SAM(text)
        exp = sam.export()
        S, E = sam.num_states, sam.num_edges
        if n >= 2:
            assert S <= 2 * n - 1
        if n >= 3:
            assert E <= 3 * n - 4
        ln, lk = exp["len"], exp["link"]
        assert lk[0] == -1 and ln[0] == 0
        assert (ln[lk[1:]] < ln[1:]).all()
        assert exp["len"][exp["last"]] == n
        # every edge goes to a longer state
        e = exp["edges"]
        if len(e):
            assert (ln[e[:, 2]] > ln[e[:, 0]]).all()


def test_walk_takes_one_hop_on_copy_stream():
    import synth
    cfg = synth.config(2, B=1)
    text = synth.copy_process(synth.rng_for(1, 0), 3000, cfg.V, 0.6, 8.0)
    sam = oracle.SAM()
    for i in range(len(text)):
        sam.extend(text[i:i + 1])
        sam.draft(3)
        assert sam.last_walk_hops == 1


def test_empty_automaton_drafts_nothing():
    sam = oracle.SAM()
    d, dl, ml = sam.draft(4)
    assert dl == 0 and ml == 0 and (d == -1).all()
    sam.extend([5])
    d, dl, ml = sam.draft(4)
    assert dl == 0 and ml == 0
    sam.extend([5])
    d, dl, ml = sam.draft(4)
    # "55": suffix "5" first ends at 0, followed by one token
    assert ml == 1 and dl == 1 and d[0] == 5
