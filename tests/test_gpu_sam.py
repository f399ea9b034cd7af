"""GPU parity of the suffix-automaton kernels against the oracle: structure
(len, link, min_endpos, transition set, state/edge numbering) and drafts are
compared bit for bit."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import sam_drafting_lossless_amd as ssl
import synth
from _parity import dev, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "abcbc.json")


def _check_chains(g, what):
    """The table's `next` field chains each state's transitions (the chain a
    clone copies): from first_edge, the chain visits exactly the rows whose
    source is that state, each once."""
    slots, fe = g["slots"], g["first_edge"]
    rows = {}
    for i, (src, _tok, _dst, _nxt) in enumerate(slots):
        if src >= 0:
            rows.setdefault(int(src), set()).add(i)
    for s in range(g["num_states"]):
        seen, e = set(), int(fe[s])
        while e != -1:
            assert e not in seen, (what, "cycle in the chain of state", s)
            assert slots[e][0] == s, (what, "chain of state", s, "reaches row", e)
            seen.add(e)
            e = int(slots[e][3])
        assert seen == rows.get(s, set()), (what, "chain of state", s)


def _compare_structure(g, o, what):
    _check_chains(g, what)
    assert g["num_states"] == len(o["len"]), what
    assert g["num_edges"] == len(o["edges"]), what
    assert g["last"] == o["last"], what
    np.testing.assert_array_equal(g["len"], o["len"], err_msg=what)
    np.testing.assert_array_equal(g["link"], o["link"], err_msg=what)
    np.testing.assert_array_equal(g["min_endpos"], o["min_endpos"], err_msg=what)
    np.testing.assert_array_equal(g["edges"], o["edges"], err_msg=what)


def test_abcbc_golden_on_gpu():
    say("[gpu] sam ABCBC")
    gd = json.load(open(GOLDEN))
    st = ssl.SamState(1, 16, 3, "cuda")
    st.extend(dev(np.array([gd["text"]], np.int32)), dev(np.array([5], np.int32)))
    e = st.export(0)
    hd = gd["hand_derived"]
    assert e["len"].tolist() == hd["len"]
    assert e["link"].tolist() == hd["link"]
    assert e["min_endpos"].tolist() == hd["min_endpos"]
    assert e["edges"].tolist() == hd["edges"]
    assert e["last"] == hd["last"] and e["status"] == 0
    d, dl, ml = st.draft(3)
    torch.cuda.synchronize()
    assert d.cpu().tolist() == [hd["draft_K3"]["draft"]]
    assert dl.item() == 2 and ml.item() == 2


@pytest.mark.parametrize("alphabet", [1, 2, 3, 8, 151936])
def test_incremental_extend_and_draft_match_oracle(alphabet):
    say(f"[gpu] sam incremental alphabet={alphabet}")
    rng = np.random.default_rng(alphabet)
    B, max_len, K = 16, 600, 5
    texts = []
    for b in range(B):
        n = int(rng.integers(1, max_len + 1))
        if alphabet > 1000:
            pool = rng.choice(alphabet, size=20, replace=False)
            t = pool[rng.integers(0, 20, n)]
        else:
            t = rng.integers(0, alphabet, n)
        texts.append(t.astype(np.int32))
    st = ssl.SamState(B, max_len, alphabet, "cuda")
    sams = [oracle.SAM() for _ in range(B)]
    pos = np.zeros(B, np.int64)
    ld = 7
    while (pos < [len(t) for t in texts]).any():
        cnt = np.array([min(int(rng.integers(0, ld + 1)), len(texts[b]) - pos[b])
                        for b in range(B)], np.int32)
        tok = np.full((B, ld), -5, np.int32)
        for b in range(B):
            tok[b, :cnt[b]] = texts[b][pos[b]:pos[b] + cnt[b]]
            sams[b].extend(tok[b, :cnt[b]])
        pos += cnt
        st.extend(dev(tok), dev(cnt))
        d, dl, ml = st.draft(K)
        d, dl, ml = d.cpu().numpy(), dl.cpu().numpy(), ml.cpu().numpy()
        for b in range(B):
            od, odl, oml = sams[b].draft(K)
            assert (d[b] == od).all() and dl[b] == odl and ml[b] == oml, b
    for b in range(B):
        _compare_structure(st.export(b), sams[b].export(), f"seq {b}")
    assert (st.status().cpu().numpy() == 0).all()


@pytest.mark.parametrize("c,nseq", [(3, 16), (4, 4)])
def test_long_copy_process_prefill(c, nseq):
    """Histories of the workloads' length (8,192 and 32,768 tokens)."""
    cfg = synth.config(c, B=nseq)
    say(f"[gpu] sam prefill {cfg.name} B={nseq} n={cfg.hist_len}")
    gt = synth.token_streams(cfg, steps=1)
    H = cfg.hist_len
    st = ssl.SamState(nseq, H + 16, cfg.V, "cuda")
    st.extend(dev(gt[:, :H]), dev(np.full(nseq, H, np.int32)))
    d, dl, ml = st.draft(cfg.K)
    d, dl, ml = d.cpu().numpy(), dl.cpu().numpy(), ml.cpu().numpy()
    for b in range(nseq):
        o = oracle.SAM(gt[b, :H])
        od, odl, oml = o.draft(cfg.K)
        assert (d[b] == od).all() and dl[b] == odl and ml[b] == oml
        _compare_structure(st.export(b), o.export(), f"seq {b}")


def test_status_bits_and_skip():
    say("[gpu] sam status")
    B, max_len = 4, 10
    st = ssl.SamState(B, max_len, 50, "cuda")
    tok = np.zeros((B, 12), np.int32)
    tok[0, :11] = np.arange(11) % 5      # 11 tokens > capacity 10
    tok[1, :3] = [1, 50, 2]              # token out of range at index 1
    tok[2, :4] = [3, 3, 3, 3]
    cnt = np.array([11, 3, 4, 13], np.int32)  # seq 3: count > ld
    st.extend(dev(tok), dev(cnt))
    s = st.status().cpu().tolist()
    assert s == [ssl.ST_SAM_CAPACITY, ssl.ST_TOKEN_RANGE, 0, ssl.ST_COUNT]
    e0, e1 = st.export(0), st.export(1)
    assert e0["n"] == 10 and e1["n"] == 1  # applied up to the failing token
    o = oracle.SAM(tok[0, :10])
    _compare_structure(e0, o.export(), "capacity seq")
    # flagged sequences are skipped from now on
    st.extend(dev(tok), dev(np.array([1, 1, 1, 0], np.int32)))
    assert st.export(0)["n"] == 10 and st.export(2)["n"] == 5


def test_zero_counts_and_empty_drafts():
    st = ssl.SamState(3, 8, 10, "cuda")
    d, dl, ml = st.draft(4)
    assert dl.cpu().tolist() == [0, 0, 0] and (d.cpu() == -1).all()
    st.extend(dev(np.zeros((3, 1), np.int32)), dev(np.array([0, 1, 1], np.int32)))
    st.extend(dev(np.zeros((3, 1), np.int32)), dev(np.array([0, 0, 1], np.int32)))
    d, dl, ml = st.draft(4)
    assert dl.cpu().tolist() == [0, 0, 1] and ml.cpu().tolist() == [0, 0, 1]
    assert d.cpu()[2].tolist() == [0, -1, -1, -1]


def test_extend_draft_matches_separate_calls():
    say("[gpu] sam_extend_draft")
    rng = np.random.default_rng(44)
    B, max_len, K, ld = 8, 400, 4, 5
    a = ssl.SamState(B, max_len, 6, "cuda")
    bst = ssl.SamState(B, max_len, 6, "cuda")
    for _ in range(60):
        cnt = rng.integers(0, ld + 1, B).astype(np.int32)
        tok = rng.integers(0, 6, (B, ld)).astype(np.int32)
        a.extend(dev(tok), dev(cnt))
        d1, l1, m1 = a.draft(K)
        d2, l2, m2 = bst.extend_draft(dev(tok), dev(cnt), K)
        torch.cuda.synchronize()
        assert torch.equal(d1, d2) and torch.equal(l1, l2) and torch.equal(m1, m2)
    for b in range(B):
        ea, eb = a.export(b), bst.export(b)
        for k in ("len", "link", "min_endpos", "edges", "text"):
            np.testing.assert_array_equal(ea[k], eb[k])
