"""Resume and determinism of the automata, on the GPU through the C ABI.

* Resume: an automaton rebuilt by one prefill of a sequence's committed
  history (its text, as sam_export returns it) equals, bit for bit, the live
  automaton that grew by fused steps (prefill, then 1..K+1 tokens a step):
  header, every state record, every raw hash-table row and the text. Blumer's
  construction and the table's first-empty-row insertion depend only on the
  token sequence ([P4] SAM-Decoding summary §3 "Update of Suffix
  Automaton"), so a caller can drop the automata and rebuild them from the
  token history.
* Determinism: the same step or extension applied twice to copies of one
  snapshot leaves byte-identical buffers and outputs."""
import numpy as np
import pytest
import torch

import sam_drafting_lossless_amd as ssl
import synth
from _parity import dev, say

pytestmark = pytest.mark.gpu


def _copy(st):
    c = ssl.SamState.__new__(ssl.SamState)
    c.B, c.max_len, c.V = st.B, st.max_len, st.V
    c.buf = st.buf.clone()
    return c


def _drive(cfg, steps, st):
    """Fused steps (spec_step) from the automata's own drafts; returns the
    per-step outputs."""
    gt = synth.token_streams(cfg, steps)
    n = np.full(cfg.B, cfg.hist_len, np.int32)
    Td = dev(np.full(cfg.B, cfg.T, np.float32))
    bufs = [st.draft(cfg.K), tuple(torch.empty_like(t) for t in st.draft(cfg.K))]
    outs = []
    for s in range(steps):
        d, dl, _ = bufs[s % 2]
        nd, ndl, nml = bufs[(s + 1) % 2]
        x = synth.target_logits(cfg, s, gt, n, device="cuda")
        out, nem, pd, status, *_ = ssl.spec_step(
            x, d, dl, Td, dev(synth.uniforms(cfg, s)), st, next_draft=nd,
            next_draft_len=ndl, next_match_len=nml)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), nem.cpu().numpy(), pd.cpu().numpy(),
                     status.cpu().numpy(), nd.cpu().numpy(), ndl.cpu().numpy()))
        n = n + outs[-1][1]
    return outs


def _prefilled(cfg, steps):
    gt = synth.token_streams(cfg, steps)
    st = ssl.SamState(cfg.B, cfg.stream_len(steps), cfg.V, "cuda")
    H = cfg.hist_len
    st.extend(dev(gt[:, :H]), dev(np.full(cfg.B, H, np.int32)))
    return st


def test_automaton_rebuilt_from_its_history_is_bit_identical():
    cfg = synth.config(3, B=48, boost=12.0, hist_len=2048)
    steps = 10
    say(f"[gpu] resume: {cfg.B} automata after {steps} fused steps, rebuilt from text")
    st = _prefilled(cfg, steps)
    outs = _drive(cfg, steps, st)
    assert max(int(o[1].max()) for o in outs) > 1  # multi-token appends happened
    live = [st.export(b) for b in range(cfg.B)]
    lens = np.array([e["n"] for e in live], np.int32)
    toks = np.full((cfg.B, int(lens.max())), -1, np.int32)
    for b, e in enumerate(live):
        toks[b, :lens[b]] = e["text"]
    re = ssl.SamState(cfg.B, st.max_len, cfg.V, "cuda")
    re.extend(dev(toks), dev(lens))
    for b in range(cfg.B):
        a, r = live[b], re.export(b)
        for k in ("n", "last", "num_states", "num_edges", "status"):
            assert a[k] == r[k], (b, k, a[k], r[k])
        for k in ("len", "link", "min_endpos", "first_edge", "text", "slots"):
            np.testing.assert_array_equal(a[k], r[k], err_msg=f"b={b} {k}")
    say(f"    {int(lens.sum())} tokens, {sum(e['num_states'] for e in live)} states")


def test_steps_and_extensions_from_one_snapshot_are_deterministic():
    cfg = synth.config(3, B=64, boost=12.0, hist_len=1024)
    say("[gpu] determinism: the same steps twice from one snapshot")
    st = _prefilled(cfg, 6)
    snap = _copy(st)
    a = _drive(cfg, 6, st)
    b = _drive(cfg, 6, snap)
    for s, (x, y) in enumerate(zip(a, b)):
        for i, (u, v) in enumerate(zip(x, y)):
            np.testing.assert_array_equal(u, v, err_msg=f"step {s} output {i}")
    assert torch.equal(st.buf, snap.buf)
    # plain extensions of varying counts, twice from one snapshot
    rng = np.random.default_rng(4)
    snap2 = _copy(st)
    for _ in range(5):
        cnt = rng.integers(0, 6, cfg.B).astype(np.int32)
        tk = rng.integers(0, cfg.V, (cfg.B, 5)).astype(np.int32)
        st.extend(dev(tk), dev(cnt))
        snap2.extend(dev(tk), dev(cnt))
    torch.cuda.synchronize()
    assert torch.equal(st.buf, snap2.buf)
