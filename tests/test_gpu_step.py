"""End-to-end parity of whole steps (draft -> verify -> extend) on the five
workloads: the GPU path and the oracle run side by side on the same device
bytes; drafts, emitted tokens and the automata must agree (T > 0 draws up to
counted ties, after which the oracle follows the GPU's tokens)."""
import numpy as np
import pytest
import torch

import oracle
import sam_drafting_lossless_amd as ssl
import synth
from _parity import Tally, compare_verify, dev, say, to_host_logits

pytestmark = pytest.mark.gpu


def _run_sam_workload(c, steps, **over):
    cfg = synth.config(c, **over)
    say(f"[gpu] steps {cfg.name} B={cfg.B} steps={steps}")
    gt = synth.token_streams(cfg, steps)
    H = cfg.hist_len
    n = np.full(cfg.B, H, np.int32)
    max_len = cfg.stream_len(steps)
    st = ssl.SamState(cfg.B, max_len, cfg.V, "cuda")
    st.extend(dev(gt[:, :H]), dev(np.full(cfg.B, H, np.int32)))
    sams = [oracle.SAM(gt[b, :H]) for b in range(cfg.B)]
    T = np.full(cfg.B, cfg.T, np.float32)
    Td = dev(T)
    ws = ssl.verify_workspace(cfg.B, cfg.K, cfg.V)
    tally = Tally()
    tokens_total = 0
    for s in range(steps):
        d, dl, ml = st.draft(cfg.K)
        x = synth.target_logits(cfg, s, gt, n, device="cuda")
        u = synth.uniforms(cfg, s)
        out, nem, pd, status = ssl.spec_verify(x, d, dl, Td, dev(u), workspace=ws)
        st.extend(out, nem)
        torch.cuda.synchronize()
        d, dl, ml = d.cpu().numpy(), dl.cpu().numpy(), ml.cpu().numpy()
        g = (out.cpu().numpy(), nem.cpu().numpy(), pd.cpu().numpy(),
             status.cpu().numpy())
        for b in range(cfg.B):
            od, odl, oml = sams[b].draft(cfg.K)
            assert (od == d[b]).all() and odl == dl[b] and oml == ml[b], (s, b)
        r = oracle.verify(to_host_logits(x), d, dl, T, u, nthreads=8)
        compare_verify(*g, r, T, u, tally, what=f"{cfg.name} step {s}")
        for b in range(cfg.B):
            sams[b].extend(g[0][b, :g[1][b]])  # identical unless a counted tie
        n = n + g[1]
        tokens_total += int(g[1].sum())
    for b in range(cfg.B):  # every automaton, bit for bit
        e, o = st.export(b), sams[b].export()
        np.testing.assert_array_equal(e["len"], o["len"])
        np.testing.assert_array_equal(e["link"], o["link"])
        np.testing.assert_array_equal(e["min_endpos"], o["min_endpos"])
        np.testing.assert_array_equal(e["edges"], o["edges"])
    assert (st.status().cpu().numpy() == 0).all()
    say(f"    mean tokens/step {tokens_total / (steps * cfg.B):.3f}")
    tally.check(cfg.name)
    return tally


def test_c1_tiny_greedy_500_steps():
    _run_sam_workload(1, 500)


def test_c2_greedy_full_size():
    _run_sam_workload(2, 6)


def test_c3_one_hot_full_size():
    _run_sam_workload(3, 4)


def test_c4_bf16_long_history():
    _run_sam_workload(4, 3)


def test_c3_shape_high_acceptance():
    """A sensitivity variant (boost +12) so that drafts are often accepted and
    the automaton grows by several tokens per step."""
    _run_sam_workload(3, 6, B=32, boost=12.0)


def test_c5_draft_model_full_size():
    cfg = synth.config(5)
    say(f"[gpu] steps {cfg.name}")
    T = np.full(cfg.B, cfg.T, np.float32)
    tally = Tally()
    for s in range(2):
        x = synth.noise(cfg, s, "cuda")
        q, draft = synth.draft_model_inputs(cfg, s, x, "cuda")
        u = synth.uniforms(cfg, s)
        dl = np.full(cfg.B, cfg.K, np.int32)
        g = ssl.spec_verify(x, dev(draft), dev(dl), dev(T), dev(u), q)
        torch.cuda.synchronize()
        g = tuple(t.cpu().numpy() for t in g)
        r = oracle.verify(x.cpu().numpy(), draft, dl, T, u, q.cpu().numpy(),
                          nthreads=8)
        compare_verify(*g, r, T, u, tally, what=f"c5 step {s}")
    tally.check()


def _run_fused_workload(c, steps, **over):
    """Same as the separate-call run, but each step is one spec_step call
    (verify + extend + next draft), with drafts ping-ponging between two
    buffers; compared against the oracle every step."""
    cfg = synth.config(c, **over)
    say(f"[gpu] fused steps {cfg.name} B={cfg.B} steps={steps}")
    gt = synth.token_streams(cfg, steps)
    H = cfg.hist_len
    n = np.full(cfg.B, H, np.int32)
    st = ssl.SamState(cfg.B, cfg.stream_len(steps), cfg.V, "cuda")
    st.extend(dev(gt[:, :H]), dev(np.full(cfg.B, H, np.int32)))
    sams = [oracle.SAM(gt[b, :H]) for b in range(cfg.B)]
    T = np.full(cfg.B, cfg.T, np.float32)
    Td = dev(T)
    ws = ssl.verify_workspace(cfg.B, cfg.K, cfg.V)
    bufs = [st.draft(cfg.K), tuple(torch.empty_like(t) for t in st.draft(cfg.K))]
    tally = Tally()
    for s in range(steps):
        d, dl, ml = bufs[s % 2]
        nd, ndl, nml = bufs[(s + 1) % 2]
        x = synth.target_logits(cfg, s, gt, n, device="cuda")
        u = synth.uniforms(cfg, s)
        out, nem, pd, status, *_ = ssl.spec_step(
            x, d, dl, Td, dev(u), st, workspace=ws, next_draft=nd,
            next_draft_len=ndl, next_match_len=nml)
        torch.cuda.synchronize()
        dh, dlh, mlh = d.cpu().numpy(), dl.cpu().numpy(), ml.cpu().numpy()
        for b in range(cfg.B):
            od, odl, oml = sams[b].draft(cfg.K)
            assert (od == dh[b]).all() and odl == dlh[b] and oml == mlh[b], (s, b)
        g = (out.cpu().numpy(), nem.cpu().numpy(), pd.cpu().numpy(),
             status.cpu().numpy())
        r = oracle.verify(to_host_logits(x), dh, dlh, T, u, nthreads=8)
        compare_verify(*g, r, T, u, tally, what=f"fused {cfg.name} step {s}")
        for b in range(cfg.B):
            sams[b].extend(g[0][b, :g[1][b]])
        n = n + g[1]
    nd, ndl, nml = bufs[steps % 2]
    ndh = nd.cpu().numpy()
    for b in range(cfg.B):
        od, odl, oml = sams[b].draft(cfg.K)
        assert (od == ndh[b]).all() and odl == int(ndl[b]) and oml == int(nml[b])
    for b in range(cfg.B):  # every automaton, bit for bit
        e, o = st.export(b), sams[b].export()
        np.testing.assert_array_equal(e["len"], o["len"])
        np.testing.assert_array_equal(e["link"], o["link"])
        np.testing.assert_array_equal(e["min_endpos"], o["min_endpos"])
        np.testing.assert_array_equal(e["edges"], o["edges"])
    assert (st.status().cpu().numpy() == 0).all()
    tally.check()


def test_fused_c1_tiny_greedy():
    _run_fused_workload(1, 300)


def test_fused_c2_greedy_full_size():
    _run_fused_workload(2, 5)


def test_fused_c3_one_hot_full_size():
    _run_fused_workload(3, 4)


def test_fused_c3_shape_high_acceptance():
    _run_fused_workload(3, 8, B=48, boost=12.0)


def test_fused_c4_bf16_long_history():
    _run_fused_workload(4, 3)


def test_fused_step_flagged_sequence_keeps_automaton():
    """A sequence whose draft_len is invalid is reported, not extended, and
    still gets a next draft from its unchanged automaton."""
    say("[gpu] fused step with a flagged sequence")
    cfg = synth.config(1, B=3, V=50, hist_len=40)
    gt = synth.token_streams(cfg, 2)
    st = ssl.SamState(3, 100, cfg.V, "cuda")
    st.extend(dev(gt[:, :40]), dev(np.full(3, 40, np.int32)))
    d, dl, ml = st.draft(cfg.K)
    dl_bad = dl.clone()
    dl_bad[1] = cfg.K + 2
    x = torch.zeros((3, cfg.K + 1, cfg.V), device="cuda")
    out, nem, pd, status, nd, ndl, nml = ssl.spec_step(
        x, d, dl_bad, dev(np.zeros(3, np.float32)), None, st)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, ssl.ST_DRAFT_LEN, 0]
    e = st.export(1)
    assert e["n"] == 40
    o = oracle.SAM(gt[1, :40])
    od, odl, oml = o.draft(cfg.K)
    assert nd[1].cpu().tolist() == od.tolist() and int(ndl[1]) == odl


def test_two_pass_calls_match_one_call_forms():
    """spec_stream followed by spec_finish gives bit-identical results to
    spec_step (automaton update) and to spec_verify (given q, residual pass),
    and the automata end up identical."""
    cfg = synth.config(3, B=48, boost=12.0)
    say("[gpu] two-pass calls vs one-call forms")
    steps = 4
    gt = synth.token_streams(cfg, steps)
    H = cfg.hist_len
    n = np.full(cfg.B, H, np.int32)
    ml_cap = cfg.stream_len(steps)
    sts = [ssl.SamState(cfg.B, ml_cap, cfg.V, "cuda") for _ in range(2)]
    for st in sts:
        st.extend(dev(gt[:, :H]), dev(np.full(cfg.B, H, np.int32)))
    Td = dev(np.full(cfg.B, cfg.T, np.float32))
    ws = [ssl.verify_workspace(cfg.B, cfg.K, cfg.V) for _ in range(2)]
    d, dl, ml = sts[0].draft(cfg.K)
    for s in range(steps):
        x = synth.target_logits(cfg, s, gt, n, device="cuda")
        u = dev(synth.uniforms(cfg, s))
        a = ssl.spec_step(x, d, dl, Td, u, sts[0], workspace=ws[0])
        ssl.spec_stream(x, d, dl, Td, u, ws[1])
        b = ssl.spec_finish(x, d, dl, Td, u, ws[1], state=sts[1])
        torch.cuda.synchronize()
        for ta, tb in zip(a, b):
            assert torch.equal(ta, tb), s
        n = n + a[1].cpu().numpy()
        d, dl, ml = a[4], a[5], a[6]
    for bq in range(cfg.B):
        ea, eb = sts[0].export(bq), sts[1].export(bq)
        for k in ("len", "link", "min_endpos", "edges"):
            np.testing.assert_array_equal(ea[k], eb[k])
    c5 = synth.config(5, B=16)
    x = synth.noise(c5, 0, "cuda")
    q, draft = synth.draft_model_inputs(c5, 0, x, "cuda")
    u = dev(synth.uniforms(c5, 0))
    T = dev(np.full(c5.B, c5.T, np.float32))
    dl = dev(np.full(c5.B, c5.K, np.int32))
    dd = dev(draft)
    a = ssl.spec_verify(x, dd, dl, T, u, q)
    w = ssl.verify_workspace(c5.B, c5.K, c5.V)
    ssl.spec_stream(x, dd, dl, T, u, w)
    b = ssl.spec_finish(x, dd, dl, T, u, w, q)
    torch.cuda.synchronize()
    for ta, tb in zip(a, b):
        assert torch.equal(ta, tb)
