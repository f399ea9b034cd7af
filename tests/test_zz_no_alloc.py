"""spec_step_noalloc (the fused step with the library's own device scratch
as its workspace, for callers that cannot allocate) against spec_step on
the same inputs, through the C ABI: two calls in a row, the second smaller
than the first, on automata copied byte for byte before the first call.
Both run the same kernels on the same bytes, so every output and the
automata afterwards must be identical; the oversized call is refused."""
import numpy as np
import pytest
import torch

import sam_drafting_lossless_amd as ssl
import synth
from _parity import dev, say

pytestmark = pytest.mark.gpu


def _case(B, K, V, T, boost, hist, seed):
    cfg = synth.config(3, B=B, V=V, K=K, T=T, boost=boost, hist_len=hist,
                       steps=4, warmup=0, seed=seed)
    gt = synth.token_streams(cfg, 4)
    st = ssl.SamState(B, cfg.stream_len(4), V, "cuda")
    st.extend(dev(gt[:, :hist]), dev(np.full(B, hist, np.int32)))
    return cfg, gt, st


def _copy(st):
    c = ssl.SamState.__new__(ssl.SamState)
    c.B, c.max_len, c.V = st.B, st.max_len, st.V
    c.buf = st.buf.clone()
    return c


def test_noalloc_step_matches_spec_step():
    # (B, K, V, T, boost, history, seed): the c3 shape with a boost that gets
    # drafts accepted, then a smaller batch with longer drafts; every fifth
    # sequence greedy
    cases = [(256, 3, 151936, 1.0, 12.0, 2048, 11),
             (24, 5, 30011, 0.7, 8.0, 700, 12)]
    for i, (B, K, V, T, boost, hist, seed) in enumerate(cases):
        say(f"[gpu] noalloc call {i}: B={B} K={K} V={V} T={T}")
        cfg, gt, st_a = _case(B, K, V, T, boost, hist, seed)
        st_b = _copy(st_a)
        d, dl, _ = st_a.draft(K)
        n = np.full(B, hist, np.int32)
        x = synth.target_logits(cfg, 0, gt, n, device="cuda")
        Tv = np.full(B, T, np.float32)
        Tv[::5] = 0.0  # some greedy sequences
        Td = dev(Tv)
        u = dev(synth.uniforms(cfg, 0))
        lp_a = torch.empty((B, K + 1), device="cuda")
        lp_b = torch.empty((B, K + 1), device="cuda")
        ga = ssl.spec_step(x, d, dl, Td, u, st_a, logprobs=lp_a)
        gb = ssl.spec_step_noalloc(x, d, dl, Td, u, st_b, logprobs=lp_b)
        torch.cuda.synchronize()
        names = ["out_tokens", "num_emitted", "p_draft", "status", "next_draft",
                 "next_draft_len", "next_match_len"]
        for nm, a, b in zip(names, ga, gb):
            assert torch.equal(a, b), (i, nm)
        assert torch.equal(lp_a.isnan(), lp_b.isnan())
        assert torch.equal(torch.nan_to_num(lp_a), torch.nan_to_num(lp_b)), i
        assert torch.equal(st_a.buf, st_b.buf), i
        assert (ga[3] == 0).all()
        nem = ga[1].cpu().numpy()
        say(f"    tokens/step {nem.mean():.2f}, max {nem.max()}")
        assert nem.max() > 1  # drafts were accepted: rows beyond 0 were read


def test_noalloc_refuses_sizes_beyond_its_scratch():
    """Sizes whose workspace exceeds the scratch are refused before anything
    is launched or read (the pointers below are never dereferenced): B = 2048,
    K = 16, V = 151936 needs 2048 x 17 x 19 partials of 16 bytes (10.6 MB);
    top_k at the c3 shape needs the truncation workspace (about 100 MB)."""
    say("[gpu] noalloc: oversized calls")
    L = ssl.lib()
    buf = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    p = buf.data_ptr()
    for B, K, V, trunc in [(2048, 16, 151936, False), (256, 3, 151936, True)]:
        assert ssl.ss_verify_workspace_bytes(B, K, V, trunc) > ssl.SCRATCH_BYTES
        rc = L.spec_step_noalloc(p, ssl.DTYPE_F32, B, K, V, p, p, p, p,
                                 p if trunc else None, None, p, 1 << 14,
                                 p, p, p, None, p, p, p, p, None)
        assert rc == ssl.SS_EWORKSPACE
        assert b"scratch" in L.ss_last_error_string()
    # and the largest c3-shaped call it serves
    assert ssl.ss_verify_workspace_bytes(256, 3, 151936) < ssl.SCRATCH_BYTES
