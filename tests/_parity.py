"""Comparison of the HIP path against the oracle, shared by the GPU tests.

Bars:
  * greedy (T = 0) outputs, drafts, automaton structure: bit-exact;
  * T > 0 accept / resample decisions: equal, except where the uniform lies
    within TIE = 1e-6 of the oracle's acceptance threshold alpha_j or of a
    normalised CDF breakpoint of its draw (such cases are counted);
  * probabilities: within 1e-5 relative of the double-precision oracle, or
    within float32's smallest normal (2^-126) absolute: the device writes
    float32 and flushes smaller values to 0.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TIE = 1e-6
P_RTOL = 1e-5
P_ATOL = float(np.finfo(np.float32).tiny)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_host_logits(x: torch.Tensor) -> np.ndarray:
    """Exact host copy of device logits (bf16 as uint16 bit patterns)."""
    if x.dtype == torch.bfloat16:
        return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return x.contiguous().cpu().numpy()


def dev(a, dtype=None):
    if a is None:
        return None
    t = torch.as_tensor(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


class Tally:
    def __init__(self):
        self.ties = 0
        self.decisions = 0

    def __repr__(self):
        return f"ties={self.ties} / decisions={self.decisions}"


def compare_verify(g_out, g_nem, g_pd, g_st, r: oracle.VerifyResult, T, u,
                   tally: Tally | None = None, what: str = ""):
    """Asserts GPU verify outputs match the oracle's. Returns the per-sequence
    mask of tie-tolerated mismatches."""
    g_out = np.asarray(g_out)
    g_nem = np.asarray(g_nem)
    g_pd = np.asarray(g_pd)
    g_st = np.asarray(g_st)
    T = np.asarray(T)
    B = g_out.shape[0]
    K = g_out.shape[1] - 1
    np.testing.assert_array_equal(g_st, r.status, err_msg=f"{what} status")
    tied = np.zeros(B, bool)
    for b in range(B):
        if r.status[b]:
            continue
        if tally is not None:
            tally.decisions += int(r.num_emitted[b])
        same = (g_nem[b] == r.num_emitted[b] and
                (g_out[b] == r.out_tokens[b]).all())
        if T[b] == 0.0:
            assert same, (f"{what} greedy mismatch b={b}: gpu {g_out[b]} "
                          f"nem {g_nem[b]} oracle {r.out_tokens[b]} nem "
                          f"{r.num_emitted[b]}")
            assert (g_pd[b] == -1).all()
            continue
        if not same:
            ag, ao = int(g_nem[b]) - 1, int(r.num_emitted[b]) - 1
            if ag != ao:
                j = min(ag, ao)
                gap = abs(float(u[b, j]) - r.alpha[b, j])
                assert gap <= TIE, (f"{what} accept mismatch b={b} j={j}: "
                                    f"u={u[b, j]!r} alpha={r.alpha[b, j]!r}")
            else:
                gap = min(abs(float(u[b, K]) - r.cdf_lo[b]),
                          abs(float(u[b, K]) - r.cdf_hi[b]))
                assert gap <= TIE, (f"{what} draw mismatch b={b}: gpu "
                                    f"{g_out[b]} oracle {r.out_tokens[b]} "
                                    f"u={u[b, K]!r} cdf=({r.cdf_lo[b]!r}, "
                                    f"{r.cdf_hi[b]!r})")
            tied[b] = True
            if tally is not None:
                tally.ties += 1
            continue
        m = r.p_draft[b] >= 0
        np.testing.assert_array_equal(g_pd[b] >= 0, m,
                                      err_msg=f"{what} p_draft mask b={b}")
        if m.any():
            np.testing.assert_allclose(g_pd[b][m], r.p_draft[b][m], rtol=P_RTOL,
                                       atol=P_ATOL, err_msg=f"{what} p_draft b={b}")
    return tied
