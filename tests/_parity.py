"""Comparison of the HIP path against the oracle, shared by the GPU tests.

Bars:
  * greedy (T = 0) outputs, drafts, automaton structure: bit-exact;
  * T > 0 accept / resample decisions: equal, except where the uniform lies
    within TIE = 1e-6 of the oracle's acceptance threshold alpha_j or of a
    normalised CDF breakpoint of its draw, at the decision where the two
    paths part (such cases are counted);
  * the excused cases are bounded: at most TIE_BUDGET of the decisions
    (TIE_FLOOR at least, for small tests), and the largest excused distance
    |u - threshold| is recorded and must stay below GAP_BOUND = 1e-7, under
    one float32 ulp at 1. The device's weights are float32 terms (exp2 of a
    float32 argument) summed in float32 partials per 32 KiB chunk, while the
    running sums and the target u * total of its draw are taken in double;
    so a normalised breakpoint it computes is off from the double-precision
    one by float32 roundings of the terms and partials (unit roundoff 6e-8
    relative, averaging out over many terms). A mismatch whose coin is
    farther than that from the oracle's threshold is a real difference. At
    V ~ 1.5e5 a breakpoint error e gives mismatches at a rate of about
    2 e V per draw, so the count budget and the gap bound together hold a
    bias of the draw to the 1e-8 scale;
  * truncation: a sequence whose top-p decision the oracle found within its
    margin of flipping is set aside before the comparison (counted, at most
    SET_ASIDE_BUDGET of the sequences, TIE_FLOOR at least);
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
TIE_BUDGET = 0.01
TIE_FLOOR = 2
GAP_BOUND = 1e-7
SET_ASIDE_BUDGET = 0.05
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
    """Counts T > 0 decisions and the excused mismatches among them."""

    def __init__(self):
        self.ties = 0
        self.decisions = 0
        self.gaps: list[float] = []
        # truncated sequences whose top-p decision the oracle found within
        # its margin of flipping, set aside before the comparison
        self.set_aside = 0
        self.sequences = 0

    def excuse(self, gap: float) -> None:
        self.ties += 1
        self.gaps.append(float(gap))

    @property
    def max_gap(self) -> float:
        return max(self.gaps, default=0.0)

    def check(self, what: str = "") -> None:
        """Asserts the excused mismatches stay within the budget and at the
        rounding scale; prints the tally."""
        say(f"    {what} {self!r}")
        budget = max(TIE_FLOOR, TIE_BUDGET * self.decisions)
        assert self.ties <= budget, f"{what}: {self!r} exceeds {budget:.1f}"
        assert self.max_gap <= GAP_BOUND, f"{what}: {self!r}"
        assert self.set_aside <= max(TIE_FLOOR, SET_ASIDE_BUDGET * self.sequences), \
            f"{what}: {self!r}"

    def __repr__(self):
        g = ", ".join(f"{x:.2e}" for x in sorted(self.gaps)[-4:])
        r = (f"ties={self.ties} / decisions={self.decisions} "
             f"max_gap={self.max_gap:.2e} [{g}]")
        if self.sequences:
            r += f" set_aside={self.set_aside} / sequences={self.sequences}"
        return r


def compare_verify(g_out, g_nem, g_pd, g_st, r: oracle.VerifyResult, T, u,
                   tally: Tally | None = None, what: str = ""):
    """Asserts GPU verify outputs match the oracle's. Returns the per-sequence
    mask of tie-tolerated mismatches. Without a tally the call's own excused
    cases are checked against the budget here; a caller that passes one
    checks it once its test is done."""
    own = tally is None
    if own:
        tally = Tally()
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
        same = (g_nem[b] == r.num_emitted[b] and
                (g_out[b] == r.out_tokens[b]).all())
        if T[b] != 0.0:
            tally.decisions += int(r.num_emitted[b])
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
            tally.excuse(gap)
            continue
        m = r.p_draft[b] >= 0
        np.testing.assert_array_equal(g_pd[b] >= 0, m,
                                      err_msg=f"{what} p_draft mask b={b}")
        if m.any():
            np.testing.assert_allclose(g_pd[b][m], r.p_draft[b][m], rtol=P_RTOL,
                                       atol=P_ATOL, err_msg=f"{what} p_draft b={b}")
    if own:
        tally.check(what)
    return tied


def compare_tree(g, r: oracle.TreeResult, T, u, tally: Tally | None = None,
                 what: str = ""):
    """Asserts GPU tree verification outputs (tokens, nodes, counts, status)
    match the oracle's. A T > 0 mismatch is excused only by the decision at
    which the two paths part: t = the first emitted position where tokens or
    nodes differ. If both paths end there with the final draw from the same
    node, the final coin must lie within TIE of a breakpoint of the oracle's
    draw; otherwise the coin of depth t must lie within TIE of one of the
    oracle's running sums at depth t (on the shared path up to t, the node
    whose children are tried is the same on both sides)."""
    out, nodes, nem, st = (np.asarray(a) for a in g)
    np.testing.assert_array_equal(st, r.status, err_msg=f"{what} status")
    own = tally is None
    if own:
        tally = Tally()
    for b in range(len(T)):
        if r.status[b]:
            continue
        same = (nem[b] == r.num_emitted[b] and (out[b] == r.out_tokens[b]).all()
                and (nodes[b] == r.out_nodes[b]).all())
        if T[b] == 0.0:
            assert same, (what, b, out[b], r.out_tokens[b], nodes[b], r.out_nodes[b])
            continue
        tally.decisions += int(r.num_emitted[b])
        if same:
            continue
        diff = (out[b] != r.out_tokens[b]) | (nodes[b] != r.out_nodes[b])
        t = int(np.flatnonzero(diff)[0])
        both_final = (t == nem[b] - 1 and t == r.num_emitted[b] - 1
                      and nodes[b, t] == r.out_nodes[b, t])
        if both_final:
            fc = float(u[b, -1])
            gap = min(abs(fc - r.cdf_lo[b]), abs(fc - r.cdf_hi[b]))
        else:
            gap = float(r.gap[b, t])
        assert gap <= TIE, (f"{what} b={b} parts at depth {t} "
                            f"({'final draw' if both_final else 'coin'}) "
                            f"gap={gap!r}: gpu {out[b]} {nodes[b]} oracle "
                            f"{r.out_tokens[b]} {r.out_nodes[b]}")
        tally.excuse(gap)
    if own:
        tally.check(what)
    return tally
