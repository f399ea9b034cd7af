"""Plain CPU oracle for the batched speculative-verify + SAM-draft step.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``sam_drafting_lossless_amd``) never imports it, and this package imports
nothing from the product.

The arithmetic lives in ``oracle.cpp`` (C++17, std::map suffix automaton,
double-precision softmax and scalar rejection sampling); this module only
marshals numpy arrays through ctypes. ``build()`` compiles it with g++.

Pages followed (cited by title and section in ``oracle.cpp``):
  [P1] "SAM投机推理：长序列强化学习训练加速利器", §1.1, §3.1.2
  [P2] m.nxbn.cn speculative-sampling guide, §2.2
  [P3] gogongxt.com notes "投机采样", "贪婪验证，拒绝采样"
  [P4] SAM-Decoding summary (volcengine), §2, §3
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

# Status bits, as the oracle defines them.
ST_TOKEN_RANGE = 1 << 1
ST_DRAFT_LEN = 1 << 2
ST_NONFINITE = 1 << 3
ST_TEMPERATURE = 1 << 4
ST_NO_UNIFORMS = 1 << 5
ST_TOP_P = 1 << 7
ST_TREE = 1 << 8


# A build with AddressSanitizer and UndefinedBehaviorSanitizer, for running
# the oracle's own tests under them (tests/test_oracle_sanitizers.py): loaded
# instead of liboracle.so when ORACLE_SANITIZE=1, in a process that preloads
# the sanitizer runtimes.
_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                  "-fno-omit-frame-pointer", "-g"]


def build(sanitize: bool = False) -> str:
    """Compile oracle.cpp into liboracle.so, or with sanitize into
    liboracle_san.so (always recompiles)."""
    out = _LIB_SAN if sanitize else _LIB
    cmd = ["g++", "-O1" if sanitize else "-O2", "-std=c++17", "-Wall", "-fPIC",
           "-shared", "-pthread", *(SANITIZE_FLAGS if sanitize else []),
           _SRC, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _LIB_SAN if os.environ.get("ORACLE_SANITIZE") == "1" else _LIB
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        build(sanitize=path == _LIB_SAN)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.orc_sam_new.restype = P
    lib.orc_sam_new.argtypes = []
    lib.orc_sam_free.argtypes = [P]
    lib.orc_sam_extend.argtypes = [P, P, i64]
    lib.orc_sam_draft.argtypes = [P, i32, P, P]
    lib.orc_sam_draft.restype = i32
    lib.orc_sam_draft_tree.argtypes = [P, i32, i32, P, P, P]
    lib.orc_sam_draft_tree.restype = i32
    for name in ("orc_sam_num_states", "orc_sam_num_edges", "orc_sam_length"):
        getattr(lib, name).argtypes = [P]
        getattr(lib, name).restype = i64
    for name in ("orc_sam_last_walk_hops", "orc_sam_last"):
        getattr(lib, name).argtypes = [P]
        getattr(lib, name).restype = i32
    lib.orc_sam_export.argtypes = [P, P, P, P, P]
    lib.orc_logprobs.argtypes = [P, i32, i32, i32, i32, P, P, P, P]
    lib.orc_logprobs.restype = None
    lib.orc_sam_match.argtypes = [P, i32, P, P, P, i64, P]
    lib.orc_sam_match.restype = None
    lib.orc_sam_static_draft.argtypes = [P, i32, P, P, i32, P, P]
    lib.orc_sam_static_draft.restype = None
    lib.orc_verify.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P,
                               P, P, P, P, P, P, P, P, P, P, P, i32]
    lib.orc_verify_tree.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P, P,
                                    P, P, P, P, P, i32]
    lib.orc_verify_tree.restype = None
    lib.orc_step.argtypes = [P, i32, i32, i32, P, i32, P, P, P, P, P,
                             P, P, P, P, P, P, P, i32]
    _lib = lib
    return lib


def _logits_arg(logits):
    """(contiguous array, dtype code): float32 is 0, bfloat16 bit patterns
    held as uint16 are 1."""
    if logits.dtype == np.float32:
        dtype = 0
    elif logits.dtype == np.uint16:
        dtype = 1
    else:
        raise TypeError("logits must be float32 or uint16 (bfloat16 bits)")
    return np.ascontiguousarray(logits), dtype


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class SAM:
    """One dynamic suffix automaton over a token history (std::map based)."""

    def __init__(self, tokens=None):
        self._lib = _load()
        self._h = self._lib.orc_sam_new()
        if tokens is not None and len(tokens):
            self.extend(tokens)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.orc_sam_free(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def extend(self, tokens) -> None:
        t = _c(np.atleast_1d(tokens), np.int32)
        self._lib.orc_sam_extend(self._h, _ptr(t), t.size)

    def draft(self, K: int):
        """Returns (draft[K] int32 padded with -1, draft_len, match_len)."""
        out = np.full(K, -1, np.int32)
        ml = np.zeros(1, np.int32)
        d = self._lib.orc_sam_draft(self._h, K, _ptr(out), _ptr(ml))
        return out, int(d), int(ml[0])

    def draft_tree(self, K: int, M: int):
        """Draft tree of up to M candidates of K tokens (see draft_tree in
        oracle.cpp). Returns (tokens [1 + M*K], parent [1 + M*K], n_nodes,
        match_len); entries past n_nodes are -1."""
        N = 1 + M * K
        tok = np.full(N, -1, np.int32)
        par = np.full(N, -1, np.int32)
        ml = np.zeros(1, np.int32)
        n = self._lib.orc_sam_draft_tree(self._h, K, M, _ptr(tok), _ptr(par), _ptr(ml))
        return tok, par, int(n), int(ml[0])

    @property
    def last_walk_hops(self) -> int:
        return int(self._lib.orc_sam_last_walk_hops(self._h))

    @property
    def num_states(self) -> int:
        return int(self._lib.orc_sam_num_states(self._h))

    @property
    def num_edges(self) -> int:
        return int(self._lib.orc_sam_num_edges(self._h))

    @property
    def length(self) -> int:
        return int(self._lib.orc_sam_length(self._h))

    @property
    def last(self) -> int:
        return int(self._lib.orc_sam_last(self._h))

    def export(self):
        """dict(len, link, min_endpos: int32[S]; edges: int32[E,3] sorted by
        (src, token); last)."""
        S, E = self.num_states, self.num_edges
        ln = np.empty(S, np.int32)
        lk = np.empty(S, np.int32)
        me = np.empty(S, np.int32)
        ed = np.empty((E, 3), np.int32)
        self._lib.orc_sam_export(self._h, _ptr(ln), _ptr(lk), _ptr(me), _ptr(ed))
        return {"len": ln, "link": lk, "min_endpos": me, "edges": ed,
                "last": self.last}

    def match(self, state, mlen, tokens, counts=None):
        """Advances match states in this automaton (used as the static
        automaton over a reference text) by tokens [B, L] (counts[b] of them
        per row, all L by default). state, mlen: int32 [B], updated in place
        (start from zeros: the root and an empty match)."""
        t = _c(tokens, np.int32)
        if t.ndim == 1:
            t = t[None, :]
        B, L = t.shape
        c = (np.full(B, L, np.int32) if counts is None
             else _c(counts, np.int32))
        assert state.dtype == np.int32 and mlen.dtype == np.int32
        assert state.flags.c_contiguous and mlen.flags.c_contiguous
        self._lib.orc_sam_match(self._h, B, _ptr(state), _ptr(mlen), _ptr(t), L,
                                _ptr(c))

    def static_draft(self, state, mlen, K: int):
        """Drafts of match states: (draft [B,K] int32, draft_len [B] int32)."""
        st = _c(state, np.int32)
        ml = _c(mlen, np.int32)
        B = st.size
        d = np.empty((B, K), np.int32)
        dl = np.empty(B, np.int32)
        self._lib.orc_sam_static_draft(self._h, B, _ptr(st), _ptr(ml), K, _ptr(d),
                                       _ptr(dl))
        return d, dl


def logprobs(logits, out_tokens, num_emitted, temperature):
    """[B, K+1] float64: log softmax(l_j / T)[out[b, j]] for j < num_emitted
    (T = 1 for greedy sequences), NaN elsewhere."""
    x, dt = _logits_arg(logits)
    B, R, V = x.shape
    out_tokens = np.asarray(out_tokens).reshape(B, R)
    num_emitted = np.asarray(num_emitted).reshape(B)
    temperature = np.asarray(temperature).reshape(B)
    out = _c(out_tokens, np.int32)
    nem = _c(num_emitted, np.int32)
    T = _c(temperature, np.float32)
    lp = np.empty((B, R), np.float64)
    _load().orc_logprobs(_ptr(x), dt, B, R - 1, V, _ptr(out), _ptr(nem), _ptr(T),
                         _ptr(lp))
    return lp


def select_drafts(static_draft, static_len, static_match, dyn_draft, dyn_len,
                  dyn_match, delta: int):
    """[P4] §3, choosing between the automata: the dynamic automaton's draft is
    preferred; the static automaton's draft is used only when its match is
    longer than the dynamic one's by more than delta (> 0). Returns (draft,
    draft_len, source) with source 1 where the static draft was taken."""
    use = np.asarray(static_match) > np.asarray(dyn_match) + delta
    draft = np.where(use[:, None], static_draft, dyn_draft).astype(np.int32)
    dl = np.where(use, static_len, dyn_len).astype(np.int32)
    return draft, dl, use.astype(np.int32)


@dataclass
class VerifyResult:
    out_tokens: np.ndarray   # [B,K+1] int32, -1 padded
    num_emitted: np.ndarray  # [B] int32
    p_draft: np.ndarray      # [B,K] float64, -1 where not computed
    alpha: np.ndarray        # [B,K] float64 min(1,p/q), NaN where unused
    cdf_lo: np.ndarray       # [B] float64 breakpoints around the final draw
    cdf_hi: np.ndarray       # [B]
    status: np.ndarray       # [B] int32
    trunc_thr: np.ndarray | None = None     # [B,K+1] threshold logit per row used
    trunc_margin: np.ndarray | None = None  # [B,K+1] top-p decision margin


def verify(logits, draft, draft_len, temperature, uniforms=None, q=None,
           nthreads: int = 1, top_k=None, top_p=None) -> VerifyResult:
    """Verify one batch.

    logits: [B,K+1,V] float32, or uint16 holding bfloat16 bit patterns.
    draft: [B,K] int32; draft_len: [B] int32; temperature: [B] float32;
    uniforms: [B,K+1] float32 or None; q: [B,K,V] float32 or None (one-hot).
    top_k: [B] int32 or None; top_p: [B] float32 or None (truncation of the
    target distribution at T > 0, see ``truncate`` in oracle.cpp).
    """
    lib = _load()
    logits, dtype = _logits_arg(logits)
    B, R, V = logits.shape
    K = R - 1
    draft = _c(draft, np.int32).reshape(B, K)
    draft_len = _c(draft_len, np.int32).reshape(B)
    temperature = _c(temperature, np.float32).reshape(B)
    if uniforms is not None:
        uniforms = _c(uniforms, np.float32).reshape(B, K + 1)
    if q is not None:
        q = _c(q, np.float32).reshape(B, K, V)
    out = np.full((B, K + 1), -1, np.int32)
    nem = np.zeros(B, np.int32)
    pd = np.empty((B, K), np.float64)
    al = np.empty((B, K), np.float64)
    lo = np.empty(B, np.float64)
    hi = np.empty(B, np.float64)
    st = np.zeros(B, np.int32)
    if top_k is not None:
        top_k = _c(top_k, np.int32).reshape(B)
    if top_p is not None:
        top_p = _c(top_p, np.float32).reshape(B)
    thr = np.empty((B, K + 1), np.float64)
    mg = np.empty((B, K + 1), np.float64)
    lib.orc_verify(_ptr(logits), dtype, B, K, V, _ptr(draft), _ptr(draft_len),
                   _ptr(q), _ptr(temperature), _ptr(uniforms), _ptr(out),
                   _ptr(nem), _ptr(pd), _ptr(al), _ptr(lo), _ptr(hi), _ptr(st),
                   _ptr(top_k), _ptr(top_p), _ptr(thr), _ptr(mg), int(nthreads))
    return VerifyResult(out, nem, pd, al, lo, hi, st, thr, mg)


@dataclass
class TreeResult:
    out_tokens: np.ndarray   # [B,N] int32, -1 padded
    out_nodes: np.ndarray    # [B,N] int32: node of each emitted token
    num_emitted: np.ndarray  # [B] int32
    gap: np.ndarray          # [B,N] float64: |u[t] - running sums| minimum
    cdf_lo: np.ndarray       # [B]
    cdf_hi: np.ndarray       # [B]
    status: np.ndarray       # [B] int32


def verify_tree(logits, tokens, parent, n_nodes, temperature, uniforms=None,
                nthreads: int = 1) -> TreeResult:
    """Verify a draft tree per sequence (see verify_tree_one in oracle.cpp).

    logits: [B,N,V] float32 or uint16 (bfloat16 bits); tokens, parent: [B,N]
    int32 (parent[b,0] = -1); n_nodes: [B]; uniforms: [B,N] (coins per depth,
    the last column the final coin)."""
    x, dt = _logits_arg(logits)
    B, N, V = x.shape
    tokens = _c(tokens, np.int32).reshape(B, N)
    parent = _c(parent, np.int32).reshape(B, N)
    n_nodes = _c(n_nodes, np.int32).reshape(B)
    temperature = _c(temperature, np.float32).reshape(B)
    if uniforms is not None:
        uniforms = _c(uniforms, np.float32).reshape(B, N)
    out = np.full((B, N), -1, np.int32)
    onode = np.full((B, N), -1, np.int32)
    nem = np.zeros(B, np.int32)
    gap = np.empty((B, N), np.float64)
    lo = np.empty(B, np.float64)
    hi = np.empty(B, np.float64)
    st = np.zeros(B, np.int32)
    _load().orc_verify_tree(_ptr(x), dt, B, N, V, _ptr(tokens), _ptr(parent),
                            _ptr(n_nodes), _ptr(temperature), _ptr(uniforms),
                            _ptr(out), _ptr(onode), _ptr(nem), _ptr(gap), _ptr(lo),
                            _ptr(hi), _ptr(st), int(nthreads))
    return TreeResult(out, onode, nem, gap, lo, hi, st)


def step(sams, logits, temperature, uniforms, nthreads: int = 1):
    """One whole oracle step over a batch of SAM objects: draft, verify,
    extend. Returns (draft, draft_len, match_len, VerifyResult)."""
    lib = _load()
    logits = np.ascontiguousarray(logits)
    dtype = 0 if logits.dtype == np.float32 else 1
    B, R, V = logits.shape
    K = R - 1
    handles = (ctypes.c_void_p * B)(*[s.handle for s in sams])
    temperature = _c(temperature, np.float32).reshape(B)
    if uniforms is not None:
        uniforms = _c(uniforms, np.float32).reshape(B, K + 1)
    dr = np.full((B, K), -1, np.int32)
    dl = np.zeros(B, np.int32)
    ml = np.zeros(B, np.int32)
    out = np.full((B, K + 1), -1, np.int32)
    nem = np.zeros(B, np.int32)
    pd = np.empty((B, K), np.float64)
    al = np.empty((B, K), np.float64)
    lo = np.empty(B, np.float64)
    hi = np.empty(B, np.float64)
    st = np.zeros(B, np.int32)
    lib.orc_step(ctypes.cast(handles, ctypes.c_void_p), B, K, V, _ptr(logits),
                 dtype, _ptr(temperature), _ptr(uniforms), _ptr(dr), _ptr(dl),
                 _ptr(ml), _ptr(out), _ptr(nem), _ptr(pd), _ptr(al), _ptr(lo),
                 _ptr(hi), _ptr(st), int(nthreads))
    return dr, dl, ml, VerifyResult(out, nem, pd, al, lo, hi, st)
