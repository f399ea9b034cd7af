"""Python binding of the MI355X speculative-verify + SAM-draft library.

Thin ctypes marshalling over ``libspecsam.so`` (C ABI in ``include/specsam.h``):
every step of the path runs in the library's HIP kernels; PyTorch provides
device memory and the stream. The names follow the C entry points:
``spec_verify``, ``sam_state_bytes``, ``sam_init``, ``sam_extend``,
``sam_draft``, ``sam_status``, ``sam_export``, ``ss_verify_workspace_bytes``.

The library must be built (``python -m sam_drafting_lossless_amd.build`` or
``__graft_entry__.build()``); importing works without it, but every call
raises if it is missing. There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so the library shares torch's HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecsam.so")

SS_OK, SS_EINVAL, SS_EWORKSPACE, SS_ELAUNCH = 0, -1, -2, -3
ST_SAM_CAPACITY = 1 << 0
ST_TOKEN_RANGE = 1 << 1
ST_DRAFT_LEN = 1 << 2
ST_NONFINITE = 1 << 3
ST_TEMPERATURE = 1 << 4
ST_NO_UNIFORMS = 1 << 5
ST_COUNT = 1 << 6
ST_TOP_P = 1 << 7
ST_TREE = 1 << 8
MAX_TREE = 64
MAX_K = 16
DTYPE_F32, DTYPE_BF16 = 0, 1

_lib = None


class SpecSamError(RuntimeError):
    pass


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise SpecSamError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m sam_drafting_lossless_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.ss_version.restype = i32
    L.ss_last_error_string.restype = ctypes.c_char_p
    L.ss_verify_workspace_bytes.argtypes = [i32, i32, i32]
    L.ss_verify_workspace_bytes.restype = sz
    L.ss_verify_workspace_bytes_ex.argtypes = [i32, i32, i32, i32]
    L.ss_verify_workspace_bytes_ex.restype = sz
    L.spec_verify.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P,
                              P, P, P, P, sz, P]
    L.spec_verify.restype = i32
    L.spec_step.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P, P, i32, P,
                            P, P, P, P, P, P, P, P, sz, P]
    L.spec_step.restype = i32
    L.spec_step_noalloc.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P, P, i32,
                                    P, P, P, P, P, P, P, P, P]
    L.spec_step_noalloc.restype = i32
    L.spec_stream.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P, P, sz, P]
    L.spec_stream.restype = i32
    L.spec_finish.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P,
                              P, P, P, P, i32, P, P, P, P, sz, P]
    L.spec_finish.restype = i32
    L.ss_tree_workspace_bytes.argtypes = [i32, i32, i32]
    L.ss_tree_workspace_bytes.restype = sz
    L.spec_verify_tree.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P,
                                   P, sz, P]
    L.spec_verify_tree.restype = i32
    L.sam_extend_draft.argtypes = [P, i32, i32, P, i32, P, i32, P, P, P, P]
    L.sam_extend_draft.restype = i32
    L.sam_state_bytes.argtypes = [i32, i32]
    L.sam_state_bytes.restype = sz
    L.sam_hash_slots.argtypes = [i32]
    L.sam_hash_slots.restype = i32
    L.sam_init.argtypes = [P, i32, i32, i32, P]
    L.sam_init.restype = i32
    L.sam_extend.argtypes = [P, i32, i32, P, i32, P, P]
    L.sam_extend.restype = i32
    L.sam_draft.argtypes = [P, i32, i32, i32, P, P, P, P]
    L.sam_draft.restype = i32
    L.sam_draft_tree.argtypes = [P, i32, i32, i32, i32, i32, P, P, P, P, P]
    L.sam_draft_tree.restype = i32
    L.sam_extend_stats.argtypes = [P, i32, i32, P, i32, P, P, P]
    L.sam_extend_stats.restype = i32
    L.sam_match.argtypes = [P, i32, i32, P, P, i32, P, i32, i32, P, P, P, P, P,
                            P, P, P]
    L.sam_match.restype = i32
    L.sam_status.argtypes = [P, i32, i32, P, P]
    L.sam_status.restype = i32
    L.sam_export.argtypes = [P, i32, i32, i32, P, P, P, P, P]
    L.sam_export.restype = i32
    _lib = L
    return L


def _check(rc: int, what: str) -> None:
    if rc != SS_OK:
        msg = lib().ss_last_error_string().decode(errors="replace")
        raise SpecSamError(f"{what} failed with code {rc}: {msg}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise SpecSamError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise SpecSamError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise SpecSamError(f"{name} must have shape {tuple(shape)}, got "
                           f"{tuple(t.shape)}")
    if not t.is_contiguous():
        raise SpecSamError(f"{name} must be contiguous")
    return t.data_ptr()


def _opt_f32(t, name, shape):
    return None if t is None else _dev(t, name, torch.float32, shape)


def _trunc_args(top_k, top_p, B):
    return (None if top_k is None else _dev(top_k, "top_k", torch.int32, (B,)),
            _opt_f32(top_p, "top_p", (B,)))


# ------------------------------------------------------------- verification --
WS_TRUNCATION = 1


def ss_verify_workspace_bytes(B: int, K: int, V: int, truncation: bool = False) -> int:
    return int(lib().ss_verify_workspace_bytes_ex(B, K, V,
                                                  WS_TRUNCATION if truncation else 0))


def verify_workspace(B: int, K: int, V: int, device=None, truncation: bool = False):
    """A workspace tensor (uint8) for spec_verify / spec_step calls of this
    size (or smaller); it needs no initialisation. `truncation`: room for
    calls that pass top_k / top_p."""
    n = ss_verify_workspace_bytes(B, K, V, truncation)
    if n == 0:
        raise SpecSamError(f"unsupported sizes B={B} K={K} V={V}")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def spec_verify(logits, draft, draft_len, temperature, uniforms=None, q=None, *,
                top_k=None, top_p=None, workspace=None, out_tokens=None,
                num_emitted=None, p_draft=None, status=None, logprobs=None,
                stream=None):
    """Verify one batch (see include/specsam.h). Returns
    (out_tokens [B,K+1] int32, num_emitted [B] int32, p_draft [B,K] float32,
    status [B] int32). `logprobs`, a [B,K+1] float32 tensor, receives the
    log-probabilities of the emitted tokens when given. `top_k` ([B] int32)
    and `top_p` ([B] float32) truncate the target at T > 0."""
    if logits.dim() != 3:
        raise SpecSamError("logits must be [B, K+1, V]")
    B, R, V = logits.shape
    K = R - 1
    if logits.dtype == torch.float32:
        dt = DTYPE_F32
    elif logits.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    else:
        raise SpecSamError("logits must be float32 or bfloat16")
    dev = logits.device
    i32 = torch.int32
    trunc = top_k is not None or top_p is not None
    if workspace is None:
        workspace = verify_workspace(B, K, V, dev, truncation=trunc)
    if out_tokens is None:
        out_tokens = torch.empty((B, R), dtype=i32, device=dev)
    if num_emitted is None:
        num_emitted = torch.empty(B, dtype=i32, device=dev)
    if p_draft is None:
        p_draft = torch.empty((B, K), dtype=torch.float32, device=dev)
    if status is None:
        status = torch.zeros(B, dtype=i32, device=dev)
    args = (
        _dev(logits, "logits"), dt, B, K, V,
        _dev(draft, "draft", i32, (B, K)),
        _dev(draft_len, "draft_len", i32, (B,)),
        None if q is None else _dev(q, "q", torch.float32, (B, K, V)),
        _dev(temperature, "temperature", torch.float32, (B,)),
        None if uniforms is None else _dev(uniforms, "uniforms", torch.float32,
                                           (B, R)),
        *_trunc_args(top_k, top_p, B),
        _dev(out_tokens, "out_tokens", i32, (B, R)),
        _dev(num_emitted, "num_emitted", i32, (B,)),
        _dev(p_draft, "p_draft", torch.float32, (B, K)),
        _opt_f32(logprobs, "logprobs", (B, R)),
        _dev(status, "status", i32, (B,)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream))
    _check(lib().spec_verify(*args), "spec_verify")
    return out_tokens, num_emitted, p_draft, status


def spec_step(logits, draft, draft_len, temperature, uniforms, state, *,
              workspace=None, out_tokens=None, num_emitted=None, p_draft=None,
              status=None, next_draft=None, next_draft_len=None,
              next_match_len=None, logprobs=None, top_k=None, top_p=None,
              stream=None):
    """One fused step (see include/specsam.h): verify the drafts, extend each
    automaton of `state` (a SamState) with the emitted tokens, and draft for
    the next step. Returns (out_tokens, num_emitted, p_draft, status,
    next_draft, next_draft_len, next_match_len); `logprobs` as spec_verify."""
    return _step(False, logits, draft, draft_len, temperature, uniforms, state,
                 workspace, out_tokens, num_emitted, p_draft, status, next_draft,
                 next_draft_len, next_match_len, logprobs, top_k, top_p, stream)


def spec_step_noalloc(logits, draft, draft_len, temperature, uniforms, state, *,
                      out_tokens=None, num_emitted=None, p_draft=None,
                      status=None, next_draft=None, next_draft_len=None,
                      next_match_len=None, logprobs=None, top_k=None, top_p=None,
                      stream=None):
    """spec_step with the library's own device scratch as its workspace (see
    include/specsam.h): the C call allocates nothing. Outputs that are not
    given are allocated here, as for spec_step; pass them all to allocate
    nothing at all. Calls that overlap on one GPU race."""
    return _step(True, logits, draft, draft_len, temperature, uniforms, state,
                 None, out_tokens, num_emitted, p_draft, status, next_draft,
                 next_draft_len, next_match_len, logprobs, top_k, top_p, stream)


SCRATCH_BYTES = 8 << 20  # SS_SCRATCH_BYTES


def _step(noalloc, logits, draft, draft_len, temperature, uniforms, state,
          workspace, out_tokens, num_emitted, p_draft, status, next_draft,
          next_draft_len, next_match_len, logprobs, top_k, top_p, stream):
    if logits.dim() != 3:
        raise SpecSamError("logits must be [B, K+1, V]")
    B, R, V = logits.shape
    K = R - 1
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}.get(logits.dtype)
    if dt is None:
        raise SpecSamError("logits must be float32 or bfloat16")
    if state.B != B:
        raise SpecSamError("state holds a different number of sequences")
    dev = logits.device
    i32 = torch.int32
    if workspace is None and not noalloc:
        workspace = verify_workspace(B, K, V, dev, truncation=(
            top_k is not None or top_p is not None))
    if out_tokens is None:
        out_tokens = torch.empty((B, R), dtype=i32, device=dev)
    if num_emitted is None:
        num_emitted = torch.empty(B, dtype=i32, device=dev)
    if p_draft is None:
        p_draft = torch.empty((B, K), dtype=torch.float32, device=dev)
    if status is None:
        status = torch.zeros(B, dtype=i32, device=dev)
    if next_draft is None:
        next_draft = torch.empty((B, K), dtype=i32, device=dev)
    if next_draft_len is None:
        next_draft_len = torch.empty(B, dtype=i32, device=dev)
    if next_match_len is None:
        next_match_len = torch.empty(B, dtype=i32, device=dev)
    args = (
        _dev(logits, "logits"), dt, B, K, V,
        _dev(draft, "draft", i32, (B, K)),
        _dev(draft_len, "draft_len", i32, (B,)),
        _dev(temperature, "temperature", torch.float32, (B,)),
        None if uniforms is None else _dev(uniforms, "uniforms", torch.float32,
                                           (B, R)),
        *_trunc_args(top_k, top_p, B),
        _dev(state.buf, "state", torch.uint8), state.max_len,
        _dev(out_tokens, "out_tokens", i32, (B, R)),
        _dev(num_emitted, "num_emitted", i32, (B,)),
        _dev(p_draft, "p_draft", torch.float32, (B, K)),
        _opt_f32(logprobs, "logprobs", (B, R)),
        _dev(status, "status", i32, (B,)),
        _dev(next_draft, "next_draft", i32, (B, K)),
        _dev(next_draft_len, "next_draft_len", i32, (B,)),
        _dev(next_match_len, "next_match_len", i32, (B,)))
    if noalloc:
        _check(lib().spec_step_noalloc(*args, _stream(stream)), "spec_step_noalloc")
    else:
        _check(lib().spec_step(*args, _dev(workspace, "workspace", torch.uint8),
                               workspace.numel(), _stream(stream)), "spec_step")
    return (out_tokens, num_emitted, p_draft, status, next_draft,
            next_draft_len, next_match_len)


def tree_workspace(B: int, N: int, V: int, device=None):
    """A workspace tensor for spec_verify_tree calls of this size."""
    n = int(lib().ss_tree_workspace_bytes(B, N, V))
    if n == 0:
        raise SpecSamError(f"unsupported sizes B={B} N={N} V={V}")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def spec_verify_tree(logits, tokens, parent, n_nodes, temperature, uniforms=None, *,
                     workspace=None, out_tokens=None, out_nodes=None,
                     num_emitted=None, status=None, stream=None):
    """Verify one draft tree per sequence (see include/specsam.h). Returns
    (out_tokens [B,N] int32, out_nodes [B,N] int32, num_emitted [B] int32,
    status [B] int32)."""
    if logits.dim() != 3:
        raise SpecSamError("logits must be [B, N, V]")
    B, N, V = logits.shape
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}.get(logits.dtype)
    if dt is None:
        raise SpecSamError("logits must be float32 or bfloat16")
    dev = logits.device
    i32 = torch.int32
    if workspace is None:
        workspace = tree_workspace(B, N, V, dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, N), dtype=i32, device=dev)
    if out_nodes is None:
        out_nodes = torch.empty((B, N), dtype=i32, device=dev)
    if num_emitted is None:
        num_emitted = torch.empty(B, dtype=i32, device=dev)
    if status is None:
        status = torch.zeros(B, dtype=i32, device=dev)
    _check(lib().spec_verify_tree(
        _dev(logits, "logits"), dt, B, N, V,
        _dev(tokens, "tokens", i32, (B, N)),
        _dev(parent, "parent", i32, (B, N)),
        _dev(n_nodes, "n_nodes", i32, (B,)),
        _dev(temperature, "temperature", torch.float32, (B,)),
        _opt_f32(uniforms, "uniforms", (B, N)),
        _dev(out_tokens, "out_tokens", i32, (B, N)),
        _dev(out_nodes, "out_nodes", i32, (B, N)),
        _dev(num_emitted, "num_emitted", i32, (B,)),
        _dev(status, "status", i32, (B,)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream)), "spec_verify_tree")
    return out_tokens, out_nodes, num_emitted, status


def _shape(logits):
    if logits.dim() != 3:
        raise SpecSamError("logits must be [B, K+1, V]")
    B, R, V = logits.shape
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}.get(logits.dtype)
    if dt is None:
        raise SpecSamError("logits must be float32 or bfloat16")
    return B, R - 1, V, dt


def spec_stream(logits, draft, draft_len, temperature, uniforms, workspace, *,
                top_k=None, top_p=None, stream=None):
    """First pass of a verification (see include/specsam.h): read the logit
    rows once and leave per-row statistics in `workspace`."""
    B, K, V, dt = _shape(logits)
    i32 = torch.int32
    _check(lib().spec_stream(
        _dev(logits, "logits"), dt, B, K, V,
        _dev(draft, "draft", i32, (B, K)),
        _dev(draft_len, "draft_len", i32, (B,)),
        _dev(temperature, "temperature", torch.float32, (B,)),
        None if uniforms is None else _dev(uniforms, "uniforms", torch.float32,
                                           (B, K + 1)),
        *_trunc_args(top_k, top_p, B),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream)), "spec_stream")


def spec_finish(logits, draft, draft_len, temperature, uniforms, workspace,
                q=None, state=None, *, out_tokens=None, num_emitted=None,
                p_draft=None, status=None, next_draft=None, next_draft_len=None,
                next_match_len=None, logprobs=None, top_k=None, top_p=None,
                stream=None):
    """Second pass (see include/specsam.h), after spec_stream with the same
    arguments and workspace. Returns (out_tokens, num_emitted, p_draft,
    status), followed by (next_draft, next_draft_len, next_match_len) when
    `state` (a SamState) is given; `logprobs` as spec_verify."""
    B, K, V, dt = _shape(logits)
    R = K + 1
    dev = logits.device
    i32 = torch.int32
    if out_tokens is None:
        out_tokens = torch.empty((B, R), dtype=i32, device=dev)
    if num_emitted is None:
        num_emitted = torch.empty(B, dtype=i32, device=dev)
    if p_draft is None:
        p_draft = torch.empty((B, K), dtype=torch.float32, device=dev)
    if status is None:
        status = torch.zeros(B, dtype=i32, device=dev)
    if state is not None:
        if state.B != B:
            raise SpecSamError("state holds a different number of sequences")
        if next_draft is None:
            next_draft = torch.empty((B, K), dtype=i32, device=dev)
        if next_draft_len is None:
            next_draft_len = torch.empty(B, dtype=i32, device=dev)
        if next_match_len is None:
            next_match_len = torch.empty(B, dtype=i32, device=dev)
    opt = lambda t, name, shape: None if t is None else _dev(t, name, i32, shape)
    _check(lib().spec_finish(
        _dev(logits, "logits"), dt, B, K, V,
        _dev(draft, "draft", i32, (B, K)),
        _dev(draft_len, "draft_len", i32, (B,)),
        None if q is None else _dev(q, "q", torch.float32, (B, K, V)),
        _dev(temperature, "temperature", torch.float32, (B,)),
        None if uniforms is None else _dev(uniforms, "uniforms", torch.float32,
                                           (B, R)),
        *_trunc_args(top_k, top_p, B),
        _dev(out_tokens, "out_tokens", i32, (B, R)),
        _dev(num_emitted, "num_emitted", i32, (B,)),
        _dev(p_draft, "p_draft", torch.float32, (B, K)),
        _opt_f32(logprobs, "logprobs", (B, R)),
        _dev(status, "status", i32, (B,)),
        None if state is None else _dev(state.buf, "state", torch.uint8),
        0 if state is None else state.max_len,
        opt(next_draft, "next_draft", (B, K)),
        opt(next_draft_len, "next_draft_len", (B,)),
        opt(next_match_len, "next_match_len", (B,)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream)), "spec_finish")
    res = (out_tokens, num_emitted, p_draft, status)
    if state is not None:
        res += (next_draft, next_draft_len, next_match_len)
    return res


# ------------------------------------------------------- suffix automaton ----
def sam_state_bytes(B: int, max_len: int) -> int:
    return int(lib().sam_state_bytes(B, max_len))


def sam_hash_slots(max_len: int) -> int:
    return int(lib().sam_hash_slots(max_len))


def sam_init(state, B: int, max_len: int, V: int, stream=None) -> None:
    _check(lib().sam_init(_dev(state, "state", torch.uint8), B, max_len, V,
                          _stream(stream)), "sam_init")


def sam_extend(state, B: int, max_len: int, tokens, counts, stream=None) -> None:
    if tokens.dim() != 2 or tokens.shape[0] != B:
        raise SpecSamError("tokens must be [B, ld]")
    _check(lib().sam_extend(_dev(state, "state", torch.uint8), B, max_len,
                            _dev(tokens, "tokens", torch.int32),
                            int(tokens.shape[1]),
                            _dev(counts, "counts", torch.int32, (B,)),
                            _stream(stream)), "sam_extend")


def sam_draft(state, B: int, max_len: int, K: int, draft=None, draft_len=None,
              match_len=None, stream=None):
    dev = state.device
    if draft is None:
        draft = torch.empty((B, K), dtype=torch.int32, device=dev)
    if draft_len is None:
        draft_len = torch.empty(B, dtype=torch.int32, device=dev)
    if match_len is None:
        match_len = torch.empty(B, dtype=torch.int32, device=dev)
    _check(lib().sam_draft(_dev(state, "state", torch.uint8), B, max_len, K,
                           _dev(draft, "draft", torch.int32, (B, K)),
                           _dev(draft_len, "draft_len", torch.int32, (B,)),
                           _dev(match_len, "match_len", torch.int32, (B,)),
                           _stream(stream)), "sam_draft")
    return draft, draft_len, match_len


def sam_extend_draft(state, B: int, max_len: int, tokens, counts, K: int,
                     draft=None, draft_len=None, match_len=None, stream=None):
    dev = state.device
    if tokens.dim() != 2 or tokens.shape[0] != B:
        raise SpecSamError("tokens must be [B, ld]")
    if draft is None:
        draft = torch.empty((B, K), dtype=torch.int32, device=dev)
    if draft_len is None:
        draft_len = torch.empty(B, dtype=torch.int32, device=dev)
    if match_len is None:
        match_len = torch.empty(B, dtype=torch.int32, device=dev)
    _check(lib().sam_extend_draft(
        _dev(state, "state", torch.uint8), B, max_len,
        _dev(tokens, "tokens", torch.int32), int(tokens.shape[1]),
        _dev(counts, "counts", torch.int32, (B,)), K,
        _dev(draft, "draft", torch.int32, (B, K)),
        _dev(draft_len, "draft_len", torch.int32, (B,)),
        _dev(match_len, "match_len", torch.int32, (B,)), _stream(stream)),
        "sam_extend_draft")
    return draft, draft_len, match_len


SAM_STATS = ("tokens", "probes", "buckets", "walk_steps", "clones",
             "copied", "redirects")


def sam_extend_stats(state, B: int, max_len: int, tokens, counts, stats=None,
                     stream=None):
    """sam_extend with work counters; returns the uint64 stats tensor [7]
    (accumulated into `stats` if given)."""
    if stats is None:
        stats = torch.zeros(len(SAM_STATS), dtype=torch.int64, device=state.device)
    if tokens.dim() != 2 or tokens.shape[0] != B:
        raise SpecSamError("tokens must be [B, ld]")
    _check(lib().sam_extend_stats(
        _dev(state, "state", torch.uint8), B, max_len,
        _dev(tokens, "tokens", torch.int32), int(tokens.shape[1]),
        _dev(counts, "counts", torch.int32, (B,)),
        _dev(stats, "stats", torch.int64, (len(SAM_STATS),)), _stream(stream)),
        "sam_extend_stats")
    return stats


def sam_status(state, B: int, max_len: int, out=None, stream=None):
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=state.device)
    _check(lib().sam_status(_dev(state, "state", torch.uint8), B, max_len,
                            _dev(out, "status_out", torch.int32, (B,)),
                            _stream(stream)), "sam_status")
    return out


def sam_export(state, B: int, max_len: int, b: int, stream=None):
    """Sequence b's automaton as host numpy arrays: dict(n, last, num_states,
    num_edges, status, len, link, min_endpos, first_edge, edges [E,3] sorted
    by (src, token), text, slots [hash_slots,4] = the raw table rows (src,
    token, dst, next)). Synchronises the stream."""
    dev = state.device
    H = sam_hash_slots(max_len)
    hdr = torch.empty(8, dtype=torch.int32, device=dev)
    st = torch.empty((2 * max_len, 4), dtype=torch.int32, device=dev)
    ed = torch.empty((H, 4), dtype=torch.int32, device=dev)
    tx = torch.empty(max_len, dtype=torch.int32, device=dev)
    _check(lib().sam_export(_dev(state, "state", torch.uint8), B, max_len, b,
                            hdr.data_ptr(), st.data_ptr(), ed.data_ptr(),
                            tx.data_ptr(), _stream(stream)), "sam_export")
    torch.cuda.synchronize(dev)
    h = hdr.cpu().numpy()
    n, last, S, E, status = (int(v) for v in h[:5])
    st = st[:S].cpu().numpy()
    ed = ed.cpu().numpy()
    slots = ed.copy()
    ed = ed[ed[:, 0] >= 0][:, :3]
    order = (ed[:, 0].astype("int64") << 32) | ed[:, 1].astype("int64")
    ed = ed[order.argsort(kind="stable")]
    return {"n": n, "last": last, "num_states": S, "num_edges": E,
            "status": status, "len": st[:, 0].copy(), "link": st[:, 1].copy(),
            "min_endpos": st[:, 2].copy(), "first_edge": st[:, 3].copy(),
            "edges": ed, "text": tx[:n].cpu().numpy(), "slots": slots}


class SamState:
    """Device buffer holding B automata of capacity max_len tokens."""

    def __init__(self, B: int, max_len: int, V: int, device="cuda", stream=None):
        n = sam_state_bytes(B, max_len)
        if n == 0:
            raise SpecSamError(f"unsupported sizes B={B} max_len={max_len}")
        self.B, self.max_len, self.V = B, max_len, V
        self.buf = torch.empty(n, dtype=torch.uint8, device=device)
        sam_init(self.buf, B, max_len, V, stream)

    def extend(self, tokens, counts, stream=None):
        sam_extend(self.buf, self.B, self.max_len, tokens, counts, stream)

    def draft(self, K: int, draft=None, draft_len=None, match_len=None,
              stream=None):
        return sam_draft(self.buf, self.B, self.max_len, K, draft, draft_len,
                         match_len, stream)

    def draft_tree(self, K: int, M: int, N: int | None = None, stream=None):
        """Draft trees (see include/specsam.h, sam_draft_tree): returns
        (tokens [B, N], parent [B, N], n_nodes [B], match_len [B]) int32,
        N = 1 + M*K by default."""
        N = 1 + M * K if N is None else N
        dev = self.buf.device
        i32 = torch.int32
        tok = torch.empty((self.B, N), dtype=i32, device=dev)
        par = torch.empty((self.B, N), dtype=i32, device=dev)
        nn = torch.empty(self.B, dtype=i32, device=dev)
        ml = torch.empty(self.B, dtype=i32, device=dev)
        _check(lib().sam_draft_tree(_dev(self.buf, "state", torch.uint8), self.B,
                                    self.max_len, K, M, N, tok.data_ptr(),
                                    par.data_ptr(), nn.data_ptr(), ml.data_ptr(),
                                    _stream(stream)), "sam_draft_tree")
        return tok, par, nn, ml

    def extend_draft(self, tokens, counts, K: int, draft=None, draft_len=None,
                     match_len=None, stream=None):
        return sam_extend_draft(self.buf, self.B, self.max_len, tokens, counts,
                                K, draft, draft_len, match_len, stream)

    def extend_stats(self, tokens, counts, stats=None, stream=None):
        return sam_extend_stats(self.buf, self.B, self.max_len, tokens, counts,
                                stats, stream)

    def status(self, out=None, stream=None):
        return sam_status(self.buf, self.B, self.max_len, out, stream)

    def export(self, b: int):
        return sam_export(self.buf, self.B, self.max_len, b)


class StaticSam:
    """The static automaton over a corpus ([P4] §3): one sequence of capacity
    len(corpus), built on the device by the same extension as the dynamic
    automata, then only read by sam_match."""

    def __init__(self, corpus, V: int, device="cuda", stream=None):
        corpus = torch.as_tensor(corpus, dtype=torch.int32, device=device)
        n = int(corpus.numel())
        if n < 1:
            raise SpecSamError("the corpus is empty")
        self.state = SamState(1, n, V, device, stream)
        self.state.extend(corpus.view(1, n).contiguous(),
                          torch.full((1,), n, dtype=torch.int32, device=device),
                          stream)
        self.max_len, self.V = n, V

    def new_match(self, B: int, device="cuda"):
        """Match states [B, 2] int32 at the root."""
        return torch.zeros((B, 2), dtype=torch.int32, device=device)

    def match(self, match, tokens=None, counts=None, K: int = 0, delta: int = 0,
              dyn=None, draft=None, draft_len=None, source=None, status=None,
              stream=None):
        """Advances `match` [B, 2] by tokens [B, L] (counts [B], all L by
        default); with K > 0 returns (draft, draft_len, source): the static
        drafts, or, with dyn = (draft, draft_len, match_len) of the dynamic
        automata, the dynamic draft unless the static match is longer by more
        than delta."""
        B = match.shape[0]
        dev = match.device
        i32 = torch.int32
        tp = cp = None
        ld = 0
        if tokens is not None:
            if tokens.dim() != 2 or tokens.shape[0] != B:
                raise SpecSamError("tokens must be [B, L]")
            ld = tokens.shape[1]
            if counts is None:
                counts = torch.full((B,), ld, dtype=i32, device=dev)
            tp = _dev(tokens, "tokens", i32)
            cp = _dev(counts, "counts", i32, (B,))
        if K > 0:
            if draft is None:
                draft = torch.empty((B, K), dtype=i32, device=dev)
            if draft_len is None:
                draft_len = torch.empty(B, dtype=i32, device=dev)
            if source is None:
                source = torch.empty(B, dtype=i32, device=dev)
        dd = dl = dm = None
        if dyn is not None:
            dd = _dev(dyn[0], "dyn draft", i32, (B, K))
            dl = _dev(dyn[1], "dyn draft_len", i32, (B,))
            dm = _dev(dyn[2], "dyn match_len", i32, (B,))
        _check(lib().sam_match(
            _dev(self.state.buf, "state", torch.uint8), self.max_len, B,
            _dev(match, "match", i32, (B, 2)), tp, ld, cp, K, delta, dd, dl, dm,
            None if draft is None else _dev(draft, "draft", i32, (B, K)),
            None if draft_len is None else _dev(draft_len, "draft_len", i32, (B,)),
            None if source is None else _dev(source, "source", i32, (B,)),
            None if status is None else _dev(status, "status", i32, (B,)),
            _stream(stream)), "sam_match")
        if K > 0:
            return draft, draft_len, source
        return None
