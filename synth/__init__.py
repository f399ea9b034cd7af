"""Seeded synthetic inputs for the speculative-verify + SAM-draft step.

This module generates inputs only. It holds none of the step's arithmetic
(no automaton, no softmax of the target, no acceptance test, no inverse CDF)
and is the one piece of code that both the oracle-side tests and the GPU side
use. Nothing here imports the oracle or the product package.

The pages measure on math/code rollouts and on prompt sets (Math500,
DAPO-MATH-17k, Spec-Bench); none of those is used. Token streams come instead
from a copy process that mimics the repetitive structure the pages describe:
with probability ``p_copy`` a span of Geometric length is copied from a
uniformly chosen earlier position (overlap allowed), otherwise a Zipf(s) token
is drawn over the vocabulary. Target logits are Gaussian noise with the
"true next token" of the stream boosted, so that drafts taken from the history
are sometimes right.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

VOCAB_QWEN = 151936


@dataclass(frozen=True)
class Config:
    """One synthetic workload."""
    name: str
    B: int
    V: int
    K: int
    T: float
    hist_len: int            # committed tokens per sequence before step 0
    p_copy: float
    span_mean: float
    sigma: float             # noise standard deviation of the target logits
    boost: float             # added to the logit of the true next token
    boost_prob: float = 1.0  # fraction of rows that get the boost
    zipf_s: float = 1.1
    dtype: str = "f32"       # "f32" or "bf16" logits in memory
    q_mode: str = "onehot"   # "onehot" (SAM drafts) or "model" (draft q given)
    draft_sigma: float = 0.0  # noise std added to the target for the draft model
    top_k: int = 0           # truncation of the target per sequence (0: off)
    top_p: float = 1.0       # (1: off)
    steps: int = 100
    warmup: int = 0
    seed: int = 0

    @property
    def rows(self) -> int:
        return self.B * (self.K + 1)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def stream_len(self, steps: int | None = None) -> int:
        """Length of each ground-truth token stream: history, then enough
        continuation that gt[n + j] exists even if every draft is accepted at
        every step."""
        s = self.steps + self.warmup if steps is None else steps
        return self.hist_len + (s + 1) * (self.K + 1)


# The five workloads. N(0, 2) and N(0, 0.5) are read as variances, so the
# standard deviations are sqrt(2) and sqrt(0.5).
CONFIGS = {
    1: Config("c1_b1_v32_k3_greedy", B=1, V=32, K=3, T=0.0, hist_len=2000,
              p_copy=0.5, span_mean=8, sigma=1.0, boost=3.0, boost_prob=0.7,
              steps=500, seed=1000),
    2: Config("c2_b64_v151936_k3_greedy", B=64, V=VOCAB_QWEN, K=3, T=0.0,
              hist_len=1024, p_copy=0.6, span_mean=8, sigma=math.sqrt(2.0),
              boost=6.0, steps=1024, seed=2000),
    3: Config("c3_b256_v151936_k3_t1_onehot", B=256, V=VOCAB_QWEN, K=3, T=1.0,
              hist_len=8192, p_copy=0.6, span_mean=8, sigma=math.sqrt(2.0),
              boost=4.0, steps=200, warmup=20, seed=3000),
    4: Config("c4_b32_v151936_k5_t0.7_bf16_long", B=32, V=VOCAB_QWEN, K=5,
              T=0.7, hist_len=32768, p_copy=0.8, span_mean=24,
              sigma=math.sqrt(2.0), boost=4.0, dtype="bf16", steps=200,
              seed=4000),
    5: Config("c5_b128_v151936_k5_t0.7_draft_model", B=128, V=VOCAB_QWEN, K=5,
              T=0.7, hist_len=0, p_copy=0.0, span_mean=1, sigma=math.sqrt(2.0),
              boost=0.0, q_mode="model", draft_sigma=math.sqrt(0.5),
              steps=100, seed=5000),
}


def config(c: int, **overrides) -> Config:
    return replace(CONFIGS[c], **overrides) if overrides else CONFIGS[c]


# ---------------------------------------------------------------------------
# Random streams. Each purpose has its own child of SeedSequence(seed) so that
# changing one does not shift the others.
# ---------------------------------------------------------------------------
STREAM_TOKENS, STREAM_BOOST_MASK, STREAM_UNIFORMS, STREAM_DRAFT = 0, 1, 2, 3
STREAM_CORPUS, STREAM_QUERY = 4, 5
STREAM_TREE = 6


def rng_for(seed: int, stream: int, *sub: int) -> np.random.Generator:
    ss = np.random.SeedSequence([seed, stream, *sub])
    return np.random.Generator(np.random.PCG64(ss))


def zipf_cdf(V: int, s: float) -> np.ndarray:
    """Cumulative table of P(rank r) proportional to r^-s, r = 1..V."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def copy_process(rng: np.random.Generator, n: int, V: int, p_copy: float,
                 span_mean: float, zipf_s: float = 1.1,
                 cdf: np.ndarray | None = None) -> np.ndarray:
    """A token stream of length n with copied spans (see module docstring).

    The first token is Zipf. Then, repeatedly: with probability p_copy copy a
    span of length L ~ Geometric(1/span_mean) on {1, 2, ...} starting at a
    uniformly chosen earlier position (token by token, so a span may overlap
    its own output; cut at n); otherwise emit one Zipf token (rank r gives
    token r - 1).
    """
    if cdf is None:
        cdf = zipf_cdf(V, zipf_s)
    out = np.empty(n, np.int32)
    if n == 0:
        return out
    pool = 4096
    zipf_tok = np.minimum(np.searchsorted(cdf, rng.random(pool), side="right"),
                          V - 1).astype(np.int32)
    zi = 0

    def next_zipf():
        nonlocal zipf_tok, zi
        if zi == pool:
            zipf_tok = np.minimum(
                np.searchsorted(cdf, rng.random(pool), side="right"),
                V - 1).astype(np.int32)
            zi = 0
        t = zipf_tok[zi]
        zi += 1
        return t

    out[0] = next_zipf()
    i = 1
    p_geo = 1.0 / span_mean
    while i < n:
        if p_copy > 0.0 and rng.random() < p_copy:
            L = int(rng.geometric(p_geo))
            src = int(rng.integers(0, i))
            L = min(L, n - i)
            if src + L <= i:
                out[i:i + L] = out[src:src + L]
            else:
                for k in range(L):
                    out[i + k] = out[src + k]
            i += L
        else:
            out[i] = next_zipf()
            i += 1
    return out


def token_streams(cfg: Config, steps: int | None = None) -> np.ndarray:
    """gt[B, stream_len] int32. gt[b, :hist_len] is the committed history;
    the rest is the continuation the synthetic target model prefers."""
    n = cfg.stream_len(steps)
    cdf = zipf_cdf(cfg.V, cfg.zipf_s)
    gt = np.empty((cfg.B, n), np.int32)
    for b in range(cfg.B):
        gt[b] = copy_process(rng_for(cfg.seed, STREAM_TOKENS, b), n, cfg.V,
                             cfg.p_copy, cfg.span_mean, cfg.zipf_s, cdf)
    return gt


def corpus(seed: int, n_docs: int, doc_len: int, V: int, eos: int,
           p_copy: float = 0.6, span_mean: float = 8.0,
           zipf_s: float = 1.1) -> np.ndarray:
    """A reference corpus for a static automaton: n_docs copy-process
    documents of doc_len tokens (each from its own seed), each followed by
    the end-of-sequence token `eos`."""
    cdf = zipf_cdf(V, zipf_s)
    parts = []
    for d in range(n_docs):
        doc = copy_process(rng_for(seed, STREAM_CORPUS, d), doc_len, V, p_copy,
                           span_mean, zipf_s, cdf)
        parts.append(doc)
        parts.append(np.array([eos], np.int32))
    return np.concatenate(parts).astype(np.int32)


def corpus_queries(seed: int, corpus_tokens: np.ndarray, B: int, n: int, V: int,
                   p_span: float = 0.5, span_mean: float = 12.0,
                   zipf_s: float = 1.1) -> np.ndarray:
    """Texts [B, n] that partly overlap a corpus: with probability p_span a
    span of length Geometric(1/span_mean) copied from a uniform corpus
    position, otherwise one Zipf token; so matches against the corpus of
    every length occur."""
    cdf = zipf_cdf(V, zipf_s)
    out = np.empty((B, n), np.int32)
    N = len(corpus_tokens)
    for b in range(B):
        rng = rng_for(seed, STREAM_QUERY, b)
        row = []
        while len(row) < n:
            if rng.random() < p_span:
                L = int(rng.geometric(1.0 / span_mean))
                a = int(rng.integers(0, N))
                row.extend(corpus_tokens[a:a + L].tolist())
            else:
                row.append(int(min(np.searchsorted(cdf, rng.random(), side="right"),
                                   V - 1)))
        out[b] = row[:n]
    return out


def uniforms(cfg: Config, step: int) -> np.ndarray:
    """[B, K+1] float32 in [0, 1): accept coins for j < K, final coin at K."""
    r = rng_for(cfg.seed, STREAM_UNIFORMS, step)
    return r.random((cfg.B, cfg.K + 1), dtype=np.float32)


def boost_mask(cfg: Config, step: int) -> np.ndarray:
    """[B, K+1] bool: which rows get the boost this step."""
    if cfg.boost_prob >= 1.0:
        return np.ones((cfg.B, cfg.K + 1), bool)
    r = rng_for(cfg.seed, STREAM_BOOST_MASK, step)
    return r.random((cfg.B, cfg.K + 1)) < cfg.boost_prob


def boost_positions(cfg: Config, gt: np.ndarray, n: np.ndarray) -> np.ndarray:
    """[B, K+1] int32: the token whose logit row j boosts, gt[b, n_b + j]."""
    idx = n.reshape(-1, 1).astype(np.int64) + np.arange(cfg.K + 1)
    return np.take_along_axis(gt, idx, axis=1).astype(np.int32)


# ---------------------------------------------------------------------------
# Noise. Generated with torch (on the CPU for small cases, on the GPU for full
# sizes); the oracle is always handed the exact bytes the GPU reads.
# ---------------------------------------------------------------------------
def noise_seed(cfg: Config, step: int) -> int:
    return cfg.seed * 1_000_003 + 7 + step


def noise(cfg: Config, step: int, device="cpu", rows_per_seq: int | None = None):
    """Target-logit noise [B, K+1, V] float32, N(0, sigma^2), seeded by step."""
    import torch
    R = cfg.K + 1 if rows_per_seq is None else rows_per_seq
    g = torch.Generator(device=device)
    g.manual_seed(noise_seed(cfg, step))
    x = torch.randn((cfg.B, R, cfg.V), generator=g, device=device,
                    dtype=torch.float32)
    if cfg.sigma != 1.0:
        x.mul_(cfg.sigma)
    return x


def target_logits(cfg: Config, step: int, gt: np.ndarray, n: np.ndarray,
                  device="cpu"):
    """The synthetic target model's logits for one step: noise plus the boost
    on gt[b, n_b + j] (rows chosen by boost_mask). Returned as a torch tensor
    in the config's storage dtype (bf16 is rounded after the boost)."""
    import torch
    x = noise(cfg, step, device)
    if cfg.boost != 0.0:
        pos = torch.as_tensor(boost_positions(cfg, gt, n), device=device,
                              dtype=torch.int64)
        msk = torch.as_tensor(boost_mask(cfg, step), device=device)
        add = torch.where(msk, cfg.boost, 0.0).to(torch.float32)
        x.scatter_add_(2, pos.unsqueeze(-1), add.unsqueeze(-1))
    if cfg.dtype == "bf16":
        x = x.to(torch.bfloat16)
    return x


def draft_model_inputs(cfg: Config, step: int, target, device="cpu"):
    """Draft-model stand-in for workloads with a given q: draft logits are the
    target's first K rows plus N(0, draft_sigma^2) noise; q = softmax(draft/T)
    (torch's library softmax, float64, stored float32); each draft token x_j is
    drawn from q_j with numpy's seeded Generator.choice.

    Returns (q [B,K,V] float32 tensor on device, draft [B,K] int32 numpy).
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(noise_seed(cfg, step) ^ 0x5A5A5A)
    t = target[:, :cfg.K, :].to(torch.float32)
    eps = torch.randn(t.shape, generator=g, device=device, dtype=torch.float32)
    dl = t + cfg.draft_sigma * eps
    q64 = torch.softmax(dl.to(torch.float64) / cfg.T, dim=-1)
    q = q64.to(torch.float32)
    qh = q64.cpu().numpy()
    rng = rng_for(cfg.seed, STREAM_DRAFT, step)
    draft = np.empty((cfg.B, cfg.K), np.int32)
    for b in range(cfg.B):
        for j in range(cfg.K):
            pr = qh[b, j]
            draft[b, j] = rng.choice(cfg.V, p=pr / pr.sum())
    return q.contiguous(), draft


# ---------------------------------------------------------------------------
# Draft trees: one tree per sequence, the shape fixed (a root with several
# candidate continuations, as drafts taken from several suffix-link ancestors
# would give), the tokens seeded per slot and distinct among siblings.
# ---------------------------------------------------------------------------
TREE8_PARENTS = (-1, 0, 0, 0, 1, 4, 5, 2)  # root, 3 candidates, one 4 deep


def draft_trees(cfg: Config, slot: int, parents=TREE8_PARENTS):
    """(tokens [B, N] int32, parent [B, N] int32, chain [B, N] bool): random
    tokens, distinct among siblings; `chain` marks the nodes on the first
    candidate's path (the ones a harness would make likely)."""
    par = np.asarray(parents, np.int32)
    N = len(par)
    r = rng_for(cfg.seed, STREAM_TREE, slot)
    tok = r.integers(0, cfg.V, (cfg.B, N)).astype(np.int32)
    tok[:, 0] = 0
    for i in range(1, N):
        for j in range(1, i):
            if par[j] == par[i]:
                same = tok[:, j] == tok[:, i]
                tok[same, i] = (tok[same, i] + 1) % cfg.V
    chain = np.zeros(N, bool)
    v = 1
    while v >= 0:
        chain[v] = True
        kids = [c for c in range(1, N) if par[c] == v]
        v = kids[0] if kids else -1
    return tok, np.tile(par, (cfg.B, 1)), np.tile(chain, (cfg.B, 1))


def tree_uniforms(cfg: Config, step: int, N: int) -> np.ndarray:
    """[B, N] float32 in [0, 1): coins per depth, the last the final coin."""
    r = rng_for(cfg.seed, STREAM_TREE + 1, step)
    return r.random((cfg.B, N), dtype=np.float32)
