"""Seeded synthetic inputs for the OTT decode-attention path.

This module only draws random tensors. It holds none of the method's
arithmetic (no norms, no quantization, no attention), so the CPU oracle
and the HIP path can both take their inputs from it without sharing any
part of the computation.

Workload shapes follow the models the OTT paper evaluates with
(Llama-2-7B/13B and Mistral-7B, "Accurate KV Cache Quantization with
Outlier Tokens Tracing", arXiv 2505.10938, sciencestack page, Figure 5
caption and the LongBench row of the blog's results section). The Key
distribution mimics the paper's observation (blog section 2.1, Figure 1
(a),(d) captions): a few outlier channels carry large magnitudes, and
inside those channels a few tokens have very small magnitude.

Recipe (every tensor is drawn in fp32 and rounded to fp16, RNE):
  * Q, V ~ N(0, 1).
  * K ~ N(0, 1); per KV head, 4 distinct "outlier channels" (shared by all
    sequences and positions) are multiplied by ``chan_scale``.
  * Each (sequence, KV head, position) is an "outlier token" with
    probability ``tok_prob``; its outlier channels are multiplied by
    ``tok_scale`` on top of that.
Every tensor comes from its own numpy PCG64 stream keyed by
(seed, tensor tag, indices), so any single (sequence, KV head) can be
regenerated alone, and any prefix of positions is stable.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

# Stream tags: the first element of every spawn key.
_TAG_CHAN = 1
_TAG_LEN = 2
_TAG_K = 3
_TAG_V = 4
_TAG_TOK = 5
_TAG_Q = 6
_TAG_SIGN = 7


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: layer shape, OTT hyper-parameters, input law."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    group_size: int        # G
    residual: int          # R
    pool_size: int         # P
    prefill: Tuple[int, int]  # prompt length drawn uniformly in [lo, hi]
    steps: int             # decode steps the workload runs
    seed: int
    chan_scale: float = 10.0
    tok_prob: float = 0.005
    tok_scale: float = 0.05
    n_outlier_channels: int = 4
    one_signed: bool = False
    retention: int = 0     # pool rule (0: the method's smallest Key norm); not an input law

    @property
    def max_prefill(self) -> int:
        return self.prefill[1]

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five layer shapes the benchmark and the parity tests use.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 128, 128, 32, 32, (512, 512), 8, seed=1),
    "llama2-7b": Workload("llama2-7b", 1, 32, 32, 128, 128, 32, 32, (4096, 4096), 64, seed=2),
    "llama2-7b-b32": Workload("llama2-7b-b32", 32, 32, 32, 128, 128, 32, 32, (3072, 4096), 64,
                              seed=3),
    "mistral-7b-gqa": Workload("mistral-7b-gqa", 8, 32, 8, 128, 128, 32, 32, (32768, 32768), 16,
                               seed=4),
    "llama2-13b-128k": Workload("llama2-13b-128k", 1, 40, 40, 128, 256, 64, 128,
                                (131072, 131072), 16, seed=5, chan_scale=15.0, tok_prob=0.002),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def outlier_channels(w: Workload, kvh: int) -> np.ndarray:
    """The KV head's outlier channels (sorted, distinct)."""
    g = _rng(w.seed, _TAG_CHAN, kvh)
    n = min(w.n_outlier_channels, w.head_dim)
    return np.sort(g.choice(w.head_dim, size=n, replace=False))


def prefill_lengths(w: Workload) -> np.ndarray:
    """Prompt length of each sequence (int64 [batch])."""
    lo, hi = w.prefill
    if lo == hi:
        return np.full(w.batch, lo, dtype=np.int64)
    g = _rng(w.seed, _TAG_LEN)
    return g.integers(lo, hi + 1, size=w.batch, dtype=np.int64)


def kv_stream(w: Workload, b: int, kvh: int, n_pos: int) -> Tuple[np.ndarray, np.ndarray]:
    """K and V of one (sequence, KV head) for positions [0, n_pos): fp16 [n_pos, d] each."""
    d = w.head_dim
    k = _rng(w.seed, _TAG_K, b, kvh).standard_normal((n_pos, d), dtype=np.float32)
    v = _rng(w.seed, _TAG_V, b, kvh).standard_normal((n_pos, d), dtype=np.float32)
    tok = _rng(w.seed, _TAG_TOK, b, kvh).random(n_pos) < w.tok_prob
    ch = outlier_channels(w, kvh)
    if ch.size:
        if w.one_signed:
            sign = np.where(_rng(w.seed, _TAG_SIGN, kvh).random(ch.size) < 0.5, -1.0, 1.0)
            k[:, ch] = np.abs(k[:, ch]) * sign.astype(np.float32)
        k[:, ch] *= np.float32(w.chan_scale)
        k[np.ix_(tok, ch)] *= np.float32(w.tok_scale)
    return k.astype(np.float16), v.astype(np.float16)


def query(w: Workload, step: int, b: int) -> np.ndarray:
    """Decode query of sequence b at decode step ``step``: fp16 [Hq, d]."""
    g = _rng(w.seed, _TAG_Q, step, b)
    return g.standard_normal((w.num_q_heads, w.head_dim), dtype=np.float32).astype(np.float16)


def queries(w: Workload, step: int) -> np.ndarray:
    """All decode queries of one step: fp16 [B, Hq, d]."""
    return np.stack([query(w, step, b) for b in range(w.batch)])


def kv_all(w: Workload, n_pos: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """K and V of every (sequence, KV head): fp16 [B, Hkv, n_pos, d] each."""
    if n_pos is None:
        n_pos = w.max_prefill + w.steps
    shape = (w.batch, w.num_kv_heads, n_pos, w.head_dim)
    K = np.empty(shape, np.float16)
    V = np.empty(shape, np.float16)
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            K[b, h], V[b, h] = kv_stream(w, b, h, n_pos)
    return K, V
