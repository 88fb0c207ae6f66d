"""CPU oracle for Outlier Tokens Tracing (OTT) quantization and decode attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module. The product
path (the HIP library and its Python binding) never calls it, and this module
imports nothing from that path.

Sources, cited by page title and section:
  [Blog]  zijie-tian.site, "Accurate KV Cache Quantization with Outlier Tokens
          Tracing" (a summary of arXiv 2505.10938): section 3.1 (outlier-token
          rule), 3.2 (Outlier Pool), 3.3 (multi-cache fused decode) and its
          flowchart, section 4 (defaults G=128, R=32), section 6 (G=256, larger P).
  [Abs]   sciencestack.ai page for arXiv 2505.10938: TL;DR, Abstract, and the
          captions of Figure 1 (smallest Key magnitude is the best retention
          criterion) and Figure 2 (decoding and quantization stages).
  [DGAP]  bittide page, section 3.2: softmax is unchanged by adding a constant to
          every logit (used only as a test property).

What the pages fix, and what this module does:
  * Three caches: 2-bit quantized KV, an FP16 residual window of recent tokens,
    and a full-precision outlier pool ([Blog] 3.3; [Abs] TL;DR).
  * Every G tokens the oldest unquantized group is processed: Key magnitudes
    are computed, the tokens with the smallest Key magnitude stay in the pool,
    the rest are quantized to 2 bits ([Blog] 3.1, 3.2, flowchart; [Abs] Fig. 2
    bottom, Fig. 1(c)).
  * Keys are quantized per channel and Values per token ([Abs] Abstract).
  * Decode multiplies the query by each kind of Key, concatenates the scores,
    takes one softmax, multiplies by each kind of Value and sums ([Blog]
    flowchart; [Abs] Fig. 2 top).

Readings taken where the pages are silent:
  R1  outlier = the P smallest squared L2 Key norms; no channel test.
  R2  squared norm = fp64 sum of exact squares in channel order 0..d-1;
      ties broken by lower position.
  R3  a token evicted from the pool joins the page being built now.
  R4  candidates at each quantize = current pool + the oldest G unquantized.
  R5  quantize when the window holds >= R+G tokens, taking the oldest G.
  R6  asymmetric uniform 2-bit quantizer: x_hat = min + code * scale,
      scale = (max - min) / 3, levels 0..3.
  R7  min and scale stored as fp16; scale = fp16_rne(fp32(max - min) / 3);
      a zero min or scale is stored as +0.
  R8  code = clamp(rint_half_even(fp32((x - min)) / fp32(scale)), 0, 3), one IEEE
      fp32 op per step; scale == 0 gives code 0.
  R9  prefill is appends plus quantize steps in position order.
  R10 score scale 1/sqrt(d), no mask; the query sees every cached token.
  R12 the pool keeps both K and V in fp16.
  R13 with grouped-query attention the caches are per KV head.
  R14 the pool keeps min(P, #candidates) entries; a page may hold fewer than G.
  R16 the comparison rules of [Abs] Fig. 1(c), built for the accuracy measurement:
      largest squared norm, or a random key per position (SplitMix64).

What pins this module (tests/test_oracle.py): hand-derived quantizer cases
(signed zeros included), the quantizer's error bound and nearest-level brute
force, fp16 rounding against Python's struct, hand-derived squared norms whose
fp64 value depends on the summation order (and the pool tie they decide),
brute-force top-P pool membership for every rule,
the SplitMix64 reference outputs, token accounting, and reductions of the
decode to textbook attention (no quantization, lossless grids, permutation
and shift invariance, closed forms). Parity with the paper's own arithmetic
is unpinned: the pages print no worked example, no codes and no outputs.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

F16 = np.float16
F32 = np.float32
F64 = np.float64


# --------------------------------------------------------------------------
# Scalar building blocks
# --------------------------------------------------------------------------

def sq_key_norm(k_rows: np.ndarray) -> np.ndarray:
    """Squared L2 norm of each fp16 Key row, as an fp64 sum in channel order.

    [Blog] 3.1 scores each candidate by its Key norm; [Abs] Fig. 1(c) picks the
    smallest Key magnitude. Squares of fp16 values are exact in fp64; the sum
    runs channel 0, 1, ..., d-1 (reading R2), so the value is reproducible.
    """
    x = np.asarray(k_rows, dtype=F16).astype(F64)
    if x.ndim == 1:
        x = x[None, :]
    acc = np.zeros(x.shape[0], dtype=F64)
    for c in range(x.shape[1]):
        acc = acc + x[:, c] * x[:, c]
    return acc


def min_scale(values_f16: np.ndarray) -> Tuple[np.float16, np.float16]:
    """(min, scale) of one quantization set, as fp16 (readings R6, R7).

    scale = fp16_rne( (fp32(max) - fp32(min)) / 3.0f ), each step one IEEE op.
    A zero min or scale is stored as +0 whatever the signs of the zeros in the
    set (reading R7: a set may hold +0 and -0, which compare equal, so "the
    minimum" names no single bit pattern; dequantized values do not depend on
    the choice). An empty set gives (+0, +0).
    """
    v = np.asarray(values_f16, dtype=F16)
    if v.size == 0:
        return F16(0.0), F16(0.0)
    lo = v.min()
    hi = v.max()
    r = F32(hi) - F32(lo)
    s = F16(r / F32(3.0))
    if lo == 0:
        lo = F16(0.0)
    if s == 0:
        s = F16(0.0)
    return F16(lo), s


def codes_of(values_f16: np.ndarray, lo: np.float16, s: np.float16) -> np.ndarray:
    """2-bit codes of fp16 values against one (min, scale) pair (reading R8)."""
    v = np.asarray(values_f16, dtype=F16)
    if F32(s) == F32(0.0):
        return np.zeros(v.shape, dtype=np.uint8)
    y = (v.astype(F32) - F32(lo)) / F32(s)
    return np.clip(np.rint(y), 0, 3).astype(np.uint8)


def dequant(lo: np.float16, s: np.float16, code) -> np.ndarray:
    """x_hat = min + code * scale, in fp64 (exact for fp16 min/scale, code <= 3)."""
    return F64(lo) + F64(s) * np.asarray(code, dtype=F64)


# --------------------------------------------------------------------------
# One quantized page
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Page:
    """One group after the outlier split: the quantized members.

    Keys: one (min, scale) per channel over the members ([Abs] Abstract,
    channel-wise Keys). Values: one (min, scale) per member token over its d
    channels ([Abs] Abstract, token-wise Values).
    """

    pos: np.ndarray        # int64 [n] member positions, ascending
    k_min: np.ndarray      # fp16 [d]
    k_scale: np.ndarray    # fp16 [d]
    k_code: np.ndarray     # uint8 [n, d]
    v_min: np.ndarray      # fp16 [n]
    v_scale: np.ndarray    # fp16 [n]
    v_code: np.ndarray     # uint8 [n, d]

    @property
    def n_valid(self) -> int:
        return int(self.pos.size)

    def k_hat(self) -> np.ndarray:
        k_min, k_scale = np.asarray(self.k_min, F64), np.asarray(self.k_scale, F64)
        return k_min[None, :] + k_scale[None, :] * self.k_code.astype(F64)

    def v_hat(self) -> np.ndarray:
        v_min, v_scale = np.asarray(self.v_min, F64), np.asarray(self.v_scale, F64)
        return v_min[:, None] + v_scale[:, None] * self.v_code.astype(F64)


def quantize_members(k: np.ndarray, v: np.ndarray, pos: np.ndarray) -> Page:
    """2-bit quantize the page members (rows in position order)."""
    n, d = k.shape
    k_min = np.zeros(d, F16)
    k_scale = np.zeros(d, F16)
    k_code = np.zeros((n, d), np.uint8)
    for c in range(d):                       # Keys: per channel
        k_min[c], k_scale[c] = min_scale(k[:, c])
        k_code[:, c] = codes_of(k[:, c], k_min[c], k_scale[c])
    v_min = np.zeros(n, F16)
    v_scale = np.zeros(n, F16)
    v_code = np.zeros((n, d), np.uint8)
    for t in range(n):                       # Values: per token
        v_min[t], v_scale[t] = min_scale(v[t, :])
        v_code[t, :] = codes_of(v[t, :], v_min[t], v_scale[t])
    return Page(np.asarray(pos, np.int64), k_min, k_scale, k_code, v_min, v_scale, v_code)


# --------------------------------------------------------------------------
# State of one (sequence, KV head)
# --------------------------------------------------------------------------

# Retention rules for the outlier pool. The method keeps the tokens with the
# smallest Key magnitude ([Abs] TL;DR and Figure 1(c), which also compares it
# with other rules; [Blog] 3.1). The other two exist for that comparison.
RETAIN_SMALLEST_NORM = 0
RETAIN_LARGEST_NORM = 1
RETAIN_RANDOM = 2

_M64 = (1 << 64) - 1


def splitmix64(seed: int) -> int:
    """First output of a SplitMix64 generator whose state is `seed` (the
    generator of Steele, Lea and Flood, in the form Vigna publishes with the
    xoshiro generators): state += 0x9E3779B97F4A7C15, then two xor-shift-multiply
    rounds and a final xor-shift."""
    z = (seed + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def retention_key(n2: float, pos: int, rule: int) -> float:
    """The value the pool keeps the smallest of (ties to the lower position):
    the squared Key norm, its negation (largest norms kept), or a random value
    in [0, 1) drawn per position (the top 53 bits of splitmix64(pos) as a
    fraction, exact in fp64)."""
    if rule == RETAIN_SMALLEST_NORM:
        return float(n2)
    if rule == RETAIN_LARGEST_NORM:
        return -float(n2)
    if rule == RETAIN_RANDOM:
        return float(splitmix64(int(pos)) >> 11) * 2.0 ** -53
    raise ValueError(f"unknown retention rule {rule}")


@dataclasses.dataclass
class Entry:
    n2: float           # squared Key norm (fp64); NaN while still in the window
    key: float          # retention key (= n2 under the method's rule); NaN in the window
    pos: int
    k: np.ndarray       # fp16 [d]
    v: np.ndarray       # fp16 [d]


class HeadOracle:
    """The three caches of one (sequence, KV head) ([Blog] 3.3)."""

    def __init__(self, head_dim: int, group_size: int, residual: int, pool_size: int,
                 retention: int = RETAIN_SMALLEST_NORM):
        self.d = head_dim
        self.G = group_size
        self.R = residual
        self.P = pool_size
        self.retention = retention
        self.pages: List[Page] = []
        self.pool: List[Entry] = []          # ascending (key, pos)
        self.recent: List[Entry] = []        # ascending pos
        self.L = 0
        # pages' positions, K_hat and V_hat concatenated, rebuilt when a page is
        # added (pages never change once made); a cache only, no arithmetic
        self._pages_cat = None
        self._pages_cat_n = None

    # -- stage: append (every step) -------------------------------------
    def append(self, k_rows: np.ndarray, v_rows: np.ndarray) -> None:
        k_rows = np.asarray(k_rows, F16).reshape(-1, self.d)
        v_rows = np.asarray(v_rows, F16).reshape(-1, self.d)
        for i in range(k_rows.shape[0]):
            self.recent.append(Entry(float("nan"), float("nan"), self.L, k_rows[i].copy(),
                                     v_rows[i].copy()))
            self.L += 1

    def ready(self) -> bool:
        """Reading R5: a group is quantized once the window holds R+G tokens."""
        return len(self.recent) >= self.R + self.G

    # -- stage: quantization (every G tokens) ---------------------------
    def quantize_group(self) -> None:
        """[Blog] flowchart, quantization branch; [Abs] Fig. 2 bottom.

        1. the G oldest window tokens are the group (R4, R5);
        2. their Key norms are computed (R2);
        3. the pool and the group compete: the P smallest norms stay in the pool
           ([Blog] 3.2), ties by position (R2) (other retention rules: the P
           smallest keys of `retention_key`);
        4. everything else, evicted pool tokens included (R3), is quantized to
           2 bits as one page (R6-R8).
        """
        assert self.ready()
        group = self.recent[: self.G]
        self.recent = self.recent[self.G:]
        norms = sq_key_norm(np.stack([e.k for e in group]))
        for e, n2 in zip(group, norms):
            e.n2 = float(n2)
            e.key = retention_key(e.n2, e.pos, self.retention)
        cands = sorted(self.pool + group, key=lambda e: (e.key, e.pos))
        keep = min(self.P, len(cands))
        self.pool = cands[:keep]
        members = sorted(cands[keep:], key=lambda e: e.pos)
        d = self.d
        k = np.stack([e.k for e in members]) if members else np.zeros((0, d), F16)
        v = np.stack([e.v for e in members]) if members else np.zeros((0, d), F16)
        pos = np.array([e.pos for e in members], np.int64)
        self.pages.append(quantize_members(k, v, pos))

    # -- views ----------------------------------------------------------
    def caches(self) -> List[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
        """The three caches as (positions, K_hat, V_hat) in fp64.

        Order: quantized pages, outlier pool, residual window ([Blog] 3.3).
        """
        d = self.d
        tag = (len(self.pages), id(self.pages[-1]) if self.pages else 0)
        if self._pages_cat_n != tag:
            if self.pages:
                self._pages_cat = (np.concatenate([p.pos for p in self.pages]),
                                   np.concatenate([p.k_hat() for p in self.pages]),
                                   np.concatenate([p.v_hat() for p in self.pages]))
            else:
                self._pages_cat = (np.zeros(0, np.int64), np.zeros((0, d)), np.zeros((0, d)))
            self._pages_cat_n = tag
        qpos, qk, qv = self._pages_cat

        def dense(entries):
            if not entries:
                return np.zeros(0, np.int64), np.zeros((0, d)), np.zeros((0, d))
            return (np.array([e.pos for e in entries], np.int64),
                    np.stack([e.k for e in entries]).astype(F64),
                    np.stack([e.v for e in entries]).astype(F64))

        return [(qpos, qk, qv), dense(self.pool), dense(self.recent)]

    def by_position(self) -> Tuple[np.ndarray, np.ndarray]:
        """K_hat and V_hat of every token, row i = position i."""
        K = np.full((self.L, self.d), np.nan)
        V = np.full((self.L, self.d), np.nan)
        for pos, kh, vh in self.caches():
            K[pos] = kh
            V[pos] = vh
        return K, V

    # -- stage: decoding (every step) -----------------------------------
    def decode(self, q: np.ndarray, sm_scale: float) -> np.ndarray:
        """[Blog] flowchart decoding branch; [Abs] Fig. 2 top.

        Scores of the query against each kind of Key are concatenated, one
        softmax is taken, and the weighted sums against each kind of Value are
        added. Returns fp64 [d].
        """
        qd = np.asarray(q, F16).astype(F64)
        parts = self.caches()
        scores = [sm_scale * (kh @ qd) for _, kh, _ in parts]
        z = np.concatenate(scores)
        if z.size == 0:
            raise ValueError("decode on an empty cache")
        p = softmax(z)
        out = np.zeros(self.d)
        start = 0
        for (_, _, vh), s in zip(parts, scores):
            out = out + p[start:start + s.size] @ vh
            start += s.size
        return out


def softmax(z: np.ndarray) -> np.ndarray:
    """exp(z - max z) / sum(exp(z - max z)), fp64."""
    z = np.asarray(z, F64)
    e = np.exp(z - z.max())
    return e / e.sum()


def textbook_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """Single-query softmax attention over explicit K, V rows (fp64)."""
    qd = np.asarray(q, F64)
    z = np.array([sm_scale * float(np.dot(K[i].astype(F64), qd)) for i in range(K.shape[0])])
    w = np.exp(z - z.max())
    return (w[:, None] * np.asarray(V, F64)).sum(axis=0) / w.sum()


# --------------------------------------------------------------------------
# Byte image of a page (the arena layout the HIP library writes)
# --------------------------------------------------------------------------

def page_nbytes(G: int, d: int) -> int:
    return G * d // 4 + d * G // 4 + 4 * d + 4 * G


def pack_page(page: Page, G: int, d: int) -> bytes:
    """Bytes of one page in the arena layout.

    [K codes: G tokens x d/4 bytes, token-major]
    [V codes: d channels x G/4 bytes, channel-major]
    [K meta: d x (fp16 min, fp16 scale)] [V meta: G x (fp16 min, fp16 scale)]
    Code i of a 4-code byte sits in bits 2i..2i+1 (channel 4j+i for K, slot 4j+i
    for V). Slots past n_valid are zero.
    """
    assert G % 4 == 0 and d % 4 == 0
    n = page.n_valid
    kc = np.zeros((G, d), np.uint8)
    kc[:n] = page.k_code
    vc = np.zeros((d, G), np.uint8)
    vc[:, :n] = page.v_code.T
    def four_per_byte(codes):  # byte j of a row = codes 4j..4j+3, code i at bits 2i
        return (codes[:, 0::4] | codes[:, 1::4] << 2 | codes[:, 2::4] << 4
                | codes[:, 3::4] << 6).astype(np.uint8)

    out = bytearray()
    out += four_per_byte(kc).tobytes()      # token t: bytes of channels 0..d-1
    out += four_per_byte(vc).tobytes()      # channel c: bytes of slots 0..G-1
    km = np.zeros((d, 2), F16)
    km[:, 0] = page.k_min
    km[:, 1] = page.k_scale
    vm = np.zeros((G, 2), F16)
    vm[:n, 0] = page.v_min
    vm[:n, 1] = page.v_scale
    out += km.astype("<f2").tobytes()
    out += vm.astype("<f2").tobytes()
    assert len(out) == page_nbytes(G, d)
    return bytes(out)


# --------------------------------------------------------------------------
# A whole layer: many (sequence, KV head) states
# --------------------------------------------------------------------------

class OTTOracle:
    """Oracle for one attention layer, optionally tracking a subset of heads.

    Each (sequence, KV head) is independent, so a parity check of a large
    layer can follow just a sample of them.
    """

    def __init__(self, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 group_size: int, residual: int, pool_size: int,
                 sm_scale: Optional[float] = None,
                 heads: Optional[Iterable[Tuple[int, int]]] = None,
                 retention: int = RETAIN_SMALLEST_NORM):
        assert num_q_heads % num_kv_heads == 0
        self.B, self.Hq, self.Hkv, self.d = batch, num_q_heads, num_kv_heads, head_dim
        self.G, self.R, self.P = group_size, residual, pool_size
        self.sm_scale = (1.0 / np.sqrt(head_dim)) if (sm_scale is None or sm_scale <= 0) \
            else float(sm_scale)
        if heads is None:
            heads = [(b, h) for b in range(batch) for h in range(num_kv_heads)]
        self.heads: Dict[Tuple[int, int], HeadOracle] = {
            (int(b), int(h)): HeadOracle(head_dim, group_size, residual, pool_size, retention)
            for b, h in heads}

    @classmethod
    def for_workload(cls, w, heads=None) -> "OTTOracle":
        return cls(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.group_size,
                   w.residual, w.pool_size, heads=heads,
                   retention=getattr(w, "retention", RETAIN_SMALLEST_NORM))

    def head(self, b: int, kvh: int) -> HeadOracle:
        return self.heads[(b, kvh)]

    def kv_head_of(self, qh: int) -> int:
        """Reading R13: query head qh reads KV head qh // (Hq / Hkv)."""
        return qh // (self.Hq // self.Hkv)

    def append(self, b: int, kvh: int, k_rows, v_rows) -> None:
        self.heads[(b, kvh)].append(k_rows, v_rows)

    def quantize_group(self) -> List[Tuple[int, int]]:
        """One group for every tracked head whose window is full (R5)."""
        done = []
        for key, st in self.heads.items():
            if st.ready():
                st.quantize_group()
                done.append(key)
        return done

    def decode(self, b: int, qh: int, q: np.ndarray) -> np.ndarray:
        return self.heads[(b, self.kv_head_of(qh))].decode(q, self.sm_scale)


def run_prefill(st: HeadOracle, k: np.ndarray, v: np.ndarray) -> None:
    """Reading R9: prefill = appends interleaved with quantize steps, in order."""
    cap = st.R + st.G
    i = 0
    n = k.shape[0]
    while i < n:
        take = min(n - i, cap - len(st.recent))
        st.append(k[i:i + take], v[i:i + take])
        i += take
        while st.ready():
            st.quantize_group()


def step(st: HeadOracle, k_row: np.ndarray, v_row: np.ndarray) -> None:
    """One decode step's cache update: append one token, then quantize if due."""
    st.append(k_row, v_row)
    while st.ready():
        st.quantize_group()
