"""Pins for the CPU oracle: it is checked against things other than itself.

Each test ties one part of the oracle to what the pages or plain mathematics
fix: hand-derived quantizer cases, IEEE rounding, the quantizer's error bound,
brute-force pool membership, token accounting, and reductions of the decode to
textbook softmax attention. The last tests plant a mistake in the oracle and
check that some pin catches it.
"""
import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import ott_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16_bits(h: str) -> np.float16:
    return np.array([int(h, 16)], np.uint16).view(np.float16)[0]


# --------------------------------------------------------------------------
# IEEE rounding used by the contract
# --------------------------------------------------------------------------

def test_fp16_rounding_matches_struct_half():
    """numpy's fp32 -> fp16 cast is round-half-even, as Python's struct 'e'."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    # exact midpoints between neighbouring fp16 values
    h = rng.integers(0x0400, 0x7800, 2000).astype(np.uint16).view(np.float16)
    mid = ((h.astype(np.float64) + np.nextafter(h, np.float16(np.inf)).astype(np.float64)) / 2)
    x = np.concatenate([x, mid.astype(np.float32), np.float32([1e-8, 3e-8, 6e-8, 65519.0])])
    ours = x.astype(np.float16)
    ref = np.array([struct.unpack("<e", struct.pack("<e", float(v)))[0] for v in x], np.float16)
    assert np.array_equal(ours.view(np.uint16), ref.view(np.uint16))


# --------------------------------------------------------------------------
# Quantizer
# --------------------------------------------------------------------------

def test_quantizer_hand_cases():
    with open(os.path.join(GOLDEN, "quantizer_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        vals = np.array([f16_bits(h) for h in c["values"]], np.float16)
        lo, s = O.min_scale(vals)
        assert lo.view(np.uint16) == f16_bits(c["min"]).view(np.uint16), c["name"]
        assert s.view(np.uint16) == f16_bits(c["scale"]).view(np.uint16), c["name"]
        assert O.codes_of(vals, lo, s).tolist() == c["codes"], c["name"]


def _random_sets(n_sets=300, seed=1):
    rng = np.random.default_rng(seed)
    for i in range(n_sets):
        n = int(rng.integers(2, 40))
        scale = float(10.0 ** rng.uniform(-2, 2))
        v = (rng.standard_normal(n) * scale + rng.uniform(-5, 5)).astype(np.float16)
        yield v


def test_quantizer_error_bound_and_extremes():
    """|x - x_hat| <= (s/2)(1 + 2^-20) for a normal-range fp16 scale; min -> code 0
    with x_hat = min exactly; max -> code 3."""
    for v in _random_sets():
        lo, s = O.min_scale(v)
        code = O.codes_of(v, lo, s)
        xh = O.dequant(lo, s, code)
        sf = float(s)
        if sf >= 2.0 ** -14:
            err = np.abs(v.astype(np.float64) - xh)
            assert err.max() <= sf / 2 * (1 + 2.0 ** -20), (v, lo, s)
        assert code[np.argmin(v)] == 0 and xh[np.argmin(v)] == float(v.min())
        if sf > 0:
            assert code[np.argmax(v)] == 3


def test_quantizer_picks_nearest_level_exactly():
    """Brute force in exact rationals: the code is a nearest level of
    {min + k*scale : k = 0..3}; only ratios within 2^-20 of a half-integer may
    go either way (fp32 rounding of the ratio)."""
    for v in _random_sets(150, seed=7):
        lo, s = O.min_scale(v)
        if float(s) == 0.0:
            continue
        code = O.codes_of(v, lo, s)
        fl, fs = Fraction(float(lo)), Fraction(float(s))
        for x, c in zip(v, code):
            fx = Fraction(float(x))
            d = [abs(fx - (fl + k * fs)) for k in range(4)]
            best = min(d)
            if d[c] == best:
                continue
            ratio = (fx - fl) / fs
            assert abs(ratio - (int(ratio) + Fraction(1, 2))) < Fraction(1, 2 ** 20), (x, c, d)


def test_scale_is_fp32_then_fp16():
    """Reading R7: scale = fp16_rne(fp32(max - min) / 3); checked in exact
    rationals for random sets (fp32 then fp16 round-to-nearest-even)."""
    def rne(fr: Fraction, mant_bits: int, emin: int) -> Fraction:
        if fr == 0:
            return fr
        e = max(fr.numerator.bit_length() - fr.denominator.bit_length(), emin)
        while Fraction(2) ** e > fr:
            e -= 1
        while Fraction(2) ** (e + 1) <= fr:
            e += 1
        e = max(e, emin)
        ulp = Fraction(2) ** (e - mant_bits)
        q, rem = divmod(fr, ulp)
        if rem * 2 > ulp or (rem * 2 == ulp and q % 2 == 1):
            q += 1
        return q * ulp

    for v in _random_sets(200, seed=3):
        lo, s = O.min_scale(v)
        r = rne(Fraction(float(v.max())) - Fraction(float(v.min())), 23, -126)
        want = rne(rne(r / 3, 23, -126), 10, -14)
        assert Fraction(float(s)) == want


# --------------------------------------------------------------------------
# Pool membership and token accounting
# --------------------------------------------------------------------------

def _tiny_stream(n, d, rng, dup_frac=0.3):
    """fp16 K rows on a coarse grid (multiples of 1/8 in [-4, 4]) so every
    squared norm is exact in fp64, with many duplicate rows (norm ties)."""
    k = (rng.integers(-32, 33, (n, d)) / 8.0).astype(np.float16)
    dup = rng.random(n) < dup_frac
    for i in np.nonzero(dup)[0]:
        k[i] = k[rng.integers(0, n)]
    v = rng.standard_normal((n, d)).astype(np.float16)
    return k, v


def _exact_sq_norm(row) -> Fraction:
    return sum(Fraction(float(x)) ** 2 for x in row)


def _order_rows(d=128):
    """Row A = [8, 2^-24 x (d-1)] and row B = A reversed (fp16)."""
    a = np.full(d, 2.0 ** -24, np.float16)
    a[0] = 8
    return a, a[::-1].copy()


def test_squared_norm_runs_in_channel_order():
    """Reading R2: the squared Key norm is an fp64 sum taken channel 0, 1, ...,
    d-1. Row A = [8, 2^-24, ..., 2^-24]: 8^2 = 64 comes first, and each 2^-48
    that follows is a quarter of the fp64 spacing at 64 (2^-46), so every partial
    sum rounds back to 64: the norm is exactly 64. Row B is A reversed: the 127
    squares 2^-48 add up exactly to 127 * 2^-48 = 31.75 * 2^-46 first, and
    64 + 31.75 * 2^-46 rounds to 64 + 32 * 2^-46 = 64 + 2^-41. A pairwise, dot
    or reversed summation gives other values for A."""
    a, b = _order_rows()
    n2 = O.sq_key_norm(np.stack([a, b]))
    assert n2[0] == 64.0
    assert n2[1] == 64.0 + 2.0 ** -41


def test_norm_order_decides_pool_ties():
    """The same rows through a quantize step (G = 4, R = 0, P = 1): row C =
    [8, 0, ..., 0] has norm exactly 64. A (position 0) ties with C (position 1),
    so the lower position keeps the pool slot; B (position 0) is larger than C
    by 2^-41, so C keeps it."""
    a, b = _order_rows()
    c = np.zeros(128, np.float16)
    c[0] = 8
    filler = np.full(128, 4.0, np.float16)      # norm 2048: never in the pool
    v = np.zeros((4, 128), np.float16)
    for first, want in ((a, [0]), (b, [1])):
        st = O.HeadOracle(128, 4, 0, 1)
        st.append(np.stack([first, c, filler, filler]), v)
        st.quantize_group()
        assert [e.pos for e in st.pool] == want


def test_signed_zero_page_metadata():
    """Reading R7 on a whole page: a Key channel whose minimum is zero, with +0
    and -0 both among the members, and a Value row holding both zeros at its
    minimum, store +0 as their min whatever order the members come in.
    Channel 0 holds {-0, +0, 3, 1.5} -> min +0, scale 1 (r = 3); Value row 0 is
    {+0, -0, 3, 0, ...} -> min +0, scale 1; Value row 1 is all -0 -> min +0,
    scale +0. Hand-derived from the definition (no oracle call builds them)."""
    d, G = 8, 4
    k = np.zeros((4, d), np.float16)
    k[:, 0] = np.float16([-0.0, 0.0, 3.0, 1.5])
    k[:, 1:] = 1.0
    v = np.zeros((4, d), np.float16)
    v[0, :3] = np.float16([0.0, -0.0, 3.0])
    v[1, :] = np.float16(-0.0)
    v[2:, :] = 1.0
    for order in ([0, 1, 2, 3], [1, 0, 3, 2]):
        kk = k[order]
        vv = v[order]
        pg = O.quantize_members(kk, vv, np.arange(4))
        b = O.pack_page(pg, G, d)
        moff = 2 * (G * d // 4)
        km = np.frombuffer(b[moff:moff + 4 * d], "<u2").reshape(d, 2)
        vm = np.frombuffer(b[moff + 4 * d:], "<u2").reshape(G, 2)
        assert km[0].tolist() == [0x0000, 0x3C00]            # +0, 1.0
        r0, r1 = order.index(0), order.index(1)
        assert vm[r0].tolist() == [0x0000, 0x3C00]
        assert vm[r1].tolist() == [0x0000, 0x0000]
        # channel 0 codes: -0 -> 0, +0 -> 0, 3 -> 3, 1.5 -> half-even 2
        assert pg.k_code[:, 0].tolist() == [[0, 0, 3, 2][i] for i in order]


@pytest.mark.parametrize("G", [2, 4, 8])
@pytest.mark.parametrize("P", [0, 1, 3, "G", "2G"])
@pytest.mark.parametrize("d", [4, 8])
def test_pool_is_bruteforce_topP(G, P, d):
    """[Blog] 3.2 / [Abs] Fig. 1(c): after every quantize step the pool is the
    P tokens of smallest Key norm among all tokens that went through a quantize
    step (positions [0, G*nb)), ties to the lower position, in that order."""
    P = {"G": G, "2G": 2 * G}.get(P, P)
    R = 3
    rng = np.random.default_rng(1000 * G + 10 * d + P)
    k, v = _tiny_stream(12 * G + 5, d, rng)
    exact = [_exact_sq_norm(row) for row in k]
    st = O.HeadOracle(d, G, R, P)
    for i in range(k.shape[0]):
        O.step(st, k[i], v[i])
        nb = len(st.pages)
        seen = sorted(range(G * nb), key=lambda p: (exact[p], p))
        assert [e.pos for e in st.pool] == seen[:P]


def test_splitmix64_matches_the_reference_outputs():
    """The generator behind the random retention rule: seeded with 1234567, the
    reference SplitMix64 (Vigna's public-domain splitmix64.c) yields these first
    five outputs; each output here is splitmix64(state) with the state advanced
    by the generator's constant between calls."""
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    state, got = 1234567, []
    for _ in range(5):
        got.append(O.splitmix64(state))
        state = (state + 0x9E3779B97F4A7C15) & ((1 << 64) - 1)
    assert got == want


@pytest.mark.parametrize("rule", [O.RETAIN_LARGEST_NORM, O.RETAIN_RANDOM])
@pytest.mark.parametrize("G,P", [(4, 3), (8, 8), (4, 9)])
def test_other_retention_rules_are_bruteforce_topP(rule, G, P):
    """The comparison rules of [Abs] Fig. 1(c): the pool is the P seen tokens of
    largest exact Key norm (ties to the lower position), or of smallest random
    key; the random key of a position is its splitmix64 value's top 53 bits,
    compared here as integers."""
    d, R = 4, 3
    rng = np.random.default_rng(7 * G + P + rule)
    k, v = _tiny_stream(12 * G + 5, d, rng)
    exact = [_exact_sq_norm(row) for row in k]
    st = O.HeadOracle(d, G, R, P, retention=rule)
    for i in range(k.shape[0]):
        O.step(st, k[i], v[i])
        nb = len(st.pages)
        if rule == O.RETAIN_LARGEST_NORM:
            seen = sorted(range(G * nb), key=lambda p: (-exact[p], p))
        else:
            seen = sorted(range(G * nb), key=lambda p: (O.splitmix64(p) >> 11, p))
        assert [e.pos for e in st.pool] == seen[:P]
        # every cached token is somewhere, once
        pos = np.concatenate([c[0] for c in st.caches()])
        assert sorted(pos.tolist()) == list(range(st.L))


@pytest.mark.parametrize("G,R,P", [(4, 2, 2), (8, 0, 3), (4, 5, 9), (8, 8, 0), (16, 4, 16)])
def test_token_accounting(G, R, P):
    """Every position is in exactly one cache; pages hold G members except the
    first (G - min(P, G)); the window keeps >= R tokens once quantizing starts
    and never reaches R+G (readings R3-R5, R14)."""
    rng = np.random.default_rng(G * 100 + R * 10 + P)
    d = 8
    k = rng.standard_normal((20 * G, d)).astype(np.float16)
    v = rng.standard_normal((20 * G, d)).astype(np.float16)
    st = O.HeadOracle(d, G, R, P)
    for i in range(k.shape[0]):
        O.step(st, k[i], v[i])
        pos = np.concatenate([c[0] for c in st.caches()])
        assert sorted(pos.tolist()) == list(range(st.L))
        assert len(st.recent) < R + G
        if st.pages:
            assert len(st.recent) >= R
        for n, pg in enumerate(st.pages):
            seen_before = min(P, G * n)
            assert pg.n_valid == G + seen_before - min(P, seen_before + G)
        assert len(st.pool) == min(P, G * len(st.pages))
        assert all(np.all(np.diff(pg.pos) > 0) for pg in st.pages)


def test_pool_catches_planted_outliers():
    """Tokens whose Keys have tiny magnitude in every channel end up in the pool."""
    w = synth.WORKLOADS["tiny"]
    K, V = synth.kv_stream(w, 0, 0, 512)
    K = K.copy()
    special = [5, 77, 200, 301]
    K[special] = (K[special].astype(np.float32) * 1e-3).astype(np.float16)
    st = O.HeadOracle(128, 128, 32, 32)
    O.run_prefill(st, K, V)
    assert set(special) <= {e.pos for e in st.pool}


# --------------------------------------------------------------------------
# Decode
# --------------------------------------------------------------------------

SM = 1.0 / np.sqrt(128)


def _state(n, G=16, R=4, P=4, d=16, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((n, d)) * scale).astype(np.float16)
    v = rng.standard_normal((n, d)).astype(np.float16)
    st = O.HeadOracle(d, G, R, P)
    O.run_prefill(st, k, v)
    return st, k, v


def test_decode_without_quantization_is_attention():
    """Before the first quantize step (L < R+G) nothing is quantized and the
    decode is plain softmax attention over the fp16 K, V."""
    st, k, v = _state(19, G=16, R=4)
    assert not st.pages
    q = np.random.default_rng(1).standard_normal(16).astype(np.float16)
    out = st.decode(q, 0.25)
    ref = O.textbook_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), 0.25)
    assert np.abs(out - ref).max() <= 1e-12


def test_decode_all_in_pool_is_attention():
    """With P >= L every quantized token stays in the pool: pages are empty and
    the decode equals attention over the fp16 K, V."""
    st, k, v = _state(70, G=8, R=2, P=80)
    assert all(p.n_valid == 0 for p in st.pages)
    q = np.random.default_rng(2).standard_normal(16).astype(np.float16)
    out = st.decode(q, 0.3)
    ref = O.textbook_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), 0.3)
    assert np.abs(out - ref).max() <= 1e-12


def _grid_stream(n_groups, G, d, rng, lead=0):
    """``lead`` tiny-norm rows, then n_groups*G rows where every K channel of a
    group lies on {a_c + j*e_c} and every V row on {b_t + j*f_t}, j in 0..3,
    with both extremes present among the group's grid rows (K) and in every V
    row, so the 2-bit quantizer is lossless on them. The tiny rows come first
    so that a pool of size ``lead`` takes them and never evicts them."""
    n = lead + n_groups * G
    K = np.zeros((n, d))
    V = np.zeros((n, d))
    a = rng.integers(1, 9, d) / 4.0                  # a_c > 0: grid norms stay large
    e = 2.0 ** rng.integers(-3, 1, d)
    j = rng.integers(0, 4, (n, d))
    for g in range(n_groups):
        first = lead if g == 0 else g * G            # grid rows of group g start here
        j[first, :] = 0
        j[first + 1, :] = 3
    K[:] = a + j * e
    K[:lead] = 1.0 / 64
    for t in range(n):
        jv = rng.integers(0, 4, d)
        jv[0], jv[1] = 0, 3
        V[t] = rng.integers(-8, 8) / 4.0 + jv * 2.0 ** int(rng.integers(-3, 1))
    return K.astype(np.float16), V.astype(np.float16)


@pytest.mark.parametrize("P", [0, 2])
def test_decode_lossless_grid_is_attention(P):
    """When every quantization set lies on a 4-level grid with both extremes
    present, x_hat = x exactly, so the three-cache decode must equal attention
    over the original K, V. With P = 2 the two tiny-norm leading tokens enter
    the pool at the first quantize and stay there, so every page holds only
    grid tokens."""
    G, R, d = 8, 4, 16
    rng = np.random.default_rng(5 + P)
    K, V = _grid_stream(7, G, d, rng, lead=P)
    st = O.HeadOracle(d, G, R, P)
    O.run_prefill(st, K, V)
    assert len(st.pages) >= 5
    if P:
        assert sorted(e.pos for e in st.pool) == list(range(P))
    Kh, Vh = st.by_position()
    assert np.array_equal(Kh, K.astype(np.float64))
    assert np.array_equal(Vh, V.astype(np.float64))
    q = np.random.default_rng(9).standard_normal(d).astype(np.float16)
    out = st.decode(q, 0.5)
    ref = O.textbook_attention(q.astype(np.float64), K.astype(np.float64), V.astype(np.float64), 0.5)
    assert np.abs(out - ref).max() <= 1e-12


def test_decode_matches_textbook_in_any_token_order():
    """The three-cache concatenation is order-free: textbook attention over the
    dequantized rows in a random order gives the same output ([Abs] Fig. 2 top)."""
    st, k, v = _state(301, G=32, R=8, P=6, d=32, seed=3)
    Kh, Vh = st.by_position()
    perm = np.random.default_rng(4).permutation(st.L)
    q = np.random.default_rng(5).standard_normal(32).astype(np.float16)
    out = st.decode(q, SM)
    ref = O.textbook_attention(q.astype(np.float64), Kh[perm], Vh[perm], SM)
    assert np.abs(out - ref).max() <= 1e-12


def test_softmax_shift_invariance():
    """[DGAP] 3.2: softmax(z + c) = softmax(z); large c must not overflow."""
    z = np.round(np.random.default_rng(6).standard_normal(50) * 4 * 2.0 ** 20) / 2.0 ** 20
    for c in (0.0, 700.0, -700.0, 2.0 ** 17):      # z + c is exact in fp64
        assert np.array_equal(O.softmax(z + c), O.softmax(z))


def test_decode_shift_of_all_keys():
    """Adding the same vector u to every Key row shifts every score by sm*q.u;
    with u on the grid spacing the quantized rows shift exactly, so the output
    must not change even when the shift is large."""
    G, R, d = 8, 4, 16
    rng = np.random.default_rng(11)
    K, V = _grid_stream(5, G, d, rng)
    u = np.full(d, 64.0)
    st0 = O.HeadOracle(d, G, R, 0)
    st1 = O.HeadOracle(d, G, R, 0)
    O.run_prefill(st0, K, V)
    O.run_prefill(st1, (K.astype(np.float64) + u).astype(np.float16), V)
    q = rng.standard_normal(d).astype(np.float16)
    a, b = st0.decode(q, 1.0), st1.decode(q, 1.0)
    assert np.abs(a - b).max() <= 1e-12


def test_decode_closed_forms():
    st, k, v = _state(1, G=8, R=2, P=1, d=16)
    q = np.random.default_rng(0).standard_normal(16).astype(np.float16)
    assert np.array_equal(st.decode(q, SM), v[0].astype(np.float64))      # L = 1 -> v
    st, k, v = _state(250, G=32, R=8, P=4, d=16, seed=8)
    _, Vh = st.by_position()
    assert np.abs(st.decode(np.zeros(16, np.float16), SM) - Vh.mean(0)).max() <= 1e-13  # q = 0
    # two tokens whose scores differ by ln 3: weights 1/4 and 3/4
    st = O.HeadOracle(4, 8, 2, 0)
    st.append(np.float16([[0, 0, 0, 0], [1, 0, 0, 0]]), np.float16([[4, 0, 0, 0], [0, 8, 0, 0]]))
    out = st.decode(np.float16([1, 0, 0, 0]), float(np.log(3.0)))
    assert np.abs(out - np.array([1.0, 6.0, 0, 0])).max() <= 1e-14


def test_p0_is_kivi_style():
    """P = 0: each page is the whole group, Keys per channel over all G tokens,
    Values per token (the KIVI-style scheme the pages compare against)."""
    st, k, v = _state(200, G=16, R=4, P=0, d=8, seed=12)
    for n, pg in enumerate(st.pages):
        assert pg.pos.tolist() == list(range(16 * n, 16 * n + 16))
        grp = k[16 * n:16 * n + 16]
        assert np.array_equal(pg.k_min, grp.min(0))
        assert np.array_equal(pg.v_min, v[16 * n:16 * n + 16].min(1))


# --------------------------------------------------------------------------
# Page byte image
# --------------------------------------------------------------------------

def test_pack_page_layout_by_hand():
    G, d = 8, 8
    kc = np.zeros((3, d), np.uint8)
    kc[0, :4] = [1, 2, 3, 0]      # byte 0 of token 0 = 1 | 2<<2 | 3<<4 = 0x39
    kc[2, 7] = 3                   # token 2, channel 7 -> byte 1 of token 2, bits 6-7
    vc = np.zeros((3, d), np.uint8)
    vc[1, 5] = 2                   # slot 1 of channel 5 -> V byte 0 of channel 5, bits 2-3
    pg = O.Page(np.array([0, 1, 2]), np.float16(np.arange(d)), np.float16(np.ones(d)), kc,
                np.float16([1.5, 2, 3]), np.float16([0.25, 0.5, 1]), vc)
    b = O.pack_page(pg, G, d)
    assert len(b) == G * d // 4 * 2 + 4 * d + 4 * G
    assert b[0] == 0x39 and b[1] == 0
    assert b[2 * 2 + 1] == 0xC0
    voff = G * d // 4
    assert b[voff + 5 * (G // 4)] == 0x08
    assert sum(b[:voff]) == 0x39 + 0xC0 and sum(b[voff:2 * voff]) == 0x08
    moff = 2 * voff
    km = np.frombuffer(b[moff:moff + 4 * d], "<f2").reshape(d, 2)
    assert km[3, 0] == 3 and km[3, 1] == 1
    vm = np.frombuffer(b[moff + 4 * d:], "<f2").reshape(G, 2)
    assert vm[0, 0] == 1.5 and vm[2, 1] == 1 and not vm[3:].any()


# --------------------------------------------------------------------------
# Planted mistakes: each must be caught by one of the pins above
# --------------------------------------------------------------------------

def test_planted_round_half_up_is_caught(monkeypatch):
    def bad_codes(values, lo, s):
        v = np.asarray(values, np.float16)
        if float(s) == 0:
            return np.zeros(v.shape, np.uint8)
        y = (v.astype(np.float32) - np.float32(lo)) / np.float32(s)
        return np.clip(np.floor(y + np.float32(0.5)), 0, 3).astype(np.uint8)
    monkeypatch.setattr(O, "codes_of", bad_codes)
    with pytest.raises(AssertionError):
        test_quantizer_hand_cases()


def test_planted_largest_norm_pool_is_caught(monkeypatch):
    monkeypatch.setattr(O, "sq_key_norm", lambda rows: -np.asarray(
        [float(np.dot(r.astype(np.float64), r.astype(np.float64))) for r in np.atleast_2d(rows)]))
    with pytest.raises(AssertionError):
        test_pool_is_bruteforce_topP(4, 3, 4)


def test_planted_dropped_evictions_are_caught(monkeypatch):
    orig = O.HeadOracle.quantize_group

    def drop_evicted(self):
        before = {e.pos for e in self.pool}
        orig(self)
        pg = self.pages[-1]
        keep = np.array([p not in before for p in pg.pos])
        self.pages[-1] = O.Page(pg.pos[keep], pg.k_min, pg.k_scale, pg.k_code[keep],
                                pg.v_min[keep], pg.v_scale[keep], pg.v_code[keep])
    monkeypatch.setattr(O.HeadOracle, "quantize_group", drop_evicted)
    with pytest.raises(AssertionError):
        test_token_accounting(4, 2, 2)


def test_planted_values_per_channel_is_caught(monkeypatch):
    """A wrong index in the Value quantizer (token t takes the parameters of
    column t instead of row t) breaks the lossless-grid pin."""
    orig = O.quantize_members

    def wrong_index(k, v, pos):
        pg = orig(k, v, pos)
        for t in range(v.shape[0]):
            lo, s = O.min_scale(v[:, t % v.shape[1]])
            pg.v_min[t], pg.v_scale[t] = lo, s
            pg.v_code[t] = O.codes_of(v[t], lo, s)
        return pg
    monkeypatch.setattr(O, "quantize_members", wrong_index)
    with pytest.raises(AssertionError):
        test_decode_lossless_grid_is_attention(0)


def test_planted_transposed_kv_is_caught(monkeypatch):
    """Using V's dequantized rows as Keys must break the attention reduction."""
    orig = O.HeadOracle.caches

    def swapped(self):
        parts = orig(self)
        return [(p, vh, kh) for p, kh, vh in parts]
    monkeypatch.setattr(O.HeadOracle, "caches", swapped)
    with pytest.raises(AssertionError):
        test_decode_without_quantization_is_attention()


def test_planted_pairwise_norm_is_caught(monkeypatch):
    """A squared norm summed pairwise (numpy's np.sum) instead of in channel order
    must break the R2 pins."""
    monkeypatch.setattr(O, "sq_key_norm", lambda rows: np.sum(
        np.atleast_2d(np.asarray(rows, np.float16)).astype(np.float64) ** 2, axis=1))
    with pytest.raises(AssertionError):
        test_squared_norm_runs_in_channel_order()
    with pytest.raises(AssertionError):
        test_norm_order_decides_pool_ties()


def test_planted_reversed_norm_is_caught(monkeypatch):
    def rev(rows):
        x = np.atleast_2d(np.asarray(rows, np.float16)).astype(np.float64)
        acc = np.zeros(x.shape[0])
        for c in range(x.shape[1] - 1, -1, -1):
            acc = acc + x[:, c] * x[:, c]
        return acc
    monkeypatch.setattr(O, "sq_key_norm", rev)
    with pytest.raises(AssertionError):
        test_squared_norm_runs_in_channel_order()


def test_planted_signed_zero_min_is_caught(monkeypatch):
    """Storing the minimum with the sign of whichever zero the scan meets first
    (numpy's min) must break the signed-zero pins."""
    def raw_min_scale(values):
        v = np.asarray(values, np.float16)
        if v.size == 0:
            return np.float16(0), np.float16(0)
        lo, hi = v.min(), v.max()
        return np.float16(lo), np.float16((np.float32(hi) - np.float32(lo)) / np.float32(3))
    monkeypatch.setattr(O, "min_scale", raw_min_scale)
    with pytest.raises(AssertionError):
        test_quantizer_hand_cases()
    with pytest.raises(AssertionError):
        test_signed_zero_page_metadata()
