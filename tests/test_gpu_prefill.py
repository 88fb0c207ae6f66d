"""GPU: ott_prefill (one launch for a whole prompt) leaves exactly the state of
the stepwise path (appends in window-sized chunks, every due quantize step in
order): counters, every page byte, member positions, the pool and the pool
before the last step, and the window, bit for bit. The stepwise path is itself checked against the oracle by
the parity tests, and the oracle-side state after ott_prefill by run_case."""
import numpy as np
import pytest

import synth
from tests.parity import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _prev_pool(layer, b, h):
    """The pool before the last quantize step (the other buffer), when that step
    had a predecessor that wrote it: (pos, n2, k, v) of its used slots."""
    nb = layer.seq_state(b)[3]
    if nb < 2:
        return None
    n = min(layer.P, layer.G * (nb - 1))
    lay = layer.layout
    slot0 = ((nb - 1) & 1) * layer.B * layer.Hkv + b * layer.Hkv + h
    d = layer.d
    return (layer._region(lay.off_pool_pos + slot0 * layer.P * 4, n * 4).copy(),
            layer._region(lay.off_pool_n2 + slot0 * layer.P * 8, n * 8).copy(),
            layer._region(lay.off_pool_k + slot0 * layer.P * d * 2, n * d * 2).copy(),
            layer._region(lay.off_pool_v + slot0 * layer.P * d * 2, n * d * 2).copy())


def _state(layer):
    """Everything either path writes (the arena is not cleared, so regions no
    step has written hold leftovers and are not compared)."""
    lay = layer.layout
    st = {"counters": layer.counters().copy()}
    nv = layer._region(lay.off_page_nvalid, layer.B * layer.Hkv * lay.pages_per_head * 4)
    nv = nv.view(np.int32).reshape(layer.B * layer.Hkv, lay.pages_per_head)
    for b in range(layer.B):
        nb = layer.seq_state(b)[3]
        for h in range(layer.Hkv):
            st[("pages", b, h)] = layer.pages_of_head(b, h, nb).copy() if nb else None
            st[("pos", b, h)] = layer.page_positions(b, h, nb).copy() if nb else None
            st[("nvalid", b, h)] = nv[b * layer.Hkv + h, :nb].copy()
            st[("pool", b, h)] = tuple(x.copy() for x in layer.pool(b, h))
            st[("prev_pool", b, h)] = _prev_pool(layer, b, h)
            st[("win", b, h)] = tuple(x.copy() for x in layer.window(b, h))
    return st


def _compare(w, lengths, keys=None):
    import torch
    from decode_attention_ott_amd import OTTLayer
    lengths = np.asarray(lengths, np.int64)
    n_pos = max(int(lengths.max()), 1)
    K, V = synth.kv_all(w, n_pos)
    if keys is not None:
        K = keys(K)
    Kd, Vd = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()
    one = OTTLayer.for_workload(w, max_seq_len=n_pos + 8)
    one.prefill(Kd, Vd, lengths)
    ref = OTTLayer.for_workload(w, max_seq_len=n_pos + 8)
    ref.prefill_stepwise(Kd, Vd, lengths)
    a, b = _state(one), _state(ref)
    assert a.keys() == b.keys()
    for key in a:
        x, y = a[key], b[key]
        if isinstance(x, tuple):
            for u, v in zip(x, y):
                assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), key
        elif x is None:
            assert y is None, key
        else:
            assert np.array_equal(x, y), key
    # host counters agree with the device's
    for bb in range(w.batch):
        assert one.seq_state(bb) == ref.seq_state(bb) == tuple(one.counters()[bb, 0])
    log(f"[prefill] {w.name} lengths {list(lengths)}: identical to the stepwise path")


def small(name, G=128, R=32, P=32, Hkv=2, seed=5, **kw):
    return synth.Workload(name, 4, 2 * Hkv, Hkv, 128, G, R, P, (1, 1), 1, seed, **kw)


@pytest.mark.parametrize("G,R,P,lengths", [
    (128, 32, 32, [0, 1, 159, 160]),       # empty, window only, one short of a page, one page
    (128, 32, 32, [1000, 417, 288, 161]),  # several pages, ragged
    (64, 16, 8, [700, 80, 81, 333]),
    (256, 64, 128, [1500, 320, 1024, 700]),
    (128, 0, 32, [512, 128, 129, 300]),    # R = 0: the window empties at each step
    (128, 32, 0, [900, 500, 33, 2]),       # P = 0
    (128, 32, 160, [1100, 700, 300, 161]), # P > G: the first page has no members
    (64, 5, 3, [401, 70, 69, 200]),        # odd window and pool sizes
])
def test_prefill_matches_stepwise(G, R, P, lengths):
    _compare(small(f"prefill-g{G}r{R}p{P}", G=G, R=R, P=P, seed=G + R + P), lengths)


@pytest.mark.parametrize("rule", [1, 2])
def test_prefill_matches_stepwise_other_retention_rules(rule):
    """Largest-norm and random retention: the one-call prefill walks the groups
    with the same rule as the stepwise quantize steps."""
    _compare(small(f"prefill-rule{rule}", retention=rule, seed=40 + rule), [1000, 417, 288, 161])


def test_prefill_with_pool_churn():
    _compare(small("prefill-churn", tok_prob=0.05, chan_scale=30.0), [1500, 1400, 900, 1501])


def test_prefill_rejects_a_nonempty_cache():
    import torch
    from decode_attention_ott_amd import OTTLayer, OttError, _lib as L
    layer = OTTLayer(1, 1, 1, 128, 128, 32, 32, max_seq_len=400)
    k = torch.zeros(1, 1, 10, 128, dtype=torch.float16, device="cuda")
    layer.append(k, k)
    before = layer.counters().copy()
    with pytest.raises(OttError, match="STATE"):
        L.ott_prefill(layer.handle, k.data_ptr(), k.data_ptr(), [10], 10, 0)
    with pytest.raises(OttError, match="CAPACITY"):
        fresh = OTTLayer(1, 1, 1, 128, 128, 32, 32, max_seq_len=5)
        L.ott_prefill(fresh.handle, k.data_ptr(), k.data_ptr(), [10], 10, 0)
    assert np.array_equal(layer.counters(), before)


def _few_norms(K):
    """Keys of 0, +1 and -1 only, most channels 0: the squared norms are small
    integers, so most keys tie with many others (and zero rows give a zero
    norm, negated to -0 under the largest-norm rule)."""
    rng = np.random.default_rng(11)
    mask = rng.random(K.shape) < 0.04
    return (np.sign(K.astype(np.float32)) * mask).astype(np.float16)


@pytest.mark.parametrize("rule", [0, 1])
def test_prefill_matches_stepwise_with_tied_keys(rule):
    """Equal keys are ranked by position: in the pool walk, and in each
    segment's selection of its smallest pairs, where a tie can fall on the
    boundary of the P smallest."""
    _compare(small(f"prefill-ties{rule}", G=64, R=16, P=40, retention=rule, seed=70 + rule),
             [3000, 2900, 1200, 3001], keys=_few_norms)


def test_prefill_long_prompt_with_a_large_pool():
    """G = 64 with P = 512: a segment's 512 smallest pairs take the spare bytes
    of two page slots; dozens of segments, each merging all earlier ones."""
    _compare(small("prefill-long", G=64, R=64, P=512, Hkv=1, seed=77), [4100, 3000, 64, 700])
