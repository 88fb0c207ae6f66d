"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: page bytes (codes and fp16 min/scale), member positions, pool
membership/order/contents, window contents, counters. Within tolerance
(max abs 2e-3, rel L2 1e-3): fp16 decode outputs.
"""
import numpy as np
import pytest

import synth
from tests.parity import check_state, log, run_case

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def small(name, B=2, Hq=2, Hkv=2, G=128, R=32, P=32, L=(400, 400), steps=8, seed=11, **kw):
    return synth.Workload(name, B, Hq, Hkv, 128, G, R, P, L, steps, seed, **kw)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ---- the tiny workload, state checked after every step ----------------------
def test_tiny_every_step():
    run_case(W["tiny"], state_every_step=True)


# ---- parameter coverage on small shapes -------------------------------------
@pytest.mark.parametrize("G,R,P,L,steps", [
    (64, 16, 8, (300, 300), 70),      # G=64, crosses quantize steps during decode
    (256, 64, 128, (700, 700), 12),   # G=256 with a large pool
    (128, 32, 0, (500, 500), 40),     # P=0: plain 2-bit cache
    (128, 0, 32, (400, 400), 12),     # R=0: the window empties at each quantize
    (128, 32, 160, (600, 600), 8),    # P > G: first page empty
    (64, 5, 3, (333, 333), 20),       # odd window and pool sizes
    (128, 128, 32, (760, 760), 12),   # R=128: window 248 of 256, a quantize at step 7
    (256, 128, 32, (1146, 1146), 10), # G=256, R=128: window 378 of 384, a quantize at step 5
    (256, 128, 128, (1146, 1146), 10),  # G=256, R=128, P=128 (the coupled setting)
    (256, 64, 512, (1082, 1082), 10), # P=512 at G=256: quantize LDS above 64 KiB, a step at 5
])
def test_parameters(G, R, P, L, steps):
    run_case(small(f"g{G}r{R}p{P}", G=G, R=R, P=P, L=L, steps=steps, seed=G + R + P),
             state_every_step=True)


# query heads per KV head: 2 and 3 (a padded group of 4), 4, 6 (a group and a
# padded one), 8 (two groups), 16 and 32 (passes of 8)
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (6, 2), (8, 2), (12, 2), (16, 2), (12, 3), (32, 2),
                                    (64, 2)])
def test_grouped_query_heads(Hq, Hkv):
    run_case(small(f"gqa{Hq}x{Hkv}", Hq=Hq, Hkv=Hkv, L=(520, 520), steps=6, seed=Hq))


@pytest.mark.parametrize("G,R,P,L,Hq", [
    (64, 16, 8, (300, 300), 8),       # G=64
    (256, 64, 128, (700, 700), 8),    # G=256 with a large pool
    (256, 64, 128, (700, 700), 32),   # G=256, 16 heads per pass
    (64, 16, 8, (300, 300), 32),      # G=64, 16 heads per pass
    (128, 32, 160, (600, 600), 8),    # P > G: first page has no members
    (128, 32, 0, (500, 500), 4),      # P=0
    (256, 128, 32, (1146, 1146), 8),  # G=256, R=128
])
def test_grouped_query_parameters(G, R, P, L, Hq):
    run_case(small(f"gqa-g{G}r{R}p{P}h{Hq}", Hq=Hq, G=G, R=R, P=P, L=L, steps=4, seed=3 * G + P),
             state_every_step=True)


def test_grouped_query_split_counts_agree():
    # past 16 splits the merge reads its partials in two rounds; at 64 most
    # splits of a 16-page head are empty
    w = small("gqa-splits", B=2, Hq=8, Hkv=2, L=(2000, 2000), steps=2)
    run_case(w, splits=[1, 2, 3, 7, 16, 17, 33, 64, 0])


def test_grouped_query_merge_rounds():
    # 6 query heads per KV head: the merging split's 256 threads take 768
    # outputs in two rounds of two, the second pair half past the end
    w = small("gqa-rounds", B=2, Hq=12, Hkv=2, L=(1500, 1500), steps=2)
    run_case(w, splits=[5, 20])


def test_grouped_query_huge_keys():
    """Outlier channels x8000 and queries x16: |q * scale| per channel exceeds
    the fp16 range, so the page's query operand is scaled down first."""
    run_case(small("gqa-hugek", Hq=8, L=(700, 700), steps=3, chan_scale=8000.0), q_scale=16.0)


def test_ragged_and_short_sequences():
    """Sequences of length 1 (window only), below R+G (no page), and longer."""
    w = small("ragged", B=5, Hq=4, Hkv=2, L=(1, 1), steps=10)
    run_case(w, lengths=[1, 50, 159, 200, 777], state_every_step=True)


def test_one_split_head_orders():
    """One split per head with more heads than CUs: 512 heads of ragged lengths
    (a whole number of rounds: the heads are dealt largest first, snaking) and
    300 heads (a partial last round: the launch keeps the identity order)."""
    for B, H in ((16, 32), (10, 30)):
        w = small(f"order{B}x{H}", B=B, Hq=H, Hkv=H, L=(300, 700), steps=3, seed=5)
        heads = [(b, (7 * b) % H) for b in range(B)]
        run_case(w, heads=heads, splits=[1], check_prefill=False)


def test_split_counts_agree():
    w = small("splits", B=2, Hq=2, Hkv=2, L=(2000, 2000), steps=3)
    run_case(w, splits=[1, 2, 3, 7, 16, 17, 40, 64, 0])


@pytest.mark.parametrize("Hq", [2, 8])
def test_split_counts_agree_at_g256(Hq):
    """G = 256 (value blocks as interleaved 32-slot stretches) on the one-head
    and the grouped-query kernel, with 1 to 16 splits over a head's pages."""
    w = small(f"splits-g256-h{Hq}", B=2, Hq=Hq, Hkv=2, G=256, R=64, P=32, L=(3000, 3000), steps=2,
              seed=29)
    run_case(w, splits=[1, 2, 5, 16, 0])


def _plant_zeros_and_norm_ties(K, V):
    """Edits the inputs of a 2-sequence, 2-head case in place.
    (0, 0): Key channel 5 non-negative with +0 and -0 scattered through it,
    channel 6 non-negative with -0 as its only zero, channel 7 all zeros of
    both signs; Value rows non-negative with zeros of both signs, of -0 only,
    or all zeros of mixed sign (every Key min/scale and Value min/scale rule
    of the signed-zero reading meets a page).
    (1, 1): Key rows whose squared norm is 64 in channel order: A = [8, 2^-24,
    ...] (exactly 64 only in channel order), C = [8, 0, ...] (exactly 64), and
    B = A reversed (64 + 2^-41), smaller than every drawn token, more of them
    than the pool holds, so the order of the norm sum decides the pool."""
    n = K.shape[2]
    p = np.arange(n)
    k = K[0, 0]
    v = V[0, 0]
    for c in (5, 6):
        k[:, c] = np.abs(k[:, c])
    k[p % 37 == 0, 5] = np.float16(-0.0)
    k[p % 41 == 0, 5] = np.float16(0.0)
    k[p % 29 == 0, 6] = np.float16(-0.0)
    k[:, 7] = np.where(p % 2 == 0, np.float16(-0.0), np.float16(0.0))
    v[:] = np.abs(v)
    r0, r1, r2 = p % 3 == 0, p % 3 == 1, p % 3 == 2
    v[r0, 3] = np.float16(-0.0)
    v[r0, 9] = np.float16(0.0)
    v[r1, :] = np.where((np.arange(v.shape[1]) % 2 == 0)[None, :], np.float16(-0.0), np.float16(0.0))
    v[r2, 11] = np.float16(-0.0)
    a = np.full(K.shape[3], 2.0 ** -24, np.float16)
    a[0] = 8
    c = np.zeros(K.shape[3], np.float16)
    c[0] = 8
    for base in (256, 650):                 # a prompt group and a group quantized while decoding
        K[1, 1, base + 2] = a
        K[1, 1, base + 3] = a[::-1]
        K[1, 1, base + 4:base + 44] = c


def test_signed_zeros_and_norm_order():
    """Bit-exact pages and pool on inputs where a stored zero min or scale could
    take either sign, and where only a channel-order fp64 norm sum gives the
    oracle's pool (the prompt's pages, then a quantize step while decoding)."""
    w = small("zeros-norms", L=(792, 792), steps=10, seed=77)
    run_case(w, plant=_plant_zeros_and_norm_ties, state_every_step=True)


def _keys_on_a_grid(K, V):
    """Keys rounded to the integers -2..2: most squared norms are small
    integers shared by many tokens."""
    K[...] = np.clip(np.rint(K.astype(np.float32)), -2.0, 2.0).astype(np.float16)


@pytest.mark.parametrize("rule", [0, 1])
def test_tied_keys_rank_by_position(rule):
    """Most keys tie, and many group keys equal the pool's largest key (such a
    token stays out of a full pool: the pool entry's position is lower). The
    prefill's segment selection and walk and the stepwise quantize steps rank
    ties by position as the oracle does; the largest-norm rule negates the
    keys (a zero norm gives -0)."""
    w = small(f"ties{rule}", B=3, Hkv=2, G=64, R=16, P=40, L=(1500, 2600), steps=70,
              seed=95 + rule, retention=rule)
    run_case(w, plant=_keys_on_a_grid, state_every_step=True)


def test_large_scores_are_safe():
    """Queries scaled x16: scores in the hundreds; the online softmax must
    rescale without overflow (softmax shift invariance)."""
    run_case(small("bigq", L=(900, 900), steps=3), q_scale=16.0)


def test_outlier_heavy_keys():
    """Many tiny-norm tokens (5%) in heavy outlier channels: the pool churns."""
    run_case(small("churn", L=(1500, 1500), steps=20, tok_prob=0.05, chan_scale=30.0),
             state_every_step=True)


@pytest.mark.parametrize("hq", [8, 2])
def test_decode_is_deterministic_and_repeatable(hq):
    # the last split to arrive merges, in split order, whichever split it is;
    # every head's arrival ticket is back at 0 after each launch
    import torch
    from decode_attention_ott_amd import OTTLayer
    w = small("det", B=2, Hq=hq, Hkv=2, L=(1200, 1200))
    K, V = synth.kv_all(w, 1200)
    layer = OTTLayer.for_workload(w, max_seq_len=1300)
    layer.prefill(torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), [1200, 1200])
    assert not layer.tickets().any()
    q = torch.from_numpy(synth.queries(w, 0)).cuda()
    outs = []
    for s in (0, 0, 5, 5, 3, 1, 5):
        layer.set_num_splits(s)
        outs.append(layer.decode(q).cpu().numpy().view(np.uint16))
        assert not layer.tickets().any(), s
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[2], outs[3])
    assert np.array_equal(outs[2], outs[6])


@pytest.mark.parametrize("hq,splits", [(8, 12), (2, 19)])
def test_split_merge_is_identical_over_many_launches(hq, splits):
    # the merging split reads the other splits' partials through device-coherent
    # loads after their ticket increments: 400 back-to-back launches, whose
    # splits finish in a different order each time, give bit-identical outputs
    import torch
    from decode_attention_ott_amd import OTTLayer
    w = small("merge-repeat", B=4, Hq=hq, Hkv=2, L=(6000, 6000))
    K, V = synth.kv_all(w, 6000)
    layer = OTTLayer.for_workload(w, max_seq_len=6100)
    layer.prefill(torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), [6000] * 4)
    layer.set_num_splits(splits)
    q = torch.from_numpy(synth.queries(w, 0)).cuda()
    first = layer.decode(q).clone()
    outs = torch.empty((400,) + tuple(first.shape), dtype=first.dtype, device=first.device)
    for i in range(400):
        layer.decode(q, out=outs[i])
    same = (outs.view(torch.int16) == first.view(torch.int16)).flatten(1).all(dim=1)
    assert bool(same.all()), f"launches differing from the first: {(~same).nonzero().flatten().tolist()[:10]}"
    assert not layer.tickets().any()


def test_capacity_error_leaves_state_unchanged():
    import torch
    from decode_attention_ott_amd import OTTLayer, OttError
    layer = OTTLayer(1, 1, 1, 128, 128, 32, 32, max_seq_len=400)
    k = torch.zeros(1, 1, 160, 128, dtype=torch.float16, device="cuda")
    layer.append(k, k)
    assert not layer.tickets().any()  # the first append clears them with the counters
    before = layer.counters().copy()
    with pytest.raises(OttError, match="CAPACITY"):
        layer.append(k[:, :, :1].contiguous(), k[:, :, :1].contiguous())
    assert np.array_equal(layer.counters(), before)
    assert layer.quantize_group() == 1
    layer.append(k[:, :, :1].contiguous(), k[:, :, :1].contiguous())
    assert layer.seq_state(0) == (161, 33, 128, 1)


def test_misaligned_rows_are_rejected_before_any_launch():
    """The kernels move fp16 rows in 16-byte pieces: inputs and outputs off a
    16-byte boundary are refused (OTT_ERR_INVALID_ARG) and leave the state as it was."""
    import torch
    from decode_attention_ott_amd import OTTLayer, OttError
    from decode_attention_ott_amd import _lib as L
    layer = OTTLayer(1, 2, 1, 128, 128, 32, 32, max_seq_len=400)
    buf = torch.zeros(2 * 8 * 128 + 8, dtype=torch.float16, device="cuda")
    k = buf[:8 * 128].view(1, 1, 8, 128)
    off = buf[1:1 + 8 * 128]  # 2 bytes past a 16-byte boundary
    assert off.data_ptr() % 16 == 2
    with pytest.raises(OttError, match="INVALID_ARG"):
        L.ott_append(layer.handle, off.data_ptr(), k.data_ptr(), [8], 8, 0)
    assert layer.seq_state(0) == (0, 0, 0, 0)
    layer.append(k, k)
    q = torch.zeros(1, 2, 128, dtype=torch.float16, device="cuda")
    out = torch.zeros(2 * 128 + 8, dtype=torch.float16, device="cuda")
    with pytest.raises(OttError, match="INVALID_ARG"):
        L.ott_decode(layer.handle, q.data_ptr(), out[1:].data_ptr(), 0)
    with pytest.raises(OttError, match="INVALID_ARG"):
        L.ott_decode(layer.handle, off.data_ptr(), out.data_ptr(), 0)
    torch.cuda.synchronize()
    assert layer.seq_state(0) == (8, 8, 0, 0)


@pytest.mark.parametrize("rule", [1, 2])
@pytest.mark.parametrize("G,R,P,Hq,steps", [(128, 32, 32, 2, 4), (64, 16, 8, 8, 70)])
def test_other_retention_rules(rule, G, R, P, Hq, steps):
    """Pool kept by largest Key norm (1) or a random key per position (2): the
    same bit-exact pool, pages and window as the oracle under that rule."""
    w = small(f"retain{rule}-g{G}h{Hq}", Hq=Hq, G=G, R=R, P=P, L=(700, 700), steps=steps,
              seed=10 * rule + G).with_(retention=rule)
    run_case(w, state_every_step=True)


def test_maximum_batch_and_pool():
    """The largest batch (512 sequences: the one-split decode deals the heads to
    CUs by size) and the largest pool (512 > G, so the first pages have no
    members), two query heads per KV head (a padded group), ragged lengths."""
    w = synth.Workload("max-b512-p512", 512, 2, 1, 128, 64, 16, 512, (100, 900), 3, seed=17)
    run_case(w, heads=[(0, 0), (137, 0), (300, 0), (511, 0)])


def test_maximum_head_ratio():
    """64 query heads per KV head (passes of 8 over every page)."""
    run_case(small("ratio64", B=1, Hq=128, Hkv=2, L=(700, 700), steps=2, seed=64))


# ---- the five layer shapes ---------------------------------------------------
def test_llama2_7b_full():
    """32 heads, 4096 context, 64 steps with a quantize at step 32: every head."""
    run_case(W["llama2-7b"])


def test_llama2_7b_b32_sampled():
    """Batch 32, ragged 3072-4096: sampled (sequence, head) pairs, all 64 steps."""
    heads = [(0, 0), (5, 31), (13, 7), (21, 16), (30, 3), (31, 30)]
    run_case(W["llama2-7b-b32"], heads=heads)


def test_mistral_gqa_sampled():
    """Batch 8 at 32K, 4 query heads per KV head, sampled heads: the window
    goes 128 -> 160, so step 31 quantizes every sequence at full shape."""
    run_case(W["mistral-7b-gqa"], heads=[(0, 0), (3, 5), (7, 7)], steps=34)


def test_llama2_13b_128k_sampled():
    """128K tokens, G = 256, R = 64, P = 128, sampled heads: the window goes
    256 -> 320, so step 63 quantizes at full shape (a 512th page)."""
    run_case(W["llama2-13b-128k"], heads=[(0, 0), (0, 23), (0, 39)], steps=66)


# ---- seeded random configurations ---------------------------------------------
def _random_configs(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([64, 128, 256]))
        R = int(rng.choice([0, 1, 7, 32, 64]))
        P = int(rng.choice([0, 1, 5, 32, 100, G + 7]))
        Hkv = int(rng.integers(1, 4))
        nq = int(rng.choice([1, 2, 3, 4, 5, 8]))
        B = int(rng.integers(1, 5))
        lengths = [int(x) for x in rng.integers(1, 4 * G + R + 40, size=B)]
        steps = int(rng.integers(1, 83))
        splits = [0, int(rng.integers(1, 9))]
        out.append((i, G, R, P, Hkv, nq, B, lengths, steps, splits))
    return out


@pytest.mark.parametrize("case", _random_configs(), ids=lambda c: f"rand{c[0]}")
def test_random_configurations(case):
    """Seeded draws over G, R, P, heads, ratio, batch, ragged lengths (from 1),
    step counts that cross quantize steps, and split counts."""
    i, G, R, P, Hkv, nq, B, lengths, steps, splits = case
    w = synth.Workload(f"rand{i}", B, Hkv * nq, Hkv, 128, G, R, P, (1, 1), steps, seed=500 + i)
    run_case(w, lengths=lengths, splits=splits, state_every_step=steps <= 16)
