"""GPU parity of ott_step, the fused decode step (append one token per
sequence, quantize full windows, decode): the same bit-exact state and the
same outputs, within tolerance, as the oracle stepping the method's stages,
through the C ABI. Covers the one-split writer (the decode work-group stores
the new token) and the split-K writer (the split merge stores it), one head
and grouped query heads, a quantize step inside the fused step, R = 0 and a
fresh handle (the separate calls), and ott_step mixed with the separate calls."""
import numpy as np
import pytest

import synth
from tests.parity import run_case

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def small(name, B=2, Hq=2, Hkv=2, G=128, R=32, P=32, L=(400, 400), steps=8, seed=11, **kw):
    return synth.Workload(name, B, Hq, Hkv, 128, G, R, P, L, steps, seed, **kw)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_step_tiny_every_step():
    run_case(W["tiny"], state_every_step=True, step_calls="step", steps=8)


# windows are 8 tokens short of full after the prompt, so step 7 quantizes
@pytest.mark.parametrize("G,R,P,L,Hq,splits", [
    (128, 32, 32, (792, 792), 2, [1]),     # one split: the decode work-group writes
    (128, 32, 32, (792, 792), 2, [5, 0]),  # split-K: the merge writes
    (128, 32, 32, (792, 792), 8, [1]),     # grouped query heads, one split
    (128, 32, 32, (792, 792), 8, [3, 0]),  # grouped query heads, split-K
    (64, 1, 8, (313, 313), 2, [1, 2]),     # R = 1: the smallest window that quantizes before the append
    (64, 2, 8, (314, 314), 4, [2, 1]),     # R = 2
    (256, 64, 128, (1082, 1082), 2, [0]),  # G = 256
    (256, 64, 128, (1082, 1082), 8, [0]),  # G = 256, grouped
    (128, 0, 32, (632, 632), 2, [0, 1]),   # R = 0: the separate calls
    (128, 32, 160, (792, 792), 2, [1]),    # P > G: first pages empty
])
def test_step_parameters(G, R, P, L, Hq, splits):
    run_case(small(f"step-g{G}r{R}p{P}h{Hq}", Hq=Hq, G=G, R=R, P=P, L=L, steps=10,
                   seed=G + R + P + Hq), splits=splits, state_every_step=True, step_calls="step")


def test_step_ragged_batch_many_quantizes():
    """Ragged lengths from 1 and 80 steps: every sequence crosses a quantize
    step at its own step (some before any page exists); state after every step."""
    w = small("step-ragged", B=6, Hq=8, Hkv=2, G=64, R=16, P=8, L=(1, 1), steps=80)
    run_case(w, lengths=[1, 40, 79, 80, 200, 333], splits=[0, 3], step_calls="step",
             state_every_step=True)


def test_step_quantizes_complete_groups_early():
    """R = 48 > G / 2 with 8 sequences at spread phases: a window's group is
    complete up to 47 steps before it is due, so a quantize launch covers
    several windows, whose pages stay invisible until their due steps; the
    state must match the oracle after every step."""
    w = small("step-early", B=8, Hq=4, Hkv=2, G=64, R=48, P=16, L=(1, 1), steps=130, seed=9)
    run_case(w, lengths=[500, 507, 514, 521, 530, 541, 552, 563], splits=[0],
             step_calls="step", state_every_step=True)


def test_step_mixed_with_separate_calls():
    w = small("step-mixed", B=3, Hq=4, Hkv=2, G=64, R=8, P=16, L=(300, 300), steps=60, seed=5)
    run_case(w, lengths=[150, 260, 301], splits=[0, 2], step_calls="mixed", state_every_step=True)


def test_step_on_the_batch_32_shape():
    """The bench's shape: batch 32 x 32 heads, ragged 3072-4096, 40 fused steps
    (several quantize steps), sampled heads."""
    heads = [(0, 0), (5, 31), (13, 7), (21, 16), (30, 3), (31, 30)]
    run_case(W["llama2-7b-b32"], heads=heads, steps=40, step_calls="step")


def test_step_from_a_fresh_handle_and_a_full_window():
    import torch
    from decode_attention_ott_amd import OTTLayer, OttError
    from oracle import ott_oracle as O
    from tests.parity import check_state, compare_outputs
    w = small("step-fresh", B=2, Hq=2, Hkv=1, G=64, R=8, P=4, L=(1, 1), steps=1)
    K, V = synth.kv_all(w, 200)
    layer = OTTLayer.for_workload(w, max_seq_len=200)
    orc = O.OTTOracle.for_workload(w)
    for t in range(100):  # the first step runs on a fresh handle (no counters yet)
        kt = torch.from_numpy(np.ascontiguousarray(K[:, :, t:t + 1])).cuda()
        vt = torch.from_numpy(np.ascontiguousarray(V[:, :, t:t + 1])).cuda()
        q = synth.queries(w, t)
        out, _ = layer.step(kt, vt, torch.from_numpy(q).cuda())
        for b in range(2):
            O.step(orc.head(b, 0), K[b, 0, t], V[b, 0, t])
        ref = np.stack([orc.decode(b, qh, q[b, qh]) for b in range(2) for qh in range(2)])
        compare_outputs(out.cpu().numpy().reshape(4, 128), ref, f"fresh step {t}")
    check_state(layer, orc, [(0, 0), (1, 0)], "after 100 fused steps")
    # a window left full by ott_append (no quantize yet) is refused, nothing enqueued
    n = layer.R + layer.G - layer.seq_state(0)[1]
    layer.append(torch.zeros(2, 1, n, 128, dtype=torch.float16, device="cuda"),
                 torch.zeros(2, 1, n, 128, dtype=torch.float16, device="cuda"))
    before = layer.counters().copy()
    z = torch.zeros(2, 1, 1, 128, dtype=torch.float16, device="cuda")
    with pytest.raises(OttError, match="STATE"):
        layer.step(z, z, torch.zeros(2, 2, 128, dtype=torch.float16, device="cuda"))
    assert np.array_equal(layer.counters(), before)


def _step_random_configs():
    from tests.test_gpu_parity import _random_configs
    return _random_configs(seed=4048)


@pytest.mark.parametrize("case", _step_random_configs(), ids=lambda c: f"srand{c[0]}")
def test_step_random_configurations(case):
    """The seeded random configurations of the separate-call parity tests
    (G, R from 0, P, heads, ratio, batch, ragged lengths from 1, step counts
    across quantize steps, split counts), each step as one ott_step."""
    i, G, R, P, Hkv, nq, B, lengths, steps, splits = case
    w = synth.Workload(f"srand{i}", B, Hkv * nq, Hkv, 128, G, R, P, (1, 1), steps, seed=900 + i)
    run_case(w, lengths=lengths, splits=splits, state_every_step=steps <= 16, step_calls="step")
