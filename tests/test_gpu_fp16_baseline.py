"""GPU parity of the fp16 baseline decode (ott_fp16_decode through the C ABI)
against the oracle's textbook attention over the same fp16 K/V rows.

Tolerance as for the OTT decode: max abs 2e-3, relative L2 1e-3 on the fp16
outputs against fp64.
"""
import numpy as np
import pytest

import synth
from oracle import ott_oracle as O
from tests.parity import compare_outputs, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(w, lens, splits, heads=None, max_len=None):
    import torch
    from decode_attention_ott_amd import _lib as L
    lens = np.asarray(lens, np.int64)
    max_len = int(max_len or lens.max())
    K, V = synth.kv_all(w, max_len)
    q = synth.queries(w, 0)
    dev = torch.device("cuda:0")
    Kd, Vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    qd = torch.from_numpy(q).to(dev)
    sm = 1.0 / np.sqrt(w.head_dim)
    nq = w.num_q_heads // w.num_kv_heads
    if heads is None:
        heads = [(b, qh) for b in range(w.batch) for qh in range(w.num_q_heads)]
    refs = {(b, qh): O.textbook_attention(q[b, qh], K[b, qh // nq, :lens[b]], V[b, qh // nq, :lens[b]], sm)
            for b, qh in heads}
    stream = torch.cuda.current_stream()
    for s in splits:
        outd = torch.full((w.batch, w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float16,
                          device=dev)
        nbytes = L.ott_fp16_decode_workspace(w.batch, w.num_q_heads, max(s, 64))
        work = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=dev)
        L.ott_fp16_decode(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, Kd.data_ptr(),
                          Vd.data_ptr(), max_len, lens, qd.data_ptr(), outd.data_ptr(), 0.0,
                          work.data_ptr(), nbytes, s, int(stream.cuda_stream))
        torch.cuda.synchronize()
        out = outd.cpu().numpy()
        gpu = np.stack([out[b, qh] for b, qh in heads])
        ref = np.stack([refs[k] for k in heads])
        mx, rel = compare_outputs(gpu, ref, f"{w.name} splits={s}")
        log(f"[fp16] {w.name} lens={lens.min()}..{lens.max()} splits={s}: max abs {mx:.2e}, rel L2 {rel:.2e}")


def small(name, B, Hq, Hkv, seed):
    return synth.Workload(name, B, Hq, Hkv, 128, 128, 32, 32, (1, 1), 1, seed)


@pytest.mark.parametrize("Hq,Hkv,lens", [
    (4, 4, [1, 17, 300]),          # one head per KV head; length 1 and a ragged tail
    (8, 2, [513, 1000]),           # 4 query heads per KV head
    (16, 2, [700, 33]),            # 8 per KV head
    (4, 2, [250, 16]),             # 2 per KV head; a length that is a whole chunk
    (6, 2, [129, 400]),            # 3 per KV head (one head per pass)
    (32, 2, [300, 301]),           # 16 per KV head (two passes of 8)
])
def test_shapes_and_split_counts(Hq, Hkv, lens):
    _run(small(f"fp16-{Hq}x{Hkv}", len(lens), Hq, Hkv, seed=Hq + Hkv), lens, splits=[1, 2, 5, 0])


def test_rows_past_the_length_are_not_read():
    """max_len above every length: the rows past each h_len hold other tokens
    and must not enter the result."""
    _run(small("fp16-maxlen", 2, 4, 2, seed=7), [100, 37], splits=[1, 3], max_len=512)


def test_llama2_7b_b32_sampled():
    """Batch 32, 32 heads, ragged 3072-4096 (the OTT bench's shape)."""
    w = synth.WORKLOADS["llama2-7b-b32"]
    lens = synth.prefill_lengths(w)
    _run(w, lens, splits=[0, 1], heads=[(0, 0), (7, 31), (19, 12), (31, 5)])


def test_mistral_gqa_sampled():
    w = synth.WORKLOADS["mistral-7b-gqa"]
    _run(w, synth.prefill_lengths(w), splits=[0], heads=[(0, 0), (3, 17), (7, 31)])


def test_llama2_13b_128k_sampled():
    """One sequence of 131072 tokens, 40 heads: many splits per head."""
    w = synth.WORKLOADS["llama2-13b-128k"]
    _run(w, synth.prefill_lengths(w), splits=[0, 64], heads=[(0, 0), (0, 39)])


def test_bad_arguments_are_rejected():
    import torch
    from decode_attention_ott_amd import _lib as L, OttError
    x = torch.zeros(1, 1, 8, 128, dtype=torch.float16, device="cuda")
    q = torch.zeros(1, 1, 128, dtype=torch.float16, device="cuda")
    with pytest.raises(OttError, match="STATE"):
        L.ott_fp16_decode(1, 1, 1, 128, x.data_ptr(), x.data_ptr(), 8, [9], q.data_ptr(),
                          q.data_ptr(), 0.0, None, 0, 1, 0)
    with pytest.raises(OttError, match="ARENA_TOO_SMALL"):
        L.ott_fp16_decode(1, 1, 1, 128, x.data_ptr(), x.data_ptr(), 8, [8], q.data_ptr(),
                          q.data_ptr(), 0.0, None, 0, 2, 0)
