"""GPU test of ott_fp16_decode_noalloc, the fp16 baseline decode for callers
that cannot allocate: its split partials live in the library's own scratch.
Checked against ott_fp16_decode (caller workspace) on two calls in a row, the
second on a smaller input, through the C ABI."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(B, Hq, Hkv, lens, seed):
    import torch
    w = synth.Workload(f"noalloc{seed}", B, Hq, Hkv, 128, 128, 32, 32, (1, 1), 1, seed=seed)
    K, V = synth.kv_all(w, max(lens))
    q = synth.queries(w, 0)
    dev = torch.device("cuda:0")
    return (torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev),
            torch.from_numpy(q).to(dev), [int(x) for x in lens])


def _run(L, noalloc, Kd, Vd, qd, lens, S, work=None):
    import torch
    B, Hkv, max_len, d = Kd.shape
    Hq = qd.shape[1]
    out = torch.full_like(qd, float("nan"))
    sp = int(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        L.ott_fp16_decode_noalloc(B, Hq, Hkv, d, Kd.data_ptr(), Vd.data_ptr(), max_len, lens,
                                  qd.data_ptr(), out.data_ptr(), 0.0, S, sp)
    else:
        nb = L.ott_fp16_decode_workspace(B, Hq, 64)
        L.ott_fp16_decode(B, Hq, Hkv, d, Kd.data_ptr(), Vd.data_ptr(), max_len, lens,
                          qd.data_ptr(), out.data_ptr(), 0.0, work.data_ptr(), nb, S, sp)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_matches_the_workspace_entry_point():
    import torch
    from decode_attention_ott_amd import _lib as L
    from tests.parity import compare_outputs
    work = torch.empty(L.ott_fp16_decode_workspace(8, 32, 64), dtype=torch.uint8, device="cuda")
    big = _case(8, 32, 8, [3000, 2047, 1, 4096, 2500, 300, 4000, 3999], seed=91)
    small = _case(2, 4, 2, [700, 129], seed=92)
    for name, (Kd, Vd, qd, lens) in (("big", big), ("small", small)):
        for S in (5, 1, 0):
            got = _run(L, True, Kd, Vd, qd, lens, S)
            want = _run(L, False, Kd, Vd, qd, lens, S, work)
            assert np.isfinite(got).all(), (name, S)
            if S > 0:  # same kernels, same split count: the same bits
                assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), (name, S)
            else:      # automatic split counts may differ (scratch vs workspace size)
                compare_outputs(got.reshape(-1, 128), want.reshape(-1, 128).astype(np.float64),
                                f"{name} auto splits")


def test_noalloc_rejects_more_splits_than_its_scratch():
    import torch
    from decode_attention_ott_amd import _lib as L
    Kd, Vd, qd, lens = _case(64, 32, 8, [200] * 64, seed=93)
    per_split = L.ott_fp16_decode_workspace(64, 32, 1 + 1) // 2
    too_many = L.FP16_DECODE_SCRATCH_BYTES // per_split + 1
    out = torch.zeros_like(qd)
    with pytest.raises(L.OttError, match="SCRATCH_TOO_SMALL"):
        L.ott_fp16_decode_noalloc(64, 32, 8, 128, Kd.data_ptr(), Vd.data_ptr(), 200, lens,
                                  qd.data_ptr(), out.data_ptr(), 0.0, too_many,
                                  int(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert not out.any()  # nothing was enqueued
