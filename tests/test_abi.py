"""CPU-side checks of the C-ABI library: it loads, exports every symbol the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?[\w\*]+\s+\**(ott_\w+)\s*\(", text, re.M))
    return names


def test_library_exports_every_declared_symbol():
    from decode_attention_ott_amd import _lib as L
    declared = _declared_symbols()
    assert {"ott_init", "ott_append", "ott_quantize_group", "ott_decode"} <= declared
    assert declared == set(L.EXPORTS)
    for name in declared:
        assert hasattr(L.lib, name), name


def _cfg(**kw):
    from decode_attention_ott_amd import _lib as L
    base = dict(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=128, group_size=128, residual=32,
                pool_size=32, max_seq_len=1000, sm_scale=0.0)
    base.update(kw)
    return L.ott_config_t(**base)


def _sizing(cfg):
    from decode_attention_ott_amd import _lib as L
    req = ctypes.c_size_t(0)
    st = L.lib.ott_init(ctypes.byref(cfg), None, 0, ctypes.byref(req), None)
    return st, req.value


def test_sizing_matches_layout_formula():
    st, req = _sizing(_cfg())
    assert st == 0
    B, Hkv, Hq, d, G, R, P, NB = 2, 2, 4, 128, 128, 32, 32, 8   # NB = ceil(1000/128)
    al = lambda x: (x + 255) // 256 * 256
    page = G * d // 4 * 2 + 4 * d + 4 * G
    assert page == 9216
    S = max(4, min(64, (8192 + B * Hkv - 1) // (B * Hkv)))
    want = (al(B * Hkv * 16) + al(B * Hkv * NB * page) + al(B * Hkv * NB * G * 4)
            + al(B * Hkv * NB * 4) + 2 * al(2 * B * Hkv * P * d * 2) + al(2 * B * Hkv * P * 4)
            + al(2 * B * Hkv * P * 8) + 2 * al(B * Hkv * (R + G) * d * 2)
            + al(B * Hq * S * (2 + d) * 4) + al(B * Hkv * 4))
    assert req == want


def test_any_head_ratio_up_to_64_is_accepted():
    for hq, hkv in [(6, 2), (10, 2), (128, 2), (7, 7)]:
        st, _ = _sizing(_cfg(num_q_heads=hq, num_kv_heads=hkv))
        assert st == 0, (hq, hkv)


@pytest.mark.parametrize("bad,status", [
    (dict(head_dim=64), 2), (dict(group_size=96), 2), (dict(group_size=32), 2),
    (dict(num_q_heads=3), 1), (dict(num_q_heads=130, num_kv_heads=2), 2),
    (dict(batch=0), 1), (dict(batch=513), 2), (dict(pool_size=-1), 1), (dict(pool_size=600), 2),
    (dict(residual=-1), 1), (dict(max_seq_len=0), 1), (dict(sm_scale=float("nan")), 1),
    (dict(retention=3), 1), (dict(retention=-1), 1),
    (dict(batch=1, num_q_heads=65536, num_kv_heads=65536), 2),
])
def test_bad_configs_are_rejected(bad, status):
    st, _ = _sizing(_cfg(**bad))
    assert st == status


def test_calls_validate_before_any_gpu_work():
    from decode_attention_ott_amd import _lib as L
    lib = L.lib
    cfg = _cfg()
    h = ctypes.c_void_p(0)
    # creating a handle without an arena is an argument error (no HIP call)
    assert lib.ott_init(ctypes.byref(cfg), None, 0, None, ctypes.byref(h)) == 1
    # an undersized or misaligned arena is rejected before any HIP call
    assert lib.ott_init(ctypes.byref(cfg), ctypes.c_void_p(4096), 16, None, ctypes.byref(h)) == 3
    assert lib.ott_init(ctypes.byref(cfg), ctypes.c_void_p(4096 + 8), 1 << 40, None,
                        ctypes.byref(h)) == 3
    n = (ctypes.c_int32 * 2)(1, 1)
    assert lib.ott_append(None, None, None, n, 1, None) == 1
    assert lib.ott_quantize_group(None, None, None) == 1
    assert lib.ott_decode(None, None, None, None) == 1
    assert lib.ott_get_layout(None, None) == 1
    assert lib.ott_set_num_splits(None, 1) == 1
    lib.ott_destroy(None)
    assert L.ott_status_string(4) == "window or sequence capacity exceeded"


def test_fp16_baseline_validates_before_any_gpu_work():
    from decode_attention_ott_amd import _lib as L
    lib = L.lib
    ln = (ctypes.c_int32 * 2)(10, 10)
    P = ctypes.c_void_p(4096)
    args = dict(batch=2, hq=4, hkv=2, d=128, k=P, v=P, max_len=16, ln=ln, q=P, out=P, sm=0.0,
                work=None, wb=0, s=1, st=None)

    def call(**kw):
        a = dict(args, **kw)
        return lib.ott_fp16_decode(a["batch"], a["hq"], a["hkv"], a["d"], a["k"], a["v"],
                                   a["max_len"], a["ln"], a["q"], a["out"], a["sm"], a["work"],
                                   a["wb"], a["s"], a["st"])
    assert call(batch=0) == 1
    assert call(hq=3) == 1                       # not a multiple of the KV heads
    assert call(d=64) == 2                       # head_dim must be 128
    assert call(k=None) == 1
    assert call(q=ctypes.c_void_p(4096 + 8)) == 1  # misaligned
    assert call(ln=(ctypes.c_int32 * 2)(10, 17)) == 5  # a length above max_len
    assert call(ln=(ctypes.c_int32 * 2)(0, 3)) == 5    # an empty sequence
    assert call(s=4) == 3                        # splits without a workspace
    assert call(s=-1) == 1
    assert L.ott_fp16_decode_workspace(2, 4, 1) == 0
    assert L.ott_fp16_decode_workspace(2, 4, 3) == 2 * 4 * 3 * 130 * 4


def test_prefill_validates_before_any_gpu_work():
    from decode_attention_ott_amd import _lib as L
    n = (ctypes.c_int32 * 2)(10, 10)
    assert L.lib.ott_prefill(None, None, None, n, 10, None) == 1


def test_init_enqueues_nothing_and_host_counts_are_checked():
    """ott_init neither reads nor writes the arena and enqueues no work: a handle
    over an arena address that is never dereferenced is created here, where no
    HIP call could succeed. The binding refuses host count lists whose length is
    not the handle's batch (the C side reads exactly `batch` entries); a decode
    of empty sequences and a quantize with no full window enqueue nothing."""
    from decode_attention_ott_amd import _lib as L
    cfg = _cfg()
    need = L.ott_init(cfg, None, 0, sizing_only=True)
    h, req = L.ott_init(cfg, 1 << 20, need)
    try:
        assert req == need
        with pytest.raises(ValueError, match="batch is 2"):
            L.ott_append(h, 4096, 4096, [1], 1, 0)
        with pytest.raises(ValueError, match="batch is 2"):
            L.ott_prefill(h, 4096, 4096, [5, 5, 5], 5, 0)
        with pytest.raises(L.OttError, match="STATE"):
            L.ott_decode(h, 4096, 4096, 0)
        assert L.ott_quantize_group(h, 0) == 0
        assert L.ott_get_seq_state(h, 1) == (0, 0, 0, 0)
        lay = L.ott_get_layout(h)
        assert lay.arena_bytes == need and lay.off_partials < need
    finally:
        L.ott_destroy(h)


def test_one_hip_runtime_whatever_the_import_order():
    # the binding imported before torch must not map a second HIP runtime
    # (torch's copy and the system copy share their sonames)
    import subprocess
    import sys
    code = ("import decode_attention_ott_amd, torch\n"
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps')"
            " if 'libamdhip64' in l or 'libhsa-runtime64' in l}))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    libs = eval(r.stdout.strip().splitlines()[-1])
    hip = [x for x in libs if "libamdhip64" in x]
    hsa = [x for x in libs if "libhsa-runtime64" in x]
    assert len(hip) == 1 and len(hsa) == 1, libs
