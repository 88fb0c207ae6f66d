"""Shared driver of the GPU parity tests: the HIP library (through the C ABI)
and the CPU oracle run the same seeded inputs; state is compared bit for bit
and decode outputs within the stated tolerance."""
from __future__ import annotations

import sys
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

import synth
from oracle import ott_oracle as O

MAX_ABS = 2e-3   # fp16 output vs fp64 oracle, per element
REL_L2 = 1e-3    # ||gpu - oracle|| / ||oracle|| over the compared rows of one step


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def first_diff(a: bytes, b: bytes) -> int:
    for i, (x, y) in enumerate(zip(a, b)):
        if x != y:
            return i
    return -1


def check_state(layer, orc: O.OTTOracle, heads: Iterable[Tuple[int, int]], where: str) -> None:
    """Bit-exact comparison of counters, pages, member positions, pool and window."""
    G, d = layer.G, layer.d
    ctr = layer.counters()
    for b, h in heads:
        st = orc.head(b, h)
        Lg, r, ring_head, nb = layer.seq_state(b)
        assert (Lg, r, nb) == (st.L, len(st.recent), len(st.pages)), (where, b, h)
        assert tuple(ctr[b, h]) == (Lg, r, ring_head, nb), (where, b, h, ctr[b, h])
        if nb:
            got = layer.pages_of_head(b, h, nb)
            ppos = layer.page_positions(b, h, nb)
            for n, pg in enumerate(st.pages):
                want = O.pack_page(pg, G, d)
                g = got[n].tobytes()
                if g != want:
                    i = first_diff(g, want)
                    raise AssertionError(f"{where}: page bytes differ at (b={b}, kvh={h}, page={n})"
                                         f" byte {i} of {len(want)}: gpu {g[i]} oracle {want[i]}")
                assert ppos[n, :pg.n_valid].tolist() == pg.pos.tolist(), (where, b, h, n)
                assert (ppos[n, pg.n_valid:] == -1).all(), (where, b, h, n)
        pos, n2, pk, pv = layer.pool(b, h)
        assert pos.tolist() == [e.pos for e in st.pool], (where, b, h, "pool membership")
        assert np.array_equal(n2, np.array([e.key for e in st.pool], np.float64)), (where, b, h)
        if st.pool:
            assert np.array_equal(pk.view(np.uint16), np.stack([e.k for e in st.pool]).view(np.uint16))
            assert np.array_equal(pv.view(np.uint16), np.stack([e.v for e in st.pool]).view(np.uint16))
        wk, wv = layer.window(b, h)
        if st.recent:
            assert np.array_equal(wk.view(np.uint16), np.stack([e.k for e in st.recent]).view(np.uint16))
            assert np.array_equal(wv.view(np.uint16), np.stack([e.v for e in st.recent]).view(np.uint16))


def compare_outputs(gpu: np.ndarray, ref: np.ndarray, where: str) -> Tuple[float, float]:
    g = gpu.astype(np.float64)
    err = np.abs(g - ref)
    mx = float(err.max())
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30))
    assert np.isfinite(g).all(), f"{where}: non-finite output"
    assert mx <= MAX_ABS and rel <= REL_L2, f"{where}: max abs {mx:.3e}, rel L2 {rel:.3e}"
    return mx, rel


def run_case(w: synth.Workload, steps: Optional[int] = None,
             heads: Optional[Sequence[Tuple[int, int]]] = None,
             lengths: Optional[Sequence[int]] = None, splits: Optional[Sequence[int]] = None,
             q_scale: float = 1.0, state_every_step: bool = False, check_prefill: bool = True,
             plant=None, step_calls: Optional[str] = None):
    """Prefill + `steps` decode steps on the GPU and in the oracle.

    heads: the (sequence, KV head) pairs the oracle follows (default: all).
    splits: split-K factors each decode is run with (default: automatic).
    plant: optional plant(K, V) that edits the drawn fp16 [B, Hkv, pos, d] inputs
    in place before either side sees them.
    step_calls: None = each step as ott_append, ott_quantize_group, ott_decode;
    "step" = each step as one ott_step (its decode with the first split count,
    the others as ott_decode afterwards); "mixed" = ott_step on even steps.
    Returns the worst (max abs, rel L2) seen.
    """
    import torch
    from decode_attention_ott_amd import OTTLayer

    steps = w.steps if steps is None else steps
    lengths = np.asarray(synth.prefill_lengths(w) if lengths is None else lengths, np.int64)
    n_pos = int(lengths.max()) + steps
    log(f"[parity] {w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} G={w.group_size}"
        f" R={w.residual} P={w.pool_size} L={lengths.min()}..{lengths.max()} steps={steps}"
        f" splits={splits} q_scale={q_scale} calls={step_calls or 'separate'}")
    K, V = synth.kv_all(w, n_pos)
    if plant is not None:
        plant(K, V)
    if heads is None:
        heads = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    heads = [(int(b), int(h)) for b, h in heads]
    nq = w.num_q_heads // w.num_kv_heads
    qrows = [(b, h * nq + i) for b, h in heads for i in range(nq)]

    layer = OTTLayer.for_workload(w, max_seq_len=n_pos)
    Kd = torch.from_numpy(K).cuda()
    Vd = torch.from_numpy(V).cuda()
    layer.prefill(Kd, Vd, lengths)
    orc = O.OTTOracle.for_workload(w, heads)
    for b, h in heads:
        O.run_prefill(orc.head(b, h), K[b, h, :lengths[b]], V[b, h, :lengths[b]])
    if check_prefill:
        check_state(layer, orc, heads, "after prefill")
    log(f"[parity] {w.name}: prefill state bit-exact on {len(heads)} heads")

    worst = (0.0, 0.0)
    bidx = np.arange(w.batch)
    for t in range(steps):
        pos = lengths + t
        kt = np.ascontiguousarray(K[bidx, :, pos][:, :, None, :])
        vt = np.ascontiguousarray(V[bidx, :, pos][:, :, None, :])
        q = (synth.queries(w, t).astype(np.float32) * np.float32(q_scale)).astype(np.float16)
        qd = torch.from_numpy(q).cuda()
        fused = step_calls == "step" or (step_calls == "mixed" and t % 2 == 0)
        split_list = list(splits or [0])
        if fused:
            layer.set_num_splits(split_list[0])
            out_step, _ = layer.step(torch.from_numpy(kt).cuda(), torch.from_numpy(vt).cuda(), qd)
        else:
            layer.append(torch.from_numpy(kt).cuda(), torch.from_numpy(vt).cuda())
            layer.quantize_group()
        for b, h in heads:
            O.step(orc.head(b, h), K[b, h, pos[b]], V[b, h, pos[b]])
        if state_every_step:
            check_state(layer, orc, heads, f"step {t}")
        ref = np.stack([orc.decode(b, qh, q[b, qh]) for b, qh in qrows])
        for i, s in enumerate(split_list):
            if fused and i == 0:
                out = out_step.cpu().numpy()
            else:
                layer.set_num_splits(s)
                out = layer.decode(qd).cpu().numpy()
            got = np.stack([out[b, qh] for b, qh in qrows])
            mx, rel = compare_outputs(got, ref, f"{w.name} step {t} splits {s}"
                                                + (" (ott_step)" if fused and i == 0 else ""))
            worst = (max(worst[0], mx), max(worst[1], rel))
    layer.set_num_splits(0)
    check_state(layer, orc, heads, "end")
    log(f"[parity] {w.name}: {steps} steps ok, worst max abs {worst[0]:.2e}, rel L2 {worst[1]:.2e}")
    layer.close()
    return worst
