"""Benchmark of the OTT decode step on one MI355X.

A step is the whole hot path for one batch: append one token per sequence,
quantize any full window, decode one query per (sequence, query head), in one
ott_step call (--separate-calls: the three calls).
Default workload: Llama-2-7B-shaped layer, batch 32, 32 heads, ragged context
3072-4096, G=128, R=32, P=32. Several independent layer states are stepped
round-robin so that consecutive steps touch different memory (the 256 MB
Infinity Cache cannot hold the working set between visits). Their prompt
lengths are moved by less than G/2 so that the states take turns at the
quantize step: any window of timed steps then holds the steady-state share of
quantize steps (one every G/B steps at ragged lengths), and the line reports
how many the timed steps held. (ott_step runs the quantize work of every
window whose group is complete in one launch, so launches are rarer.)

Prints one JSON line (rank 0, N=1 only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "OTT decode-attention tokens/s + achieved HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBS = 8000.0
# sources of the one-head decode kernel (its split merge included); the
# grouped-head kernel adds its own file
MHA_SOURCES = ("decode_attention_ott_amd/csrc/ott_decode.hip",
               "decode_attention_ott_amd/csrc/ott_decode_common.h",
               "decode_attention_ott_amd/csrc/ott_mx.h",
               "decode_attention_ott_amd/csrc/ott_device.h",
               "decode_attention_ott_amd/csrc/ott_kernels.h")
GQA_SOURCES = MHA_SOURCES + ("decode_attention_ott_amd/csrc/ott_decode_gqa.hip",)


def algorithmic_decode_bytes(layer) -> int:
    """Bytes one decode must move: per (sequence, KV head) 512 per page (K min/scale),
    68 per quantized token (32 B K codes + 32 B V codes + 4 B V min/scale), 512 per
    fp16 pool or window token (K and V); plus 512 per query head (q in, out)."""
    total = 0
    for b in range(layer.B):
        L, r_cnt, _, nb = layer.seq_state(b)
        pc = min(layer.P, layer.G * nb)
        nq = L - pc - r_cnt
        total += layer.Hkv * (512 * nb + 68 * nq + 512 * (pc + r_cnt))
    return total + 512 * layer.B * layer.Hq


def auto_states(w, lengths) -> int:
    """States per lap so that one lap reads >= 3 x 256 MB (3..8), raised to the
    next count coprime with the quantize period (see staggered_lengths)."""
    page = w.group_size * w.head_dim // 2 + 4 * w.head_dim + 4 * w.group_size
    per_head = [(int(L) // w.group_size) * page + (w.pool_size + w.residual + w.group_size // 2) * 4 * w.head_dim
                for L in lengths]
    state = w.num_kv_heads * sum(per_head)
    n = int(min(8, max(3, -(-3 * 256e6 // max(state, 1)))))
    period = quantize_period(w)
    while period and math.gcd(n, period) != 1:
        n += 1
    return n


def quantize_period(w) -> int:
    """Steps between two quantize steps of one state in the full-step timing: G / B
    when ragged lengths spread the B windows evenly over the G phases (0 when B
    does not divide G), G when every sequence has the same length (the windows
    fill together)."""
    G, B = w.group_size, w.batch
    if w.prefill[0] == w.prefill[1]:
        return G
    return G // B if G % B == 0 else 0


def staggered_lengths(w, lengths, n_states: int):
    """Per-state prompt lengths for the full-step timing. A window quantizes
    every G appended tokens, at a step fixed by its length mod G. Each length
    is moved by less than G/2 (kept inside a ragged workload's range by whole
    groups) so that the states, stepped round-robin, take turns at quantizing:
    - ragged lengths: within a state the B sequences reach a full window at
      evenly spread steps, one every Pi = G/B steps;
    - equal lengths: a state's B windows stay in step (they fill together, as
      in the workload), Pi = G;
    with S states coprime to Pi, state s's quantize steps fall on the global
    steps i = S t + s that are multiples of Pi. Every Pi-th global step then
    quantizes (one sequence, or a whole batch of equal lengths), whatever the
    first timed step, so a window of K steps holds K/Pi (+-1) quantize steps:
    the steady-state share. Returns [n_states][B] int64."""
    G, R, C, B = w.group_size, w.residual, w.residual + w.group_size, w.batch
    lo, hi = w.prefill
    L0 = np.asarray(lengths, np.int64)
    period = quantize_period(w)

    def first_due(L):  # state-step at which a prompt of L tokens first quantizes
        r = L - G * ((L - R) // G) if L >= R + G else L
        return (C - 1 - r) % G

    spread = lo != hi
    order = np.argsort([first_due(int(L)) for L in L0], kind="stable")
    out = []
    for s in range(n_states):
        a_s = (s * G) // (B * n_states) if spread else (s * G) // n_states
        if period:
            a_s = next(a for a in range(period) if (n_states * a + s) % period == 0)
        Ls = L0.copy()
        for k, b in enumerate(order):
            # this sequence's quantize step mod G
            tau = (a_s + (k * G) // B) % G if spread else a_s
            r = R + (G - 1 - tau) % G            # window after the prompt, in [R, C)
            L = int(L0[b])
            d = (r - L) % G
            if d >= G // 2:
                d -= G
            L += d
            while L > hi and L - G >= max(lo, R + G):
                L -= G
            while L < lo and L + G <= hi:
                L += G
            Ls[b] = L
        out.append(Ls)
    return out


def decode_kernel_name(w) -> str:
    """The decode kernel a workload's decode-only loop launches, as rocprofv3
    names it (with several splits, the last split of each head to finish merges
    them inside the same launch; the fused step launches the same template with
    `true`)."""
    nq = w.num_q_heads // w.num_kv_heads
    if nq == 1:
        return f"decode_kernel<{w.group_size}, false>"
    na = 2 if nq % 8 == 0 else 1  # groups of 4 query heads per pass
    return f"decode_gqa_kernel<{w.group_size}, {na}, false>"


def decode_sources(w):
    return MHA_SOURCES if w.num_q_heads == w.num_kv_heads else GQA_SOURCES


def kernel_source_hash(w, read=None) -> str:
    """Hash of the sources the workload's decode kernels are built from (read(path)
    -> bytes may supply another version of them)."""
    h = hashlib.sha256()
    for p in decode_sources(w):
        if read is None:
            with open(os.path.join(ROOT, p), "rb") as f:
                h.update(f.read())
        else:
            h.update(read(p))
    return h.hexdigest()[:16]


def load_traffic(w):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if they
    were taken on the current source of the workload's decode kernels."""
    path = os.path.join(ROOT, "profiles", f"decode_{w.name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_source_hash(w):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, lengths, budget_s: float = 12.0):
    """The oracle, single-threaded, on a bounded sample: whole (sequence, KV head)
    units taken in order until the time budget is spent; each runs prefill
    (untimed) then decode steps (append + quantize + decode of every query head
    of the unit). Scaled to the full batch: tokens/s = B / (per-unit step time
    * B * Hkv). The oracle's quantize step is also timed on its own: every
    quantize_group call of the first unit's prefill (a full group against a
    pool)."""
    try:
        import threadpoolctl
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpoolctl = threadpool_limits = None
    import synth
    from oracle import ott_oracle as O
    nq = w.num_q_heads // w.num_kv_heads
    steps = 8
    t_step, n_unit = 0.0, 0
    q_times = []
    ctx = threadpool_limits(1) if threadpool_limits else None
    blas = []
    if threadpoolctl is not None:
        blas = [f"{i.get('internal_api')} {i.get('version')} x{i.get('num_threads')}"
                for i in threadpoolctl.threadpool_info()]
    t_all = time.perf_counter()
    try:
        for b in range(w.batch):
            for h in range(w.num_kv_heads):
                K, V = synth.kv_stream(w, b, h, int(lengths[b]) + steps)
                st = O.HeadOracle(w.head_dim, w.group_size, w.residual, w.pool_size)
                if n_unit == 0:  # time each quantize step of this prefill
                    qg = st.quantize_group

                    def timed_qg(qg=qg):
                        t = time.perf_counter()
                        qg()
                        q_times.append(time.perf_counter() - t)
                    st.quantize_group = timed_qg
                    O.run_prefill(st, K[:lengths[b]], V[:lengths[b]])
                    del st.quantize_group
                else:
                    O.run_prefill(st, K[:lengths[b]], V[:lengths[b]])
                qs = [synth.query(w, t, b)[h * nq:(h + 1) * nq] for t in range(steps)]
                sm = 1.0 / np.sqrt(w.head_dim)
                t0 = time.perf_counter()
                for t in range(steps):
                    O.step(st, K[lengths[b] + t], V[lengths[b] + t])
                    for i in range(nq):
                        st.decode(qs[t][i], sm)
                t_step += (time.perf_counter() - t0) / steps
                n_unit += 1
                if time.perf_counter() - t_all > budget_s:
                    break
            if time.perf_counter() - t_all > budget_s:
                break
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    per_unit = t_step / n_unit
    full_step = per_unit * w.batch * w.num_kv_heads
    q_mean = float(np.mean(q_times)) if q_times else None
    return {"value": w.batch / full_step, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_unit} (sequence, KV head) units of {w.name} x {steps} decode steps "
                      f"(append+quantize+decode of {nq} query head(s)), fp64 numpy, 1 thread; "
                      f"scaled to {w.batch}x{w.num_kv_heads} units",
            "s_per_step": full_step,
            "host_cores": len(os.sched_getaffinity(0)), "blas_threads_used": 1,
            "blas": blas, "numpy": np.__version__,
            "quantize_group_s_per_head": q_mean, "quantize_group_calls_timed": len(q_times),
            "quantize_group_s_per_step": (q_mean * w.batch * w.num_kv_heads / w.group_size
                                          if q_mean else None)}


def time_launches(launch, n_targets: int, stream, min_launches: int = 20) -> float:
    """Median over 5 laps of the mean duration (us) of back-to-back launches,
    launch(i) for i = 0, 1, ... round-robin over n_targets, timed with HIP events
    on `stream` (the stream the kernels are launched on)."""
    import torch
    per_lap = n_targets * -(-min_launches // n_targets)
    for i in range(n_targets):
        launch(i)
    laps = []
    for _ in range(5):
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        d0.record(stream)
        for i in range(per_lap):
            launch(i % n_targets)
        d1.record(stream)
        torch.cuda.synchronize()
        laps.append(1e3 * d0.elapsed_time(d1) / per_lap)
    return sorted(laps)[len(laps) // 2]


def fp16_baseline(w, K, V, lens, qd, outd, stream) -> dict:
    """The fp16 baseline decode (ott_fp16_decode) on the same K/V rows and lengths:
    decode-only time and HBM rate. Algorithmic bytes: 512 per token and KV head
    (K and V rows) plus 512 per query head (q in, out). One cache copy suffices:
    a launch reads far more than the 256 MB Infinity Cache."""
    import torch
    from decode_attention_ott_amd import _lib as L
    lens = [int(x) for x in lens]
    max_len = max(lens)
    dev = qd.device
    Kd = torch.from_numpy(np.ascontiguousarray(K[:, :, :max_len])).to(dev)
    Vd = torch.from_numpy(np.ascontiguousarray(V[:, :, :max_len])).to(dev)
    nbytes = L.ott_fp16_decode_workspace(w.batch, w.num_q_heads, 256)
    work = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=dev)
    sp = int(stream.cuda_stream)

    def launch(_i):
        L.ott_fp16_decode(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, Kd.data_ptr(),
                          Vd.data_ptr(), max_len, lens, qd.data_ptr(), outd.data_ptr(), 0.0,
                          work.data_ptr(), nbytes, 0, sp)
    us = time_launches(launch, 1, stream)
    nbytes_alg = 512 * w.num_kv_heads * sum(lens) + 512 * w.batch * w.num_q_heads
    del Kd, Vd, work
    torch.cuda.empty_cache()
    nq = w.num_q_heads // w.num_kv_heads
    hg = 8 if nq % 8 == 0 else 4 if nq % 4 == 0 else 2 if nq % 2 == 0 else 1
    return {"kernel": f"fp16_decode_kernel<{hg}>", "decode_us": round(us, 2),
            "alg_bytes_per_launch": int(nbytes_alg),
            "achieved_gbs": round(nbytes_alg / (us * 1e-6) / 1e9, 1)}


def sweep_batch(args, batches):
    """OTT decode vs the fp16 baseline decode, decode-only, for each batch size
    (the workload's shape otherwise): one JSON line per batch size."""
    import torch
    import synth
    from decode_attention_ott_amd import OTTLayer, _lib as L
    base = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)
    for B in batches:
        w = base.with_(batch=B)
        lengths = synth.prefill_lengths(w)
        n_states = auto_states(w, lengths)
        print(f"[sweep] batch {B}: generating inputs, {n_states} states", file=sys.stderr, flush=True)
        K, V = synth.kv_all(w, int(lengths.max()) + 1)
        Kd, Vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
        layers = []
        for _ in range(n_states):
            lay = OTTLayer.for_workload(w, max_seq_len=int(lengths.max()) + 1)
            lay.prefill(Kd, Vd, lengths)
            layers.append(lay)
        del Kd, Vd
        qd = torch.from_numpy(synth.queries(w, 0)).to(dev)
        outd = torch.empty(B, w.num_q_heads, w.head_dim, dtype=torch.float16, device=dev)
        ott_us = time_launches(lambda i: L.ott_decode(layers[i].handle, qd.data_ptr(),
                                                      outd.data_ptr(), sp), n_states, stream)
        ott_bytes = sum(algorithmic_decode_bytes(l) for l in layers) / n_states
        del layers
        torch.cuda.empty_cache()
        fb = fp16_baseline(w, K, V, lengths, qd, outd, stream)
        print(json.dumps({
            "sweep": "batch", "workload": w.name, "batch": B,
            "context": f"{w.prefill[0]}-{w.prefill[1]}",
            "ott_decode_us": round(ott_us, 2), "ott_tokens_per_s": round(B / (ott_us * 1e-6), 1),
            "ott_gbs": round(ott_bytes / (ott_us * 1e-6) / 1e9, 1),
            "fp16_decode_us": fb["decode_us"],
            "fp16_tokens_per_s": round(B / (fb["decode_us"] * 1e-6), 1),
            "fp16_gbs": fb["achieved_gbs"],
            "speedup": round(fb["decode_us"] / ott_us, 3)}), flush=True)


def time_prefill(args, reps: int = 5) -> None:
    """ott_prefill of the workload's prompts into an empty cache: one JSON line
    with the median over `reps` calls (after one untimed call) of the time between
    HIP events on the launch stream around the call (layers are made beforehand).
    Prompt bytes: the K and V rows of every prompt token and KV head (512 bytes),
    each read at least once."""
    import torch
    import synth
    from decode_attention_ott_amd import OTTLayer
    w = synth.WORKLOADS[args.workload]
    lengths = synth.prefill_lengths(w)
    print(f"[prefill] generating {w.name} prompts", file=sys.stderr, flush=True)
    K, V = synth.kv_all(w, int(lengths.max()))
    dev = torch.device("cuda:0")
    Kd, Vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    del K, V
    stream = torch.cuda.current_stream()
    times = []
    for rep in range(reps + 1):
        lay = OTTLayer.for_workload(w, max_seq_len=int(lengths.max()) + 1)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lay.prefill(Kd, Vd, lengths)
        e1.record(stream)
        torch.cuda.synchronize()
        if rep:
            times.append(1e3 * e0.elapsed_time(e1))
        lay.close()
        print(f"[prefill] call {rep} done", file=sys.stderr, flush=True)
    us = sorted(times)[len(times) // 2]
    tokens = int(np.sum(lengths))
    prompt_bytes = tokens * w.num_kv_heads * 2 * w.head_dim * 2
    print(json.dumps({
        "prefill": w.name, "batch": w.batch, "kv_heads": w.num_kv_heads,
        "context": f"{w.prefill[0]}-{w.prefill[1]}", "G": w.group_size, "P": w.pool_size,
        "prefill_us": round(us, 1), "prompt_tokens_per_s": round(tokens / (us * 1e-6), 1),
        "prompt_gb": round(prompt_bytes / 1e9, 3),
        "prompt_gbs": round(prompt_bytes / (us * 1e-6) / 1e9, 1),
        "calls_us": [round(t, 1) for t in times]}), flush=True)


def accuracy(args, batch: int = 8):
    """Attention-output error of the OTT decode against exact attention over the
    same fp16 tokens (the fp16 baseline kernel), for the plain 2-bit cache
    (P = 0), the pages' pool size (P = 32) and a larger pool (P = 128), for the
    comparison pool rules, and for G = 256 with larger R and P, on the
    workload's Key law and on its one-signed outlier-channel variant. The
    workload's shape with `batch` sequences; one JSON line per setting. The
    L1 loss is the mean absolute error over every output element (the measure
    of the pages' retention-criterion comparison); relative L1 divides the summed
    absolute error by the summed absolute exact output."""
    import torch
    import synth
    from decode_attention_ott_amd import OTTLayer, _lib as L
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)
    for one_signed in (False, True):
        base = synth.WORKLOADS[args.workload].with_(batch=batch, one_signed=one_signed)
        lengths = synth.prefill_lengths(base)
        K, V = synth.kv_all(base, int(lengths.max()))
        Kd, Vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
        # two query sets: the workload's N(0, 1) queries, and queries pointed at
        # one token: 10 x the unit Key of the token with the smallest Key norm
        # among the first L - R - G positions (tokens that go through a
        # quantize step), so that token takes most of the weight
        qs = {"random": synth.queries(base, 0)}
        nq = base.num_q_heads // base.num_kv_heads
        peaked = np.empty_like(qs["random"])
        for b in range(batch):
            n_q = max(1, int(lengths[b]) - base.residual - base.group_size)
            for h in range(base.num_kv_heads):
                kk = K[b, h, :n_q].astype(np.float64)
                t = int(np.argmin((kk * kk).sum(axis=1)))
                peaked[b, h * nq:(h + 1) * nq] = (10.0 * kk[t] / np.linalg.norm(kk[t])).astype(np.float16)
        qs["peaked on the smallest-norm token"] = peaked
        nbytes = L.ott_fp16_decode_workspace(batch, base.num_q_heads, 256)
        work = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=dev)
        refs = {}
        for name, qh in qs.items():
            qd = torch.from_numpy(qh).to(dev)
            ref = torch.empty(batch, base.num_q_heads, base.head_dim, dtype=torch.float16, device=dev)
            L.ott_fp16_decode(batch, base.num_q_heads, base.num_kv_heads, base.head_dim,
                              Kd.data_ptr(), Vd.data_ptr(), int(lengths.max()), lengths,
                              qd.data_ptr(), ref.data_ptr(), 0.0, work.data_ptr(), nbytes, 0, sp)
            refs[name] = (qd, ref)
        # the method's rule at P = 0, 32, 128; the comparison rules of the pages'
        # Figure 1(c) (largest Key norm, random) at P = 32; G = 256 with R = 64,
        # 128 and P = 32, 128 (a larger group needs a larger window and pool)
        settings = [(128, base.residual, P, rule)
                    for P, rule in ((0, 0), (32, 0), (128, 0), (32, 1), (32, 2))]
        settings += [(256, R, P, 0) for R in (64, 128) for P in (32, 128)]
        for G, R, P, rule in settings:
            w = base.with_(group_size=G, residual=R, pool_size=P, retention=rule)
            lay = OTTLayer.for_workload(w, max_seq_len=int(lengths.max()))
            lay.prefill(Kd, Vd, lengths)
            for name, (qd, ref) in refs.items():
                out = torch.empty_like(ref)
                L.ott_decode(lay.handle, qd.data_ptr(), out.data_ptr(), sp)
                torch.cuda.synchronize()
                r = ref.double()
                e = out.double() - r
                rel = (e.norm(dim=-1) / r.norm(dim=-1)).flatten()
                l1 = float(e.abs().mean())
                print(json.dumps({
                    "accuracy": "attention output vs exact fp16-cache attention",
                    "workload": w.name, "batch": batch, "one_signed_outlier_channels": one_signed,
                    "queries": name, "G": w.group_size, "R": w.residual, "P": P,
                    "retention": ["smallest Key norm", "largest Key norm", "random"][rule],
                    "l1_loss": round(l1, 7),
                    "rel_l1": round(float(e.abs().sum() / r.abs().sum()), 5),
                    "rel_l2_total": round(float(e.norm() / r.norm()), 5),
                    "rel_l2_per_head_mean": round(float(rel.mean()), 5),
                    "rel_l2_per_head_max": round(float(rel.max()), 5),
                    "max_abs": round(float(e.abs().max()), 5)}), flush=True)
            del lay
        del Kd, Vd, work
        torch.cuda.empty_cache()


def sweep_params(args):
    """OTT decode-only time for G, R and P varied one at a time around the
    workload's values (G in {64, 128, 256}, R in {32, 64, 128}, P in {0, 32, 128}),
    then G = 256 with R in {64, 128} and P in {32, 128} together (a larger group
    wants a larger window and pool): one JSON line per setting with the
    algorithmic bytes per quantized and per cached token-head, decode time,
    tokens/s and the HBM fraction."""
    import torch
    import synth
    from decode_attention_ott_amd import OTTLayer, _lib as L
    base = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)
    lengths = synth.prefill_lengths(base)
    K, V = synth.kv_all(base, int(lengths.max()) + 1)
    Kd, Vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    del K, V
    qd = torch.from_numpy(synth.queries(base, 0)).to(dev)
    outd = torch.empty(base.batch, base.num_q_heads, base.head_dim, dtype=torch.float16, device=dev)
    settings = [dict(group_size=g) for g in (64, 128, 256)]
    settings += [dict(residual=r) for r in (64, 128)]
    settings += [dict(pool_size=p) for p in (0, 128)]
    settings += [dict(group_size=256, residual=r, pool_size=p) for r in (64, 128) for p in (32, 128)]
    for kw in settings:
        w = base.with_(**kw)
        n_states = auto_states(w, lengths)
        print(f"[sweep] {kw}: {n_states} states", file=sys.stderr, flush=True)
        layers = []
        for _ in range(n_states):
            lay = OTTLayer.for_workload(w, max_seq_len=int(lengths.max()) + 1)
            lay.prefill(Kd, Vd, lengths)
            layers.append(lay)
        us = time_launches(lambda i: L.ott_decode(layers[i].handle, qd.data_ptr(), outd.data_ptr(),
                                                  sp), n_states, stream)
        nbytes = sum(algorithmic_decode_bytes(l) for l in layers) / n_states
        tokens = w.num_kv_heads * int(lengths.sum())
        page = w.group_size * w.head_dim // 2 + 4 * w.head_dim + 4 * w.group_size
        print(json.dumps({
            "sweep": "params", "workload": w.name, "G": w.group_size, "R": w.residual,
            "P": w.pool_size, "page_bytes": page,
            "bytes_per_quantized_token_head": round(page / w.group_size, 2),
            "bytes_per_cached_token_head": round(nbytes / tokens, 2),
            "decode_us": round(us, 2), "tokens_per_s": round(w.batch / (us * 1e-6), 1),
            "alg_bytes_per_launch": int(nbytes),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)
        del layers
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="llama2-7b-b32")
    ap.add_argument("--states", type=int, default=0,
                    help="independent layer states stepped round-robin (0: enough that one lap "
                         "over them reads >= 3 x 256 MB, the Infinity Cache size; 3..8)")
    ap.add_argument("--splits", type=int, default=0, help="split-K factor (0 = library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-calls", action="store_true",
                    help="time each step as ott_append + ott_quantize_group + ott_decode instead "
                         "of one ott_step")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="before warm-up, one device-to-device copy of this many MiB; its "
                         "rocprofv3 FETCH_SIZE/WRITE_SIZE readings calibrate the counters")
    ap.add_argument("--no-fp16-baseline", action="store_true",
                    help="skip timing the fp16 baseline decode on the same K/V")
    ap.add_argument("--sweep-batch", default="",
                    help="comma-separated batch sizes: print OTT vs fp16 decode-only lines "
                         "for each instead of the bench line")
    ap.add_argument("--accuracy", action="store_true",
                    help="print the OTT output error against exact attention for P = 0, 32, 128")
    ap.add_argument("--prefill", action="store_true",
                    help="time ott_prefill of the workload's prompts (one JSON line)")
    ap.add_argument("--sweep-params", action="store_true",
                    help="print OTT decode-only lines for G, R and P varied one at a time")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this OTT build has no multi-GPU path "
              "(each (sequence, KV head) is independent, so sharding heads or sequences needs no exchange).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from decode_attention_ott_amd import OTTLayer, _lib as L

    if args.accuracy:
        accuracy(args)
        return
    if args.prefill:
        time_prefill(args)
        return
    if args.sweep_params:
        sweep_params(args)
        return
    if args.sweep_batch:
        sweep_batch(args, [int(x) for x in args.sweep_batch.split(",")])
        return
    w = synth.WORKLOADS[args.workload]
    lengths = synth.prefill_lengths(w)
    if args.states <= 0:
        args.states = auto_states(w, lengths)
    # per-state prompt lengths whose windows take turns at quantizing, so that
    # the timed steps hold the steady-state share of quantize steps
    state_lengths = staggered_lengths(w, lengths, args.states)
    n_steps_state = (args.warmup + args.steps + args.states - 1) // args.states + 1
    n_pos = int(max(Ls.max() for Ls in state_lengths)) + n_steps_state
    print(f"[bench] generating {w.name} inputs ({n_pos} positions)", file=sys.stderr, flush=True)
    K, V = synth.kv_all(w, n_pos)
    dev = torch.device("cuda:0")
    Kd = torch.from_numpy(K).to(dev)
    Vd = torch.from_numpy(V).to(dev)
    layers = []
    for i in range(args.states):
        lay = OTTLayer.for_workload(w, max_seq_len=n_pos)
        lay.prefill(Kd, Vd, state_lengths[i])
        lay.set_num_splits(args.splits)
        layers.append(lay)
        print(f"[bench] state {i} prefilled", file=sys.stderr, flush=True)
    # per-state new tokens (each state's next positions) and queries, resident on
    # the device: kt[s][t] = the rows at positions state_lengths[s] + t
    bidx = np.arange(w.batch)
    kt = np.stack([np.stack([K[bidx, :, Ls + t][:, :, None, :] for t in range(n_steps_state)])
                   for Ls in state_lengths])
    vt = np.stack([np.stack([V[bidx, :, Ls + t][:, :, None, :] for t in range(n_steps_state)])
                   for Ls in state_lengths])
    ktd = torch.from_numpy(np.ascontiguousarray(kt)).to(dev)
    vtd = torch.from_numpy(np.ascontiguousarray(vt)).to(dev)
    qd = torch.from_numpy(np.stack([synth.queries(w, t) for t in range(args.warmup + args.steps)])).to(dev)
    outd = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float16, device=dev)
    del Kd, Vd
    torch.cuda.synchronize()

    if args.copy_probe_mb:
        n = args.copy_probe_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)
    ones = [1] * w.batch

    quantized = [0, 0]  # steps whose decode sees a new page, sequences quantized

    def step(i):
        """One step of state i % states: ott_step (append + quantize + decode in
        one call), or the three calls with --separate-calls."""
        s = i % args.states
        lay = layers[s]
        t = i // args.states
        if args.separate_calls:
            L.ott_append(lay.handle, ktd[s, t].data_ptr(), vtd[s, t].data_ptr(), ones, 1, sp)
            n = L.ott_quantize_group(lay.handle, sp)
            L.ott_decode(lay.handle, qd[i].data_ptr(), outd.data_ptr(), sp)
        else:
            n = L.ott_step(lay.handle, ktd[s, t].data_ptr(), vtd[s, t].data_ptr(), qd[i].data_ptr(),
                           outd.data_ptr(), sp)
        quantized[0] += n > 0
        quantized[1] += n
        return lay

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    quantized[:] = [0, 0]
    t_start.record(stream)
    for j in range(args.steps):
        step(args.warmup + j)
    t_end.record(stream)
    torch.cuda.synchronize()
    # quantize steps (a window's group becoming a page) in the timed steps; with
    # ott_step their work runs in fewer launches (every complete group at once)
    timed_quantize = {"steps_with_a_quantize": quantized[0], "sequences": quantized[1],
                      "steady_state_steps_with_a_quantize_per_step":
                          round(1.0 / quantize_period(w), 5) if quantize_period(w) else None}
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    tokens_per_s = w.batch * args.steps / (total_ms / 1e3)
    # The decode alone, launched back to back over the states (state is not
    # modified by a decode): 5 laps of >= 20 launches each, the median lap's
    # per-launch duration is the figure the roofline uses.
    dec_bytes = [algorithmic_decode_bytes(lay) for lay in layers]
    q_last = qd[args.warmup + args.steps - 1]
    dec_only_us = time_launches(
        lambda i: L.ott_decode(layers[i].handle, q_last.data_ptr(), outd.data_ptr(), sp),
        args.states, stream)
    n_dec = 5 * args.states * -(-20 // args.states)
    bytes_per_launch = sum(dec_bytes) / len(dec_bytes)
    achieved = bytes_per_launch / (dec_only_us * 1e-6) / 1e9
    traffic = load_traffic(w)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": decode_kernel_name(w),
                "decode_us": round(dec_only_us, 2),
                "decode_launches": n_dec,
                "alg_bytes_per_launch": int(bytes_per_launch)}
    fp16 = None
    if not args.no_fp16_baseline:
        print("[bench] timing the fp16 baseline decode", file=sys.stderr, flush=True)
        # the lengths the OTT states hold at the timed decodes
        lens_now = [layers[0].seq_state(b)[0] for b in range(w.batch)]
        del layers
        torch.cuda.empty_cache()
        fp16 = fp16_baseline(w, K, V, lens_now, q_last, outd, stream)
        fp16["speedup_ott_vs_fp16"] = round(fp16["decode_us"] / dec_only_us, 3)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, lengths)
    res = {"metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8e4m3-digit x fp4-code MFMA, fp32 accumulate",
           "data": "synthetic",
           "config": {"workload": w.name, "batch": w.batch, "num_q_heads": w.num_q_heads,
                      "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                      "context": f"{w.prefill[0]}-{w.prefill[1]}", "G": w.group_size,
                      "R": w.residual, "P": w.pool_size, "states": args.states,
                      "splits": args.splits or "auto",
                      "storage": "2-bit K/V codes, fp16 min/scale, fp16 pool and window",
                      "step": "append 1 token per sequence + quantize full windows + decode, as "
                              + ("ott_append + ott_quantize_group + ott_decode" if args.separate_calls
                                 else "one ott_step"),
                      "state_lengths": "each state's prompt lengths moved by < G/2 so the states "
                                       "take turns at quantizing (steady-state share per step)"},
           "timed_quantize": timed_quantize,
           "roofline": roofline, "cpu_baseline": cpu, "fp16_baseline": fp16}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
