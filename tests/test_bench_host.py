"""Host logic of bench.py, on the CPU: the one-GPU guard, the staggered state
lengths that make every timed window hold the steady-state share of quantize
steps, and the gate that keeps stale traffic counters off the bench line."""
import math
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synth


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _quantize_steps(w, state_lengths, n_steps, first):
    """Global steps in [first, first + n_steps) at which some window of some
    state is due, stepping the states round-robin one token per step: a window
    holding r tokens after its prompt is full (R + G) after C - r appends, and
    every G appends after that."""
    G, R = w.group_size, w.residual
    C = R + G
    n = len(state_lengths)
    due = set()
    for s, Ls in enumerate(state_lengths):
        for L in Ls:
            L = int(L)
            r = L - G * ((L - R) // G) if L >= R + G else L
            t = C - r                          # appends until full (1-based state step)
            while True:
                i = n * (t - 1) + s            # global step of this state step
                if i >= first + n_steps:
                    break
                if i >= first:
                    due.add(i)
                t += G
    return due


@pytest.mark.parametrize("name", ["llama2-7b-b32", "mistral-7b-gqa", "llama2-13b-128k", "llama2-7b"])
def test_staggered_states_take_turns_at_quantizing(name):
    w = synth.WORKLOADS[name]
    G = w.group_size
    lo, hi = w.prefill
    L0 = synth.prefill_lengths(w)
    n = bench.auto_states(w, L0)
    period = bench.quantize_period(w)
    assert 3 <= n and (period == 0 or math.gcd(n, period) == 1)
    states = bench.staggered_lengths(w, L0, n)
    assert len(states) == n
    for Ls in states:
        moved = (np.asarray(Ls) - L0) % G
        moved = np.where(moved >= G // 2, moved - G, moved)
        assert (np.abs(moved) < G // 2).all()          # less than G/2, up to whole groups
        if hi - lo >= G:
            assert ((Ls >= lo) & (Ls <= hi)).all()
    if not period:
        return
    # any window of timed steps holds the steady-state share, K / period, +-1
    for first, K in ((5, 20), (16, 64), (0, 3 * period), (7, 384)):
        got = len(_quantize_steps(w, states, K, first))
        assert abs(got - K / period) <= 1, (first, K, got)


def test_every_state_quantizes_at_its_own_phase():
    # the three batch-32 states, ragged: within a state the 32 windows are due
    # at 32 different steps mod G (one every G / B steps)
    w = synth.WORKLOADS["llama2-7b-b32"]
    G, R = w.group_size, w.residual
    L0 = synth.prefill_lengths(w)
    for Ls in bench.staggered_lengths(w, L0, bench.auto_states(w, L0)):
        r = np.array([L - G * ((L - R) // G) for L in Ls])
        phases = (R + G - r) % G
        assert len(set(phases.tolist())) == w.batch
        assert len(set((phases % (G // w.batch)).tolist())) == 1


def test_traffic_counters_are_used_only_for_the_sources_they_were_taken_on(monkeypatch):
    w = synth.WORKLOADS["llama2-7b-b32"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda _w, read=None: "not-the-sources")
    assert bench.load_traffic(w) is None


def test_the_source_hash_covers_every_decode_source():
    w = synth.WORKLOADS["mistral-7b-gqa"]
    real = bench.kernel_source_hash(w)
    for p in bench.decode_sources(w):
        def read(path, _p=p):
            with open(os.path.join(bench.ROOT, path), "rb") as f:
                data = f.read()
            return data + b"\n" if path == _p else data
        assert bench.kernel_source_hash(w, read=read) != real, p
