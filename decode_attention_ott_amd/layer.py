"""OTTLayer: one attention layer's OTT caches behind the C ABI.

Torch is used for device memory and the current stream only; the calls go
straight to libott.so (see _lib.py). Read-back helpers copy arena regions to
the host for inspection (tests, snapshots); they do no computation of the
method.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib as L

ALIGN = 256


def _stream() -> int:
    return int(torch.cuda.current_stream().cuda_stream)


class OTTLayer:
    def __init__(self, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int = 128,
                 group_size: int = 128, residual: int = 32, pool_size: int = 32,
                 max_seq_len: int = 4096, sm_scale: float = 0.0, device="cuda",
                 retention: int = 0):
        self.cfg = L.ott_config_t(batch, num_q_heads, num_kv_heads, head_dim, group_size,
                                  residual, pool_size, max_seq_len, sm_scale, retention)
        self.B, self.Hq, self.Hkv, self.d = batch, num_q_heads, num_kv_heads, head_dim
        self.G, self.R, self.P = group_size, residual, pool_size
        self.max_seq_len = max_seq_len
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        need = L.ott_init(self.cfg, None, 0, sizing_only=True)
        self._buf = torch.empty(need + ALIGN, dtype=torch.uint8, device=self.device)
        off = (-self._buf.data_ptr()) % ALIGN
        self.arena = self._buf[off:off + need]
        self.handle, _ = L.ott_init(self.cfg, self.arena.data_ptr(), need)
        self.layout = L.ott_get_layout(self.handle)

    @classmethod
    def for_workload(cls, w, max_seq_len: Optional[int] = None, **kw) -> "OTTLayer":
        if max_seq_len is None:
            max_seq_len = w.max_prefill + w.steps
        kw.setdefault("retention", getattr(w, "retention", 0))
        return cls(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.group_size,
                   w.residual, w.pool_size, max_seq_len, **kw)

    # -- the four calls ------------------------------------------------------
    def append(self, k: torch.Tensor, v: torch.Tensor, n_new: Optional[Sequence[int]] = None):
        """k, v: fp16 [B, Hkv, n, d] on the device; n_new[b] <= n tokens per sequence."""
        self._check_kv(k, v)
        n = k.shape[2]
        if n_new is None:
            n_new = [n] * self.B
        L.ott_append(self.handle, k.data_ptr(), v.data_ptr(), n_new, n, _stream())

    def quantize_group(self) -> int:
        return L.ott_quantize_group(self.handle, _stream())

    def decode(self, q: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """q: fp16 [B, Hq, d] on the device; returns fp16 [B, Hq, d]."""
        if q.dtype != torch.float16 or q.device != self.device or not q.is_contiguous() \
                or tuple(q.shape) != (self.B, self.Hq, self.d):
            raise ValueError(f"q must be contiguous fp16 [{self.B}, {self.Hq}, {self.d}] on "
                             f"{self.device}, got {q.dtype} {tuple(q.shape)} on {q.device}")
        if out is None:
            out = torch.empty_like(q)
        elif out.dtype != torch.float16 or tuple(out.shape) != tuple(q.shape) \
                or not out.is_contiguous() or out.device != self.device:
            raise ValueError("out must be a contiguous fp16 tensor shaped like q")
        L.ott_decode(self.handle, q.data_ptr(), out.data_ptr(), _stream())
        return out

    def step(self, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor,
             out: Optional[torch.Tensor] = None):
        """One decode step (append one token per sequence, quantize full windows,
        decode) through ott_step. k, v: fp16 [B, Hkv, 1, d]; q: fp16 [B, Hq, d].
        Returns (out, sequences quantized)."""
        self._check_kv(k, v)
        if k.shape[2] != 1:
            raise ValueError("a step appends one token per sequence")
        if q.dtype != torch.float16 or q.device != self.device or not q.is_contiguous() \
                or tuple(q.shape) != (self.B, self.Hq, self.d):
            raise ValueError(f"q must be contiguous fp16 [{self.B}, {self.Hq}, {self.d}]")
        if out is None:
            out = torch.empty_like(q)
        n = L.ott_step(self.handle, k.data_ptr(), v.data_ptr(), q.data_ptr(), out.data_ptr(),
                       _stream())
        return out, n

    def set_num_splits(self, s: int) -> None:
        L.ott_set_num_splits(self.handle, s)

    def seq_state(self, b: int):
        """(L, r_cnt, ring_head, nb) of sequence b."""
        return L.ott_get_seq_state(self.handle, b)

    def close(self) -> None:
        if getattr(self, "handle", None):
            L.ott_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- helpers ---------------------------------------------------------------
    def _check_kv(self, k, v):
        for name, t in (("k", k), ("v", v)):
            if t.dtype != torch.float16 or t.device != self.device or not t.is_contiguous() \
                    or t.dim() != 4 or t.shape[0] != self.B or t.shape[1] != self.Hkv \
                    or t.shape[3] != self.d:
                raise ValueError(f"{name} must be contiguous fp16 [{self.B}, {self.Hkv}, n, "
                                 f"{self.d}] on {self.device}")
        if k.shape != v.shape:
            raise ValueError("k and v shapes differ")

    def prefill(self, K: torch.Tensor, V: torch.Tensor, lengths: Sequence[int]) -> None:
        """Tokens [0, lengths[b]) of K, V (fp16 [B, Hkv, >=max(lengths), d] on the
        device) into the cache. An empty cache takes the whole prompt in one
        ott_prefill call; otherwise the tokens go through prefill_stepwise."""
        lengths = [int(x) for x in lengths]
        if all(self.seq_state(b)[0] == 0 for b in range(self.B)):
            self._check_kv(K, V)
            if max(lengths) > K.shape[2]:
                raise ValueError("lengths exceed the rows of K and V")
            L.ott_prefill(self.handle, K.data_ptr(), V.data_ptr(), lengths, K.shape[2],
                          _stream())
            return
        self.prefill_stepwise(K, V, lengths)

    def prefill_stepwise(self, K: torch.Tensor, V: torch.Tensor, lengths: Sequence[int]) -> None:
        """Appends tokens [0, lengths[b]) of K, V (fp16 [B, Hkv, >=max(lengths), d] on
        the device) in chunks that fit the window, quantizing whenever a window
        is full: the ordinary append/quantize sequence, in position order."""
        lengths = [int(x) for x in lengths]
        cap = self.R + self.G
        done = [self.seq_state(b)[0] for b in range(self.B)]
        while True:
            room = [cap - self.seq_state(b)[1] for b in range(self.B)]
            n_new = [max(0, min(lengths[b] - done[b], room[b])) for b in range(self.B)]
            if not any(n_new):
                break
            s0 = min(done[b] for b in range(self.B) if n_new[b] > 0)
            # all sequences move together from position 0, so a common start works
            starts = {done[b] for b in range(self.B) if n_new[b] > 0}
            if len(starts) != 1:
                raise ValueError("prefill needs every sequence to start at the same position")
            n = max(n_new)
            kc = K[:, :, s0:s0 + n].contiguous()
            vc = V[:, :, s0:s0 + n].contiguous()
            self.append(kc, vc, n_new)
            for b in range(self.B):
                done[b] += n_new[b]
            while self.quantize_group():
                pass

    # -- read-back (host copies of arena regions) ------------------------------
    def _region(self, off: int, nbytes: int) -> np.ndarray:
        torch.cuda.synchronize(self.device)
        return self.arena[off:off + nbytes].cpu().numpy()

    def counters(self) -> np.ndarray:
        """int32 [B, Hkv, 4]: {L, r_cnt, ring_head, nb} as the device holds them."""
        n = self.B * self.Hkv * 4 * 4
        return self._region(self.layout.off_counters, n).view(np.int32).reshape(self.B, self.Hkv, 4)

    def tickets(self) -> np.ndarray:
        """uint32 [B, Hkv]: split arrivals of the running decode (0 between launches)."""
        n = self.B * self.Hkv * 4
        return self._region(self.layout.off_tickets, n).view(np.uint32).reshape(self.B, self.Hkv)

    def page_bytes(self, b: int, kvh: int, n: int) -> bytes:
        pb = self.layout.page_bytes
        bh = b * self.Hkv + kvh
        off = self.layout.off_pages + (bh * self.layout.pages_per_head + n) * pb
        return self._region(off, pb).tobytes()

    def pages_of_head(self, b: int, kvh: int, count: int) -> np.ndarray:
        pb = self.layout.page_bytes
        bh = b * self.Hkv + kvh
        off = self.layout.off_pages + bh * self.layout.pages_per_head * pb
        return self._region(off, count * pb).reshape(count, pb)

    def page_positions(self, b: int, kvh: int, count: int) -> np.ndarray:
        bh = b * self.Hkv + kvh
        off = self.layout.off_page_pos + bh * self.layout.pages_per_head * self.G * 4
        return self._region(off, count * self.G * 4).view(np.int32).reshape(count, self.G)

    def pool(self, b: int, kvh: int):
        """Live pool of (b, kvh): (pos int32 [n], n2 fp64 [n], k fp16 [n, d], v fp16 [n, d])."""
        L_, r_cnt, head, nb = self.seq_state(b)
        n = min(self.P, self.G * nb)
        buf = nb & 1
        bh = b * self.Hkv + kvh
        BH = self.B * self.Hkv
        slot0 = buf * BH + bh
        lay = self.layout
        pos = self._region(lay.off_pool_pos + slot0 * self.P * 4, n * 4).view(np.int32)
        n2 = self._region(lay.off_pool_n2 + slot0 * self.P * 8, n * 8).view(np.float64)
        kk = self._region(lay.off_pool_k + slot0 * self.P * self.d * 2, n * self.d * 2)
        vv = self._region(lay.off_pool_v + slot0 * self.P * self.d * 2, n * self.d * 2)
        return (pos, n2, kk.view(np.float16).reshape(n, self.d),
                vv.view(np.float16).reshape(n, self.d))

    def window(self, b: int, kvh: int):
        """Window tokens of (b, kvh) oldest first: (k fp16 [r, d], v fp16 [r, d])."""
        L_, r_cnt, head, nb = self.seq_state(b)
        C = self.R + self.G
        bh = b * self.Hkv + kvh
        lay = self.layout
        rk = self._region(lay.off_ring_k + bh * C * self.d * 2, C * self.d * 2)
        rv = self._region(lay.off_ring_v + bh * C * self.d * 2, C * self.d * 2)
        rk = rk.view(np.float16).reshape(C, self.d)
        rv = rv.view(np.float16).reshape(C, self.d)
        idx = [(head + i) % C for i in range(r_cnt)]
        return rk[idx], rv[idx]
