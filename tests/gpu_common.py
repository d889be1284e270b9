"""Helpers for the GPU parity tests: upload seeded workloads, run decode trajectories through the
C ABI, and pick the sampled checkpoint steps. Nothing here computes attention."""
from __future__ import annotations

import numpy as np
import torch

from workloads import DecodeWorkload


def upload(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """Stored input values -> device tensor (bf16 bit patterns become torch.bfloat16)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def kv_torch_dtype(dtype: str) -> torch.dtype:
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def sample_steps(T: int, n: int, m: int, seed: int = 0, extra: int = 16, crossings: int = 24,
                 full: bool = False) -> list[int]:
    """Checkpoints: {1, 2, n-1, n, n+1, 2n, 1000, T-1, T}, the steps where the live row count
    crosses a multiple of 64 (at most `crossings`, evenly spaced), and `extra` seeded random
    steps; all clipped to [1, T]."""
    s = {1, 2, n - 1, n, n + 1, 2 * n, 1000, T - 1, T}
    cross = []
    for t in range(1, T + 1):
        L0 = m + (t - 1 if full else min(n, t - 1))
        L1 = m + (t if full else min(n, t))
        if L0 // 64 != L1 // 64:
            cross.append(t)
    if len(cross) > crossings:
        idx = np.linspace(0, len(cross) - 1, crossings).round().astype(int)
        cross = [cross[i] for i in idx]
    s |= set(cross)
    rng = np.random.default_rng(seed)
    s |= set(rng.integers(1, T + 1, size=extra).tolist())
    return sorted(t for t in s if 1 <= t <= T)


class Trajectory:
    """Device copies of a decode workload and a cache built from it."""

    def __init__(self, wa, wl: DecodeWorkload, mode: int, storage: torch.Tensor | None = None,
                 paged=None):
        """`paged` (a workloads.PagedPrefix): build the cache over the shared token pool and its
        page table instead of copying wl's gathered prefixes."""
        self.wl = wl
        self.wa = wa
        self.mode = mode
        if paged is None:
            self.pk = upload(wl.prefix_k, wl.dtype) if wl.prefix_k.shape[0] else None
            self.pv = upload(wl.prefix_v, wl.dtype) if wl.prefix_v.shape[0] else None
        else:
            self.pk = self.pv = None
            pool = dict(pool_k=upload(paged.pool_k, wl.dtype), pool_v=upload(paged.pool_v, wl.dtype),
                        prefix_table=torch.from_numpy(paged.table).cuda())
        self.q = upload(wl.q, wl.dtype)
        self.k = upload(wl.k, wl.dtype)
        self.v = upload(wl.v, wl.dtype)
        ragged = bool((wl.steps != wl.steps.max()).any())
        self.active = None
        if ragged:
            act = np.stack([wl.active(t) for t in range(1, wl.T + 1)])
            self.active = torch.from_numpy(act).cuda()
        max_steps = wl.steps if mode == wa.MODE_FULL_CAUSAL else None
        window = wl.window if mode == wa.MODE_RSWA else None
        extra = pool if paged is not None else {}
        self.cache = wa.RswaCache(self.pk, self.pv, wl.prefix_len, window, mode=mode,
                                  max_steps=max_steps, kv_dtype=kv_torch_dtype(wl.dtype),
                                  storage=storage, **extra)

    def run(self, checkpoints, out_dtype=torch.float32, t_end: int | None = None,
            fused: bool = False, raw: bool = False):
        """Run steps 1..t_end (append then decode, or the fused step); return
        {t: out [B, H, D]} at the checkpoints (float32 numpy, or the raw output tensor copy)."""
        wl = self.wl
        t_end = wl.T if t_end is None else t_end
        out = torch.zeros((wl.batch, 16, 128), dtype=out_dtype, device="cuda")
        keep = set(checkpoints)
        res = {}
        for t in range(1, t_end + 1):
            act = None if self.active is None else self.active[t - 1]
            if fused:
                self.cache.step(self.q[t - 1], self.k[t - 1], self.v[t - 1], out, active=act)
            else:
                self.cache.append(self.k[t - 1], self.v[t - 1], act)
                self.cache.decode(self.q[t - 1], out, active=act)
            if t in keep:
                res[t] = out.clone() if raw else out.float().cpu().numpy()
        torch.cuda.synchronize()
        return res
