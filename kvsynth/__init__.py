"""Seeded synthetic KV caches for ChunkKV compression.

This module only draws inputs.  It holds none of the method's arithmetic (no
scores, no softmax, no selection), so both the oracle side and the HIP side
may use it.  Workload shapes stand in for the pages' long-context workloads,
whose datasets and model weights are not available: Llama-3-8B-shaped caches
(32 query heads, 8 KV heads, head_dim 128) at 8k/32k tokens, the chunk-size
and fixed-KV-size ablation shapes, and a 70B-shaped batch (64 query heads).

Distributions:
  * window queries ~ N(0, 1);
  * keys z * s with z ~ N(0, 1) and a per-(layer, KV head, channel) scale
    s = exp(0.5 * N(0, 1)) (log-normal(0, 0.5)), standing in for key outlier
    channels;
  * values ~ N(0, 1);
  * optional planted "hot" chunks: their keys get + amp * u, where u is the
    unit mean direction of the KV group's window queries.  Adjacent layers
    share 80% of their hot chunks.
bf16 tensors are rounded from fp32 with round-to-nearest-even (torch's cast).

Layouts (what the C-ABI takes):
  q_win[L][B][w][H_q][d]    window queries (row r <-> position T_b - w + r)
  k, v [L][sum_b T_b][H_kv][d]  packed token-major caches
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16"
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_lens: tuple
    window: int
    chunk: int
    l_max: tuple               # per sequence
    n_reuse: int
    planted: str = "none"      # "none" | "tiny" | "layers"

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _budget(T: int, ratio: float) -> int:
    # "x% budget" means L_max = floor(x * T)
    return int(math.floor(ratio * T + 1e-9))


WORKLOADS = {
    # 1 layer, 1 KV head, 1 query head, d=64, T=1000, fp32, 5 planted chunks
    "tiny-fp32-d64-T1000": Workload(
        "tiny-fp32-d64-T1000", "f32", 1, 1, 1, 64, (1000,), 8, 10, (100,), 1, "tiny"),
    # one Llama-3-8B-shaped layer at 8k tokens, 10% budget
    "llama3-8b-1layer-T8192": Workload(
        "llama3-8b-1layer-T8192", "bf16", 1, 32, 8, 128, (8192,), 32, 10,
        (_budget(8192, 0.10),), 1),
    # the 32-layer Llama-3-8B-shaped stack at 32k tokens, 10% budget, index reuse 2
    "llama3-8b-32layer-T32768": Workload(
        "llama3-8b-32layer-T32768", "bf16", 32, 32, 8, 128, (32768,), 32, 10,
        (3276,), 2, "layers"),
    # chunk-size / fixed-KV-size sweep point (c and L_max overridden per point)
    "llama3-8b-csweep-T16384": Workload(
        "llama3-8b-csweep-T16384", "bf16", 1, 32, 8, 128, (16384,), 32, 10, (512,), 1),
    # 70B-shaped batch of four sequences, 20% budget, index reuse 2
    "llama-70b-80layer-4seq": Workload(
        "llama-70b-80layer-4seq", "bf16", 80, 64, 8, 128, (131072, 65536, 32768, 16384), 64,
        10, tuple(_budget(t, 0.20) for t in (131072, 65536, 32768, 16384)), 2, "layers"),
}

CSWEEP_CHUNKS = (3, 5, 10, 20, 30)
CSWEEP_LMAX = (128, 256, 512)


def seq_starts(wl: Workload) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(wl.seq_lens)]).astype(np.int64)


def make_tiny(seed: int = 0):
    """The tiny fp32 case: numpy default_rng(seed), drawn as Q[1000,1,64], K, V.

    Returns dict(q_full, k, v, planted) as float32 numpy arrays; planted holds
    the 5 chunk ids (from chunks 0..98, i.e. not the window's chunk) whose keys
    were shifted by +2 (two standard deviations) along the unit mean direction
    of the 8 window queries.
    """
    wl = WORKLOADS["tiny-fp32-d64-T1000"]
    T, d, w, c = wl.seq_lens[0], wl.head_dim, wl.window, wl.chunk
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, 1, d)).astype(np.float32)
    k = rng.standard_normal((T, 1, d)).astype(np.float32)
    v = rng.standard_normal((T, 1, d)).astype(np.float32)
    planted = np.sort(rng.choice((T - w) // c, size=5, replace=False)).astype(np.int64)
    u = q[T - w:, 0, :].astype(np.float64).mean(axis=0)
    u = (u / np.linalg.norm(u)).astype(np.float32)
    for j in planted:
        k[j * c:(j + 1) * c, 0, :] += 2.0 * u
    return dict(q_full=q, k=k, v=v, planted=planted)


def _hot_sets(rng: np.random.Generator, n_layers: int, n_heads: int, n_chunks: int,
              n_hot: int, n_excl: int):
    """Per (layer, head) hot chunk ids; adjacent layers share 80% of them."""
    cand = n_chunks - n_excl
    n_hot = max(0, min(n_hot, cand))
    keep = int(math.floor(0.8 * n_hot))
    out = []
    prev = [rng.choice(cand, n_hot, replace=False) for _ in range(n_heads)]
    out.append(prev)
    for _ in range(1, n_layers):
        cur = []
        for h in range(n_heads):
            kept = rng.choice(prev[h], keep, replace=False)
            rest = np.setdiff1d(np.arange(cand), kept)
            fresh = rng.choice(rest, n_hot - keep, replace=False)
            cur.append(np.concatenate([kept, fresh]))
        out.append(cur)
        prev = cur
    return out


def make_cache(wl: Workload, device="cpu", seed: int = 0, layers: Optional[range] = None):
    """Draw window queries and K/V caches for the workload on ``device``.

    Each layer l uses its own torch generator seeded 1000*l + tensor_id + seed
    (tensor ids: 0 queries, 1 key noise, 2 key scales, 3 values), so any layer
    can be regenerated alone.  Returns dict(q_win [L,B,w,Hq,d], k, v
    [L,sumT,Hkv,d], hot: per-layer list of per-(seq, head) hot chunk ids or
    None).
    """
    if wl.planted == "tiny":
        raise ValueError("use make_tiny() for the tiny workload")
    layers = range(wl.n_layers) if layers is None else layers
    L = len(layers)
    B = len(wl.seq_lens)
    T_tot = wl.total_tokens
    Hq, Hkv, d, w, c = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.chunk
    G = Hq // Hkv
    starts = seq_starts(wl)
    dt = wl.torch_dtype
    q_win = torch.empty((L, B, w, Hq, d), dtype=dt, device=device)
    k = torch.empty((L, T_tot, Hkv, d), dtype=dt, device=device)
    v = torch.empty((L, T_tot, Hkv, d), dtype=dt, device=device)
    hot_all = None
    if wl.planted == "layers":
        rng = np.random.default_rng(seed + 7)
        per_seq = []
        for b, T in enumerate(wl.seq_lens):
            C = -(-T // c)
            n_excl = C - (T - w) // c          # chunks touching the window
            per_seq.append(_hot_sets(rng, wl.n_layers, Hkv, C, wl.l_max[b] // c, n_excl))
        hot_all = [[per_seq[b][l] for b in range(B)] for l in layers]
    for li, l in enumerate(layers):
        gens = [torch.Generator(device=device) for _ in range(4)]
        for tid, g in enumerate(gens):
            g.manual_seed(1000 * l + tid + seed)
        qf = torch.randn((B, w, Hq, d), generator=gens[0], device=device)
        z = torch.randn((T_tot, Hkv, d), generator=gens[1], device=device)
        s = torch.exp(0.5 * torch.randn((Hkv, d), generator=gens[2], device=device))
        kf = z * s
        vf = torch.randn((T_tot, Hkv, d), generator=gens[3], device=device)
        if hot_all is not None:
            amp = 2.0 * torch.sqrt((s * s).mean(dim=1))          # [Hkv]
            for b in range(B):
                u = qf[b].reshape(w, Hkv, G, d).mean(dim=(0, 2))  # [Hkv, d]
                u = u / u.norm(dim=1, keepdim=True)
                t0 = int(starts[b])
                for h in range(Hkv):
                    ids = torch.as_tensor(np.sort(hot_all[li][b][h]), device=device)
                    tok = (ids[:, None] * c + torch.arange(c, device=device)[None, :]).reshape(-1)
                    tok = tok[tok < wl.seq_lens[b]] + t0
                    kf[tok, h, :] += amp[h] * u[h]
        q_win[li] = qf.to(dt)
        k[li] = kf.to(dt)
        v[li] = vf.to(dt)
        del qf, z, kf, vf
    return dict(q_win=q_win, k=k, v=v, hot=hot_all)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a bf16 tensor as a host uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_array(t: torch.Tensor) -> np.ndarray:
    """Host numpy view for the oracle: float32 as is, bf16 as raw bits."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().contiguous().cpu().numpy()
