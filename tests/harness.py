"""Shared helpers for the GPU parity tests: run the HIP path through the C-ABI
binding, pull results to the host, and compare one (layer, sequence, KV head)
unit against the CPU oracle.

Parity bar (ChunkKV page section 4.1 Algorithm 1; Kara eq. (1)):
  * chunk scores: |S_gpu - S_ref| <= RTOL * |S_ref| + ATOL with RTOL 1e-3 for
    bf16 inputs (fp32 accumulation) and 1e-5 for fp32 inputs; ATOL = 1e-30 is
    only an fp32-underflow floor (far below any score these inputs produce);
  * selection + index build: the oracle's TopK and index build applied to the
    GPU's own fp32 scores must reproduce the GPU's indices exactly (the same
    decision in the same precision); against the oracle's fp64 scores the
    selected chunk sets may differ only inside the band of scores within
    tolerance of the k-th largest;
  * gather: K'/V' rows are bit-exact copies of the rows the indices name, and
    output rows beyond n keep their poison pattern.
"""
from __future__ import annotations

import numpy as np
import torch

import kvsynth
import oracle
from kv_cache_compression_win_amd import chunkkv as ck

RTOL = {ck.BF16: 1e-3, ck.F32: 1e-5}
ATOL = 1e-30
POISON_BYTE = 0x7B
POISON_INDEX = -7


def tdtype(dtype: int):
    return torch.float32 if dtype == ck.F32 else torch.bfloat16


class Case:
    """One compress_layers problem with inputs already on the GPU.

    q_win [L, B, w, Hq, d], k/v [L, sum T, Hkv, d] torch tensors on cuda.
    """

    def __init__(self, dtype, seq_lens, l_max, n_q_heads, n_kv_heads, head_dim, window, chunk,
                 n_reuse, q_win, k, v, n_score_layers=None, kv_strides=None):
        self.dtype, self.seq_lens, self.l_max = dtype, list(seq_lens), list(l_max)
        self.Hq, self.Hkv, self.d, self.w, self.c = n_q_heads, n_kv_heads, head_dim, window, chunk
        self.n_reuse = n_reuse
        self.q_win, self.k, self.v = q_win, k, v
        self.L = k.shape[0]
        self.starts = np.concatenate([[0], np.cumsum(self.seq_lens)]).astype(np.int64)
        self.prob = ck.make_problem(dtype, seq_lens, l_max, n_q_heads, n_kv_heads, head_dim, window,
                                    chunk, kv_strides=kv_strides)
        self.plan = ck.plan(self.prob)
        self.n_score_layers = n_score_layers

    def run(self, phase_events=None):
        L, d = self.L, self.d
        bufs = ck.Buffers(self.prob, L, self.n_reuse, d, tdtype(self.dtype), "cuda",
                          n_score_layers=self.n_score_layers)
        bufs.k_out.view(torch.uint8).fill_(POISON_BYTE)
        bufs.v_out.view(torch.uint8).fill_(POISON_BYTE)
        bufs.indices.fill_(POISON_INDEX)
        qs = [self.q_win[l] if l % self.n_reuse == 0 else None for l in range(L)]
        ck.compress_layers(self.prob, self.n_reuse, qs, [self.k[l] for l in range(L)],
                           [self.v[l] for l in range(L)], [bufs.k_out[l] for l in range(L)],
                           [bufs.v_out[l] for l in range(L)], bufs.scores, bufs.indices, bufs.lengths,
                           bufs.workspace, bufs.ws_bytes, phase_events=phase_events)
        torch.cuda.synchronize()
        self.bufs = bufs
        A = bufs.n_anchor
        self.scores = bufs.scores.cpu().numpy().reshape(A, -1)
        self.indices = bufs.indices.cpu().numpy().reshape(A, -1)
        self.lengths = bufs.lengths.cpu().numpy().reshape(A, -1)
        return self

    # -- per-unit accessors -------------------------------------------------
    def C(self, b):
        return -(-self.seq_lens[b] // self.c)

    def kk(self, b):
        return self.l_max[b] // self.c

    def gpu_scores(self, l, b, h):
        a = l // self.n_reuse
        o = self.plan["score_off"][b] + h * self.C(b)
        return self.scores[a, o:o + self.C(b)]

    def gpu_indices(self, l, b, h):
        a = l // self.n_reuse
        n = int(self.lengths[a, b * self.Hkv + h])
        o = self.plan["index_off"][b] + h * self.plan["l_cap"][b]
        return self.indices[a, o:o + n], self.indices[a, o + n:o + self.plan["l_cap"][b]]

    def host_q(self, l, b):
        return kvsynth.host_array(self.q_win[l, b])              # [w, Hq, d]

    def host_kv(self, t, l, b):
        s0, s1 = int(self.starts[b]), int(self.starts[b + 1])
        return kvsynth.host_array(t[l, s0:s1])                    # [T, Hkv, d]

    def out_rows(self, which, l, b, h):
        o = self.plan["index_off"][b] + h * self.plan["l_cap"][b]
        t = self.bufs.k_out if which == "k" else self.bufs.v_out
        return kvsynth.host_array(t[l, o:o + self.plan["l_cap"][b]])


def check_scores(s_gpu, s_ref, dtype, where=""):
    rtol = RTOL[dtype]
    err = np.abs(s_gpu.astype(np.float64) - s_ref)
    bad = err > rtol * np.abs(s_ref) + ATOL
    assert not bad.any(), (f"{where}: {bad.sum()} chunk scores out of tolerance; worst rel "
                           f"{(err / np.maximum(np.abs(s_ref), 1e-300)).max():.3e}")


def check_selection(s_gpu, s_ref, idx_gpu, T, w, c, kk, dtype, where=""):
    # exact: the oracle's TopK + index build on the GPU's own fp32 scores
    sel_g = oracle.topk(s_gpu.astype(np.float64), kk)
    idx_from_g = oracle.indices(T, w, c, sel_g)
    assert np.array_equal(idx_gpu, idx_from_g), f"{where}: GPU indices differ from TopK of its scores"
    # band: against the fp64 oracle selection
    sel_r = oracle.topk(s_ref, kk)
    assert sel_g.size == sel_r.size
    if 0 < kk < s_ref.size:
        tau = np.sort(s_ref)[::-1][kk - 1]
        band = set(np.nonzero(np.abs(s_ref - tau) <= RTOL[dtype] * tau + ATOL)[0].tolist())
        assert set(sel_g.tolist()) - band == set(sel_r.tolist()) - band, \
            f"{where}: selected chunks differ outside the tolerance band"
    else:
        assert np.array_equal(sel_g, sel_r)
    # invariants of the index list
    assert np.all(np.diff(idx_gpu) > 0)
    assert set(range(T - w, T)) <= set(idx_gpu.tolist())
    assert idx_gpu.size <= min(T, kk * c + w)
    return sel_g, sel_r


def check_gather(case, l, b, h, idx_gpu):
    n = idx_gpu.size
    for which, t in (("k", case.k), ("v", case.v)):
        src = case.host_kv(t, l, b)
        out = case.out_rows(which, l, b, h)
        ref = oracle.gather(src, idx_gpu, h)
        assert np.array_equal(out[:n].view(np.uint8), ref.view(np.uint8)), \
            f"layer {l} seq {b} head {h}: {which}' rows are not bit-exact copies"
        assert np.all(out[n:].view(np.uint8) == POISON_BYTE), \
            f"layer {l} seq {b} head {h}: {which}' rows beyond n were written"


def check_unit(case, l, b, h, s_ref=None):
    """Full parity check of one (layer, sequence, head) unit; returns s_ref."""
    T, w, c, kk = case.seq_lens[b], case.w, case.c, case.kk(b)
    where = f"layer {l} seq {b} head {h}"
    a = (l // case.n_reuse) * case.n_reuse
    if s_ref is None:
        s_ref = oracle.chunk_scores(case.host_q(a, b), case.host_kv(case.k, a, b), h, case.Hq, w, c)
    s_gpu = case.gpu_scores(l, b, h)
    check_scores(s_gpu, s_ref, case.dtype, where)
    idx, tail = case.gpu_indices(l, b, h)
    check_selection(s_gpu, s_ref, idx, T, w, c, kk, case.dtype, where)
    assert np.all(tail == POISON_INDEX), f"{where}: index entries beyond n were written"
    check_gather(case, l, b, h, idx)
    return s_ref


def random_case(dtype, seq_lens, l_max, Hq, Hkv, d, w, c, n_layers=1, n_reuse=1, seed=0, scale_k=1.0,
                **kw):
    """Gaussian inputs drawn on the GPU (layout as the C-ABI takes it)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    T = int(sum(seq_lens))
    dt = tdtype(dtype)
    q = torch.randn((n_layers, len(seq_lens), w, Hq, d), generator=g, device="cuda").to(dt)
    k = (scale_k * torch.randn((n_layers, T, Hkv, d), generator=g, device="cuda")).to(dt)
    v = torch.randn((n_layers, T, Hkv, d), generator=g, device="cuda").to(dt)
    return Case(dtype, seq_lens, l_max, Hq, Hkv, d, w, c, n_reuse, q, k, v, **kw)
