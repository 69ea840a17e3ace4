"""GPU parity of chunkkv_decode_attention, the consumer of the compacted cache,
against the oracle's decode attention (softmax(q . k / sqrt(d)) weights of the
Kara page, eq. (1)).

Inputs are synthetic compacted caches written on the host (random kept rows,
random lengths from 0 to L_cap, the rows past each length poisoned with NaN so
that reading one shows), never the library's own outputs.  Tolerance: every
output is a convex combination of kept value rows, computed from exactly
widened inputs with fp32 accumulation in a fixed order, so the error is a few
fp32 roundings of the largest value: |o_gpu - o_ref| <= 1e-5 * (max|v| + |o_ref|).
"""
import numpy as np
import pytest
import torch

import kvsynth
import oracle
from kv_cache_compression_win_amd import chunkkv as ck

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _bits(a, dtype):
    """Host array of the cache dtype (bf16 as raw uint16 patterns) and its torch form."""
    if dtype == ck.F32:
        t = torch.from_numpy(a.astype(np.float32))
        return t.numpy(), t
    t = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    return kvsynth.bf16_bits(t), t


def _run(dtype, seq_lens, l_max, Hq, Hkv, d, w, c, seed, lengths=None):
    rng = np.random.default_rng(seed)
    prob = ck.make_problem(dtype, seq_lens, l_max, Hq, Hkv, d, w, c)
    pl = ck.plan(prob)
    rows = pl["index_elems"]
    B, G = len(seq_lens), Hq // Hkv
    kh, kt = _bits(rng.standard_normal((rows, d)) * 2, dtype)
    vh, vt = _bits(rng.standard_normal((rows, d)), dtype)
    qh, qt = _bits(rng.standard_normal((B, Hq, d)), dtype)
    if lengths is None:
        lengths = np.array([rng.integers(0, pl["l_cap"][b] + 1) for b in range(B) for _ in range(Hkv)],
                           dtype=np.int32)
    # poison every row past its length: NaN in both caches
    nan = torch.tensor(float("nan"), dtype=kt.dtype)
    for b in range(B):
        for h in range(Hkv):
            o = pl["index_off"][b] + h * pl["l_cap"][b]
            kt[o + int(lengths[b * Hkv + h]):o + pl["l_cap"][b]] = nan
            vt[o + int(lengths[b * Hkv + h]):o + pl["l_cap"][b]] = nan
    kh = kt.numpy() if dtype == ck.F32 else kvsynth.bf16_bits(kt)
    vh = vt.numpy() if dtype == ck.F32 else kvsynth.bf16_bits(vt)
    ws_n = ck.decode_workspace_bytes(prob)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    out = torch.full((B, Hq, d), 12345.0, dtype=torch.float32, device="cuda")
    ck.decode_attention(prob, qt.cuda(), kt.cuda(), vt.cuda(), torch.from_numpy(lengths).cuda(), out, ws, ws_n)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            n = int(lengths[b * Hkv + h])
            o = pl["index_off"][b] + h * pl["l_cap"][b]
            ref = oracle.decode_attention(qh[b, h * G:(h + 1) * G], kh[o:o + n], vh[o:o + n])
            vmax = float(np.abs(vt[o:o + n].float().numpy()).max()) if n else 0.0
            err = np.abs(got[b, h * G:(h + 1) * G] - ref)
            assert np.all(err <= TOL * (vmax + np.abs(ref))), (b, h, n, float(err.max()))
    return got


@pytest.mark.parametrize("dtype,d,Hq,Hkv", [
    (ck.BF16, 128, 32, 8),     # Llama-3-8B heads (G = 4)
    (ck.BF16, 128, 64, 8),     # 70B-shaped heads (G = 8)
    (ck.BF16, 128, 24, 2),     # G = 12: two passes over the kept rows
    (ck.F32, 64, 8, 2),        # fp32 cache
    (ck.BF16, 96, 6, 3),       # 12 pieces per row
    (ck.BF16, 8, 4, 1),        # one 16-byte piece per row
    (ck.F32, 256, 4, 2),       # 64 pieces per row
    (ck.F32, 64, 16, 2),       # one-wave kernel, fp32, 8 query heads per pass
    (ck.BF16, 96, 24, 3),      # workgroup kernel, 8 query heads per pass
    (ck.F32, 256, 12, 1),      # workgroup kernel, G = 12: two passes
])
def test_decode_matches_oracle(dtype, d, Hq, Hkv):
    # two sequences whose budgets span several 256-row blocks and a ragged last block
    _run(dtype, [4000, 1300], [700, 300], Hq, Hkv, d, 16, 10, seed=d + Hq)


def test_decode_edge_lengths_and_many_sequences():
    # lengths 0 (zeros out), 1, exactly one block, one block + 1 and L_cap;
    # eleven sequences force two launches
    lens = [3000] * 11
    prob = ck.make_problem(ck.BF16, lens, [600] * 11, 8, 2, 128, 16, 10)
    lc = ck.plan(prob)["l_cap"][0]
    choice = [0, 1, 256, 257, lc, 17]
    lengths = np.array([choice[i % len(choice)] for i in range(22)], dtype=np.int32)
    got = _run(ck.BF16, lens, [600] * 11, 8, 2, 128, 16, 10, seed=5, lengths=lengths)
    assert np.all(got[0, 0:4] == 0.0)            # sequence 0, KV head 0 keeps no rows


def test_decode_after_compression_workload():
    # the shapes of the 8k layer: decode over a cache of L_cap rows per head
    wl = kvsynth.WORKLOADS["llama3-8b-1layer-T8192"]
    _run(ck.BF16, wl.seq_lens, wl.l_max, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.chunk,
         seed=8)


@pytest.mark.parametrize("d", [128, 96])   # the one-wave kernel and the workgroup kernel
def test_decode_graph_replays_match_eager(d):
    # the call only launches kernels, so it can be captured; every replay
    # (with eager work and synchronisation between) equals the eager output
    prob = ck.make_problem(ck.BF16, [5000], [900], 16, 4, d, 16, 10)
    pl = ck.plan(prob)
    g = torch.Generator(device="cuda")
    g.manual_seed(d)
    k = torch.randn((pl["index_elems"], d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((pl["index_elems"], d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((1, 16, d), generator=g, device="cuda").to(torch.bfloat16)
    lengths = torch.tensor([pl["l_cap"][0], 1, 0, 333], dtype=torch.int32, device="cuda")
    ws_n = ck.decode_workspace_bytes(prob)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    eager = torch.empty((1, 16, d), dtype=torch.float32, device="cuda")
    ck.decode_attention(prob, q, k, v, lengths, eager, ws, ws_n)
    torch.cuda.synchronize()
    out = torch.zeros_like(eager)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        ck.decode_attention(prob, q, k, v, lengths, out, ws, ws_n)
    for rep in range(3):
        out.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        del scratch
