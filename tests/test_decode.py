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


def _run(dtype, seq_lens, l_max, Hq, Hkv, d, w, c, seed, lengths=None, rows=None):
    """Decode over a host-written compacted cache checked against the oracle.
    rows(rng, pl, q) may give the (k, v) float arrays of all index_elems rows
    (default: N(0, 2) keys, N(0, 1) values); q is the [B, Hq, d] query array."""
    rng = np.random.default_rng(seed)
    prob = ck.make_problem(dtype, seq_lens, l_max, Hq, Hkv, d, w, c)
    pl = ck.plan(prob)
    n_rows = pl["index_elems"]
    B, G = len(seq_lens), Hq // Hkv
    q_f = rng.standard_normal((B, Hq, d))
    if rows is None:
        k_f, v_f = rng.standard_normal((n_rows, d)) * 2, rng.standard_normal((n_rows, d))
    else:
        k_f, v_f = rows(rng, pl, q_f)
    kh, kt = _bits(k_f, dtype)
    vh, vt = _bits(v_f, dtype)
    qh, qt = _bits(q_f, dtype)
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


# Work split of the decode call, as the library documents it: rows of 16
# pieces of 16 bytes take the one-wave kernel (about 2048 items, 32-row
# steps), other rows the workgroup kernel (about 512 items, 64-row steps);
# an item's block is a multiple of the step.
WAVE_ITEMS, WAVE_ROWS = 2048, 32
WG_ITEMS, WG_ROWS = 512, 64


def _steps_per_item(prob, dtype, d, Hq, Hkv):
    """Steps per full work item of the decode call on problem prob; the
    workspace size the library asks for must match the same split."""
    pl = ck.plan(prob)
    n_rows = Hkv * sum(pl["l_cap"])
    wave = d * (4 if dtype == ck.F32 else 2) == 256
    items, step = (WAVE_ITEMS, WAVE_ROWS) if wave else (WG_ITEMS, WG_ROWS)
    rpb = -(-max(-(-n_rows // items), step) // step) * step
    blocks = sum(Hkv * -(-lc // rpb) for lc in pl["l_cap"])
    need = blocks * (Hq // Hkv) * (d + 4) * 4
    assert ck.decode_workspace_bytes(prob) == -(-need // 256) * 256
    return rpb // step


def _full_or_random_lengths(pl, Hkv, seed):
    """Every other (sequence, head) keeps all L_cap rows (full work items,
    every step taken); the rest a random count."""
    rng = np.random.default_rng(seed)
    return np.array([pl["l_cap"][b] if (b + h) % 2 == 0 else rng.integers(0, pl["l_cap"][b] + 1)
                     for b in range(len(pl["l_cap"])) for h in range(Hkv)], dtype=np.int32)


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
    # two sequences with budgets of a few hundred rows: one step per work
    # item, a ragged last block per head
    _run(dtype, [4000, 1300], [700, 300], Hq, Hkv, d, 16, 10, seed=d + Hq)


def _monotone_rows(direction):
    """Keys along each head's mean query direction with a strength that rises
    (direction +1) or falls (-1) over the kept rows: with +1 every step's
    maximum exceeds the running one (the value sums are rescaled at every step
    with a finite running maximum), with -1 the first step holds it."""
    def rows(rng, pl, q):
        n_rows, d = pl["index_elems"], q.shape[2]
        k = rng.standard_normal((n_rows, d)) * 0.3
        v = rng.standard_normal((n_rows, d))
        B, Hq = q.shape[0], q.shape[1]
        Hkv = pl["length_elems"] // B
        G = Hq // Hkv
        for b in range(B):
            lc = pl["l_cap"][b]
            for h in range(Hkv):
                u = q[b, h * G:(h + 1) * G].mean(axis=0)
                u = u / np.linalg.norm(u)
                ramp = np.linspace(0.0, 1.0, lc) if direction > 0 else np.linspace(1.0, 0.0, lc)
                o = pl["index_off"][b] + h * lc
                k[o:o + lc] += (6.0 * np.sqrt(d) / 4.0) * ramp[:, None] * u[None, :]
        return k, v
    return rows


@pytest.mark.parametrize("dtype,d,Hq,Hkv,T,l_max,min_steps", [
    (ck.BF16, 128, 8, 2, 60000, 50000, 2),     # one-wave kernel: 100032 rows, 2 steps of 32
    (ck.F32, 64, 8, 1, 200000, 190000, 3),     # one-wave kernel, fp32: 3 steps
    (ck.BF16, 96, 12, 4, 30000, 29000, 4),     # workgroup kernel: 116064 rows, 4 steps of 64
    (ck.F32, 256, 8, 2, 40000, 30000, 2),      # workgroup kernel, 64 pieces per row: 2 steps
    (ck.BF16, 128, 24, 2, 70000, 69000, 3),    # one-wave kernel, G = 12 (two passes of query heads): 3 steps
])
def test_decode_multi_step_items(dtype, d, Hq, Hkv, T, l_max, min_steps):
    # caches large enough that every full work item walks several steps: the
    # next step's keys and values are requested during the current one, and
    # the running maximum and value sums carry over between steps
    prob = ck.make_problem(dtype, [T], [l_max], Hq, Hkv, d, 16, 10)
    assert _steps_per_item(prob, dtype, d, Hq, Hkv) >= min_steps
    pl = ck.plan(prob)
    _run(dtype, [T], [l_max], Hq, Hkv, d, 16, 10, seed=T + d,
         lengths=_full_or_random_lengths(pl, Hkv, seed=T))


@pytest.mark.parametrize("direction", [1, -1])
@pytest.mark.parametrize("d", [128, 96])      # the one-wave kernel and the workgroup kernel
def test_decode_running_max_moves(direction, d):
    # logits that rise (or fall) along the kept rows, over several steps per item
    T, l_max, Hq, Hkv = 80000, 75000, 8, 2
    prob = ck.make_problem(ck.BF16, [T], [l_max], Hq, Hkv, d, 16, 10)
    assert _steps_per_item(prob, ck.BF16, d, Hq, Hkv) >= 2
    pl = ck.plan(prob)
    lengths = np.array([pl["l_cap"][0]] * Hkv, dtype=np.int32)
    _run(ck.BF16, [T], [l_max], Hq, Hkv, d, 16, 10, seed=d + direction, lengths=lengths,
         rows=_monotone_rows(direction))


def test_decode_full_cache_of_32k_layer():
    # layer 0 of the 32-layer 32k stack with every token kept (L_max = T):
    # 262144 rows over 8 KV heads, 4 steps per one-wave item; the compacted
    # cache is the layer's K/V made head-major on the host side of the test
    wl = kvsynth.WORKLOADS["llama3-8b-32layer-T32768"].with_(n_layers=1)
    cache = kvsynth.make_cache(wl, device="cuda", seed=0)
    T, Hq, Hkv, d = wl.seq_lens[0], wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    prob = ck.make_problem(ck.BF16, [T], [T], Hq, Hkv, d, wl.window, wl.chunk)
    assert _steps_per_item(prob, ck.BF16, d, Hq, Hkv) == 4
    k_out = cache["k"][0].permute(1, 0, 2).contiguous().reshape(-1, d)
    v_out = cache["v"][0].permute(1, 0, 2).contiguous().reshape(-1, d)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    q = torch.randn((1, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    lengths = torch.full((Hkv,), T, dtype=torch.int32, device="cuda")
    ws_n = ck.decode_workspace_bytes(prob)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    out = torch.empty((1, Hq, d), dtype=torch.float32, device="cuda")
    ck.decode_attention(prob, q, k_out, v_out, lengths, out, ws, ws_n)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    qh, kh, vh = kvsynth.bf16_bits(q.cpu()), kvsynth.bf16_bits(k_out.cpu()), kvsynth.bf16_bits(v_out.cpu())
    G = Hq // Hkv
    for h in range(Hkv):
        ref = oracle.decode_attention(qh[0, h * G:(h + 1) * G], kh[h * T:(h + 1) * T], vh[h * T:(h + 1) * T])
        vmax = float(v_out[h * T:(h + 1) * T].abs().max().float())
        err = np.abs(got[0, h * G:(h + 1) * G] - ref)
        assert np.all(err <= TOL * (vmax + np.abs(ref))), (h, float(err.max()))


def test_decode_70b_shaped_compressed_cache():
    # the 70B-shaped batch's compacted cache (4 sequences of 131072 / 65536 /
    # 32768 / 16384 tokens at a 20% budget, 8 KV heads, G = 8): 395088 rows,
    # 7 steps per one-wave item; synthetic kept rows written on the host
    wl = kvsynth.WORKLOADS["llama-70b-80layer-4seq"]
    prob = ck.make_problem(ck.BF16, wl.seq_lens, wl.l_max, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                           wl.window, wl.chunk)
    assert _steps_per_item(prob, ck.BF16, wl.head_dim, wl.n_q_heads, wl.n_kv_heads) == 7
    pl = ck.plan(prob)
    _run(ck.BF16, wl.seq_lens, wl.l_max, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.chunk,
         seed=70, lengths=_full_or_random_lengths(pl, wl.n_kv_heads, seed=70))


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
