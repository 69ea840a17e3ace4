"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle.

Method: ChunkKV page, section 4.1 (Algorithm 1) and 4.2 (Algorithm 2);
softmax(QK^T/sqrt(d)) from Kara eq. (1).  Tolerances and the selection band
rule are in tests/harness.py.  Small cases are checked on every unit; the
workload-sized cases (the 8k layer, the 32-layer 32k stack that the benchmark
times, the chunk-size sweep and the 70B-shaped batch) check sampled units
against the oracle and properties on all units.
"""
import concurrent.futures
import os

import numpy as np
import pytest
import torch

import kvsynth
import oracle
from harness import (ATOL, POISON_BYTE, POISON_INDEX, RTOL, Case, check_gather, check_scores, check_selection,
                     check_unit, random_case)
from kv_cache_compression_win_amd import chunkkv as ck

pytestmark = pytest.mark.gpu

POOL = concurrent.futures.ThreadPoolExecutor(max_workers=max(8, min(16, os.cpu_count() or 8)))


def _all_units(case, layers=None):
    layers = range(case.L) if layers is None else layers
    anchors = sorted({(l // case.n_reuse) * case.n_reuse for l in layers})
    jobs = {}
    for a in anchors:
        for b in range(len(case.seq_lens)):
            for h in range(case.Hkv):
                jobs[(a, b, h)] = POOL.submit(oracle.chunk_scores, case.host_q(a, b),
                                              case.host_kv(case.k, a, b), h, case.Hq, case.w, case.c)
    for l in layers:
        a = (l // case.n_reuse) * case.n_reuse
        for b in range(len(case.seq_lens)):
            for h in range(case.Hkv):
                check_unit(case, l, b, h, s_ref=jobs[(a, b, h)].result())


# ------------------------------------------------------------ small shapes --

def test_tiny_fp32_workload():
    # 1 layer, 1 KV head, 1 query head, d=64, T=1000, fp32, 5 planted chunks;
    # w=8, c=10, L_max=100.  Generic (VALU) score path.
    d = kvsynth.make_tiny()
    wl = kvsynth.WORKLOADS["tiny-fp32-d64-T1000"]
    q = torch.from_numpy(d["q_full"][-wl.window:]).cuda()[None, None]     # [1,1,w,1,64]
    k = torch.from_numpy(d["k"]).cuda()[None]
    v = torch.from_numpy(d["v"]).cuda()[None]
    case = Case(ck.F32, wl.seq_lens, wl.l_max, 1, 1, 64, wl.window, wl.chunk, 1, q, k, v).run()
    check_unit(case, 0, 0, 0)
    sel = oracle.topk(case.gpu_scores(0, 0, 0).astype(np.float64), 10)
    assert set(d["planted"].tolist()) <= set(sel.tolist())


@pytest.mark.parametrize("c", [1, 2, 3, 5, 8, 10, 16, 20, 30, 32, 64])
def test_bf16_mfma_chunk_sizes(c):
    # MFMA path for every statically laid-out chunk size: several spans and
    # groups per head, a ragged last span and a short last chunk.
    T = 1737
    case = random_case(ck.BF16, [T], [T // 7], 8, 2, 128, 32, c, seed=c).run()
    _all_units(case)


@pytest.mark.parametrize("dtype,d,c,Hq,Hkv,w", [
    (ck.F32, 128, 10, 8, 2, 16),     # fp32 inputs
    (ck.BF16, 64, 10, 8, 2, 16),     # head_dim without an MFMA path
    (ck.BF16, 128, 7, 4, 1, 32),     # chunk size without a static layout
    (ck.BF16, 128, 100, 4, 2, 8),    # chunk size beyond the MFMA layouts
    (ck.F32, 32, 3, 2, 2, 4),
    (ck.F32, 64, 10, 64, 1, 64),     # G*w = 4096 rows, the largest supported (3-chunk spans)
])
def test_generic_path(dtype, d, c, Hq, Hkv, w):
    case = random_case(dtype, [1201], [300], Hq, Hkv, d, w, c, seed=d + c).run()
    _all_units(case)


@pytest.mark.parametrize("Hq,Hkv,w,c", [
    (3, 1, 5, 10), (24, 8, 7, 10), (8, 8, 32, 10),    # one row block, padding rows
    (64, 8, 64, 10), (64, 8, 64, 32),                 # 4 row blocks (the 70B shape)
    (64, 8, 64, 5), (64, 8, 64, 20),                  # 4 row blocks, 1 and 4 tiles per group
    (16, 2, 32, 10), (16, 2, 32, 5),                  # 2 row blocks, 2 KV heads
    (32, 4, 48, 10),                                  # 3 row blocks
    (64, 1, 64, 10), (32, 2, 256, 10),                # G*w = 4096, the largest supported: 32 row blocks
])
def test_mfma_row_blocks(Hq, Hkv, w, c):
    # G*w not a multiple of 32 (padding rows), and G*w > 128 (several row
    # blocks per head, each its own workgroup; blocks of one span range are
    # placed on one XCD when the worker counts allow).
    case = random_case(ck.BF16, [1500], [160], Hq, Hkv, 128, w, c, seed=Hq * w + c).run()
    _all_units(case)


@pytest.mark.parametrize("name,T,l_max,w,c", [
    ("k_zero_window_only", 700, 9, 32, 10),
    ("k_covers_all", 700, 700, 32, 10),
    ("k_above_C", 700, 5000, 32, 10),
    ("window_is_everything", 96, 10, 96, 10),
    ("chunk_longer_than_T", 90, 200, 16, 128),
    ("single_token_window", 333, 50, 1, 10),
    ("window_plus_one", 33, 10, 32, 10),
    ("one_chunk_left", 75, 70, 5, 10),
    ("all_of_20000_chunks", 20000, 20000, 16, 1),   # 1024-thread select, every chunk kept
])
def test_edge_cases(name, T, l_max, w, c):
    case = random_case(ck.BF16, [T], [l_max], 8, 2, 128, w, c, seed=T + w).run()
    _all_units(case)
    n = case.lengths[0]
    kk = l_max // c
    C = -(-T // c)
    if kk >= C or w == T:
        assert np.all(n == T)
    if kk == 0:
        assert np.all(n == w)


@pytest.mark.parametrize("dtype,d,c,T", [(ck.BF16, 128, 10, 3001), (ck.BF16, 128, 1, 2500),
                                         (ck.F32, 64, 10, 1201), (ck.BF16, 128, 2, 9001),
                                         (ck.BF16, 128, 1, 12000),    # C = 12000: 32 scores per thread
                                         (ck.BF16, 128, 1, 20000),    # C = 20000: 1024 threads x 32 scores
                                         (ck.BF16, 128, 1, 40000)])   # C = 40000 > 32768: scores re-read
def test_tied_scores_lower_id_first(dtype, d, c, T):
    # all-zero keys: every logit is 0, so every full chunk gets the same score
    # (c/T per row) and only the short last chunk differs; the top-k must take
    # the lowest chunk ids (ChunkKV page, section 4.1: ties are broken towards
    # the lower chunk id).
    l_max = T // 5
    case = random_case(dtype, [T], [l_max], 8, 2, d, 16, c, seed=T, scale_k=0.0).run()
    _all_units(case)
    kk = l_max // c
    for h in range(2):
        idx, _ = case.gpu_indices(0, 0, h)
        assert np.array_equal(idx[:kk * c], np.arange(kk * c))


def test_scores_underflow_to_zero():
    # very peaked attention: most chunk scores are exactly 0 in fp32 and the
    # k-th largest is 0, so the selection breaks a tie among the zero chunks.
    case = random_case(ck.BF16, [5000], [2000], 8, 2, 128, 16, 2, seed=5, scale_k=300.0).run()
    _all_units(case)
    for h in range(2):
        s = case.gpu_scores(0, 0, h)
        assert np.count_nonzero(s) < 1000 < s.size


def test_ragged_batch_and_many_sequences():
    # independent sequences packed along the token axis, each with its own
    # T_b and L_max,b; 11 sequences force several launches per phase.
    lens = [1000, 2500, 33, 64, 640, 641, 129, 3000, 50, 777, 1024]
    lmax = [100, 250, 5, 64, 0, 700, 20, 300, 49, 77, 1024]
    case = random_case(ck.BF16, lens, lmax, 8, 2, 128, 32, 10, seed=5).run()
    _all_units(case)


def _draw_problem(seed):
    """A seeded random problem: dtype, head_dim, GQA shape, window, chunk size
    (MFMA-supported or not), ragged sequences, budgets from 0 to above T, layer
    count and reuse interval; sizes bounded so the oracle takes about a second."""
    rng = np.random.default_rng(1000 + seed)
    dtype = ck.BF16 if rng.random() < 0.75 else ck.F32
    if dtype == ck.BF16:
        d = 128 if rng.random() < 0.7 else int(rng.choice([8, 64, 96, 256]))
    else:
        d = int(rng.choice([8, 32, 64, 100]))   # rows of 32..400 bytes (head_dim >= 8)
    Hkv = int(rng.choice([1, 2, 3, 8]))
    G = int(rng.choice([1, 2, 4, 5]))
    w = int(rng.integers(1, 49))
    while G * w > 192:
        w //= 2
    c = int(rng.choice([1, 2, 3, 4, 5, 7, 10, 11, 16, 20, 33, 64, 100]))
    B = int(rng.integers(1, 4))
    lens = [int(rng.integers(w, 6001)) for _ in range(B)]
    n_layers = int(rng.integers(1, 5))
    n_reuse = int(rng.integers(1, 4))
    anchors = -(-n_layers // n_reuse)
    # oracle work: anchors x sum(T) x Hkv x G*w x d multiply-adds
    budget = 1e9
    cost = anchors * sum(lens) * Hkv * G * w * d
    if cost > budget:
        f = budget / cost
        lens = [max(w, int(t * f)) for t in lens]
    lmax = []
    for t in lens:
        u = rng.random()
        lmax.append(0 if u < 0.15 else t if u < 0.3 else int(rng.integers(0, t + 50)))
    return dict(dtype=dtype, d=d, Hq=G * Hkv, Hkv=Hkv, w=w, c=c, lens=lens, lmax=lmax,
                n_layers=n_layers, n_reuse=n_reuse)


@pytest.mark.parametrize("seed", range(64))
def test_random_problems(seed):
    p = _draw_problem(seed)
    print("problem", p, flush=True)
    case = random_case(p["dtype"], p["lens"], p["lmax"], p["Hq"], p["Hkv"], p["d"], p["w"], p["c"],
                       n_layers=p["n_layers"], n_reuse=p["n_reuse"], seed=seed).run()
    _all_units(case)


@pytest.mark.parametrize("n_reuse", [1, 2, 3, 9])
def test_layer_index_reuse(n_reuse):
    # Algorithm 2: anchor layers score, the others gather their own K/V with
    # the anchor's indices.  The workspace holds one scoring layer only, so
    # anchors are scored in several launches.
    case = random_case(ck.BF16, [900, 1300], [90, 200], 8, 2, 128, 16, 10, n_layers=5,
                       n_reuse=n_reuse, seed=n_reuse, n_score_layers=1).run()
    _all_units(case)
    assert case.scores.shape[0] == -(-5 // n_reuse)


@pytest.mark.parametrize("n_reuse", [1, 2])
def test_more_layers_than_one_launch(n_reuse):
    # more than 32 layers in one call: the scoring layers are split over
    # several launches (32 at most each) and so are the gathers.
    case = random_case(ck.BF16, [300, 517], [40, 60], 8, 2, 128, 16, 10, n_layers=35,
                       n_reuse=n_reuse, seed=35 + n_reuse).run()
    _all_units(case)
    assert case.scores.shape[0] == -(-35 // n_reuse)


def test_graph_capture_replays_match_eager():
    # chunkkv_compress_layers allocates nothing and records no memsets, so a
    # call can be captured in a HIP graph; every replay (with eager work and
    # synchronisations between them) must reproduce the eager outputs bit for
    # bit.
    case = random_case(ck.BF16, [4096, 1500], [400, 150], 32, 8, 128, 32, 10, n_layers=4, n_reuse=2,
                       seed=7).run()
    _all_units(case)            # the eager outputs the replays must equal match the oracle
    ref = case.bufs
    L = case.L
    bufs = ck.Buffers(case.prob, L, case.n_reuse, case.d, torch.bfloat16, "cuda")
    qs = [case.q_win[l] if l % case.n_reuse == 0 else None for l in range(L)]
    stream = torch.cuda.Stream()
    args = (case.prob, case.n_reuse, qs, [case.k[l] for l in range(L)], [case.v[l] for l in range(L)],
            [bufs.k_out[l] for l in range(L)], [bufs.v_out[l] for l in range(L)], bufs.scores, bufs.indices,
            bufs.lengths, bufs.workspace, bufs.ws_bytes)
    with torch.cuda.stream(stream):
        ck.compress_layers(*args, stream=stream)      # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        ck.compress_layers(*args, stream=stream)
    torch.cuda.synchronize()
    outs = (bufs.scores, bufs.indices, bufs.lengths, bufs.k_out, bufs.v_out)
    refs = (ref.scores, ref.indices, ref.lengths, ref.k_out, ref.v_out)
    for rep in range(3):
        # eager work between replays: the same poison as the eager run (rows
        # past each head's length are left untouched by the library)
        for t in (bufs.scores, bufs.lengths, bufs.k_out, bufs.v_out):
            t.view(torch.uint8).fill_(POISON_BYTE)
        bufs.indices.fill_(POISON_INDEX)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, refs):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), rep


# ------------------------------------------- exchange mode and its fallback --
# With CHUNKKV_SCORE_PATH=exchange (read by the library at every call), bf16
# caches with head_dim 128, one 128-row block per head and a chunk size with
# an exchange kernel are scored in one persistent launch whose spans exchange
# per-row statistics (no chunk partials in memory); by default they take the
# chunk-partial path (score kernel writing U, then the combine).
# CHUNKKV_SPIN_LIMIT=0 makes every exchange span give up waiting for its
# head's row statistics and spill its partials (the head's last span scores
# them).

@pytest.mark.parametrize("c", [4, 5, 6, 8, 10, 15, 16, 25])
def test_exchange_spill_path_equals_normal_path(c, monkeypatch):
    # two sequences, three scoring layers: every span spilled gives the same
    # bits as every span scored from LDS (same products, same order)
    monkeypatch.setenv("CHUNKKV_SCORE_PATH", "exchange")
    case = random_case(ck.BF16, [3000, 1700], [300, 170], 32, 8, 128, 32, c, n_layers=3, n_reuse=1,
                       seed=100 + c).run()
    s_norm, i_norm, l_norm = case.scores.copy(), case.indices.copy(), case.lengths.copy()
    _all_units(case)
    monkeypatch.setenv("CHUNKKV_SPIN_LIMIT", "0")
    case.run()
    assert np.array_equal(case.scores.view(np.uint32), s_norm.view(np.uint32))
    assert np.array_equal(case.indices, i_norm) and np.array_equal(case.lengths, l_norm)
    _all_units(case)


@pytest.mark.parametrize("seq_lens,l_max,n_layers", [([8192], [819], 1),             # the 8k layer's shape
                                                      ([32768], [3276], 2),
                                                      ([1000, 2500, 33, 640, 3000, 777, 1024, 50, 129],
                                                       [100, 250, 5, 0, 300, 77, 1024, 49, 20], 2)])
def test_exchange_path_matches_oracle(seq_lens, l_max, n_layers, monkeypatch):
    # the exchange kernel on the 8k layer's shape, two 32k layers and nine
    # ragged sequences (two launches); it agrees with the default
    # chunk-partial path within tolerance
    case = random_case(ck.BF16, seq_lens, l_max, 32, 8, 128, 32, 10, n_layers=n_layers, seed=len(seq_lens)).run()
    _all_units(case)
    s_part = case.scores.copy()
    monkeypatch.setenv("CHUNKKV_SCORE_PATH", "exchange")
    case.run()
    err = np.abs(case.scores.astype(np.float64) - s_part)
    assert np.all(err <= 2 * RTOL[ck.BF16] * np.abs(s_part.astype(np.float64)) + ATOL)
    _all_units(case)


def test_strided_kv_layout():
    # K/V with a padded head stride (d + 64 elements) and token stride.
    Hkv, d, T = 2, 128, 1100
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    big_k = torch.randn((1, T, Hkv, d + 64), generator=g, device="cuda").to(torch.bfloat16)
    big_v = torch.randn((1, T, Hkv, d + 64), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((1, 1, 32, 8, d), generator=g, device="cuda").to(torch.bfloat16)
    k = big_k[..., :d]
    v = big_v[..., :d]
    case = Case(ck.BF16, [T], [110], 8, Hkv, d, 32, 10, 1, q, big_k, big_v,
                kv_strides=(Hkv * (d + 64), d + 64))
    case.run()
    # the oracle sees the logical [T, Hkv, d] view
    case.k, case.v = k.contiguous(), v.contiguous()
    _all_units(case)


def test_per_layer_entry_points_match_driver():
    # chunkkv_score / chunkkv_select / chunkkv_gather called one by one give
    # bit-identical results to chunkkv_compress_layers on the same layer.
    case = random_case(ck.BF16, [1500, 700], [150, 70], 32, 8, 128, 32, 10, seed=3).run()
    pl = case.plan
    ws_n = ck.workspace_bytes(case.prob, 1)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    scores = torch.empty(pl["scores_elems"], dtype=torch.float32, device="cuda")
    idx = torch.full((pl["index_elems"],), POISON_INDEX, dtype=torch.int32, device="cuda")
    lens = torch.empty(pl["length_elems"], dtype=torch.int32, device="cuda")
    ko = torch.empty((pl["index_elems"], 128), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    ck.score(case.prob, case.q_win[0], case.k[0], scores, ws, ws_n)
    ck.select(case.prob, scores, idx, lens)
    ck.gather(case.prob, case.k[0], case.v[0], idx, lens, ko, vo)
    torch.cuda.synchronize()
    assert np.array_equal(scores.cpu().numpy(), case.scores[0])
    assert np.array_equal(idx.cpu().numpy(), case.indices[0])
    assert np.array_equal(lens.cpu().numpy(), case.lengths[0])
    for b in range(2):
        for h in range(8):
            o = pl["index_off"][b] + h * pl["l_cap"][b]
            n = int(case.lengths[0][b * 8 + h])
            assert torch.equal(ko[o:o + n], case.bufs.k_out[0, o:o + n])
            assert torch.equal(vo[o:o + n], case.bufs.v_out[0, o:o + n])


def test_deterministic():
    a = random_case(ck.BF16, [2000], [200], 32, 8, 128, 32, 10, seed=9).run()
    s1, i1 = a.scores.copy(), a.indices.copy()
    a.run()
    assert np.array_equal(s1, a.scores) and np.array_equal(i1, a.indices)


@pytest.mark.parametrize("dtype,d,c", [(ck.BF16, 128, 10),    # events on the score and gather kernels
                                       (ck.F32, 64, 10),      # events recorded between the phases' kernels
                                       (ck.BF16, 128, 2)])    # two passes over the keys: markers
def test_phase_events(dtype, d, c):
    case = random_case(dtype, [4096], [400], 32, 8, d, 32, c, n_layers=4, n_reuse=2, seed=2)
    ev = ck.PhaseEvents()
    case.run(phase_events=ev)
    times = [ev.elapsed_ms(i, i + 1) for i in range(ck.N_PHASE_EVENTS - 1)]
    assert all(t >= 0 for t in times) and ev.elapsed_ms(0, ck.N_PHASE_EVENTS - 1) > 0


# -------------------------------------------------------- workload sizes --

def _props_all_units(case):
    """Properties that hold for every unit at any size."""
    G = case.Hq // case.Hkv
    for a in range(case.scores.shape[0]):
        for b, T in enumerate(case.seq_lens):
            C, kk = case.C(b), case.kk(b)
            for h in range(case.Hkv):
                s = case.gpu_scores(a * case.n_reuse, b, h).astype(np.float64)
                assert abs(s.sum() - G * case.w) <= RTOL[case.dtype] * G * case.w
                idx, _ = case.gpu_indices(a * case.n_reuse, b, h)
                assert np.array_equal(idx, oracle.indices(T, case.w, case.c, oracle.topk(s, kk)))


def _gather_all_layers_on_gpu(case):
    """Bit-exact gather check of every layer, sequence and head on the GPU."""
    for l in range(case.L):
        a = l // case.n_reuse
        for b in range(len(case.seq_lens)):
            s0 = int(case.starts[b])
            for h in range(case.Hkv):
                idx, _ = case.gpu_indices(l, b, h)
                it = torch.from_numpy(idx.astype(np.int64)).cuda() + s0
                o = case.plan["index_off"][b] + h * case.plan["l_cap"][b]
                for t, out in ((case.k, case.bufs.k_out), (case.v, case.bufs.v_out)):
                    ref = t[l, :, h, :].index_select(0, it)
                    got = out[l, o:o + idx.size]
                    assert torch.equal(ref.view(torch.int16), got.view(torch.int16)), (l, b, h)


def test_llama3_8b_layer_T8192():
    wl = kvsynth.WORKLOADS["llama3-8b-1layer-T8192"]
    cache = kvsynth.make_cache(wl, device="cuda", seed=0)
    case = Case(ck.BF16, wl.seq_lens, wl.l_max, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window,
                wl.chunk, wl.n_reuse, cache["q_win"], cache["k"], cache["v"]).run()
    _all_units(case)


def test_llama3_8b_32layer_T32768_all_units():
    # The workload the benchmark times, in the same launch configuration:
    # every one of its 16 scoring layers x 8 KV heads against the oracle
    # (about 1 s of host time per unit), each with its reusing layer.
    wl = kvsynth.WORKLOADS["llama3-8b-32layer-T32768"]
    cache = kvsynth.make_cache(wl, device="cuda", seed=0)
    case = Case(ck.BF16, wl.seq_lens, wl.l_max, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window,
                wl.chunk, wl.n_reuse, cache["q_win"], cache["k"], cache["v"]).run()
    _props_all_units(case)
    _gather_all_layers_on_gpu(case)
    _all_units(case)


def test_chunk_size_sweep_T16384():
    # every chunk size and budget of the sweep, every KV head against the
    # oracle (the scores of a 16384-token head cost about 0.7 s of host time)
    wl = kvsynth.WORKLOADS["llama3-8b-csweep-T16384"]
    cache = kvsynth.make_cache(wl, device="cuda", seed=0)
    refs = {}
    for c in kvsynth.CSWEEP_CHUNKS:
        for h in range(wl.n_kv_heads):
            refs[(c, h)] = POOL.submit(oracle.chunk_scores, kvsynth.host_array(cache["q_win"][0, 0]),
                                       kvsynth.host_array(cache["k"][0]), h, wl.n_q_heads, wl.window, c)
    for c in kvsynth.CSWEEP_CHUNKS:
        for l_max in kvsynth.CSWEEP_LMAX:
            case = Case(ck.BF16, wl.seq_lens, (l_max,), wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                        wl.window, c, 1, cache["q_win"], cache["k"], cache["v"]).run()
            _props_all_units(case)
            for h in range(wl.n_kv_heads):
                check_unit(case, 0, 0, h, s_ref=refs[(c, h)].result())


def test_llama70b_batch_sampled():
    # 70B-shaped batch (64 query heads, 8 KV heads, w=64, four sequences of
    # 131072/65536/32768/16384 tokens in one launch, 20% budget, reuse 2);
    # 4 of the 80 layers.
    wl = kvsynth.WORKLOADS["llama-70b-80layer-4seq"].with_(n_layers=4)
    cache = kvsynth.make_cache(wl, device="cuda", seed=0)
    case = Case(ck.BF16, wl.seq_lens, wl.l_max, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window,
                wl.chunk, wl.n_reuse, cache["q_win"], cache["k"], cache["v"]).run()
    _props_all_units(case)
    _gather_all_layers_on_gpu(case)
    # the oracle on every head of the 32768- and 16384-token sequences and on
    # two heads of each longer one, for both scoring layers (a 131072-token
    # unit costs about 20 s of host time; about 260 s in all, spread over
    # the host's threads)
    units = [(a, b, h) for a in (0, 2) for b in (2, 3) for h in range(case.Hkv)]
    units += [(a, b, h) for a in (0, 2) for b, hs in ((0, (5, 2)), (1, (1, 6))) for h in hs]
    jobs = {(a, b, h): POOL.submit(oracle.chunk_scores, case.host_q(a, b), case.host_kv(case.k, a, b),
                                   h, case.Hq, case.w, case.c) for (a, b, h) in units}
    for (a, b, h), fut in jobs.items():
        s_ref = fut.result()
        for l in (a, a + 1):
            check_unit(case, l, b, h, s_ref=s_ref)


# --------------------------------------------------- selection on any input --

def _adversarial_scores(rng, C, with_pos_nan):
    s = rng.random(C).astype(np.float32)
    bits = s.view(np.uint32)
    r = rng.random(C)
    bits[r < 0.15] = np.float32(-1.5).view(np.uint32)      # negative
    bits[(r >= 0.15) & (r < 0.25)] = 0x80000000             # -0
    bits[(r >= 0.25) & (r < 0.32)] = 0xFFC00000             # negative NaN
    bits[(r >= 0.32) & (r < 0.35)] = 0x7F800000             # +inf
    if with_pos_nan:
        bits[(r >= 0.35) & (r < 0.38)] = 0x7FC00000         # positive NaN
    return bits.view(np.float32)


@pytest.mark.parametrize("T,c,w,l_max", [(2000, 10, 16, 300),       # register path (C = 200)
                                         (90001, 10, 32, 9000),     # C = 9001: 32 scores per thread
                                         (200001, 10, 32, 20000),   # C = 20001: 1024 threads x 32 scores
                                         (400001, 10, 32, 40000)])  # C = 40001 > 32768: scores re-read
def test_select_any_scores_stays_in_range(T, c, w, l_max):
    # chunkkv_select takes caller scores: a score with the sign bit set counts
    # as 0 and the rest are ordered by bit pattern, so exactly k chunks are
    # selected and the index list never leaves [0, T) or exceeds L_cap.
    Hkv = 2
    prob = ck.make_problem(ck.BF16, [T], [l_max], 4, Hkv, 128, w, c)
    pl = ck.plan(prob)
    C = -(-T // c)
    kk = l_max // c
    rng = np.random.default_rng(T)
    for with_pos_nan in (False, True):
        host = np.concatenate([_adversarial_scores(rng, C, with_pos_nan) for _ in range(Hkv)])
        scores = torch.from_numpy(host).cuda()
        indices = torch.full((pl["index_elems"],), POISON_INDEX, dtype=torch.int32, device="cuda")
        lengths = torch.zeros(Hkv, dtype=torch.int32, device="cuda")
        ck.select(prob, scores, indices, lengths)
        torch.cuda.synchronize()
        idx_all, n_all = indices.cpu().numpy(), lengths.cpu().numpy()
        L_cap = int(pl["l_cap"][0])
        for h in range(Hkv):
            n = int(n_all[h])
            idx = idx_all[h * L_cap:h * L_cap + n]
            assert n <= L_cap
            assert np.all(idx_all[h * L_cap + n:(h + 1) * L_cap] == POISON_INDEX)
            assert np.all(np.diff(idx) > 0) and idx[0] >= 0 and idx[-1] < T
            assert set(range(T - w, T)) <= set(idx.tolist())
            if not with_pos_nan:
                s = host[h * C:(h + 1) * C].astype(np.float64)
                s = np.where(np.signbit(s), 0.0, s)            # sign bit -> 0
                sel = oracle.topk(s, kk)
                assert np.array_equal(idx, oracle.indices(T, w, c, sel))


def _digit_scores(rng, C, kind):
    """Scores whose bit patterns share their top 8, 16 or 24 bits (the select
    must resolve the k-th largest in a later radix digit), tie in large groups,
    or are all distinct; fp32 patterns of non-negative values."""
    if kind == "distinct":
        return rng.random(C).astype(np.float32)
    if kind == "ties":
        return rng.integers(0, 5, C).astype(np.float32) / 4.0
    shared = {"share8": 8, "share16": 16, "share24": 24}[kind]
    base = np.uint32(0x3f000000)
    low = rng.integers(0, 1 << (31 - shared), C, dtype=np.uint64).astype(np.uint32)
    bits = (base & np.uint32(~((1 << (31 - shared)) - 1) & 0x7fffffff)) | low
    return bits.view(np.float32)


@pytest.mark.parametrize("C", [1, 63, 64, 65, 512, 513, 1025, 4096, 4097, 8193])
@pytest.mark.parametrize("kind", ["distinct", "ties", "share8", "share16", "share24"])
def test_select_threshold_bits(C, kind):
    # chunkkv_select against the oracle's full-sort top-k on score sets whose
    # k-th largest differs from its neighbours only in the low 23, 15 or 7
    # bits of its pattern (the bitwise threshold search must run through all
    # of them), tie at the k-th score, or sit on either side of the register
    # layouts' chunk limits (1, 2, 8 and 16 scores per thread of 512);
    # budgets from one chunk to all but one.
    c, w = 4, 3
    T = C * c - 1 if C > 1 else 3
    Hkv = 2
    rng = np.random.default_rng(C * 31 + len(kind))
    for kk in sorted({1, max(1, C // 3), max(1, C - 1)}):
        prob = ck.make_problem(ck.F32, [T], [kk * c], 4, Hkv, 64, w, c)
        pl = ck.plan(prob)
        host = np.concatenate([_digit_scores(rng, C, kind) for _ in range(Hkv)])
        scores = torch.from_numpy(host).cuda()
        indices = torch.full((pl["index_elems"],), POISON_INDEX, dtype=torch.int32, device="cuda")
        lengths = torch.zeros(Hkv, dtype=torch.int32, device="cuda")
        ck.select(prob, scores, indices, lengths)
        torch.cuda.synchronize()
        idx_all, n_all = indices.cpu().numpy(), lengths.cpu().numpy()
        L_cap = int(pl["l_cap"][0])
        for h in range(Hkv):
            s = host[h * C:(h + 1) * C].astype(np.float64)
            want = oracle.indices(T, w, c, oracle.topk(s, min(kk, C)))
            n = int(n_all[h])
            assert n == len(want) <= L_cap, (kind, C, kk, h)
            assert np.array_equal(idx_all[h * L_cap:h * L_cap + n], want), (kind, C, kk, h)
            assert np.all(idx_all[h * L_cap + n:(h + 1) * L_cap] == POISON_INDEX)


def test_gather_clamps_caller_indices_and_lengths():
    # chunkkv_gather with caller-made indices and lengths: lengths are
    # clamped into [0, L_cap] and index values into [0, T); rows past the
    # clamped length keep their poison.
    T, c, w, l_max, Hkv, d = 700, 10, 16, 200, 3, 128
    prob = ck.make_problem(ck.BF16, [T], [l_max], 6, Hkv, d, w, c)
    pl = ck.plan(prob)
    L_cap = int(pl["l_cap"][0])
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    k = torch.randn((T, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((T, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    rng = np.random.default_rng(5)
    idx_h = rng.integers(-3 * T, 3 * T, size=pl["index_elems"]).astype(np.int32)
    idx_h[:5] = [np.iinfo(np.int32).min, -1, T, T - 1, np.iinfo(np.int32).max]
    len_h = np.array([L_cap + 50, -4, L_cap // 2], dtype=np.int32)
    ko = torch.empty((pl["index_elems"], d), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    ko.view(torch.uint8).fill_(POISON_BYTE)
    vo.view(torch.uint8).fill_(POISON_BYTE)
    ck.gather(prob, k, v, torch.from_numpy(idx_h).cuda(), torch.from_numpy(len_h).cuda(), ko, vo)
    torch.cuda.synchronize()
    kh, vh = kvsynth.host_array(k), kvsynth.host_array(v)
    ko_h, vo_h = kvsynth.host_array(ko), kvsynth.host_array(vo)
    for h in range(Hkv):
        n = min(max(int(len_h[h]), 0), L_cap)
        rows = np.clip(idx_h[h * L_cap:h * L_cap + n].astype(np.int64), 0, T - 1)
        for out, src in ((ko_h, kh), (vo_h, vh)):
            blk = out[h * L_cap:(h + 1) * L_cap]
            assert np.array_equal(blk[:n].view(np.uint16), src[rows, h].view(np.uint16))
            assert np.all(blk[n:].view(np.uint8) == POISON_BYTE)
