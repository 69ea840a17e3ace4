"""GPU parity of chunkkv_compress_layers_hybrid: the hybrid layer policy of
the ChunkKV page, section 5.7 (chunk-level selection in the lower layers,
token-level, c = 1, in the upper ones) as a per-layer chunk size, with
Algorithm 2 (section 4.2) restarting at every change of chunk size.

Every anchor's scores, selection and every layer's gathered rows are checked
against the oracle run on each run of layers with that run's chunk size, and
the whole output against one chunkkv_compress_layers call per run, bit for
bit.
"""
import numpy as np
import pytest
import torch

import oracle
from harness import POISON_BYTE, POISON_INDEX, check_scores, check_selection, tdtype
from kv_cache_compression_win_amd import chunkkv as ck
import kvsynth

pytestmark = pytest.mark.gpu


def _inputs(dtype, seq_lens, L, Hq, Hkv, d, w, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dt = tdtype(dtype)
    T = int(sum(seq_lens))
    q = torch.randn((L, len(seq_lens), w, Hq, d), generator=g, device="cuda").to(dt)
    k = torch.randn((L, T, Hkv, d), generator=g, device="cuda").to(dt)
    v = torch.randn((L, T, Hkv, d), generator=g, device="cuda").to(dt)
    return q, k, v


def _runs(chunks):
    runs, l = [], 0
    while l < len(chunks):
        e = l
        while e < len(chunks) and chunks[e] == chunks[l]:
            e += 1
        runs.append((l, e, chunks[l]))
        l = e
    return runs


def _hybrid(prob, chunks, n_reuse, q, k, v, d, dt):
    L = len(chunks)
    hb = ck.HybridBuffers(prob, chunks, n_reuse, d, dt)
    for t in hb.k_out + hb.v_out:
        t.view(torch.uint8).fill_(POISON_BYTE)
    hb.indices.fill_(POISON_INDEX)
    qs = []
    for l0, e, _ in _runs(chunks):
        qs += [q[l] if (l - l0) % n_reuse == 0 else None for l in range(l0, e)]
    ck.compress_layers_hybrid(prob, chunks, n_reuse, qs, [k[l] for l in range(L)], [v[l] for l in range(L)],
                              hb.k_out, hb.v_out, hb.scores, hb.indices, hb.lengths, hb.workspace, hb.ws_bytes)
    torch.cuda.synchronize()
    return hb


CASES = [
    # (dtype, seq_lens, l_max, Hq, Hkv, d, w, layer chunk sizes, n_reuse)
    (ck.BF16, [700, 333], [140, 70], 8, 2, 128, 16, [10, 10, 10, 10, 1, 1, 1, 1], 2),
    (ck.BF16, [900], [300], 8, 2, 128, 16, [10, 10, 4, 1, 1, 10], 2),
    (ck.F32, [500, 64], [100, 30], 4, 2, 64, 8, [8, 8, 8, 1, 1], 3),
    # more anchors in one run than one launch scores (36 > 32) and more
    # sequences than one launch holds (9 > 8), every layer an anchor
    (ck.BF16, [300, 200, 257, 128, 199, 310, 64, 96, 150], [60, 40, 51, 25, 39, 62, 12, 19, 30], 8, 2, 128, 16,
     [10] * 36 + [1] * 4, 1),
]


def _check_oracle(hb, dtype, seq_lens, l_max, Hq, Hkv, d, w, chunks, n_reuse, q, k, v):
    """Every anchor's scores and selection and every layer's gathered rows of
    a hybrid call against the oracle's Algorithm 2 on each run of layers."""
    hp = hb.hplan
    scores, indices, lengths = hb.scores.cpu().numpy(), hb.indices.cpu().numpy(), hb.lengths.cpu().numpy()
    starts = np.concatenate([[0], np.cumsum(seq_lens)]).astype(np.int64)
    anchor = 0
    for l0, e, c in _runs(chunks):
        pl = ck.plan(ck.make_problem(dtype, seq_lens, l_max, Hq, Hkv, d, w, c))
        for b, T in enumerate(seq_lens):
            s0, s1 = int(starts[b]), int(starts[b + 1])
            qs = [kvsynth.host_array(q[l, b]) if (l - l0) % n_reuse == 0 else None for l in range(l0, e)]
            ks = [kvsynth.host_array(k[l, s0:s1]) for l in range(l0, e)]
            vs = [kvsynth.host_array(v[l, s0:s1]) for l in range(l0, e)]
            ref = oracle.compress_layers(qs, ks, vs, Hq, w, c, l_max[b], n_reuse)
            C, cap = ref["C"], int(pl["l_cap"][b])
            assert cap == ref["l_cap"]
            for i, l in enumerate(range(l0, e)):
                a = anchor + i // n_reuse
                where = f"layer {l} (chunk {c}) seq {b}"
                for h in range(Hkv):
                    so = hp["score_block_off"][a] + pl["score_off"][b] + h * C
                    io = hp["index_block_off"][a] + pl["index_off"][b] + h * cap
                    n = int(lengths[hp["length_block_off"][a] + b * Hkv + h])
                    s_ref = ref["scores"][(i // n_reuse) * n_reuse, h]
                    s_gpu = scores[so:so + C]
                    idx = indices[io:io + n]
                    if (l - l0) % n_reuse == 0:
                        check_scores(s_gpu, s_ref, dtype, where)
                        check_selection(s_gpu, s_ref, idx, T, w, c, l_max[b] // c, dtype, where)
                        assert np.all(indices[io + n:io + cap] == POISON_INDEX), where
                    # the binding's view of the same head
                    kk, vv, pos = hb.kept(l, b, h)
                    assert np.array_equal(pos.cpu().numpy(), idx), where
                    # gathered rows: this layer's own K/V at the anchor's indices
                    ro = pl["index_off"][b] + h * cap
                    assert kk.shape[0] == vv.shape[0] == n, where
                    assert kk.data_ptr() == hb.k_out[l][ro:].data_ptr(), where
                    assert vv.data_ptr() == hb.v_out[l][ro:].data_ptr(), where
                    for t, name in ((hb.k_out[l], "k"), (hb.v_out[l], "v")):
                        got = kvsynth.host_array(t[ro:ro + cap])
                        src = ks[i] if name == "k" else vs[i]
                        assert np.array_equal(got[:n].view(np.uint8), src[idx, h].view(np.uint8)), where
                        assert np.all(got[n:].view(np.uint8) == POISON_BYTE), where
        anchor += -(-(e - l0) // n_reuse)
    assert anchor == hp["n_anchor"]


@pytest.mark.parametrize("dtype,seq_lens,l_max,Hq,Hkv,d,w,chunks,n_reuse", CASES)
def test_hybrid_matches_oracle_per_run(dtype, seq_lens, l_max, Hq, Hkv, d, w, chunks, n_reuse):
    L = len(chunks)
    q, k, v = _inputs(dtype, seq_lens, L, Hq, Hkv, d, w, seed=len(chunks) + sum(seq_lens))
    prob = ck.make_problem(dtype, seq_lens, l_max, Hq, Hkv, d, w, chunks[0])
    hb = _hybrid(prob, chunks, n_reuse, q, k, v, d, tdtype(dtype))
    _check_oracle(hb, dtype, seq_lens, l_max, Hq, Hkv, d, w, chunks, n_reuse, q, k, v)


def test_hybrid_graph_replays_match_eager():
    # the hybrid call allocates nothing and issues only kernel launches, so it
    # can be captured in a HIP graph; every replay (eager poison fills and
    # synchronisations between them) reproduces the eager outputs, which are
    # themselves checked against the oracle
    dtype, seq_lens, l_max, Hq, Hkv, d, w, chunks, n_reuse = CASES[1]
    L = len(chunks)
    dt = tdtype(dtype)
    q, k, v = _inputs(dtype, seq_lens, L, Hq, Hkv, d, w, seed=11)
    prob = ck.make_problem(dtype, seq_lens, l_max, Hq, Hkv, d, w, chunks[0])
    ref = _hybrid(prob, chunks, n_reuse, q, k, v, d, dt)
    _check_oracle(ref, dtype, seq_lens, l_max, Hq, Hkv, d, w, chunks, n_reuse, q, k, v)
    hb = ck.HybridBuffers(prob, chunks, n_reuse, d, dt)
    qs = [q[l] for l in range(L)]
    stream = torch.cuda.Stream()
    args = (prob, chunks, n_reuse, qs, [k[l] for l in range(L)], [v[l] for l in range(L)], hb.k_out, hb.v_out,
            hb.scores, hb.indices, hb.lengths, hb.workspace, hb.ws_bytes)
    with torch.cuda.stream(stream):
        ck.compress_layers_hybrid(*args, stream=stream)      # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        ck.compress_layers_hybrid(*args, stream=stream)
    torch.cuda.synchronize()
    outs = [hb.scores, hb.indices, hb.lengths] + hb.k_out + hb.v_out
    refs = [ref.scores, ref.indices, ref.lengths] + ref.k_out + ref.v_out
    for rep in range(3):
        for t in [hb.scores, hb.lengths] + hb.k_out + hb.v_out:
            t.view(torch.uint8).fill_(POISON_BYTE)
        hb.indices.fill_(POISON_INDEX)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, refs)):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), (rep, i)


@pytest.mark.parametrize("dtype,seq_lens,l_max,Hq,Hkv,d,w,chunks,n_reuse", CASES[:2] + CASES[3:])
def test_hybrid_equals_one_call_per_run(dtype, seq_lens, l_max, Hq, Hkv, d, w, chunks, n_reuse):
    L = len(chunks)
    dt = tdtype(dtype)
    q, k, v = _inputs(dtype, seq_lens, L, Hq, Hkv, d, w, seed=7)
    prob = ck.make_problem(dtype, seq_lens, l_max, Hq, Hkv, d, w, chunks[0])
    hb = _hybrid(prob, chunks, n_reuse, q, k, v, d, dt)
    hp = hb.hplan
    anchor = 0
    for l0, e, c in _runs(chunks):
        pc = ck.make_problem(dtype, seq_lens, l_max, Hq, Hkv, d, w, c)
        n = e - l0
        bufs = ck.Buffers(pc, n, n_reuse, d, dt, "cuda")
        bufs.k_out.view(torch.uint8).fill_(POISON_BYTE)
        bufs.v_out.view(torch.uint8).fill_(POISON_BYTE)
        bufs.indices.fill_(POISON_INDEX)
        qs = [q[l] if (l - l0) % n_reuse == 0 else None for l in range(l0, e)]
        ck.compress_layers(pc, n_reuse, qs, [k[l] for l in range(l0, e)], [v[l] for l in range(l0, e)],
                           [bufs.k_out[i] for i in range(n)], [bufs.v_out[i] for i in range(n)], bufs.scores,
                           bufs.indices, bufs.lengths, bufs.workspace, bufs.ws_bytes)
        torch.cuda.synchronize()
        na = bufs.n_anchor
        for name, whole, part, off in (("scores", hb.scores, bufs.scores, "score_block_off"),
                                       ("indices", hb.indices, bufs.indices, "index_block_off"),
                                       ("lengths", hb.lengths, bufs.lengths, "length_block_off")):
            seg = whole[hp[off][anchor]:hp[off][anchor + na]]
            assert torch.equal(seg.view(torch.int32), part.view(torch.int32)), (name, l0, c)
        for i, l in enumerate(range(l0, e)):
            assert torch.equal(hb.k_out[l].view(torch.uint8), bufs.k_out[i].view(torch.uint8)), (l, c)
            assert torch.equal(hb.v_out[l].view(torch.uint8), bufs.v_out[i].view(torch.uint8)), (l, c)
        anchor += na


def test_hybrid_phase_events_bracket_the_call():
    dtype, seq_lens, l_max, Hq, Hkv, d, w, chunks, n_reuse = CASES[0]
    L = len(chunks)
    q, k, v = _inputs(dtype, seq_lens, L, Hq, Hkv, d, w, seed=3)
    prob = ck.make_problem(dtype, seq_lens, l_max, Hq, Hkv, d, w, chunks[0])
    hb = ck.HybridBuffers(prob, chunks, n_reuse, d, tdtype(dtype))
    qs = [q[l] for l in range(L)]     # extra queries on reusing layers are ignored
    ev = ck.PhaseEvents()
    ck.compress_layers_hybrid(prob, chunks, n_reuse, qs, [k[l] for l in range(L)], [v[l] for l in range(L)],
                              hb.k_out, hb.v_out, hb.scores, hb.indices, hb.lengths, hb.workspace, hb.ws_bytes,
                              phase_events=ev)
    torch.cuda.synchronize()
    score_ms, gather_ms = ev.elapsed_ms(0, 1), ev.elapsed_ms(2, 3)
    assert score_ms > 0 and gather_ms > 0
    assert ev.elapsed_ms(1, 2) >= 0
