"""GPU parity of chunkkv_gather_paged, the compaction written into fixed-size
pages of consecutive KV rows (the PagedAttention block layout, Kara page,
section 2), against the oracle: its index_select of each head's kept rows
(ChunkKV page, section 4.1) placed by its page layout.  Bit-exact.

Inputs are synthetic: random K/V bit patterns, ascending unique kept
positions and lengths drawn on the host (0 and L_cap included), block tables
that list a random permutation of a larger pool.  Every pool byte the copy
must not write holds a poison pattern that is checked afterwards.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_win_amd import chunkkv as ck

pytestmark = pytest.mark.gpu

POISON = 0xA5


def _run(dtype, seq_lens, l_max, Hkv, d, page_rows, seed, extra_pages=7, bad_ids=False, lengths=None):
    rng = np.random.default_rng(seed)
    prob = ck.make_problem(dtype, seq_lens, l_max, Hkv, Hkv, d, 16, 10)
    pl = ck.plan(prob)
    B = len(seq_lens)
    T_all = int(sum(seq_lens))
    host_t = np.int32 if dtype == ck.F32 else np.int16
    kh = rng.integers(np.iinfo(host_t).min, np.iinfo(host_t).max, size=(T_all, Hkv, d), dtype=host_t)
    vh = rng.integers(np.iinfo(host_t).min, np.iinfo(host_t).max, size=(T_all, Hkv, d), dtype=host_t)
    idx = np.zeros(pl["index_elems"], dtype=np.int32)
    if lengths is None:
        lengths = np.array([rng.integers(0, pl["l_cap"][b] + 1) for b in range(B) for _ in range(Hkv)],
                           dtype=np.int32)
    for b in range(B):
        for h in range(Hkv):
            n = int(lengths[b * Hkv + h])
            o = pl["index_off"][b] + h * pl["l_cap"][b]
            idx[o:o + n] = np.sort(rng.choice(seq_lens[b], size=n, replace=False))
    max_pages = max(-(-int(x) // page_rows) for x in pl["l_cap"])
    n_pages = B * Hkv * max_pages + extra_pages
    table = rng.permutation(n_pages)[:B * Hkv * max_pages].astype(np.int32).reshape(B * Hkv, max_pages)
    if bad_ids:
        table[::3, 0] = -1
        table[1::3, -1] = n_pages
    row_bytes = d * np.dtype(host_t).itemsize
    kp = torch.full((n_pages, page_rows, row_bytes), POISON, dtype=torch.uint8, device="cuda")
    vp = torch.full_like(kp, POISON)
    ck.gather_paged(prob, torch.from_numpy(kh).cuda(), torch.from_numpy(vh).cuda(), torch.from_numpy(idx).cuda(),
                    torch.from_numpy(lengths).cuda(), torch.from_numpy(table).cuda(), max_pages, page_rows,
                    n_pages, kp, vp)
    torch.cuda.synchronize()
    got_k, got_v = kp.cpu().numpy(), vp.cpu().numpy()
    want_k = np.full((n_pages, page_rows, row_bytes), POISON, dtype=np.uint8)
    want_v = want_k.copy()
    tok0 = np.concatenate([[0], np.cumsum(seq_lens)])
    for b in range(B):
        for h in range(Hkv):
            n = int(lengths[b * Hkv + h])
            o = pl["index_off"][b] + h * pl["l_cap"][b]
            for src, want in ((kh, want_k), (vh, want_v)):
                rows = oracle.gather(src[tok0[b]:tok0[b + 1]], idx[o:o + n], h)
                oracle.to_pages(rows.view(np.uint8).reshape(n, row_bytes), table[b * Hkv + h], page_rows, want)
    assert np.array_equal(got_k, want_k)
    assert np.array_equal(got_v, want_v)


@pytest.mark.parametrize("dtype,d,page_rows", [
    (ck.BF16, 128, 256),   # pages of 256 tokens, the pages' example size
    (ck.BF16, 128, 16),
    (ck.F32, 64, 7),       # ragged pages
    (ck.BF16, 8, 1),       # one row per page, one 16-byte piece per row
    (ck.F32, 256, 4096),   # one page per head
])
def test_gather_paged_matches_oracle(dtype, d, page_rows):
    _run(dtype, [4000, 1300], [700, 300], 4, d, page_rows, seed=d + page_rows)


def test_gather_paged_skips_out_of_range_pages():
    _run(ck.BF16, [3000], [500], 6, 128, 32, seed=2, bad_ids=True)


def test_gather_paged_many_sequences_and_edge_lengths():
    # eleven sequences (two launches of at most eight), lengths 0 and L_cap
    lens = [257, 4096, 1000, 33, 5000, 800, 2049, 640, 100, 3000, 1500]
    prob = ck.make_problem(ck.BF16, lens, [600] * 11, 2, 2, 128, 16, 10)
    l_cap = ck.plan(prob)["l_cap"]
    lengths = np.array([(0 if i % 3 == 0 else int(l_cap[i // 2])) for i in range(22)], dtype=np.int32)
    _run(ck.BF16, lens, [600] * 11, 2, 128, 64, seed=11, lengths=lengths)


def test_gather_paged_graph_replays_match_eager():
    T, Hkv, d, rows = 3000, 4, 128, 64
    prob = ck.make_problem(ck.BF16, [T], [500], Hkv, Hkv, d, 16, 10)
    pl = ck.plan(prob)
    rng = np.random.default_rng(4)
    kh = rng.integers(-2**15, 2**15 - 1, size=(T, Hkv, d), dtype=np.int16)
    vh = rng.integers(-2**15, 2**15 - 1, size=(T, Hkv, d), dtype=np.int16)
    L = int(pl["l_cap"][0])
    idx = np.concatenate([np.sort(rng.choice(T, size=L, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    lengths = np.array([L, 7, 0, L // 2], dtype=np.int32)
    max_pages = -(-L // rows)
    n_pages = Hkv * max_pages
    table = rng.permutation(n_pages).astype(np.int32)
    args = [torch.from_numpy(x).cuda() for x in (kh, vh, idx, lengths, table)]
    eager_k = torch.full((n_pages, rows, 2 * d), POISON, dtype=torch.uint8, device="cuda")
    eager_v = torch.full_like(eager_k, POISON)
    ck.gather_paged(prob, *args, max_pages, rows, n_pages, eager_k, eager_v)
    torch.cuda.synchronize()
    kp, vp = torch.empty_like(eager_k), torch.empty_like(eager_v)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        ck.gather_paged(prob, *args, max_pages, rows, n_pages, kp, vp)
    for rep in range(3):
        kp.fill_(POISON)
        vp.fill_(POISON)
        scratch = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(kp, eager_k) and torch.equal(vp, eager_v), rep
        del scratch
