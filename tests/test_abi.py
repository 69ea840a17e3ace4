"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/chunkkv.h declares, and validates arguments on the host
(chunkkv_plan is host-only; invalid calls return before any launch).

Output sizes follow the pages' formulas (ChunkKV page section 4.1,
Algorithm 1): C = ceil(T/c), k = floor(L_max/c), L_cap = min(T, k*c + w).
"""
import ctypes
import math
import os
import re

import pytest

from kv_cache_compression_win_amd import chunkkv as ck

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "chunkkv.h")


def test_library_exports_every_declared_symbol():
    decl = set(re.findall(r"\b(chunkkv_[a-z_]+)\s*\(", open(HEADER).read()))
    assert decl == set(ck.SYMBOLS)
    L = ck.lib()
    for name in decl:
        assert getattr(L, name) is not None


def _p(**kw):
    args = dict(dtype=ck.BF16, seq_lens=[1000], l_max=[100], n_q_heads=8, n_kv_heads=2, head_dim=128,
                window=8, chunk=10)
    args.update(kw)
    return ck.make_problem(**args)


@pytest.mark.parametrize("seq_lens,l_max,w,c", [
    ([32768], [3276], 32, 10), ([8192], [819], 32, 10), ([16384], [128], 32, 3),
    ([131072, 65536, 32768, 16384], [26214, 13107, 6553, 3276], 64, 10), ([1000], [100], 8, 10),
    ([50, 7, 1000], [0, 7, 10000], 7, 9)])
def test_plan_sizes_follow_the_formulas(seq_lens, l_max, w, c):
    pl = ck.plan(_p(seq_lens=seq_lens, l_max=l_max, window=w, chunk=c))
    Hkv = 2
    C = [math.ceil(t / c) for t in seq_lens]
    cap = [min(t, (lm // c) * c + w) for t, lm in zip(seq_lens, l_max)]
    assert pl["scores_elems"] == Hkv * sum(C)
    assert pl["index_elems"] == Hkv * sum(cap)
    assert pl["length_elems"] == Hkv * len(seq_lens)
    assert pl["l_cap"] == cap
    assert pl["score_off"] == [Hkv * sum(C[:b]) for b in range(len(C))]
    assert pl["index_off"] == [Hkv * sum(cap[:b]) for b in range(len(cap))]
    assert all(x <= lm + w for x, lm in zip(cap, l_max))
    assert pl["workspace_bytes"] > 0


def test_workspace_grows_with_layers_per_launch():
    p = _p(seq_lens=[32768], l_max=[3276], n_q_heads=32, n_kv_heads=8, window=32)
    assert ck.workspace_bytes(p, 16) > ck.workspace_bytes(p, 1) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), ck.ERR_INVALID_ARG),
    (dict(n_q_heads=6, n_kv_heads=4), ck.ERR_INVALID_ARG),
    (dict(window=0), ck.ERR_INVALID_ARG),
    (dict(chunk=0), ck.ERR_INVALID_ARG),
    (dict(window=1001, n_q_heads=2, n_kv_heads=2), ck.ERR_INVALID_ARG),
    (dict(l_max=[-1]), ck.ERR_INVALID_ARG),
    (dict(seq_lens=[0]), ck.ERR_INVALID_ARG),
    (dict(head_dim=4), ck.ERR_UNSUPPORTED),
    (dict(head_dim=260), ck.ERR_UNSUPPORTED),
    (dict(head_dim=12), ck.ERR_UNSUPPORTED),
    (dict(n_q_heads=4096, n_kv_heads=1, window=8), ck.ERR_UNSUPPORTED),
    (dict(kv_strides=(1000, 100)), ck.ERR_UNSUPPORTED),
    (dict(kv_strides=(0, 128)), ck.ERR_INVALID_ARG),
])
def test_plan_rejects_invalid_problems(kw, status):
    with pytest.raises(ck.ChunkKVError) as e:
        ck.plan(_p(**kw))
    assert e.value.status == status
    assert ck.last_error()


def test_null_problem_and_null_outputs():
    L = ck.lib()
    assert L.chunkkv_plan(None, None, None, None, None) == ck.ERR_INVALID_ARG
    p = _p()
    assert L.chunkkv_plan(p.ref, None, None, None, None) == ck.ERR_INVALID_ARG
    assert ck.lib().chunkkv_workspace_bytes(p.ref, 0) == 0


def test_entry_points_validate_before_launch():
    # Every failure below is decided on the host; nothing reaches a device.
    L = ck.lib()
    p = _p()
    dummy = 1 << 20  # a non-NULL, 16-byte-aligned address that is never touched
    assert L.chunkkv_score(p.ref, None, dummy, dummy, dummy, 1 << 30, None) == ck.ERR_INVALID_ARG
    assert L.chunkkv_score(p.ref, dummy, dummy, dummy, None, 1 << 30, None) == ck.ERR_WORKSPACE
    assert L.chunkkv_score(p.ref, dummy, dummy, dummy, dummy, 16, None) == ck.ERR_WORKSPACE
    assert L.chunkkv_score(p.ref, dummy + 2, dummy, dummy, dummy, 1 << 30, None) == ck.ERR_UNSUPPORTED
    assert L.chunkkv_select(p.ref, None, dummy, dummy, None) == ck.ERR_INVALID_ARG
    assert L.chunkkv_gather(p.ref, dummy, dummy, dummy, dummy, None, dummy, None) == ck.ERR_INVALID_ARG
    assert L.chunkkv_gather(p.ref, dummy + 8, dummy, dummy, dummy, dummy, dummy, None) == ck.ERR_UNSUPPORTED
    P = ctypes.c_void_p * 2
    tab = P(dummy, dummy)
    half = P(dummy, None)
    args = (ctypes.cast(tab, ctypes.c_void_p),) * 5 + (dummy, dummy, dummy, dummy, 1 << 30, None, None)
    assert L.chunkkv_compress_layers(p.ref, 0, 1, *args) == ck.ERR_INVALID_ARG
    assert L.chunkkv_compress_layers(p.ref, 2, 0, *args) == ck.ERR_INVALID_ARG
    # layer 1 scores when n_reuse = 1, so its NULL query pointer is an error;
    # with n_reuse = 2 the NULL is allowed and validation passes that check.
    bad_q = (ctypes.cast(half, ctypes.c_void_p),) + args[1:]
    assert L.chunkkv_compress_layers(p.ref, 2, 1, *bad_q) == ck.ERR_INVALID_ARG
    small_ws = args[:8] + (16,) + args[9:]
    assert L.chunkkv_compress_layers(p.ref, 2, 2, *(bad_q[:8] + (16,) + bad_q[9:])) == ck.ERR_WORKSPACE
    assert L.chunkkv_compress_layers(p.ref, 2, 1, *small_ws) == ck.ERR_WORKSPACE


def test_gather_paged_validates_before_launch():
    # The paged gather's checks are host-side too: NULL buffers, empty pages,
    # a block table too short for the longest kept run, misaligned pages.
    L = ck.lib()
    p = _p()
    dummy = 1 << 20
    l_cap = max(int(x) for x in ck.plan(p)["l_cap"])
    rows = 16
    need = -(-l_cap // rows)

    def call(table=dummy, max_pages=need, page_rows=rows, n_pages=64, kp=dummy):
        return L.chunkkv_gather_paged(p.ref, dummy, dummy, dummy, dummy, table, max_pages, page_rows,
                                      n_pages, kp, dummy, None)

    assert call(table=None) == ck.ERR_INVALID_ARG
    assert call(page_rows=0) == ck.ERR_INVALID_ARG
    assert call(n_pages=0) == ck.ERR_INVALID_ARG
    assert call(max_pages=need - 1) == ck.ERR_INVALID_ARG
    assert call(kp=dummy + 4) == ck.ERR_UNSUPPORTED


def test_decode_attention_validates_before_launch():
    L = ck.lib()
    p = _p()
    dummy = 1 << 20
    need = L.chunkkv_decode_workspace_bytes(p.ref)
    assert need > 0 and need % 16 == 0
    args = dict(q=dummy, k=dummy, v=dummy, lens=dummy, out=dummy, ws=dummy, n=need)

    def call(**kw):
        a = {**args, **kw}
        return L.chunkkv_decode_attention(p.ref, a["q"], a["k"], a["v"], a["lens"], a["out"], a["ws"], a["n"],
                                          None)

    assert call(q=None) == ck.ERR_INVALID_ARG
    assert call(q=dummy + 2) == ck.ERR_UNSUPPORTED
    assert call(ws=dummy + 8) == ck.ERR_UNSUPPORTED
    assert call(n=need - 16) == ck.ERR_WORKSPACE
    assert call(ws=None) == ck.ERR_WORKSPACE


def test_decode_attention_static_validates_before_launch():
    # The static-scratch variant rejects, on the host, problems whose decode
    # partials need more than the library's 16 MiB array, and the same bad
    # arguments as chunkkv_decode_attention.
    L = ck.lib()
    dummy = 1 << 20
    big = ck.make_problem(ck.BF16, [131072], [131072], 128, 8, 128, 32, 10)   # G = 16, all rows kept
    assert L.chunkkv_decode_workspace_bytes(big.ref) > ck.STATIC_SCRATCH_BYTES
    assert L.chunkkv_decode_attention_static(big.ref, dummy, dummy, dummy, dummy, dummy, None) == ck.ERR_WORKSPACE
    assert "static scratch" in ck.last_error()
    p = _p()
    assert L.chunkkv_decode_attention_static(p.ref, None, dummy, dummy, dummy, dummy, None) == ck.ERR_INVALID_ARG
    assert L.chunkkv_decode_attention_static(p.ref, dummy, dummy + 2, dummy, dummy, dummy, None) == ck.ERR_UNSUPPORTED
    assert L.chunkkv_decode_attention_static(None, dummy, dummy, dummy, dummy, dummy, None) == ck.ERR_INVALID_ARG


def test_plan_hybrid_blocks_follow_each_runs_plan():
    # runs of equal chunk size (ChunkKV page, section 5.7, as a per-layer c):
    # [0-2] c = 10, [3-4] c = 1, [5] c = 4; Algorithm 2 restarts at each run,
    # so with n_reuse = 2 the anchors are layers 0, 2, 3 and 5
    p = _p(seq_lens=[1000, 333], l_max=[100, 40])
    chunks = [10, 10, 10, 1, 1, 4]
    hp = ck.plan_hybrid(p, chunks, 2)
    anchors = [0, 2, 3, 5]
    assert hp["n_anchor"] == len(anchors)
    per_c = {c: ck.plan(_p(seq_lens=[1000, 333], l_max=[100, 40], chunk=c)) for c in set(chunks)}
    so = io = lo = 0
    for a, l in enumerate(anchors):
        assert (hp["score_block_off"][a], hp["index_block_off"][a], hp["length_block_off"][a]) == (so, io, lo)
        pl = per_c[chunks[l]]
        so, io, lo = so + pl["scores_elems"], io + pl["index_elems"], lo + pl["length_elems"]
    assert (hp["score_block_off"][-1], hp["index_block_off"][-1], hp["length_block_off"][-1]) == (so, io, lo)
    assert hp["kv_out_rows"] == [per_c[c]["index_elems"] for c in chunks]
    # every run scores all its anchors at once: runs of 2, 1 and 1 anchors
    n_run_anchors = {10: 2, 1: 1, 4: 1}
    assert hp["workspace_bytes"] == max(
        ck.workspace_bytes(_p(seq_lens=[1000, 333], l_max=[100, 40], chunk=c), n) for c, n in n_run_anchors.items())
    # one chunk size for every layer: the blocks of chunkkv_compress_layers
    one = ck.plan_hybrid(p, [10] * 5, 2)
    pl = per_c[10]
    assert one["n_anchor"] == 3
    assert one["score_block_off"] == [a * pl["scores_elems"] for a in range(4)]
    assert one["index_block_off"] == [a * pl["index_elems"] for a in range(4)]


def test_hybrid_entry_points_validate_before_launch():
    L = ck.lib()
    p = _p()
    with pytest.raises(ck.ChunkKVError) as e:
        ck.plan_hybrid(p, [10, 10, 0, 0], 1)
    assert e.value.status == ck.ERR_INVALID_ARG and "layers 2-3" in ck.last_error()
    with pytest.raises(ck.ChunkKVError) as e:
        ck.plan_hybrid(p, [10, 1], 0)
    assert e.value.status == ck.ERR_INVALID_ARG
    assert L.chunkkv_plan_hybrid(p.ref, None, 2, 1, None, None, None, None, None, None) == ck.ERR_INVALID_ARG
    dummy = 1 << 20
    chunks = (ctypes.c_int32 * 4)(10, 10, 10, 1)
    P = ctypes.c_void_p * 4
    full = P(dummy, dummy, dummy, dummy)
    q_gap = P(dummy, None, dummy, None)      # layer 3 starts a run: it scores
    q_ok = P(dummy, None, dummy, dummy)
    tab = ctypes.cast(full, ctypes.c_void_p)

    def call(q, ws_bytes):
        return L.chunkkv_compress_layers_hybrid(p.ref, ctypes.cast(chunks, ctypes.c_void_p), 4, 2,
                                                ctypes.cast(q, ctypes.c_void_p), tab, tab, tab, tab, dummy, dummy,
                                                dummy, dummy, ws_bytes, None, None)

    assert call(q_gap, 1 << 30) == ck.ERR_INVALID_ARG and "q_win[3]" in ck.last_error()
    assert call(q_ok, 16) == ck.ERR_WORKSPACE
