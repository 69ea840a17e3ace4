"""chunkkv_decode_attention_static (the library's per-GPU static scratch
instead of a caller workspace) against chunkkv_decode_attention on the same
inputs: two calls in a row, the second on a smaller problem, each equal to
the workspace entry point's output bit for bit (same kernels, same work split,
same arithmetic order)."""
import numpy as np
import pytest
import torch

import kvsynth
from kv_cache_compression_win_amd import chunkkv as ck

pytestmark = pytest.mark.gpu


def _inputs(prob, Hq, d, seed):
    pl = ck.plan(prob)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    rows = pl["index_elems"]
    k = (2 * torch.randn((rows, d), generator=g, device="cuda")).to(torch.bfloat16)
    v = torch.randn((rows, d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((prob.n_seqs, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    Hkv = pl["length_elems"] // prob.n_seqs
    rng = np.random.default_rng(seed)
    lens = [pl["l_cap"][b] if (b + h) % 2 == 0 else int(rng.integers(0, pl["l_cap"][b] + 1))
            for b in range(prob.n_seqs) for h in range(Hkv)]
    return q, k, v, torch.tensor(lens, dtype=torch.int32, device="cuda")


def _both(prob, Hq, d, seed):
    q, k, v, lens = _inputs(prob, Hq, d, seed)
    ws_n = ck.decode_workspace_bytes(prob)
    assert ws_n <= ck.STATIC_SCRATCH_BYTES
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    want = torch.full((prob.n_seqs, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full_like(want, float("nan"))
    ck.decode_attention(prob, q, k, v, lens, want, ws, ws_n)
    ck.decode_attention_static(prob, q, k, v, lens, got)
    torch.cuda.synchronize()
    assert not torch.isnan(want).any()
    assert torch.equal(got, want)


def test_static_scratch_matches_workspace_entry_point_twice():
    # first call: the 70B-shaped batch's compacted cache (4 sequences, 8 KV
    # heads, G = 8; about 7.5 MB of partials), then a smaller one (a 4k
    # sequence, G = 4) that reuses the array the first call left behind
    wl = kvsynth.WORKLOADS["llama-70b-80layer-4seq"]
    big = ck.make_problem(ck.BF16, wl.seq_lens, wl.l_max, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window,
                          wl.chunk)
    _both(big, wl.n_q_heads, wl.head_dim, seed=1)
    small = ck.make_problem(ck.BF16, [4096], [400], 32, 8, 128, 32, 10)
    assert ck.decode_workspace_bytes(small) < ck.decode_workspace_bytes(big)
    _both(small, 32, 128, seed=2)


def test_static_scratch_workgroup_kernel_and_rejection():
    # the workgroup kernel (rows of 12 pieces), then a problem beyond the
    # array, rejected on the host before anything is launched
    p = ck.make_problem(ck.BF16, [30000, 5000], [20000, 800], 12, 4, 96, 16, 10)
    _both(p, 12, 96, seed=3)
    big = ck.make_problem(ck.BF16, [131072], [131072], 128, 8, 128, 32, 10)
    with pytest.raises(ck.ChunkKVError) as e:
        ck.decode_attention_static(big, 16, 16, 16, 16, 16, stream=0)
    assert e.value.status == ck.ERR_WORKSPACE
