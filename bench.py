#!/usr/bin/env python3
"""Benchmark of ChunkKV prefill-time KV-cache compression on one MI355X.

A step is one chunkkv_compress_layers call over the whole synthetic cache:
observe-window scoring, chunk sums, top-k, recent-window merge and K/V gather
on every layer, with layer-wise index reuse (ChunkKV page, section 4.1
Algorithm 1 and section 4.2 Algorithm 2).  Inputs are resident in HBM before
the timed region.

Prints one JSON line: layer-tokens/s (sum over layers of the tokens
compressed, per second), the score kernel's achieved HBM bandwidth against
the 8 TB/s MI355X peak (the library's phase events, taken at the score
kernel's own start and end on the launch stream), and the CPU oracle timed
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KV tokens compressed/sec per layer·head-set + achieved HBM GB/s (% of peak)"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, MI355X


SCORE_SOURCES = ("kv_cache_compression_win_amd/csrc/score_mfma.hip",
                 "kv_cache_compression_win_amd/csrc/chunkkv_internal.h")


def profile_record(summary: str, workload: str, key: str):
    """Value `key` of the machine-readable line in the committed rocprofv3
    summary profiles/<summary>_<workload>.md, or None when there is none or
    the score kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{summary}_{workload}.md")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("{") and key in line:
                rec = json.loads(line)
    if rec is None:
        return None
    h = hashlib.sha256()
    for rel in SCORE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return rec[key] if h.hexdigest() == rec["source_sha256"] else None


def counted_traffic(workload: str):
    """HBM bytes per score-kernel launch (FETCH_SIZE + WRITE_SIZE, scaled by a
    plain copy's readings)."""
    return profile_record("hbm_counters", workload, "traffic_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="llama3-8b-32layer-T32768")
    ap.add_argument("--layers", type=int, default=None, help="use the first N layers only")
    ap.add_argument("--cpu-baseline", choices=("on", "off"), default="on")
    ap.add_argument("--context", choices=("on", "off"), default="on",
                    help="after the timed steps, also time the 8-layer slice and a 1 GiB device copy")
    ap.add_argument("--cpu-anchor-pairs", type=int, default=0,
                    help="oracle sample: this many (scoring, reusing) layer pairs, all KV heads "
                         "(0: every layer of the workload)")
    ap.add_argument("--context-70b", choices=("on", "off"), default="on",
                    help="after everything else, also time the 70B-shaped 80-layer batch (about 107 GB of HBM)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the benchmark, run a plain device copy of this many MiB "
                         "(reference kernel for scaling the HBM byte counters)")
    return ap.parse_args()


def copy_calibration(mib: int, reps: int = 5):
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give
    the factor between counter readings and bytes moved."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / reps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps, "ms": ms,
                      "copy_gbps": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


def copy_peak(n: int, start, stop, step_gbps: float, reps: int = 5):
    """A plain 1 GiB device-to-device copy timed on the same stream: the
    measured copy rate (read + write bytes) that the step is compared with."""
    import torch
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    stop.record()
    torch.cuda.synchronize()
    gbps = 2 * n / (start.elapsed_time(stop) / reps * 1e-3) / 1e9
    return {"gbps": gbps, "what": "1 GiB device-to-device copy (torch copy_), read + write bytes",
            "step_hbm_frac": step_gbps / gbps}


def graph_time_us(fn, args, start, stop, n_in=20):
    """Device time of one fn() call in microseconds: n_in calls captured in a
    HIP graph (fn must only launch kernels), the graph replayed args.steps
    times, so host launch costs do not enter."""
    import torch
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        for _ in range(n_in):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / (args.steps * n_in) * 1e3


def decode_context(wl, cache, prob, bufs, args, start, stop):
    """Decode attention of one new query per query head over layer 0's
    compacted cache, against the same kernel over that layer's full cache (every
    token kept: l_max = T), per layer, device time from graph replays."""
    import torch
    from kv_cache_compression_win_amd import chunkkv as ck
    B, Hq, d = len(wl.seq_lens), wl.n_q_heads, wl.head_dim
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    q = torch.randn((B, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")

    def timed(p, k_out, v_out, lengths):
        ws_n = ck.decode_workspace_bytes(p)
        ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
        return graph_time_us(lambda: ck.decode_attention(p, q, k_out, v_out, lengths, out, ws, ws_n),
                             args, start, stop)

    nh = B * wl.n_kv_heads
    lens_c = bufs.lengths[:nh]
    kept = int(lens_c.sum().item())
    us_c = timed(prob, bufs.k_out[0], bufs.v_out[0], lens_c)
    # the full cache of layer 0, head-major, from the library itself with every token kept
    prob_f = ck.make_problem(ck.BF16, wl.seq_lens, wl.seq_lens, Hq, wl.n_kv_heads, d, wl.window, wl.chunk)
    bf = ck.Buffers(prob_f, 1, 1, d, torch.bfloat16, "cuda")
    ck.compress_layers(prob_f, 1, [cache["q_win"][0]], [cache["k"][0]], [cache["v"][0]], [bf.k_out[0]],
                       [bf.v_out[0]], bf.scores, bf.indices, bf.lengths, bf.workspace, bf.ws_bytes)
    us_f = timed(prob_f, bf.k_out[0], bf.v_out[0], bf.lengths[:nh])
    full = sum(wl.seq_lens) * wl.n_kv_heads
    return {"per_layer_us": {"compressed": us_c, "full": us_f}, "speedup": us_f / us_c,
            "rows": {"compressed": kept, "full": full},
            # each kept K and V row is read once
            "hbm_gbps": {"compressed": 2 * kept * d * 2 / (us_c * 1e-6) / 1e9,
                         "full": 2 * full * d * 2 / (us_f * 1e-6) / 1e9}}


def paged_context(wl, cache, prob, bufs, args, start, stop, page_rows=256):
    """Layer 0's compaction written into pool pages of page_rows rows through a
    shuffled block table (the PagedAttention block layout, Kara page,
    section 2), against the contiguous gather of the same layer; device time
    from graph replays."""
    import torch
    from kv_cache_compression_win_amd import chunkkv as ck
    from kv_cache_compression_win_amd import accounting
    pl = ck.plan(prob)
    d, nh = wl.head_dim, len(wl.seq_lens) * wl.n_kv_heads
    idx, lens = bufs.indices[:pl["index_elems"]], bufs.lengths[:nh]
    max_pages = max(-(-int(x) // page_rows) for x in pl["l_cap"])
    n_pages = nh * max_pages
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    table = torch.randperm(n_pages, generator=g, device="cuda").to(torch.int32)
    kp = torch.empty((n_pages, page_rows, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    ko, vo = bufs.k_out[0], bufs.v_out[0]
    k0, v0 = cache["k"][0], cache["v"][0]

    def timed(fn):
        return graph_time_us(fn, args, start, stop)

    us_p = timed(lambda: ck.gather_paged(prob, k0, v0, idx, lens, table, max_pages, page_rows, n_pages, kp, vp))
    us_c = timed(lambda: ck.gather(prob, k0, v0, idx, lens, ko, vo))
    kept = int(lens.sum().item())
    nbytes = accounting.gather_bytes(kept, d, 2)
    return {"page_rows": page_rows, "n_pages": n_pages, "per_layer_us": {"paged": us_p, "contiguous": us_c},
            "hbm_gbps": {"paged": nbytes / (us_p * 1e-6) / 1e9, "contiguous": nbytes / (us_c * 1e-6) / 1e9}}


def reuse_context(wl, cache, prob, args, start, stop, reuse=(1, 2, 4)):
    """Layer-wise index reuse (ChunkKV page, section 4.2, Algorithm 2): the
    same stack compressed with N_reuse = 1 (every layer scores), 2 and 4, one
    chunkkv_compress_layers call per step, so the cost that reuse removes is
    measured directly."""
    import torch
    from kv_cache_compression_win_amd import chunkkv as ck
    L = wl.n_layers
    ks, vs = [cache["k"][l] for l in range(L)], [cache["v"][l] for l in range(L)]
    out = {}
    for nr in reuse:
        b = ck.Buffers(prob, L, nr, wl.head_dim, torch.bfloat16, "cuda")
        qs = [cache["q_win"][l] if l % nr == 0 else None for l in range(L)]

        def call():
            ck.compress_layers(prob, nr, qs, ks, vs, [b.k_out[l] for l in range(L)],
                               [b.v_out[l] for l in range(L)], b.scores, b.indices, b.lengths, b.workspace,
                               b.ws_bytes)

        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            call()
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / args.steps
        out[f"n_reuse_{nr}"] = {"scoring_layers": -(-L // nr), "ms_per_step": ms,
                                "value": L * sum(wl.seq_lens) / (ms * 1e-3), "unit": "layer-tokens/s"}
        del b
        torch.cuda.empty_cache()
    return out


def hybrid_policy(wl, prob, bufs, qs, ks, vs, kos, vos, n_reuse, args, start, stop):
    """The hybrid layer policy (ChunkKV page, section 5.7): the lower half of
    the layers keeps chunk size c, the upper half scores single tokens (c = 1,
    same L_max and reuse), in one chunkkv_compress_layers_hybrid call with a
    per-layer chunk size (index reuse restarts at the upper half)."""
    import torch
    from kv_cache_compression_win_amd import chunkkv as ck
    L = len(ks)
    half = (L // 2 // n_reuse) * n_reuse
    chunks = [wl.chunk] * half + [1] * (L - half)
    hb = ck.HybridBuffers(prob, chunks, n_reuse, wl.head_dim, torch.bfloat16, "cuda")

    def call():
        # half is a multiple of n_reuse: the scoring layers are those of the uniform policy
        ck.compress_layers_hybrid(prob, chunks, n_reuse, qs, ks, vs, hb.k_out, hb.v_out, hb.scores, hb.indices,
                                  hb.lengths, hb.workspace, hb.ws_bytes)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    del hb
    return {"layers": f"0-{half - 1} at c = {wl.chunk}, {half}-{L - 1} at c = 1 (one call)", "ms_per_step": ms,
            "value": L * sum(wl.seq_lens) / (ms * 1e-3), "unit": "layer-tokens/s"}


def selection_overlap(bufs, wl, n_reuse, plan):
    """Mean Jaccard index of the chunk sets selected by consecutive scoring
    layers (sequence 0, every KV head), from the indices the library wrote;
    a chunk counts as selected when one of its tokens before the recent
    window is kept."""
    import numpy as np
    T, c, w, H = wl.seq_lens[0], wl.chunk, wl.window, wl.n_kv_heads
    n_anchor = bufs.n_anchor
    idx = bufs.indices.view(n_anchor, -1).cpu().numpy()
    lens = bufs.lengths.view(n_anchor, -1).cpu().numpy()
    L_cap, off = plan["l_cap"][0], plan["index_off"][0]

    def chunks(a, h):
        kept = idx[a, off + h * L_cap: off + h * L_cap + lens[a, h]]
        return set((kept[kept < T - w] // c).tolist())

    sets = [[chunks(a, h) for h in range(H)] for a in range(n_anchor)]
    jac = [len(sets[a][h] & sets[a + 1][h]) / max(1, len(sets[a][h] | sets[a + 1][h]))
           for a in range(n_anchor - 1) for h in range(H)]
    return {"mean_jaccard": float(np.mean(jac)) if jac else None,
            "pairs": f"scoring layers l and l + {n_reuse}, sequence 0, all {H} KV heads"}


# Host multiply-adds per second of one oracle thread (the fp64 score loop),
# used only to bound the default CPU sample.
ORACLE_MACS_PER_THREAD = 4.0e8
CPU_BUDGET_S = 60.0


def cpu_baseline(wl, cache, n_pairs: int):
    """Time the CPU oracle, as it stands, on the workload's own inputs copied
    to the host: for every (scoring layer, KV head) of sequence 0, Algorithm 1
    (fp64 scores, full-sort top-k, index build) on the scoring layer and the
    row copies of K and V of that layer and of the layers reusing its indices.
    n_pairs > 0 takes only the first n_pairs scoring layers; n_pairs = 0 takes
    every layer of the workload when its estimated cost fits CPU_BUDGET_S of
    wall time, else the largest leading sample that does (labelled)."""
    import oracle
    import kvsynth
    oracle.build(force=False)
    T = wl.seq_lens[0]
    n_anchor = -(-wl.n_layers // wl.n_reuse)
    threads = max(1, min(os.cpu_count() or 1, 16))
    rows = wl.window * (wl.n_q_heads // wl.n_kv_heads)
    unit_s = rows * T * wl.head_dim / ORACLE_MACS_PER_THREAD
    fit = max(1, int(CPU_BUDGET_S * threads / (unit_s * wl.n_kv_heads)))
    pairs = min(n_anchor, n_pairs if n_pairs > 0 else fit)
    whole = pairs == n_anchor and len(wl.seq_lens) == 1
    groups = {a * wl.n_reuse: [l for l in range(a * wl.n_reuse, min((a + 1) * wl.n_reuse, wl.n_layers))]
              for a in range(pairs)}
    layers = [l for g in groups.values() for l in g]
    host = {l: (kvsynth.host_array(cache["k"][l, :T]), kvsynth.host_array(cache["v"][l, :T]))
            for l in layers}
    qh = {a: kvsynth.host_array(cache["q_win"][a, 0]) for a in groups}
    kk = wl.l_max[0] // wl.chunk

    def unit(args):
        a, h = args
        s = oracle.chunk_scores(qh[a], host[a][0], h, wl.n_q_heads, wl.window, wl.chunk)
        idx = oracle.indices(T, wl.window, wl.chunk, oracle.topk(s, kk))
        for l in groups[a]:
            oracle.gather(host[l][0], idx, h)
            oracle.gather(host[l][1], idx, h)

    jobs = [(a, h) for a in sorted(groups) for h in range(wl.n_kv_heads)]
    threads = max(1, min(len(jobs), threads))
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(unit, jobs))
    dt = time.perf_counter() - t0
    layer_tokens = len(layers) * T
    # one thread: the first two units of the same sample, one after the other
    n1 = min(2, len(jobs))
    t1 = time.perf_counter()
    for job in jobs[:n1]:
        unit(job)
    dt1 = time.perf_counter() - t1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    what = ("the whole workload" if whole else
            f"a sample: layers {layers[0]}-{layers[-1]} of {wl.n_layers}, sequence 0 only")
    return {"value": layer_tokens / dt, "unit": "layer-tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"{what} (T={T}, {len(layers)} layers, all {wl.n_kv_heads} KV heads): "
                       f"fp64 scoring + full-sort top-k + index build on the {len(groups)} scoring layers, "
                       f"row copies on all {len(layers)}; {dt:.2f} s wall on {threads} threads"),
            "single_thread": {"value": layer_tokens * n1 / len(jobs) / dt1, "unit": "layer-tokens/s",
                              "sample": f"{n1} of the {len(jobs)} (scoring layer, KV head) units, {dt1:.2f} s"},
            "host": {"cpu_model": model, "logical_cpus": os.cpu_count()}}


def layer_latency_context(name, args, start, stop, chunk=None, l_max=None, calls=40, blocks=5, copies=16):
    """A single-layer compress_layers call (score, select and gather of one
    layer): median and minimum over blocks of back-to-back calls, once on the
    same input (which the 256 MB last-level cache may partly hold between
    calls) and once rotating over `copies` copies of the input in distinct
    memory (together larger than that cache), so that every call reads its
    keys and kept rows from HBM."""
    import torch
    import kvsynth
    from kv_cache_compression_win_amd import chunkkv as ck
    wl = kvsynth.WORKLOADS[name]
    cache = kvsynth.make_cache(wl, device="cuda", seed=0)
    c = chunk or wl.chunk
    lm = l_max or wl.l_max
    prob = ck.make_problem(ck.BF16, wl.seq_lens, lm, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, c)
    bufs = ck.Buffers(prob, 1, 1, wl.head_dim, torch.bfloat16, "cuda")

    inputs = [(cache["q_win"][0], cache["k"][0], cache["v"][0])]
    inputs += [tuple(x.clone() for x in inputs[0]) for _ in range(copies - 1)]

    def call(i):
        q, k, v = inputs[i]
        ck.compress_layers(prob, 1, [q], [k], [v], [bufs.k_out[0]], [bufs.v_out[0]], bufs.scores, bufs.indices,
                           bufs.lengths, bufs.workspace, bufs.ws_bytes)

    def timed(rotate):
        us = []
        for _ in range(blocks):
            start.record()
            for j in range(calls):
                call(j % copies if rotate else 0)
            stop.record()
            torch.cuda.synchronize()
            us.append(start.elapsed_time(stop) / calls * 1e3)
        return us

    for j in range(max(args.warmup, copies)):
        call(j % copies)
    torch.cuda.synchronize()
    same = timed(False)
    rot = timed(True)
    in_bytes = sum(x.numel() * x.element_size() for x in inputs[0])
    return {"workload": name, "chunk": c, "l_max": list(lm), "us_per_call_median": statistics.median(same),
            "us_per_call_min": min(same), "blocks": blocks, "calls_per_block": calls,
            "rotated_inputs": {"copies": copies, "input_mb_per_copy": round(in_bytes / 2**20, 1),
                               "us_per_call_median": statistics.median(rot), "us_per_call_min": min(rot)}}


def context_70b(args):
    """The 70B-shaped batch (80 layers, 64 query heads, 8 KV heads, four
    packed sequences of 131072 / 65536 / 32768 / 16384 tokens, 20% budget,
    index reuse 2), inputs resident in HBM: 5 timed steps of the whole stack
    (median, minimum and mean step), and the score kernel alone on the first
    64 layers (32 scoring layers: one score launch, its own start and end
    events) against the dense bf16 MFMA peak and the HBM peak."""
    import torch
    import kvsynth
    from kv_cache_compression_win_amd import accounting
    from kv_cache_compression_win_amd import chunkkv as ck
    wl = kvsynth.WORKLOADS["llama-70b-80layer-4seq"]
    cache = kvsynth.make_cache(wl, device="cuda", seed=0)
    L, nr, e = wl.n_layers, wl.n_reuse, 2
    prob = ck.make_problem(ck.BF16, wl.seq_lens, wl.l_max, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window,
                           wl.chunk)
    bufs = ck.Buffers(prob, L, nr, wl.head_dim, torch.bfloat16, "cuda")
    qs = [cache["q_win"][l] if l % nr == 0 else None for l in range(L)]
    ks = [cache["k"][l] for l in range(L)]
    vs = [cache["v"][l] for l in range(L)]
    kos = [bufs.k_out[l] for l in range(L)]
    vos = [bufs.v_out[l] for l in range(L)]

    def step(n, events=None):
        ck.compress_layers(prob, nr, qs[:n], ks[:n], vs[:n], kos[:n], vos[:n], bufs.scores, bufs.indices,
                           bufs.lengths, bufs.workspace, bufs.ws_bytes, phase_events=events)

    for _ in range(2):
        step(L)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    evs[0].record()
    for i in range(5):
        step(L)
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(5)]
    mean_ms = evs[0].elapsed_time(evs[5]) / 5
    n_anchor = -(-L // nr)
    kept = bufs.lengths.view(n_anchor, -1).sum(dim=1).tolist()
    step_bytes = (n_anchor * accounting.score_bytes(wl.seq_lens, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                                                    wl.window, wl.chunk, e)
                  + sum(accounting.select_bytes(wl.seq_lens, wl.n_kv_heads, wl.chunk, k) for k in kept)
                  + accounting.gather_bytes(sum(kept[l // nr] for l in range(L)), wl.head_dim, e))
    # the score kernel of the first 32 scoring layers (one launch)
    n64 = 64
    sev = [ck.PhaseEvents() for _ in range(3)]
    for ev in sev:
        step(n64, ev)
    torch.cuda.synchronize()
    score_ms = statistics.median(ev.elapsed_ms(0, 1) for ev in sev)
    a64 = n64 // nr
    flops = a64 * 2 * wl.window * wl.n_q_heads * wl.head_dim * sum(wl.seq_lens)
    kbytes = a64 * (sum(wl.seq_lens) * wl.n_kv_heads * wl.head_dim * e
                    + len(wl.seq_lens) * wl.window * wl.n_q_heads * wl.head_dim * e)
    tflops = flops / (score_ms * 1e-3) / 1e12
    gbps = kbytes / (score_ms * 1e-3) / 1e9
    out = {"workload": wl.name, "steps": 5, "ms_per_step_mean": mean_ms, "ms_per_step_median": statistics.median(ms),
           "ms_per_step_min": min(ms), "value": L * sum(wl.seq_lens) / (mean_ms * 1e-3), "unit": "layer-tokens/s",
           "step_hbm": {"achieved": step_bytes / (mean_ms * 1e-3) / 1e9,
                        "frac": step_bytes / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "algorithmic_bytes": step_bytes},
           "score_kernel": {"layers": "first 64 layers: 32 scoring layers in one score launch", "ms": score_ms,
                            "mfma": {"achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "algorithmic_flops": flops},
                            "hbm": {"achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                    "frac": gbps / HBM_PEAK_GBPS, "algorithmic_bytes": kbytes}}}
    del cache, bufs
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: ChunkKV compression here has no multi-GPU path "
              "(every (layer, sequence, KV head) unit is independent, so sequences, heads or "
              "layers would be split across GPUs without any exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return

    import kvsynth
    from kv_cache_compression_win_amd import accounting
    from kv_cache_compression_win_amd import chunkkv as ck

    wl = kvsynth.WORKLOADS[args.workload]
    if args.layers:
        wl = wl.with_(n_layers=args.layers)
    assert wl.dtype == "bf16"
    torch.cuda.set_device(0)
    dev = "cuda"
    print(f"[bench] generating {wl.name} ({wl.n_layers} layers, T={list(wl.seq_lens)}) on {dev}",
          file=sys.stderr, flush=True)
    cache = kvsynth.make_cache(wl, device=dev, seed=0)
    torch.cuda.synchronize()

    L, n_reuse = wl.n_layers, wl.n_reuse
    prob = ck.make_problem(ck.BF16, wl.seq_lens, wl.l_max, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                           wl.window, wl.chunk)
    bufs = ck.Buffers(prob, L, n_reuse, wl.head_dim, torch.bfloat16, dev)
    qs = [cache["q_win"][l] if l % n_reuse == 0 else None for l in range(L)]
    ks = [cache["k"][l] for l in range(L)]
    vs = [cache["v"][l] for l in range(L)]
    kos = [bufs.k_out[l] for l in range(L)]
    vos = [bufs.v_out[l] for l in range(L)]

    def step(events=None):
        ck.compress_layers(prob, n_reuse, qs, ks, vs, kos, vos, bufs.scores, bufs.indices,
                           bufs.lengths, bufs.workspace, bufs.ws_bytes, phase_events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # every timed step takes the score phase's two events (at the score
    # kernel's own start and end when it is one launch); the gather-phase
    # events stay unset, as events between a step's kernels cost time
    evs = [ck.PhaseEvents() for _ in range(args.steps)]
    score_only = [[e.handles[0], e.handles[1], None, None] for e in evs]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the timed steps fall into at least 3 blocks (as many as steps allow, at
    # most 4), each bracketed by stream events, for a median and a minimum
    n_blocks = min(args.steps, max(3, min(4, args.steps)))
    bounds = [round(i * args.steps / n_blocks) for i in range(n_blocks + 1)]
    block_evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_blocks + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        if i in bounds:
            block_evs[bounds.index(i)].record()
        step(score_only[i])
    block_evs[n_blocks].record()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps
    block_ms = [block_evs[j].elapsed_time(block_evs[j + 1]) / (bounds[j + 1] - bounds[j]) for j in range(n_blocks)]

    def mean_ms(i, j):
        return sum(e.elapsed_ms(i, j) for e in evs) / len(evs)

    ph = {"score": mean_ms(0, 1)}
    ph["rest_of_step"] = ms_step - ph["score"]

    # algorithmic bytes (kept-token counts from the actual lengths)
    n_anchor = bufs.n_anchor
    kept_per_anchor = bufs.lengths.view(n_anchor, -1).sum(dim=1).tolist()
    kept_total = sum(kept_per_anchor[l // n_reuse] for l in range(L))
    e = 2
    k_bytes = sum(wl.seq_lens) * wl.n_kv_heads * wl.head_dim * e
    q_bytes = len(wl.seq_lens) * wl.window * wl.n_q_heads * wl.head_dim * e
    score_kernel_bytes = n_anchor * (k_bytes + q_bytes)
    step_bytes = (n_anchor * accounting.score_bytes(wl.seq_lens, wl.n_q_heads, wl.n_kv_heads,
                                                     wl.head_dim, wl.window, wl.chunk, e)
                  + sum(accounting.select_bytes(wl.seq_lens, wl.n_kv_heads, wl.chunk, kept)
                        for kept in kept_per_anchor)
                  + accounting.gather_bytes(kept_total, wl.head_dim, e))
    score_gbps = score_kernel_bytes / (ph["score"] * 1e-3) / 1e9
    # the score contraction: 2 * (G*w rows) * d per key token and KV head
    score_flops = n_anchor * 2 * wl.window * wl.n_q_heads * wl.head_dim * sum(wl.seq_lens)
    score_tflops = score_flops / (ph["score"] * 1e-3) / 1e12
    step_gbps = step_bytes / (ms_step * 1e-3) / 1e9
    layer_tokens = L * sum(wl.seq_lens)
    value = layer_tokens / (ms_step * 1e-3)

    out = {
        "metric": METRIC, "value": value, "unit": "layer-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "n_layers": L, "seq_lens": list(wl.seq_lens),
                   "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "window": wl.window, "chunk": wl.chunk,
                   "l_max": list(wl.l_max), "n_reuse": n_reuse, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "kernel": "score_mfma_kernel", "achieved": score_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": score_gbps / HBM_PEAK_GBPS,
                     "traffic": counted_traffic(wl.name),
                     "algorithmic_bytes_per_launch": score_kernel_bytes,
                     "avg_launch_ms": ph["score"]},
        "score_mfma": {"achieved": score_tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": score_tflops / MFMA_BF16_PEAK_TFLOPS, "algorithmic_flops_per_launch": score_flops,
                       "busy_counted": profile_record("mfma_counters", wl.name, "mfma_busy_frac")},
        "step_hbm": {"achieved": step_gbps, "frac": step_gbps / HBM_PEAK_GBPS,
                     "algorithmic_bytes": step_bytes},
        "phases_ms": ph,
        "timing": {"blocks": n_blocks, "steps_per_block": [bounds[j + 1] - bounds[j] for j in range(n_blocks)],
                   "ms_per_step_blocks": block_ms, "ms_per_step_median": statistics.median(block_ms),
                   "ms_per_step_min": min(block_ms),
                   "what": "the timed steps in consecutive blocks, stream events between steps; value uses the "
                           "mean over all timed steps"},
        "wall_s_timed": wall,
    }
    # context outside the timed region: the 8-layer slice (its first 8
    # layers: 4 scoring + 4 reusing), per-phase durations and a plain device
    # copy of 1 GiB
    extra = {}
    if args.context == "on" and L > 8:
        def slice8():
            ck.compress_layers(prob, n_reuse, qs[:8], ks[:8], vs[:8], kos[:8], vos[:8], bufs.scores,
                               bufs.indices, bufs.lengths, bufs.workspace, bufs.ws_bytes)
        for _ in range(args.warmup):
            slice8()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            slice8()
        stop.record()
        torch.cuda.synchronize()
        ms8 = start.elapsed_time(stop) / args.steps
        extra["slice_8_layers"] = {"ms_per_call": ms8, "value": 8 * sum(wl.seq_lens) / (ms8 * 1e-3),
                                   "unit": "layer-tokens/s"}
    if args.context == "on":
        # workload diagnostic: overlap of the chunks selected by consecutive
        # scoring layers (the synthetic caches share 80% of the planted hot
        # chunks between adjacent layers), mean Jaccard index over the heads
        extra["selection_overlap"] = selection_overlap(bufs, wl, n_reuse, ck.plan(prob))
        # per-phase durations from separate steps that take all four phase
        # events (score | combine + select | gather); the extra events cost a
        # few microseconds per step, so these steps are not the timed ones
        evs_all = [ck.PhaseEvents() for _ in range(args.steps)]
        for e_all in evs_all:
            step(e_all)
        torch.cuda.synchronize()

        def mean_all(i, j):
            return sum(x.elapsed_ms(i, j) for x in evs_all) / len(evs_all)

        g_bytes = accounting.gather_bytes(kept_total, wl.head_dim, e)
        g_ms = mean_all(2, 3)
        g_gbps = g_bytes / (g_ms * 1e-3) / 1e9
        extra["phase_breakdown"] = {
            "score_ms": mean_all(0, 1), "combine_select_ms": mean_all(1, 2), "gather_ms": g_ms,
            "gather_hbm": {"achieved": g_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": g_gbps / HBM_PEAK_GBPS, "algorithmic_bytes": g_bytes}}
    if args.context == "on":
        extra["decode"] = decode_context(wl, cache, prob, bufs, args, start, stop)
        extra["paged_output"] = paged_context(wl, cache, prob, bufs, args, start, stop)
    if args.context == "on" and L >= 4 and wl.chunk > 1:
        extra["hybrid_policy"] = hybrid_policy(wl, prob, bufs, qs, ks, vs, kos, vos, n_reuse, args,
                                               start, stop)
    if args.context == "on" and L >= 4:
        extra["index_reuse"] = reuse_context(wl, cache, prob, args, start, stop)
    n_copy = 1 << 30 if args.context == "on" else 0
    if n_copy:
        extra["copy_peak"] = copy_peak(n_copy, start, stop, step_gbps)
    out.update(extra)
    if args.context == "on":
        # single-layer calls: bound by launch and latency more than by bytes
        extra_l = {"llama3-8b-1layer-T8192": layer_latency_context("llama3-8b-1layer-T8192", args, start, stop),
                   "llama3-8b-csweep-T16384 (c = 10, L_max = 512)":
                       layer_latency_context("llama3-8b-csweep-T16384", args, start, stop, chunk=10, l_max=(512,))}
        out["single_layer_calls"] = extra_l
    if args.cpu_baseline == "on":
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, cache, args.cpu_anchor_pairs)
    if args.context == "on" and args.context_70b == "on" and wl.name != "llama-70b-80layer-4seq":
        print("[bench] the 70B-shaped batch (context)", file=sys.stderr, flush=True)
        del cache, bufs, qs, ks, vs, kos, vos
        torch.cuda.empty_cache()
        out["llama_70b_80layer_4seq"] = context_70b(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
