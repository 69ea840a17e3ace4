"""Thin ctypes binding of libchunkkv.so (the C-ABI in include/chunkkv.h).

Argument marshalling only: every step of the compression runs in the HIP
library.  Entry points keep the C names (``chunkkv_plan`` -> ``plan`` etc.).
Tensors are passed by ``data_ptr()``; plain integers are taken as raw device
pointers.  There is no fallback: if the library is missing or a call returns
a non-OK status, a ``ChunkKVError`` is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libchunkkv.so")

F32, BF16 = 0, 1
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
N_PHASE_EVENTS = 4

SYMBOLS = ("chunkkv_plan", "chunkkv_workspace_bytes", "chunkkv_score", "chunkkv_select",
           "chunkkv_gather", "chunkkv_compress_layers", "chunkkv_decode_workspace_bytes",
           "chunkkv_decode_attention", "chunkkv_decode_attention_static", "chunkkv_gather_paged",
           "chunkkv_plan_hybrid", "chunkkv_compress_layers_hybrid", "chunkkv_last_error")
STATIC_SCRATCH_BYTES = 16 << 20


class ChunkKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"chunkkv status {status}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
        ("seq_start", ctypes.POINTER(ctypes.c_int64)), ("l_max", ctypes.POINTER(ctypes.c_int64)),
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32), ("chunk", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("kv_stride_tok", ctypes.c_int64), ("kv_stride_head", ctypes.c_int64),
        ("q_stride_seq", ctypes.c_int64), ("q_stride_row", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
    ]


class Sizes(ctypes.Structure):
    _fields_ = [("scores_elems", ctypes.c_int64), ("index_elems", ctypes.c_int64),
                ("length_elems", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t)]


_lib = None
_hip = None


def lib() -> ctypes.CDLL:
    """Load libchunkkv.so (raises if it has not been built).

    torch is imported first so that the library binds to the HIP runtime
    torch already uses (one runtime per process).
    """
    global _lib
    if _lib is None:
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ChunkKVError(ERR_UNSUPPORTED,
                               f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        P = ctypes.POINTER(Problem)
        L.chunkkv_plan.restype = ctypes.c_int
        L.chunkkv_plan.argtypes = [P, ctypes.POINTER(Sizes), vp, vp, vp]
        L.chunkkv_workspace_bytes.restype = sz
        L.chunkkv_workspace_bytes.argtypes = [P, i32]
        L.chunkkv_score.restype = ctypes.c_int
        L.chunkkv_score.argtypes = [P, vp, vp, vp, vp, sz, vp]
        L.chunkkv_select.restype = ctypes.c_int
        L.chunkkv_select.argtypes = [P, vp, vp, vp, vp]
        L.chunkkv_gather.restype = ctypes.c_int
        L.chunkkv_gather.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        L.chunkkv_compress_layers.restype = ctypes.c_int
        L.chunkkv_compress_layers.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                              vp, vp]
        L.chunkkv_decode_workspace_bytes.restype = sz
        L.chunkkv_decode_workspace_bytes.argtypes = [P]
        L.chunkkv_decode_attention.restype = ctypes.c_int
        L.chunkkv_decode_attention.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
        L.chunkkv_decode_attention_static.restype = ctypes.c_int
        L.chunkkv_decode_attention_static.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.chunkkv_gather_paged.restype = ctypes.c_int
        L.chunkkv_gather_paged.argtypes = [P, vp, vp, vp, vp, vp, i32, i32, i64, vp, vp, vp]
        L.chunkkv_plan_hybrid.restype = ctypes.c_int
        L.chunkkv_plan_hybrid.argtypes = [P, vp, i32, i32, vp, vp, vp, vp, vp, vp]
        L.chunkkv_compress_layers_hybrid.restype = ctypes.c_int
        L.chunkkv_compress_layers_hybrid.argtypes = [P, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                                     vp, vp]
        L.chunkkv_last_error.restype = ctypes.c_char_p
        L.chunkkv_last_error.argtypes = []
        _lib = L
    return _lib


def hip_runtime() -> ctypes.CDLL:
    """The process's HIP runtime (the one libchunkkv.so is bound to)."""
    global _hip
    if _hip is None:
        lib()
        H = ctypes.CDLL("libamdhip64.so.7")
        H.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        H.hipEventDestroy.argtypes = [ctypes.c_void_p]
        H.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        H.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        _hip = H
    return _hip


class PhaseEvents:
    """CHUNKKV_N_PHASE_EVENTS raw hipEvent_t handles for chunkkv_compress_layers'
    phase_events argument: start and end of the scoring phase, start and end
    of the gather phase, on the launch stream (taken at the kernel's own start
    and end where a phase is one launch)."""

    def __init__(self):
        H = hip_runtime()
        self.handles = []
        for _ in range(N_PHASE_EVENTS):
            h = ctypes.c_void_p()
            if H.hipEventCreate(ctypes.byref(h)) != 0:
                raise ChunkKVError(ERR_HIP, "hipEventCreate failed")
            self.handles.append(h.value)

    def elapsed_ms(self, i: int, j: int) -> float:
        H = hip_runtime()
        if H.hipEventSynchronize(self.handles[j]) != 0:
            raise ChunkKVError(ERR_HIP, "hipEventSynchronize failed")
        ms = ctypes.c_float()
        if H.hipEventElapsedTime(ctypes.byref(ms), self.handles[i], self.handles[j]) != 0:
            raise ChunkKVError(ERR_HIP, "hipEventElapsedTime failed (event not recorded?)")
        return ms.value

    def __del__(self):
        if _hip is not None:
            for h in getattr(self, "handles", []):
                _hip.hipEventDestroy(h)


def last_error() -> str:
    return lib().chunkkv_last_error().decode()


def _check(status: int) -> None:
    if status != OK:
        raise ChunkKVError(status, last_error())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


@dataclass
class ProblemHandle:
    """A chunkkv_problem plus the host arrays it points to (kept alive here)."""
    struct: Problem
    seq_start: ctypes.Array
    l_max: ctypes.Array

    @property
    def ref(self):
        return ctypes.byref(self.struct)

    @property
    def n_seqs(self) -> int:
        return self.struct.n_seqs


def make_problem(dtype: int, seq_lens: Sequence[int], l_max: Sequence[int], n_q_heads: int,
                 n_kv_heads: int, head_dim: int, window: int, chunk: int,
                 kv_strides: Optional[tuple] = None, q_strides: Optional[tuple] = None,
                 seq_start0: int = 0) -> ProblemHandle:
    """Build a chunkkv_problem.  Default strides are the packed layouts
    K/V[sum T][H_kv][d] and window queries [B][w][H_q][d]."""
    B = len(seq_lens)
    starts = [seq_start0]
    for t in seq_lens:
        starts.append(starts[-1] + int(t))
    ss = (ctypes.c_int64 * (B + 1))(*starts)
    lm = (ctypes.c_int64 * B)(*[int(x) for x in l_max])
    kv_st, kv_sh = kv_strides if kv_strides else (n_kv_heads * head_dim, head_dim)
    q_ss, q_sr, q_sh = q_strides if q_strides else (window * n_q_heads * head_dim, n_q_heads * head_dim,
                                                    head_dim)
    st = Problem(dtype, B, ss, lm, n_q_heads, n_kv_heads, head_dim, window, chunk, 0,
                 kv_st, kv_sh, q_ss, q_sr, q_sh)
    return ProblemHandle(st, ss, lm)


def plan(prob: ProblemHandle) -> dict:
    """chunkkv_plan: output sizes, per-sequence offsets and L_cap (host only)."""
    sz = Sizes()
    B = prob.n_seqs
    so, io, lc = (ctypes.c_int64 * B)(), (ctypes.c_int64 * B)(), (ctypes.c_int64 * B)()
    _check(lib().chunkkv_plan(prob.ref, ctypes.byref(sz), ctypes.addressof(so), ctypes.addressof(io),
                              ctypes.addressof(lc)))
    return dict(scores_elems=sz.scores_elems, index_elems=sz.index_elems,
                length_elems=sz.length_elems, workspace_bytes=sz.workspace_bytes,
                score_off=list(so), index_off=list(io), l_cap=list(lc))


def workspace_bytes(prob: ProblemHandle, n_score_layers: int = 1) -> int:
    n = lib().chunkkv_workspace_bytes(prob.ref, n_score_layers)
    if n == 0:
        raise ChunkKVError(ERR_INVALID_ARG, last_error() or "invalid problem")
    return n


def score(prob, q_win, k, scores, workspace, workspace_nbytes: int, stream=None) -> None:
    _check(lib().chunkkv_score(prob.ref, _ptr(q_win), _ptr(k), _ptr(scores), _ptr(workspace),
                               workspace_nbytes, _stream(stream)))


def select(prob, scores, indices, lengths, stream=None) -> None:
    _check(lib().chunkkv_select(prob.ref, _ptr(scores), _ptr(indices), _ptr(lengths),
                                _stream(stream)))


def gather(prob, k, v, indices, lengths, k_out, v_out, stream=None) -> None:
    _check(lib().chunkkv_gather(prob.ref, _ptr(k), _ptr(v), _ptr(indices), _ptr(lengths),
                                _ptr(k_out), _ptr(v_out), _stream(stream)))


def gather_paged(prob, k, v, indices, lengths, block_table, max_pages: int, page_rows: int, n_pages: int,
                 k_pages, v_pages, stream=None) -> None:
    """chunkkv_gather_paged: the kept rows written into pool pages
    [n_pages][page_rows][head_dim] listed by block_table [B * H_kv][max_pages]."""
    _check(lib().chunkkv_gather_paged(prob.ref, _ptr(k), _ptr(v), _ptr(indices), _ptr(lengths),
                                      _ptr(block_table), max_pages, page_rows, n_pages, _ptr(k_pages),
                                      _ptr(v_pages), _stream(stream)))


def decode_workspace_bytes(prob: ProblemHandle) -> int:
    n = lib().chunkkv_decode_workspace_bytes(prob.ref)
    if n == 0:
        raise ChunkKVError(ERR_INVALID_ARG, last_error() or "invalid problem")
    return n


def decode_attention(prob, q_dec, k_out, v_out, lengths, out, workspace, workspace_nbytes: int,
                     stream=None) -> None:
    """chunkkv_decode_attention: one decode query per query head over the
    compacted cache (out fp32 [n_seqs][n_q_heads][head_dim])."""
    _check(lib().chunkkv_decode_attention(prob.ref, _ptr(q_dec), _ptr(k_out), _ptr(v_out), _ptr(lengths),
                                          _ptr(out), _ptr(workspace), workspace_nbytes, _stream(stream)))


def decode_attention_static(prob, q_dec, k_out, v_out, lengths, out, stream=None) -> None:
    """chunkkv_decode_attention_static: decode_attention with the library's
    own per-GPU static scratch (STATIC_SCRATCH_BYTES) instead of a workspace."""
    _check(lib().chunkkv_decode_attention_static(prob.ref, _ptr(q_dec), _ptr(k_out), _ptr(v_out), _ptr(lengths),
                                                 _ptr(out), _stream(stream)))


def compress_layers(prob, n_reuse: int, q_win: Sequence, k: Sequence, v: Sequence, k_out: Sequence,
                    v_out: Sequence, scores, indices, lengths, workspace, workspace_nbytes: int,
                    stream=None, phase_events: Optional[Sequence] = None) -> None:
    n = len(k)
    P = ctypes.c_void_p * n
    qt = P(*[_ptr(x) for x in q_win])
    kt, vt = P(*[_ptr(x) for x in k]), P(*[_ptr(x) for x in v])
    kot, vot = P(*[_ptr(x) for x in k_out]), P(*[_ptr(x) for x in v_out])
    ev = None
    if phase_events is not None:
        hs = phase_events.handles if isinstance(phase_events, PhaseEvents) else list(phase_events)
        ev = (ctypes.c_void_p * N_PHASE_EVENTS)(*hs)
    _check(lib().chunkkv_compress_layers(
        prob.ref, n, n_reuse, ctypes.cast(qt, ctypes.c_void_p), ctypes.cast(kt, ctypes.c_void_p),
        ctypes.cast(vt, ctypes.c_void_p), ctypes.cast(kot, ctypes.c_void_p),
        ctypes.cast(vot, ctypes.c_void_p), _ptr(scores), _ptr(indices), _ptr(lengths),
        _ptr(workspace), workspace_nbytes, _stream(stream),
        None if ev is None else ctypes.cast(ev, ctypes.c_void_p)))


def plan_hybrid(prob, layer_chunk: Sequence[int], n_reuse: int) -> dict:
    """chunkkv_plan_hybrid: per-anchor block offsets (with the totals as the
    last entry), each layer's K'/V' row count and the workspace size."""
    n = len(layer_chunk)
    ch = (ctypes.c_int32 * n)(*layer_chunk)
    na = ctypes.c_int32(0)
    so, io, lo = (ctypes.c_int64 * (n + 1))(), (ctypes.c_int64 * (n + 1))(), (ctypes.c_int64 * (n + 1))()
    rows = (ctypes.c_int64 * n)()
    ws = ctypes.c_size_t(0)
    _check(lib().chunkkv_plan_hybrid(prob.ref, ctypes.cast(ch, ctypes.c_void_p), n, n_reuse, ctypes.byref(na),
                                     ctypes.cast(so, ctypes.c_void_p), ctypes.cast(io, ctypes.c_void_p),
                                     ctypes.cast(lo, ctypes.c_void_p), ctypes.cast(rows, ctypes.c_void_p),
                                     ctypes.byref(ws)))
    a = na.value
    return {"n_anchor": a, "score_block_off": list(so[:a + 1]), "index_block_off": list(io[:a + 1]),
            "length_block_off": list(lo[:a + 1]), "kv_out_rows": list(rows), "workspace_bytes": ws.value}


def compress_layers_hybrid(prob, layer_chunk: Sequence[int], n_reuse: int, q_win: Sequence, k: Sequence,
                           v: Sequence, k_out: Sequence, v_out: Sequence, scores, indices, lengths, workspace,
                           workspace_nbytes: int, stream=None, phase_events: Optional[Sequence] = None) -> None:
    n = len(k)
    if len(layer_chunk) != n:
        raise ValueError("layer_chunk needs one chunk size per layer")
    ch = (ctypes.c_int32 * n)(*layer_chunk)
    P = ctypes.c_void_p * n
    qt = P(*[_ptr(x) for x in q_win])
    kt, vt = P(*[_ptr(x) for x in k]), P(*[_ptr(x) for x in v])
    kot, vot = P(*[_ptr(x) for x in k_out]), P(*[_ptr(x) for x in v_out])
    ev = None
    if phase_events is not None:
        hs = phase_events.handles if isinstance(phase_events, PhaseEvents) else list(phase_events)
        ev = (ctypes.c_void_p * N_PHASE_EVENTS)(*hs)
    _check(lib().chunkkv_compress_layers_hybrid(
        prob.ref, ctypes.cast(ch, ctypes.c_void_p), n, n_reuse, ctypes.cast(qt, ctypes.c_void_p),
        ctypes.cast(kt, ctypes.c_void_p), ctypes.cast(vt, ctypes.c_void_p), ctypes.cast(kot, ctypes.c_void_p),
        ctypes.cast(vot, ctypes.c_void_p), _ptr(scores), _ptr(indices), _ptr(lengths), _ptr(workspace),
        workspace_nbytes, _stream(stream), None if ev is None else ctypes.cast(ev, ctypes.c_void_p)))


class HybridBuffers:
    """Device outputs and workspace of one compress_layers_hybrid call
    (layout from plan_hybrid), allocated with torch (memory plumbing only)."""

    def __init__(self, prob: ProblemHandle, layer_chunk: Sequence[int], n_reuse: int, head_dim: int, dtype,
                 device="cuda"):
        import torch
        hp = plan_hybrid(prob, layer_chunk, n_reuse)
        self.hplan = hp
        self.ws_bytes = hp["workspace_bytes"]
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.scores = torch.empty(hp["score_block_off"][-1], dtype=torch.float32, device=device)
        self.indices = torch.empty(hp["index_block_off"][-1], dtype=torch.int32, device=device)
        self.lengths = torch.empty(hp["length_block_off"][-1], dtype=torch.int32, device=device)
        self.k_out = [torch.empty((r, head_dim), dtype=dtype, device=device) for r in hp["kv_out_rows"]]
        self.v_out = [torch.empty((r, head_dim), dtype=dtype, device=device) for r in hp["kv_out_rows"]]
        self.n_reuse = n_reuse
        self.n_kv_heads = prob.struct.n_kv_heads
        # runs of equal chunk size: (first layer, end, first anchor, that chunk size's plan)
        self.runs = []
        l, a = 0, 0
        while l < len(layer_chunk):
            e = l
            while e < len(layer_chunk) and layer_chunk[e] == layer_chunk[l]:
                e += 1
            st = Problem.from_buffer_copy(prob.struct)
            st.chunk = int(layer_chunk[l])
            self.runs.append((l, e, a, plan(ProblemHandle(st, prob.seq_start, prob.l_max))))
            a += -(-(e - l) // n_reuse)
            l = e

    def kept(self, layer: int, seq: int, head: int):
        """As Buffers.kept, for a compress_layers_hybrid call into these
        buffers: the layer's run gives its chunk size, anchor and offsets."""
        for l0, e, a0, pl in self.runs:
            if l0 <= layer < e:
                break
        else:
            raise IndexError(f"layer {layer} outside the plan")
        hp = self.hplan
        a = a0 + (layer - l0) // self.n_reuse
        cap = pl["l_cap"][seq]
        n = int(self.lengths[hp["length_block_off"][a] + seq * self.n_kv_heads + head])
        r0 = pl["index_off"][seq] + head * cap
        i0 = hp["index_block_off"][a] + r0
        return self.k_out[layer][r0:r0 + n], self.v_out[layer][r0:r0 + n], self.indices[i0:i0 + n]


class Buffers:
    """Device outputs and workspace of one compress_layers call, allocated
    with torch (memory plumbing only)."""

    def __init__(self, prob: ProblemHandle, n_layers: int, n_reuse: int, head_dim: int, dtype,
                 device="cuda", n_score_layers: Optional[int] = None):
        import torch
        pl = plan(prob)
        self.plan = pl
        self.n_anchor = -(-n_layers // n_reuse)
        ns = self.n_anchor if n_score_layers is None else n_score_layers
        self.ws_bytes = workspace_bytes(prob, max(1, min(ns, 32)))
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.scores = torch.empty(self.n_anchor * pl["scores_elems"], dtype=torch.float32, device=device)
        self.indices = torch.empty(self.n_anchor * pl["index_elems"], dtype=torch.int32, device=device)
        self.lengths = torch.empty(self.n_anchor * pl["length_elems"], dtype=torch.int32, device=device)
        self.k_out = torch.empty((n_layers, pl["index_elems"], head_dim), dtype=dtype, device=device)
        self.v_out = torch.empty((n_layers, pl["index_elems"], head_dim), dtype=dtype, device=device)
        self.n_reuse = n_reuse
        self.n_kv_heads = prob.struct.n_kv_heads

    def kept(self, layer: int, seq: int, head: int):
        """(K' rows, V' rows, kept token positions) of KV head `head` of
        sequence `seq` in layer `layer` after a compress_layers call into these
        buffers: views of the outputs, n rows each, n being the head's length
        of the layer's anchor (read from the device, so this synchronises)."""
        pl = self.plan
        a = layer // self.n_reuse
        cap = pl["l_cap"][seq]
        n = int(self.lengths[a * pl["length_elems"] + seq * self.n_kv_heads + head])
        r0 = pl["index_off"][seq] + head * cap
        i0 = a * pl["index_elems"] + r0
        return self.k_out[layer, r0:r0 + n], self.v_out[layer, r0:r0 + n], self.indices[i0:i0 + n]
