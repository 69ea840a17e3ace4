"""ctypes wrapper of the plain CPU oracle (oracle/chunkkv_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only users.  The product package never
imports this module and shares no code with it.

Arrays are numpy: fp32 inputs as ``float32``, bf16 inputs as their raw 16-bit
patterns in ``uint16``.  Layouts follow the pages' statement of the problem
(ChunkKV page, section 4.1, Algorithm 1): per sequence ``q[t_q, H_q, d]`` (only
the last ``w`` rows are read), ``k``/``v[T, H_kv, d]``.

Parity note: every function here is pinned by ``tests/test_oracle.py`` against
closed forms, invariants, brute force and library routines; none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "chunkkv_oracle.c")
# CHUNKKV_ORACLE_LIB points the wrapper at another build of the oracle; the
# mutation test uses it to load copies with planted mistakes.
_LIB_PATH = os.environ.get("CHUNKKV_ORACLE_LIB") or os.path.join(_HERE, "libchunkkv_oracle.so")

F32, BF16 = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/libchunkkv_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.orc_num_chunks.restype = i64
        L.orc_num_chunks.argtypes = [i64, i64]
        L.orc_num_keep_chunks.restype = i64
        L.orc_num_keep_chunks.argtypes = [i64, i64]
        L.orc_chunk_scores.restype = i32
        L.orc_chunk_scores.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32, i32,
                                       vp, i64, i64, vp, i64, i64, vp]
        L.orc_topk.restype = i64
        L.orc_topk.argtypes = [i64, i64, vp, vp]
        L.orc_indices.restype = i64
        L.orc_indices.argtypes = [i64, i32, i32, i64, vp, vp]
        L.orc_gather.restype = None
        L.orc_gather.argtypes = [i64, vp, i32, i32, vp, i64, i64, i32, vp]
        L.orc_decode_attention.restype = i32
        L.orc_decode_attention.argtypes = [i32, i64, i32, i32, vp, vp, vp, vp]
        L.orc_compress_layers.restype = i32
        L.orc_compress_layers.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32, i64,
                                          i32, i32, vp, i64, i64, vp, vp, i64, i64,
                                          vp, vp, i64, vp, vp, vp]
        _lib = L
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def num_chunks(T: int, c: int) -> int:
    return int(lib().orc_num_chunks(T, c))


def num_keep_chunks(l_max: int, c: int) -> int:
    return int(lib().orc_num_keep_chunks(l_max, c))


def chunk_scores(q: np.ndarray, k: np.ndarray, h: int, n_q_heads: int, w: int, c: int) -> np.ndarray:
    """Chunk scores of KV head ``h`` (Algorithm 1 steps 1-3), float64 [C]."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    t_q, hq, d = q.shape
    T, hkv, dk = k.shape
    assert hq == n_q_heads and dk == d and q.dtype == k.dtype
    out = np.empty(num_chunks(T, c), dtype=np.float64)
    rc = lib().orc_chunk_scores(_dtype_code(k), T, t_q, hq, hkv, h, d, w, c,
                                _ptr(q), hq * d, d, _ptr(k), hkv * d, d, _ptr(out))
    if rc != 0:
        raise ValueError(f"orc_chunk_scores failed with status {rc}")
    return out


def topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Selected chunk ids (Algorithm 1 step 4), ascending int32."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    sel = np.empty(max(1, min(k, s.size)), dtype=np.int32)
    n = lib().orc_topk(s.size, k, _ptr(s), _ptr(sel))
    if n < 0:
        raise ValueError(f"orc_topk failed with status {-n}")
    return sel[:n].copy()


def indices(T: int, w: int, c: int, sel: np.ndarray) -> np.ndarray:
    """Kept token positions (Algorithm 1 steps 5-6), ascending int32."""
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    out = np.empty(T, dtype=np.int32)
    n = lib().orc_indices(T, w, c, sel.size, _ptr(sel), _ptr(out))
    if n < 0:
        raise ValueError(f"orc_indices failed with status {-n}")
    return out[:n].copy()


def gather(src: np.ndarray, idx: np.ndarray, head: int) -> np.ndarray:
    """index_select of head ``head`` rows of ``src[T, H_kv, d]`` -> [n, d]."""
    src = np.ascontiguousarray(src)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, hkv, d = src.shape
    dst = np.empty((idx.size, d), dtype=src.dtype)
    lib().orc_gather(idx.size, _ptr(idx), src.itemsize, d, _ptr(src), hkv * d, d, head, _ptr(dst))
    return dst


def to_pages(rows: np.ndarray, table: np.ndarray, page_rows: int, pool: np.ndarray) -> None:
    """Write one head's kept rows ``rows[n, d]`` into the page pool
    ``pool[n_pages, page_rows, d]`` in place: the cache as fixed-size blocks of
    consecutive KV rows, as PagedAttention keeps it (Kara page, section 2).
    Row i goes to row ``i % page_rows`` of page ``table[i // page_rows]``; a
    page id outside ``[0, n_pages)`` leaves its rows unwritten.  Plain loop
    over the rows: small cases only."""
    n_pages = pool.shape[0]
    for i in range(rows.shape[0]):
        page = int(table[i // page_rows])
        if 0 <= page < n_pages:
            pool[page, i % page_rows] = rows[i]


def decode_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Decode attention of the G queries ``q[G, d]`` over one head's kept rows
    ``k[n, d]``, ``v[n, d]`` (softmax(q . k / sqrt(d)) weights, Kara eq. (1)),
    float64 [G, d]; zeros when n == 0."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    G, d = q.shape
    n = k.shape[0]
    assert k.shape == (n, d) and v.shape == (n, d) and q.dtype == k.dtype == v.dtype
    out = np.empty((G, d), dtype=np.float64)
    rc = lib().orc_decode_attention(_dtype_code(k), n, G, d, _ptr(q), _ptr(k), _ptr(v), _ptr(out))
    if rc != 0:
        raise ValueError(f"orc_decode_attention failed with status {rc}")
    return out


def compress_one(q, k, v, n_q_heads, w, c, l_max):
    """Algorithm 1 on one layer of one sequence, all KV heads.

    Returns (scores[H_kv, C] float64, list of index arrays, list of K' [n, d],
    list of V' [n, d]).
    """
    T, hkv, d = k.shape
    scores = np.stack([chunk_scores(q, k, h, n_q_heads, w, c) for h in range(hkv)])
    kk = num_keep_chunks(l_max, c)
    idxs, kouts, vouts = [], [], []
    for h in range(hkv):
        idx = indices(T, w, c, topk(scores[h], kk))
        idxs.append(idx)
        kouts.append(gather(k, idx, h))
        vouts.append(gather(v, idx, h))
    return scores, idxs, kouts, vouts


def l_cap(T: int, w: int, c: int, l_max: int) -> int:
    """Largest possible number of kept tokens: min(T, floor(L_max/c)*c + w)."""
    return min(T, num_keep_chunks(l_max, c) * c + w)


def compress_layers(qs, ks, vs, n_q_heads, w, c, l_max, n_reuse):
    """Algorithm 2 for one sequence.

    qs/ks/vs: lists (one per layer) of [t_q, H_q, d] / [T, H_kv, d] arrays
    (qs[l] may be None where l % n_reuse != 0).
    Returns dict with scores [L, H_kv, C] (NaN on reusing layers), indices
    [L, H_kv, l_cap], lengths [L, H_kv], k_out/v_out [L, H_kv, l_cap, d].
    """
    L = len(ks)
    T, hkv, d = ks[0].shape
    dt = ks[0].dtype
    cap = l_cap(T, w, c, l_max)
    C = num_chunks(T, c)
    t_q = next(q.shape[0] for q in qs if q is not None)
    qs = [None if q is None else np.ascontiguousarray(q) for q in qs]
    ks = [np.ascontiguousarray(x) for x in ks]
    vs = [np.ascontiguousarray(x) for x in vs]
    k_out = np.zeros((L, hkv, cap, d), dtype=dt)
    v_out = np.zeros((L, hkv, cap, d), dtype=dt)
    scores = np.full((L, hkv, C), np.nan)
    indices_ = np.full((L, hkv, cap), -1, dtype=np.int32)
    lengths = np.zeros((L, hkv), dtype=np.int64)
    P = ctypes.c_void_p * L
    qp = P(*[None if q is None else _ptr(q) for q in qs])
    rc = lib().orc_compress_layers(
        _dtype_code(ks[0]), T, t_q, n_q_heads, hkv, d, w, c, l_max, L, n_reuse,
        qp, n_q_heads * d, d, P(*[_ptr(x) for x in ks]), P(*[_ptr(x) for x in vs]),
        hkv * d, d, P(*[_ptr(k_out[l]) for l in range(L)]),
        P(*[_ptr(v_out[l]) for l in range(L)]), cap, _ptr(scores), _ptr(indices_),
        _ptr(lengths))
    if rc != 0:
        raise ValueError(f"orc_compress_layers failed with status {rc}")
    return dict(scores=scores, indices=indices_, lengths=lengths, k_out=k_out, v_out=v_out,
                l_cap=cap, C=C)
