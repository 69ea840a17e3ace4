"""Byte accounting for ChunkKV compression (no device code, no method math).

Algorithmic bytes are what the method must move, not what an implementation
happens to move:
  * a scoring (anchor) layer reads every key of every KV head once and the
    window queries, and writes C fp32 chunk scores per head;
  * selection reads the scores and writes the kept indices;
  * every layer's gather reads the kept K and V rows and writes K' and V'
    (4 * n * d * elem_bytes per head), reading the n indices.
"""
from __future__ import annotations


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """KV-cache footprint of one token: K and V rows of every layer and head."""
    return 2 * n_layers * n_kv_heads * head_dim * elem_bytes


def score_bytes(seq_lens, n_q_heads, n_kv_heads, head_dim, window, chunk, elem_bytes) -> int:
    """One anchor layer's score phase: K read + window queries + fp32 scores."""
    k_read = sum(seq_lens) * n_kv_heads * head_dim * elem_bytes
    q_read = len(seq_lens) * window * n_q_heads * head_dim * elem_bytes
    s_write = sum(-(-t // chunk) for t in seq_lens) * n_kv_heads * 4
    return k_read + q_read + s_write


def select_bytes(seq_lens, n_kv_heads, chunk, total_kept) -> int:
    """One anchor layer's selection: read the scores, write indices and lengths."""
    return (sum(-(-t // chunk) for t in seq_lens) * n_kv_heads * 4 + total_kept * 4
            + len(seq_lens) * n_kv_heads * 4)


def gather_bytes(total_kept, head_dim, elem_bytes) -> int:
    """One layer's gather: read kept K and V rows, write K' and V', read indices."""
    return 4 * total_kept * head_dim * elem_bytes + total_kept * 4
