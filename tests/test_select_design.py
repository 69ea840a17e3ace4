"""CPU checks of the two facts the selection kernels are built on (ChunkKV
page, section 4.1, Algorithm 1 steps 4-6), each written here as plain Python
and compared with the oracle's TopK and index build on many random cases:

1. the threshold search: on keys that are fp32 bit patterns of scores >= 0
   (a pattern with the sign bit set counting as 0), building the largest
   pattern tau with #{key >= tau} >= k greedily from the top bit (bit 30
   alone, then two bits per step, three candidates counted at once), and
   stopping as soon as exactly k keys reach the prefix, yields the k-th
   largest key when it runs to the end; and in every case the keys above tau
   plus the first k - #{key > tau} keys equal to tau in id order are exactly
   the oracle's TopK (score descending, lower id first) -- so exactly min(k, C)
   chunks are selected whatever the bit patterns are;
2. the index list: with j_w = floor((T - w) / c), the first chunk that reaches
   the recent window, the kept tokens in ascending order are the c tokens of
   every selected chunk j < j_w followed by [j_w * c, T) if chunk j_w is
   selected, else [T - w, T) -- the oracle's sorted union of the selected
   chunks' tokens and the window.

This is the algorithm, not the HIP code: the GPU parity tests check the
kernels themselves against the oracle.
"""
import numpy as np
import pytest

import oracle


def _key(pattern: np.ndarray) -> np.ndarray:
    p = pattern.astype(np.uint32)
    return np.where(p >> np.uint32(31), np.uint32(0), p)


def _greedy_threshold(keys: np.ndarray, k: int):
    """tau and #{key >= tau}, as the kernels build them (0 < k < C)."""
    tau, n_ge = 0, len(keys)
    n1 = int(np.count_nonzero(keys >= (1 << 30)))
    if n1 >= k:
        tau, n_ge = 1 << 30, n1
    bit = 28
    while bit >= 0 and n_ge != k:
        counts = [int(np.count_nonzero(keys >= (tau | (m << bit)))) for m in (1, 2, 3)]
        for m in (3, 2, 1):
            if counts[m - 1] >= k:
                tau, n_ge = tau | (m << bit), counts[m - 1]
                break
        bit -= 2
    return tau, n_ge


def _select(keys: np.ndarray, k: int) -> np.ndarray:
    """Selected chunk ids (ascending) under the kernels' threshold and tie rule."""
    C = len(keys)
    if k >= C:
        return np.arange(C, dtype=np.int32)
    if k == 0:
        return np.zeros(0, dtype=np.int32)
    tau, n_ge = _greedy_threshold(keys, k)
    above = keys > tau
    if n_ge == k:   # exactly k reach tau: they are the selection
        return np.nonzero(keys >= tau)[0].astype(np.int32)
    need = k - int(np.count_nonzero(above))
    eq = np.nonzero(keys == tau)[0][:need]
    return np.sort(np.concatenate([np.nonzero(above)[0], eq])).astype(np.int32)


def _index_list(T: int, w: int, c: int, sel: np.ndarray) -> np.ndarray:
    j_w = (T - w) // c
    head = [np.arange(j * c, j * c + c) for j in sel if j < j_w]
    tail0 = j_w * c if j_w in set(sel.tolist()) else T - w
    parts = head + [np.arange(tail0, T)]
    return np.concatenate(parts).astype(np.int32)


def _patterns(rng, C: int, kind: str) -> np.ndarray:
    if kind == "scores":      # positive scores spanning many binades
        return np.exp(rng.normal(-4.0, 3.0, C)).astype(np.float32).view(np.uint32)
    if kind == "ties":        # few distinct values: many equal keys at tau
        return rng.choice(np.array([0.0, 0.25, 0.5, 1.0, 3.0], np.float32), C).view(np.uint32)
    if kind == "close":       # values a few ulps apart
        base = np.float32(0.0123).view(np.uint32)
        return (base + rng.integers(0, 6, C)).astype(np.uint32)
    # arbitrary 32-bit patterns: negatives, -0, NaNs of both signs, +-inf
    return rng.integers(0, 1 << 32, C, dtype=np.uint64).astype(np.uint32)


@pytest.mark.parametrize("kind", ["scores", "ties", "close", "any"])
def test_threshold_and_tie_rule_equal_oracle_topk(kind):
    rng = np.random.default_rng(7)
    for _ in range(300):
        C = int(rng.integers(1, 400))
        k = int(rng.integers(0, C + 3))
        keys = _key(_patterns(rng, C, kind))
        sel = _select(keys, k)
        assert len(sel) == min(k, C)
        # the oracle's TopK on the same order: the keys' unsigned order is the
        # scores' order for patterns below 2^31, so rank by key as a float64
        ref = oracle.topk(keys.astype(np.float64), k)
        assert np.array_equal(sel, ref), (kind, C, k)
        if 0 < k < C:
            tau, n_ge = _greedy_threshold(keys, k)
            kth = np.sort(keys)[::-1][k - 1]
            if n_ge != k:   # ran to the end: tau is the k-th largest key itself
                assert tau == kth
            else:           # stopped early: tau is a prefix at or below the k-th largest
                assert tau <= kth and np.count_nonzero(keys >= tau) == k


def test_index_list_equals_oracle_union():
    rng = np.random.default_rng(11)
    for _ in range(500):
        c = int(rng.integers(1, 40))
        T = int(rng.integers(1, 3000))
        w = int(rng.integers(1, T + 1))
        C = -(-T // c)
        n_sel = int(rng.integers(0, C + 1))
        sel = np.sort(rng.choice(C, n_sel, replace=False)).astype(np.int32)
        got = _index_list(T, w, c, sel)
        assert np.array_equal(got, oracle.indices(T, w, c, sel)), (T, w, c, n_sel)
