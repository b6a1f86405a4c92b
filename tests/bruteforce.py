"""Brute-force NumPy checkers that pin the CPU oracle on tiny inputs.

Each function computes one step of the layer a different way from the oracle (full sorts,
exhaustive enumeration, dense library products), so that a slip in the oracle's loops shows
up as a mismatch.  Used only by the tests.
"""
from __future__ import annotations

import itertools

import numpy as np


def topk_by_sort(keys: np.ndarray, k: int, allowed: np.ndarray | None = None) -> np.ndarray:
    """Per row: the k allowed columns of largest key, ties to the lower column, by a full
    lexicographic sort of (-key, column)."""
    T, E = keys.shape
    out = np.empty((T, k), np.int32)
    cols = np.arange(E)
    for t in range(T):
        kk = keys[t].astype(np.float64)
        c = cols if allowed is None else cols[allowed[t]]
        order = np.lexsort((c, -kk[c]))
        out[t] = c[order[:k]]
    return out


def group_mask_by_enumeration(keys: np.ndarray, n_groups: int, topk_groups: int,
                              per_group: int) -> np.ndarray:
    """Group-limited routing mask by exhaustive enumeration of group subsets.

    Group score: fp32 sum of the group's top `per_group` keys, largest first.  Among all
    subsets of `topk_groups` groups, the kept one is the lexicographically best when each
    subset is listed in rank order (score desc, group asc) -- i.e. no unkept group outranks a
    kept one."""
    T, E = keys.shape
    gs = E // n_groups
    mask = np.zeros((T, E), bool)
    for t in range(T):
        sc = []
        for g in range(n_groups):
            kg = np.sort(keys[t, g * gs:(g + 1) * gs].astype(np.float32))[::-1][:per_group]
            s = np.float32(0.0)
            for v in kg:
                s = np.float32(s + v)
            sc.append(s)

        def before(a, b):
            return sc[a] > sc[b] or (sc[a] == sc[b] and a < b)

        best = None
        for sub in itertools.combinations(range(n_groups), topk_groups):
            ok = all(not before(o, s) for s in sub for o in range(n_groups) if o not in sub)
            if ok:
                assert best is None, "two admissible group subsets"
                best = sub
        for g in best:
            mask[t, g * gs:(g + 1) * gs] = True
    return mask


def permutation_by_argsort(idx: np.ndarray, E: int):
    """counts/offsets/pos/src by a stable argsort of the flattened expert ids."""
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")        # src: rows in expert order, ascending pair
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    pos = np.empty_like(flat)
    pos[order] = np.arange(len(flat))
    return counts, offsets, pos.reshape(idx.shape).astype(np.int32), order.astype(np.int32)


def dense_swiglu(x: np.ndarray, w1: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """Dense SwiGLU FFN with library matrix products: (silu(x W_g^T) * (x W_u^T)) W2^T."""
    I = w1.shape[0] // 2
    g = x @ w1[:I].T
    u = x @ w1[I:].T
    return ((g / (1.0 + np.exp(-g))) * u) @ w2.T


def e4m3_values() -> np.ndarray:
    """All 256 E4M3 (OCP 'FN') codes decoded straight from the bit-field definition."""
    v = np.empty(256)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v[c] = np.nan
        elif e == 0:
            v[c] = (m / 8.0) * 2.0 ** -6
        else:
            v[c] = (1 + m / 8.0) * 2.0 ** (e - 7)
        if s:
            v[c] = -v[c]
    return v


def e4m3_nearest(a: np.ndarray) -> np.ndarray:
    """Nearest non-negative finite E4M3 code to each a >= 0 by exhaustive search over the
    127 finite codes 0x00..0x7E; exact ties go to the even code; a > 448 saturates."""
    vals = e4m3_values()[:127]
    a = np.minimum(np.asarray(a, np.float64), 448.0)
    d = np.abs(a[..., None] - vals)
    dmin = d.min(-1, keepdims=True)
    cand = d == dmin
    n_c = cand.sum(-1)
    first = cand.argmax(-1)
    # two candidates at equal distance: take the one with even code
    second = 126 - np.flip(cand, -1).argmax(-1)
    pick = np.where((n_c > 1) & (first % 2 == 1), second, first)
    return pick.astype(np.uint8)
