"""Softmax attention over dequantized K^/V^, in fp64.

Decode: query head h reads KV head g = h // G (G = Hq / Hkv, contiguous
groups); scores s_t = sm * q_h . K^_{t,g}, weights w = exp(s - max s) / sum,
output o_h = sum_t w_t V^_{t,g}.  Prefill: query i of a chunk starting at
absolute position p0 sees keys 0..p0+i inclusive, after the whole chunk has
been appended, so its own keys are read back quantized ("KV at 9 KB a token",
How it works: prefill attention reads the compressed cache directly).

The pages ask that every long sum be kept in real FP32 or better ("Half the
Cache, Twice the Context", section "The cliff is in the accumulator"): the
oracle keeps everything in fp64.

``split_partials`` / ``merge_partials`` restate split-K (flash-decoding): each
split p of the keys keeps (m_p, l_p, o_p) = (max score, sum of exp(s - m_p),
sum of exp(s - m_p) V^), and the merge rescales by exp(m_p - M).  In exact
arithmetic the merge equals the unsplit softmax; that invariant pins it.

Pins (tests/test_oracle_pool_attention.py): ctx_len = 1 gives o = V^_0;
constant scores give the mean of V^; a dominant key returns its value row; a
loop reference on tiny shapes; the split/merge identity; prefill's last row
equals decode at the same length.  scores: with K[t, g] = (g + 1) * ones and
unit queries every score of head h is sm * D * (h // G + 1) (the GQA
mapping); unit-vector keys return the scaled query row; keys parallel to the
query give sm * c * |q|^2; softmax of the scores applied to V is decode's
output.  planted_rank: worked cases with ties.
"""

from __future__ import annotations

import numpy as np


def _softmax(s):
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def decode(q, K, V, sm: float):
    """q [Hq][D]; K, V [T][Hkv][D] -> out [Hq][D] (fp64)."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    Hq, Hkv = q.shape[0], K.shape[1]
    G = Hq // Hkv
    out = np.empty((Hq, q.shape[1]), np.float64)
    for h in range(Hq):
        g = h // G
        s = sm * (K[:, g, :] @ q[h])
        out[h] = _softmax(s) @ V[:, g, :]
    return out


def scores(q, K, sm: float):
    """Raw logits [Hq][T] of one decode step (fp64)."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    G = q.shape[0] // K.shape[1]
    return np.stack([sm * (K[:, h // G, :] @ q[h]) for h in range(q.shape[0])])


def prefill(q, K, V, sm: float, q_start: int, rows=None):
    """q [n][Hq][D] at absolute positions q_start.. ; K, V [T][Hkv][D], T >= q_start + n.

    Returns out [len(rows)][Hq][D] for the requested chunk rows (default all).
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n, Hq = q.shape[0], q.shape[1]
    G = Hq // K.shape[1]
    rows = range(n) if rows is None else rows
    out = np.empty((len(rows), Hq, q.shape[2]), np.float64)
    for r, i in enumerate(rows):
        end = q_start + i + 1
        for h in range(Hq):
            g = h // G
            s = sm * (K[:end, g, :] @ q[i, h])
            out[r, h] = _softmax(s) @ V[:end, g, :]
    return out


def prefill_dense(q, K, V, sm: float, q_start: int):
    """The same causal prefill as ``prefill``, as one fp64 matrix product per
    query head over the whole chunk: scores [n][T] with keys past a row's
    position masked out, row softmax, then the product with V.  For checking
    every row of a long chunk (one product per head instead of a vector product
    per row and head); pinned against ``prefill`` in
    tests/test_oracle_pool_attention.py."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n, Hq, D = q.shape
    T = q_start + n
    G = Hq // K.shape[1]
    visible = np.arange(T)[None, :] <= (q_start + np.arange(n))[:, None]       # [n][T]
    out = np.empty((n, Hq, D), np.float64)
    for h in range(Hq):
        g = h // G
        s = sm * (q[:, h, :] @ K[:T, g, :].T)
        s = np.where(visible, s, -np.inf)
        out[:, h, :] = _softmax(s) @ V[:T, g, :]
    return out


def split_partials(s, Vg, bounds):
    """Per split [a, b): (m, l, o) for scores s [T] and values Vg [T][D]."""
    parts = []
    for a, b in bounds:
        if b <= a:
            parts.append((-np.inf, 0.0, np.zeros(Vg.shape[1])))
            continue
        m = s[a:b].max()
        e = np.exp(s[a:b] - m)
        parts.append((m, e.sum(), e @ Vg[a:b]))
    return parts


def merge_partials(parts):
    M = max(m for m, _, _ in parts)
    num = sum(np.exp(m - M) * o for m, l, o in parts if l > 0)
    den = sum(np.exp(m - M) * l for m, l, o in parts if l > 0)
    return num / den


def planted_rank(s_row, pos: int) -> int:
    """1 + number of keys scoring strictly above the planted one (ties favour it)."""
    s_row = np.asarray(s_row)
    return 1 + int(np.count_nonzero(s_row > s_row[pos]))
