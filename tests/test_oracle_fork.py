"""Oracle pins: prefix sharing between sequences (fork).

A child that starts with the parent's first n tokens shares the parent's whole
pages and gets a copy of the page the prefix only partly fills ("The KV cache
and prompt reuse", What a sequence is made of).  Pinned by:
  * the child reads back exactly the parent's first n tokens;
  * the child's continuation reads back exactly what a fresh sequence of the
    same tokens, appended on its own, reads back;
  * the parent reads back the same before and after the child appends, and
    its own continuation equals a fresh sequence as well;
  * a fork on a page boundary copies nothing.
"""

import numpy as np
import pytest

from oracle import pool
from synth import WORKLOADS, kv_rows

FORMATS = ["q2", "q8", "bf16", "q2w", "q2r"]


def _rows(n, lane=0):
    w = WORKLOADS["tiny"]
    k, v = kv_rows(w, 0, lane, n)
    return k.float().numpy(), v.float().numpy()


def _dims(fmt):
    return 128 if fmt == "q8" else 256


def _fresh(fmt, k, v, pieces):
    D = _dims(fmt)
    p = pool.OraclePool(fmt, 2, 4, D, 8)
    bt = np.arange(8, dtype=np.int32)
    start = 0
    for n in pieces:
        for layer in range(2):
            p.append(layer, 0, bt, start, k[start:start + n, :, :D], v[start:start + n, :, :D])
        start += n
    return [p.gather(layer, bt, start, seq=0) for layer in range(2)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("n", [150, 128])
def test_fork_prefix_then_continuations(fmt, n):
    D = _dims(fmt)
    k, v = _rows(260)
    kc, vc = _rows(260, lane=1)          # the child's own continuation
    kc[:n], vc[:n] = k[:n], v[:n]
    p = pool.OraclePool(fmt, 2, 4, D, 12, fill=0x3C)
    pbt = np.array([7, 2, 9, 4, 11], np.int32)
    for layer in range(2):
        p.append(layer, 0, pbt, 0, k[:100, :, :D], v[:100, :, :D])
        p.append(layer, 0, pbt, 100, k[100:n, :, :D], v[100:n, :, :D])
    before = [p.gather(layer, pbt, n, seq=0) for layer in range(2)]
    cbt = np.concatenate([pbt[:n // 64], np.array([0, 5, 1, 8, 3], np.int32)])[:5]
    page_copy = p.data[pbt[n // 64]].copy() if n % 64 else None
    p.fork(0, pbt, 1, cbt, n)
    if n % 64:
        assert np.array_equal(p.data[cbt[n // 64]], page_copy)
    for layer in range(2):   # the child reads the parent's prefix exactly
        K, V = p.gather(layer, cbt, n, seq=1)
        assert np.array_equal(K, before[layer][0]) and np.array_equal(V, before[layer][1])
    for layer in range(2):   # the child appends its own tokens
        p.append(layer, 1, cbt, n, kc[n:230, :, :D], vc[n:230, :, :D])
    want = _fresh(fmt, kc, vc, (n, 230 - n))
    for layer in range(2):
        K, V = p.gather(layer, cbt, 230, seq=1)
        assert np.array_equal(K, want[layer][0]) and np.array_equal(V, want[layer][1])
    for layer in range(2):   # the parent did not change, and continues on its own pages
        K, V = p.gather(layer, pbt, n, seq=0)
        assert np.array_equal(K, before[layer][0]) and np.array_equal(V, before[layer][1])
        p.append(layer, 0, pbt, n, k[n:260, :, :D], v[n:260, :, :D])
    want = _fresh(fmt, k, v, (n, 260 - n))
    for layer in range(2):
        K, V = p.gather(layer, pbt, 260, seq=0)
        assert np.array_equal(K, want[layer][0]) and np.array_equal(V, want[layer][1])


def test_fork_refusals():
    k, v = _rows(200)
    p = pool.OraclePool("q2w", 1, 4, 256, 8)
    pbt = np.array([0, 1, 2, 3], np.int32)
    p.append(0, 0, pbt, 0, k[:200], v[:200])
    with pytest.raises(ValueError):      # the shared pages must be the parent's
        p.fork(0, pbt, 1, np.array([0, 5, 6, 7], np.int32), 150)
    with pytest.raises(ValueError):      # the open page must be copied, not shared
        p.fork(0, pbt, 1, np.array([0, 1, 2, 7], np.int32), 150)
    with pytest.raises(ValueError):      # a window fork ends in the parent's last page
        p.fork(0, pbt, 1, np.array([0, 1, 6, 7], np.int32), 150)
