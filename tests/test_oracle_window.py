"""Oracle pins: the 2-bit format with an exact window of the last page.

"The KV cache and prompt reuse" (What a sequence is made of) has the
compressed format hold its most recent keys unquantized.  Read here: with A
tokens of a (sequence, layer) appended, the tokens of page floor((A - 1) / 64)
are read exact, every earlier token through the 2-bit codec.  Pinned by:
  * the pages equal a plain 2-bit pool's byte for byte (the body is the 2-bit
    format, whose codec has its own pins);
  * a sequence inside one page attends exactly as a plain loop over the input
    rows does (brute force, no quantization anywhere);
  * the last page reads back as the appended rows, earlier pages as the codec's
    rows, and the boundary moves when a new page opens;
  * a dominant key in the window returns its exact value row, where the plain
    2-bit pool returns the dequantized one.
"""

import math

import numpy as np
import pytest

from oracle import attention, codec, pool
from synth import WORKLOADS, kv_rows, queries


def _rows(n):
    w = WORKLOADS["tiny"]
    k, v = kv_rows(w, 0, 0, n)
    return w, k.float().numpy(), v.float().numpy()


def _loop_attention(q, K, V, sm):
    """Softmax attention written as plain loops (fp64), GQA head h -> h // G."""
    Hq, D = q.shape
    T, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D))
    for h in range(Hq):
        g = h // G
        s = [sm * sum(float(q[h, d]) * float(K[t, g, d]) for d in range(D)) for t in range(T)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        for t in range(T):
            out[h] += (e[t] / z) * V[t, g].astype(np.float64)
    return out


def _append_pieces(p, k, v, pieces, bt):
    start = 0
    for n in pieces:
        p.append(0, 0, bt, start, k[start:start + n], v[start:start + n])
        start += n
    return start


def test_pages_equal_a_plain_2bit_pool():
    w, k, v = _rows(200)
    bt = np.array([2, 0, 3, 1], np.int32)
    a = pool.OraclePool("q2w", 1, 4, 256, 4)
    b = pool.OraclePool("q2", 1, 4, 256, 4)
    _append_pieces(a, k, v, (64, 70, 1, 65), bt)
    _append_pieces(b, k, v, (64, 70, 1, 65), bt)
    assert np.array_equal(a.data, b.data)


def test_sequence_inside_one_page_attends_exactly():
    w, k, v = _rows(50)
    D = 32   # a slice of the dims keeps the loop reference quick
    k, v = k[..., :D].copy(), v[..., :D].copy()
    q = queries(w, 0, 1)[0].float().numpy()[:, :D]
    p = pool.OraclePool("q2w", 1, 4, D, 2)
    bt = np.array([1], np.int32)
    _append_pieces(p, k, v, (7, 30, 13), bt)
    for ctx in (1, 17, 50):
        K, V = p.gather(0, bt, ctx, seq=0)
        assert np.array_equal(K, k[:ctx]) and np.array_equal(V, v[:ctx])
        got = attention.decode(q, K, V, w.sm_scale)
        want = _loop_attention(q, k[:ctx], v[:ctx], w.sm_scale)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_body_is_the_codec_and_last_page_is_exact():
    w, k, v = _rows(200)
    bt = np.array([3, 1, 0, 2], np.int32)
    p = pool.OraclePool("q2w", 1, 4, 256, 4)
    _append_pieces(p, k, v, (64, 70, 1, 65), bt)
    assert p.window_start(0, 0) == 192
    K, V = p.gather(0, bt, 200, seq=0)
    Kq = codec.q2_dequantize(*codec.q2_quantize(k))
    Vq = codec.q2_dequantize(*codec.q2_quantize(v))
    assert np.array_equal(K[:192], Kq[:192]) and np.array_equal(V[:192], Vq[:192])
    assert np.array_equal(K[192:], k[192:]) and np.array_equal(V[192:], v[192:])
    assert not np.array_equal(Kq[192:], k[192:])   # the window really differs from the codec
    # a context that ends before the window reads the 2-bit rows only
    K, V = p.gather(0, bt, 150, seq=0)
    assert np.array_equal(K, Kq[:150]) and np.array_equal(V, Vq[:150])
    # the whole-sequence shortcut gives the same rows
    K2, V2 = pool.dequantized_rows("q2w", k, v)
    K, V = p.gather(0, bt, 200, seq=0)
    assert np.array_equal(K, K2) and np.array_equal(V, V2)


def test_window_moves_when_a_new_page_opens():
    w, k, v = _rows(129)
    bt = np.array([0, 1, 2], np.int32)
    p = pool.OraclePool("q2w", 1, 4, 256, 3)
    _append_pieces(p, k, v, (100, 28), bt)           # 128 tokens: page 1 is full and exact
    K, _ = p.gather(0, bt, 128, seq=0)
    assert p.window_start(0, 0) == 64
    assert np.array_equal(K[64:], k[64:128])
    p.append(0, 0, bt, 128, k[128:129], v[128:129])
    assert p.window_start(0, 0) == 128
    K, V = p.gather(0, bt, 129, seq=0)
    Kq = codec.q2_dequantize(*codec.q2_quantize(k))
    assert np.array_equal(K[64:128], Kq[64:128])     # page 1 now reads compressed
    assert np.array_equal(K[128], k[128]) and np.array_equal(V[128], v[128])


def test_dominant_window_key_returns_its_exact_value():
    w, k, v = _rows(100)
    q = queries(w, 0, 1)[0].float().numpy()
    t = 97
    for g in range(4):   # key t of head g points along the query of head 4g, 40x its norm
        u = q[4 * g] / np.linalg.norm(q[4 * g])
        k[t, g] = (40.0 * u).astype(np.float32)
    k = (k.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)   # keep them bf16 numbers
    bt = np.array([0, 1], np.int32)
    a = pool.OraclePool("q2w", 1, 4, 256, 2)
    b = pool.OraclePool("q2", 1, 4, 256, 2)
    _append_pieces(a, k, v, (100,), bt)
    _append_pieces(b, k, v, (100,), bt)
    oa = attention.decode(q, *a.gather(0, bt, 100, seq=0), w.sm_scale)
    ob = attention.decode(q, *b.gather(0, bt, 100), w.sm_scale)
    Vq = codec.q2_dequantize(*codec.q2_quantize(v))
    for g in range(4):
        np.testing.assert_allclose(oa[4 * g], v[t, g], atol=1e-9)
        np.testing.assert_allclose(ob[4 * g], Vq[t, g], atol=1e-9)
    assert np.abs(v[t] - Vq[t]).max() > 0.1


def test_refusals():
    w, k, v = _rows(80)
    bt = np.array([0, 1], np.int32)
    p = pool.OraclePool("q2w", 1, 4, 256, 2)
    p.append(0, 0, bt, 0, k[:40], v[:40])
    with pytest.raises(ValueError):
        p.append(0, 0, bt, 41, k[41:50], v[41:50])   # not sequential
    with pytest.raises(ValueError):
        p.gather(0, bt, 41, seq=0)                   # beyond the appended tokens
