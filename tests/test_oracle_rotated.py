"""Oracle pins: the Hadamard-rotated 2-bit variant.

The rotated variant quantizes H k (H the unnormalised Sylvester
Walsh-Hadamard matrix) and reads back H k^_r / D; V is the 2-bit format's.
Pinned by:
  * the fp32 butterfly transform equals the product with scipy's Hadamard
    matrix exactly on small-integer rows (every fp32 operation exact) and to
    fp32 rounding on bf16 rows; the inverse undoes it;
  * the error bound the rotation keeps: ||k^ - k||_2 <= scale_r / 2 per row,
    because H / sqrt(D) is orthogonal and every rotated element is within
    scale_r / 2 of its code; V reads back as the plain 2-bit codec's rows;
  * scores over the read-back rows equal (H q) . x^_r / D, the identity the
    decode kernel uses;
  * on rows with the channel outliers of "Half the Cache, Twice the Context"
    (every 16th key channel x4), rotation lowers the 2-bit error of K, as
    that page's closing notes lead one to expect.
"""

import numpy as np
import scipy.linalg

from oracle import codec, pool
from synth import WORKLOADS, kv_rows, queries


def _rows(n=200):
    w = WORKLOADS["tiny"]
    k, v = kv_rows(w, 0, 0, n)
    return w, k.float().numpy(), v.float().numpy()


def test_butterflies_equal_the_hadamard_matrix():
    H = scipy.linalg.hadamard(256).astype(np.float64)
    rng = np.random.default_rng(3)
    xi = rng.integers(-4, 5, size=(5, 256)).astype(np.float32)
    assert np.array_equal(codec.hadamard_rows(xi).astype(np.float64), xi.astype(np.float64) @ H.T)
    assert np.array_equal(codec.unrotate_rows(codec.hadamard_rows(xi)), xi.astype(np.float64))
    _, k, _ = _rows(8)
    x = k[:, 0, :]
    got = codec.hadamard_rows(x).astype(np.float64)
    want = x.astype(np.float64) @ H.T
    assert np.max(np.abs(got - want) / (np.abs(want) + 1e-3)) < 1e-5
    H128 = scipy.linalg.hadamard(128).astype(np.float64)
    xi = rng.integers(-3, 4, size=(3, 128)).astype(np.float32)
    assert np.array_equal(codec.hadamard_rows(xi).astype(np.float64), xi.astype(np.float64) @ H128.T)


def test_rotated_error_bound_and_score_identity():
    w, k, v = _rows(200)
    p = pool.OraclePool("q2r", 1, 4, 256, 4)
    bt = np.array([2, 0, 3, 1], np.int32)
    p.append(0, 0, bt, 0, k[:120], v[:120])
    p.append(0, 0, bt, 120, k[120:], v[120:])
    K, V = p.gather(0, bt, 200)
    _, sk, _ = codec.q2_quantize(codec.hadamard_rows(k))
    ek = np.linalg.norm(K - k.astype(np.float64), axis=-1)
    assert np.all(ek <= 0.5 * sk * (1 + 1e-5))
    assert np.array_equal(V, codec.q2_dequantize(*codec.q2_quantize(v)))
    # scores in the original basis equal (H q) . x^_r / D over the raw rotated rows
    Kr = p._gather_pages(0, bt, 200)[0].astype(np.float64)
    q = queries(w, 0, 1)[0].float().numpy().astype(np.float64)
    for h in (0, 5, 15):
        g = h // 4
        direct = K[:, g, :] @ q[h]
        via_hq = Kr[:, g, :] @ (scipy.linalg.hadamard(256) @ q[h]) / 256
        np.testing.assert_allclose(direct, via_hq, rtol=1e-10, atol=1e-10)


def test_rotation_lowers_the_2bit_key_error_under_channel_outliers():
    _, k, v = _rows(256)
    Kq = codec.q2_dequantize(*codec.q2_quantize(k)).astype(np.float64)
    Kr, _ = pool.dequantized_rows("q2r", k, v)
    plain = np.linalg.norm(Kq - k) / np.linalg.norm(k)
    rot = np.linalg.norm(Kr - k) / np.linalg.norm(k)
    assert rot < 0.8 * plain, (plain, rot)
