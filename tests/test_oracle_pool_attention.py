"""Oracle pins: pool append / gather and fp64 attention (closed forms, invariants, loops)."""

import math

import numpy as np
import pytest

from oracle import attention, codec, layout, pool
from synth import WORKLOADS, kv_rows, page_permutation, queries

F32 = np.float32


def _c0_rows(n=256):
    w = WORKLOADS["tiny"]
    k, v = kv_rows(w, 0, 0, n)
    return w, k.float().numpy(), v.float().numpy()


@pytest.mark.parametrize("fmt", ["q2", "q8", "bf16"])
def test_append_gather_is_permutation_invariant(fmt):
    w, k, v = _c0_rows()
    D = 128 if fmt == "q8" else 256
    k, v = k[..., :D].copy(), v[..., :D].copy()
    outs = []
    for salt in (0, 1):
        bt = page_permutation(w, 6, salt=salt)[:4]
        p = pool.OraclePool(fmt, 1, 4, D, 6)
        start = 0
        for n in (100, 1, 27, 64, 64):   # ragged chunks, one crossing page ends
            p.append(0, 0, bt, start, k[start:start + n], v[start:start + n])
            start += n
        outs.append(p.gather(0, bt, 256))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    K, V = pool.dequantized_rows(fmt, k, v)
    assert np.array_equal(outs[0][0], K) and np.array_equal(outs[0][1], V)


def test_bf16_pool_stores_rows_as_given_at_their_byte_offsets():
    # the exact format: the gather returns the appended rows bit for bit, and
    # the bytes sit where the block layout puts them (K row t at 2 D t, V
    # element (d, t) at 128 D + 2 (64 d + t)), read back here by hand
    w, k, v = _c0_rows(100)
    D, H = 256, 4
    p = pool.OraclePool("bf16", 2, H, D, 5, fill=0x5A)
    bt = np.array([3, 0], np.int32)
    p.append(1, 0, bt, 0, k[:70], v[:70])
    p.append(1, 0, bt, 70, k[70:], v[70:])
    K, V = p.gather(1, bt, 100)
    assert np.array_equal(K, k) and np.array_equal(V, v)
    for page in (1, 2, 4):
        assert np.all(p.data[page] == 0x5A)
    kbits = k.view(np.uint32) >> 16
    vbits = v.view(np.uint32) >> 16
    for t, h, d in ((0, 0, 0), (63, 3, 255), (64, 1, 7), (99, 2, 128), (37, 0, 200)):
        page, slot = int(bt[t // 64]), t % 64
        base = (1 * H + h) * layout.bf16_block_bytes(D)   # layer 1
        ko = base + 2 * D * slot + 2 * d
        vo = base + 128 * D + 2 * (64 * d + slot)
        assert int(p.data[page, ko]) | int(p.data[page, ko + 1]) << 8 == kbits[t, h, d]
        assert int(p.data[page, vo]) | int(p.data[page, vo + 1]) << 8 == vbits[t, h, d]
    # layer 0 of the used pages was never written
    assert np.all(p.data[3, :H * layout.bf16_block_bytes(D)] == 0x5A)
    with pytest.raises(AssertionError):   # rows off the bf16 grid are refused
        p.append(1, 0, bt, 0, k[:1] * np.float32(1.0001), v[:1])


def test_append_leaves_other_slots_and_pages_alone():
    w, k, v = _c0_rows(100)
    p = pool.OraclePool("q2", 1, 4, 256, 6, fill=0xA5)
    bt = np.array([4, 1], np.int32)
    p.append(0, 0, bt, 0, k, v)
    for page in (0, 2, 3, 5):
        assert np.all(p.data[page] == 0xA5)
    for h in range(4):
        blk = p.block(1, 0, h)
        assert np.all(blk.k_codes[36:] == 0xA5)             # slots 36..63 of the 2nd page
        assert np.all(blk.k_meta[36:].view(np.uint8) == 0xA5)
        fill_slots = layout.unpack2_vrow(np.full((1, 16), 0xA5, np.uint8))[0]
        assert np.all(layout.unpack2_vrow(blk.v_codes)[:, 36:] == fill_slots[36:])   # V slots 36..63


def test_q8_partial_page_then_full_page_equals_full_quantization():
    w, k, v = _c0_rows(128)
    k, v = k[..., :128].copy(), v[..., :128].copy()
    p = pool.OraclePool("q8", 1, 4, 128, 2)
    bt = np.array([1, 0], np.int32)
    p.append(0, 7, bt, 0, k[:10], v[:10])
    c10, s10 = codec.q8_quantize_k_page(k[:10])
    assert np.array_equal(p.block(1, 0, 2).k_codes[:10], c10[:, 2])
    assert np.array_equal(p.block(1, 0, 2).k_scale, s10[2])
    p.append(0, 7, bt, 10, k[10:75], v[10:75])
    c64, s64 = codec.q8_quantize_k_page(k[:64])
    for h in range(4):
        assert np.array_equal(p.block(1, 0, h).k_codes, c64[:, h])
        assert np.array_equal(p.block(1, 0, h).k_scale, s64[h])
    cn, sn = codec.q8_quantize_k_page(k[64:75])
    assert np.array_equal(p.block(0, 0, 1).k_codes[:11], cn[:, 1])


# ------------------------------------------------------------ attention --

def _loop_decode(q, K, V, sm):
    Hq, D = len(q), len(q[0])
    T, Hkv = len(K), len(K[0])
    G = Hq // Hkv
    out = []
    for h in range(Hq):
        g = h // G
        s = [sm * sum(q[h][d] * K[t][g][d] for d in range(D)) for t in range(T)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        out.append([sum(e[t] * V[t][g][d] for t in range(T)) / z for d in range(D)])
    return out


def test_decode_matches_loop_reference():
    rng = np.random.default_rng(31)
    q = rng.normal(0, 1, (4, 6))
    K = rng.normal(0, 1, (9, 2, 6))
    V = rng.normal(0, 1, (9, 2, 6))
    got = attention.decode(q, K, V, 0.4)
    ref = np.array(_loop_decode(q.tolist(), K.tolist(), V.tolist(), 0.4))
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_decode_closed_forms():
    rng = np.random.default_rng(32)
    V = rng.normal(0, 1, (50, 2, 8))
    q = rng.normal(0, 1, (4, 8))
    # one token: output is that token's value row
    K = rng.normal(0, 1, (1, 2, 8))
    o = attention.decode(q, K, V[:1], 0.3)
    assert np.allclose(o, V[0, [0, 0, 1, 1]], rtol=0, atol=1e-15)
    # identical keys: uniform weights, output is the mean value
    K = np.zeros((50, 2, 8))
    o = attention.decode(q, K, V, 0.3)
    assert np.allclose(o, V.mean(axis=0)[[0, 0, 1, 1]], rtol=1e-14)
    # one dominant key
    K = rng.normal(0, 0.01, (50, 2, 8))
    K[17] = 1e3 * q[[0, 2]]
    o = attention.decode(q, K, V, 1.0)
    assert np.allclose(o[[0, 2]], V[17], atol=1e-12)


def test_split_merge_equals_softmax():
    rng = np.random.default_rng(33)
    s = rng.normal(0, 3, 1000)
    Vg = rng.normal(0, 1, (1000, 16))
    w = np.exp(s - s.max())
    ref = (w / w.sum()) @ Vg
    for P in (1, 3, 16, 128):
        cuts = np.linspace(0, 1000, P + 1).astype(int)
        bounds = list(zip(cuts[:-1], cuts[1:]))
        got = attention.merge_partials(attention.split_partials(s, Vg, bounds))
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-15)
    # empty splits contribute nothing
    got = attention.merge_partials(attention.split_partials(s, Vg, [(0, 500), (500, 500), (500, 1000)]))
    assert np.allclose(got, ref, rtol=1e-12)


def test_prefill_rows_equal_decode_at_their_length():
    rng = np.random.default_rng(34)
    K = rng.normal(0, 1, (40, 2, 8))
    V = rng.normal(0, 1, (40, 2, 8))
    q = rng.normal(0, 1, (6, 4, 8))
    out = attention.prefill(q, K, V, 0.35, q_start=34)
    for i in range(6):
        assert np.allclose(out[i], attention.decode(q[i], K[:35 + i], V[:35 + i], 0.35), rtol=1e-14)


def test_planted_rank():
    s = np.array([0.1, 3.0, 2.0, 3.0, -1.0])
    assert attention.planted_rank(s, 1) == 1       # tie with index 3 counts in its favour
    assert attention.planted_rank(s, 2) == 3
    assert attention.planted_rank(s, 4) == 5


def test_flat_attention_at_131072_keeps_all_mass():
    """Identical keys over 131072 tokens: fp64 softmax keeps the whole mass (the
    bf16 register of the flat-sum table would keep 0.001953 of it)."""
    T = 131072
    s = np.zeros(T)
    w = np.exp(s - s.max())
    assert abs(w.sum() / T - 1.0) < 1e-15
    Vg = np.ones((T, 1))
    o = attention.merge_partials(attention.split_partials(s, Vg, [(0, T // 2), (T // 2, T)]))
    assert abs(o[0] - 1.0) < 1e-14


def test_c0_pipeline_oracle_runs():
    w, k, v = _c0_rows()
    K, V = pool.dequantized_rows("q2", k, v)
    q = queries(w, 0, 1)[0].float().numpy()
    o = attention.decode(q, K, V, w.sm_scale)
    assert o.shape == (16, 256) and np.all(np.isfinite(o))


def test_scores_gqa_head_mapping_closed_form():
    """Query head h reads KV head h // G: with K[t, g] = (g + 1) * ones and
    q_h = ones, every score of head h is sm * D * (h // G + 1).  Reading
    KV head h % Hkv instead, or the wrong axis, changes the values."""
    T, Hkv, G, D, sm = 5, 2, 4, 8, 0.3
    K = np.stack([np.full((T, D), g + 1.0) for g in range(Hkv)], axis=1)
    q = np.ones((Hkv * G, D))
    s = attention.scores(q, K, sm)
    assert s.shape == (Hkv * G, T)
    for h in range(Hkv * G):
        assert np.all(s[h] == sm * D * (h // G + 1))


def test_scores_against_basis_keys_and_parallel_keys():
    """Keys that are the unit vectors e_t give scores sm * q_h[t] (the query
    row itself, so a transposed operand fails); keys c_t * q_h give
    sm * c_t * |q_h|^2."""
    rng = np.random.default_rng(31)
    D, sm = 6, 0.125
    q = rng.standard_normal((2, D))                     # Hq = 2, Hkv = 1
    K = np.eye(D)[:, None, :]                           # [T = D][1][D]
    s = attention.scores(q, K, sm)
    assert np.array_equal(s, sm * q)
    c = np.array([0.5, -2.0, 3.0])
    K2 = (c[:, None] * q[0][None, :])[:, None, :]       # three keys parallel to q_0
    s2 = attention.scores(q[:1], K2, sm)[0]
    assert np.allclose(s2, sm * c * np.dot(q[0], q[0]), rtol=1e-15, atol=0)


def test_scores_give_the_decode_weights():
    """softmax of the raw logits, applied to V, is the decode output (decode
    itself is pinned by its own closed forms above)."""
    w, k, v = _c0_rows(200)
    q = queries(w, 0, 1)[0].float().numpy()
    K, V = pool.dequantized_rows("q2", k, v)
    s = attention.scores(q, K, w.sm_scale)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    G = w.group
    out = np.stack([p[h] @ np.asarray(V[:, h // G], np.float64) for h in range(w.n_q_heads)])
    assert np.allclose(out, attention.decode(q, K, V, w.sm_scale), rtol=1e-12, atol=1e-14)


def test_planted_rank_counts_strictly_higher_scores():
    s = np.array([0.1, 0.5, 0.5, 0.3])
    assert attention.planted_rank(s, 1) == 1   # tied with slot 2: ties favour the planted key
    assert attention.planted_rank(s, 2) == 1
    assert attention.planted_rank(s, 3) == 3   # 0.5 and 0.5 above it
    assert attention.planted_rank(s, 0) == 4


@pytest.mark.parametrize("fmt,D", [("q2", 256), ("q2", 128), ("q8", 128), ("q8", 256)])
def test_sequence_blocks_equal_the_token_by_token_pool(fmt, D):
    """The whole-sequence page images equal the pool image that appends one
    token at a time (OraclePool), block by block."""
    w, k, v = _c0_rows(192)
    k, v = k[..., :D].copy(), v[..., :D].copy()
    H = k.shape[1]
    bt = np.array([2, 0, 1], np.int32)
    p = pool.OraclePool(fmt, 2, H, D, 3, fill=0x3C)
    start = 0
    for n in (70, 1, 57, 64):
        p.append(1, 0, bt, start, k[start:start + n], v[start:start + n])
        start += n
    blocks = pool.sequence_blocks(fmt, k, v)
    assert blocks.shape == (3, H, layout.block_bytes(fmt, D))
    bb = layout.block_bytes(fmt, D)
    for lp in range(3):
        for h in range(H):
            off = (1 * H + h) * bb                       # layer 1
            assert np.array_equal(p.data[bt[lp], off:off + bb], blocks[lp, h]), (lp, h)


def test_prefill_dense_equals_the_row_loop():
    rng = np.random.default_rng(41)
    n, T0, Hq, Hkv, D = 9, 23, 4, 2, 16
    q = rng.standard_normal((n, Hq, D))
    K = rng.standard_normal((T0 + n, Hkv, D))
    V = rng.standard_normal((T0 + n, Hkv, D))
    a = attention.prefill(q, K, V, 0.25, T0)
    b = attention.prefill_dense(q, K, V, 0.25, T0)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)
