"""Oracle pins: page layout (packing) against loop references and byte totals."""

import numpy as np

from oracle import accounting, layout


def _pack_loop(codes):
    n = len(codes)
    out = []
    for b in range(n // 4):
        v = 0
        for j in range(4):
            v |= int(codes[4 * b + j]) << (2 * j)
        out.append(v)
    return out


def test_pack2_matches_loop():
    rng = np.random.default_rng(21)
    for n in (64, 128, 256):
        c = rng.integers(0, 4, (5, n)).astype(np.uint8)
        p = layout.pack2(c)
        for r in range(5):
            assert list(p[r]) == _pack_loop(c[r])
        assert np.array_equal(layout.unpack2(p, n), c)


def test_block_sizes_match_token_bytes():
    for L, H, D in ((16, 4, 256), (1, 4, 256), (2, 2, 128)):
        assert L * H * layout.q2_block_bytes(D) == accounting.page_bytes("q2", L, H, D)
    assert 32 * 8 * layout.q8_block_bytes(128) == accounting.page_bytes("q8", 32, 8, 128)
    assert layout.q2_block_bytes(256) == 2 * 64 * 72  # K and V rows of 64 tokens
    for L, H, D in ((16, 4, 256), (32, 8, 128)):
        assert L * H * layout.bf16_block_bytes(D) == accounting.page_bytes("bf16", L, H, D)
    assert layout.bf16_block_bytes(256) == 2 * 64 * 512  # the page's 512 B per head per token


def test_v_plane_write_touches_only_its_slot():
    buf = np.full(layout.q2_block_bytes(256), 0xA5, np.uint8)
    blk = layout.Q2Block(buf, 256)
    rng = np.random.default_rng(22)
    before = buf.copy()
    c = rng.integers(0, 4, 256).astype(np.uint8)
    blk.write_v(37, c, np.float32(0.5), np.float32(-1.0))
    codes = layout.unpack2_vrow(blk.v_codes)            # [D][64]
    old = layout.unpack2_vrow(before[16 * 256:32 * 256].reshape(256, 16))
    assert np.array_equal(codes[:, 37], c)
    mask = np.ones(64, bool)
    mask[37] = False
    assert np.array_equal(codes[:, mask], old[:, mask])
    assert np.array_equal(buf[:16 * 256], before[:16 * 256])  # K plane untouched


def test_k_row_layout_positions():
    buf = np.zeros(layout.q2_block_bytes(128), np.uint8)
    blk = layout.Q2Block(buf, 128)
    c = np.zeros(128, np.uint8)
    c[5] = 3  # dim 5 -> byte 1, bits 2..3
    blk.write_k(2, c, np.float32(1.0), np.float32(0.0))
    row_off = 2 * 128 // 4
    assert buf[row_off + 1] == 3 << 2 and buf[row_off:row_off + 32].sum() == 12
    assert np.frombuffer(buf[32 * 128 + 16:32 * 128 + 24].tobytes(), np.float32).tolist() == [1.0, 0.0]


def test_v_row_word_layout_matches_loop():
    """slot 16b + 4w + r sits in word w at bit 16(r % 2) + 4b + 2(r // 2)."""
    rng = np.random.default_rng(23)
    c = rng.integers(0, 4, (7, 64)).astype(np.uint8)
    p = layout.pack2_vrow(c)
    for r in range(7):
        for w in range(4):
            word = 0
            for b in range(4):
                for q in range(4):
                    word |= int(c[r, 16 * b + 4 * w + q]) << (16 * (q % 2) + 4 * b + 2 * (q // 2))
            assert int.from_bytes(bytes(p[r, 4 * w:4 * w + 4]), "little") == word
            # nibble n of the 0x33333333 mask: slot 16 (n % 4) + 4w + n // 4 (r in {0, 1})
            lo = [(word >> (4 * n)) & 3 for n in range(8)]
            assert lo == [c[r, 16 * (n % 4) + 4 * w + n // 4] for n in range(8)]
            hi = [(word >> (4 * n + 2)) & 3 for n in range(8)]
            assert hi == [c[r, 16 * (n % 4) + 4 * w + 2 + n // 4] for n in range(8)]
    assert np.array_equal(layout.unpack2_vrow(p), c)
    # every (word, bit) pair is used by exactly one slot
    assert len({layout.v_slot_word_bit(s) for s in range(64)}) == 64


def test_v_plane_word_offsets_tile_the_plane():
    for D in (128, 256):
        offs = sorted(layout.v_word_offset(D, d, w) for d in range(D) for w in range(4))
        assert offs == list(range(0, 16 * D, 4))
        for d in range(D):
            if d % 32 < 16:
                for half in (0, 1):
                    a = layout.v_word_offset(D, d, 2 * half)
                    assert layout.v_word_offset(D, d, 2 * half + 1) == a + 4
                    assert layout.v_word_offset(D, d + 16, 2 * half) == a + 8  # dims d, d+16 adjacent
