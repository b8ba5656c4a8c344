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


def _golden_rows(golden, kind):
    return [r[1:] for r in golden("layout_cases.txt") if r[0] == kind]


def test_hand_derived_code_positions(golden):
    """One code in an all-zero block sets exactly the byte worked out by hand
    in tests/golden/layout_cases.txt (independently of the oracle's index
    arithmetic)."""
    rows = _golden_rows(golden, "code")
    assert len(rows) >= 10
    for fmt, D, plane, slot, dim, code, byte, value, *_ in rows:
        D, slot, dim, code, byte, value = int(D), int(slot), int(dim), int(code), int(byte), int(value, 16)
        if fmt == "q2":
            buf = np.zeros(layout.q2_block_bytes(D), np.uint8)
            blk = layout.Q2Block(buf, D)
            row = np.zeros(D, np.uint8)
            row[dim] = code
            (blk.write_k if plane == "K" else blk.write_v)(slot, row, np.float32(0), np.float32(0))
        else:
            buf = np.zeros(layout.q8_block_bytes(D), np.uint8)
            blk = layout.Q8Block(buf, D)
            if plane == "K":
                blk.k_codes[slot, dim] = code
            else:
                blk.v_codes[dim, slot] = code
        nz = np.nonzero(buf)[0]
        assert list(nz) == [byte], (fmt, D, plane, slot, dim, list(nz))
        assert int(buf[byte]) == value


def test_hand_derived_metadata_positions(golden):
    for fmt, D, field, slot, scale, mn, off, hexbytes, *_ in _golden_rows(golden, "meta"):
        D, slot, off = int(D), int(slot), int(off)
        buf = np.zeros(layout.q2_block_bytes(D), np.uint8)
        blk = layout.Q2Block(buf, D)
        (blk.write_k if field == "K" else blk.write_v)(slot, np.zeros(D, np.uint8), np.float32(scale), np.float32(mn))
        assert buf[off:off + 8].tobytes().hex() == hexbytes
        assert np.count_nonzero(buf) == np.count_nonzero(np.frombuffer(bytes.fromhex(hexbytes), np.uint8))
    for fmt, D, field, idx, x, off, hexbytes, *_ in _golden_rows(golden, "scale"):
        D, idx, off = int(D), int(idx), int(off)
        buf = np.zeros(layout.q8_block_bytes(D), np.uint8)
        blk = layout.Q8Block(buf, D)
        (blk.k_scale if field == "K" else blk.v_scale)[idx] = np.float32(x)
        assert buf[off:off + 4].tobytes().hex() == hexbytes
        assert np.count_nonzero(buf) == np.count_nonzero(np.frombuffer(bytes.fromhex(hexbytes), np.uint8))


def test_block_image_is_frozen():
    """The whole 2-bit block image of a fixed code pattern equals the stored
    vector (tests/golden/q2_block_d128.hex, written by
    tests/golden/make_layout_golden.py through the oracle): a change of the
    block format anywhere shows as a difference here."""
    import importlib.util
    import os
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    spec = importlib.util.spec_from_file_location("make_layout_golden", os.path.join(here, "make_layout_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    buf = mod.pattern_block()
    stored = bytearray()
    with open(os.path.join(here, "q2_block_d128.hex")) as f:
        for line in f:
            if line.startswith("#"):
                continue
            off, hx = line.split()
            assert int(off) == len(stored)
            stored += bytes.fromhex(hx)
    assert bytes(stored) == buf.tobytes()
    # spot checks by hand: K row 0 of codes (0, 3, 2, 1, ...) packs to 0x6c;
    # K metadata of slot 1 is (2.0, -0.125)
    assert stored[0] == 0 | 3 << 2 | 2 << 4 | 1 << 6 == 0x6C
    assert np.frombuffer(bytes(stored[32 * 128 + 8:32 * 128 + 16]), np.float32).tolist() == [2.0, -0.125]
