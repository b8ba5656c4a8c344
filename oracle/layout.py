"""Byte layout of a pool page, written out as plain packing loops.

A page holds 64 tokens of every layer and every KV head ("Pages hold 64
tokens", KV at 9 KB a token, How it works; one ``kv_page_bytes`` figure per
pool, section "See it, control it").  Inside a page, the data of one
(layer, KV head) pair is one contiguous block at
``((layer * Hkv) + head) * block_bytes``.

2-bit block (D dims; 72 B per token per head at D = 256, as the page's table):
    [0,        16*D)   K codes, token-major: row t (D/4 bytes) at t*D/4
    [16*D,     32*D)   V codes, dim-major, in two halves of 32 token slots
    [32*D,     32*D+512)  K metadata: 64 x [fp32 scale, fp32 min]
    [32*D+512, 32*D+1024) V metadata: 64 x [fp32 scale, fp32 min]
  K rows pack dims least-significant-bits first: dim j sits in byte j // 4 at
  bit 2 * (j % 4).  The V codes of a dim are four 32-bit little-endian words;
  token slot s = 16b + 4w + r (b = s // 16, w = (s // 4) % 4, r = s % 4) sits
  in word w at bits 16 * (r % 2) + 4 * b + 2 * (r // 2).  Masking a word with
  0x33333333 therefore yields the eight slots with r in {0, 1}, one per 4-bit
  nibble, and masking it shifted right by two the eight slots with r in {2, 3}.
  Words 0-1 of every dim form the first half of the V plane, words 2-3 the
  second; inside a half the 8 bytes of dims d and d + 16 (d % 32 < 16) are
  adjacent, so the 8-byte pieces of dim d sit at
  half * 8D + 16 * (16 * (d // 32) + d % 16) + 8 * ((d // 16) % 2).

8-bit block (D dims):
    [0,      64*D)   K codes int8, token-major: row t at t*D
    [64*D,  128*D)   V codes int8, dim-major:   row d (64 bytes) at 64*d
    [128*D, 132*D)   K scales: fp32 per channel (one set per page)
    [132*D, 132*D+256) V scales: fp32 per token slot

bf16 block (D dims; 512 B per head per token, the BF16 row of the page's
table, so 65,536 B a token at the 27B geometry):
    [0,       128*D)  K, bf16 bit patterns, token-major: row t (2D bytes) at 2*D*t
    [128*D,   256*D)  V, bf16 bit patterns, dim-major:   row d (128 bytes) at 128*d
  The exact cache the pages compare every compressed format against, kept in
  the same paged pool so that the same gather reads it.

The arrangement inside a block is not fixed by the pages (they give only the
bytes per head per token); the byte totals match them exactly.  Pinned by
closed forms: block sizes reproduce 9,216 B/token at the 27B geometry and the
pack/unpack pair is checked element by element on seeded codes with a loop
reference in tests/test_oracle_layout.py.
"""

from __future__ import annotations

import numpy as np

PAGE = 64


def q2_block_bytes(D: int) -> int:
    return 32 * D + 1024


def q8_block_bytes(D: int) -> int:
    return 132 * D + 256


def bf16_block_bytes(D: int) -> int:
    return 256 * D


def block_bytes(fmt: str, D: int) -> int:
    if fmt == "q2":
        return q2_block_bytes(D)
    if fmt == "q8":
        return q8_block_bytes(D)
    if fmt == "bf16":
        return bf16_block_bytes(D)
    raise ValueError(fmt)


def block_offset(fmt: str, layer: int, head: int, n_kv_heads: int, D: int) -> int:
    return (layer * n_kv_heads + head) * block_bytes(fmt, D)


# --------------------------------------------------------- 2-bit packing --

def pack2(codes) -> np.ndarray:
    """codes uint8 [..., n] in 0..3 (n % 4 == 0) -> bytes [..., n/4], element j at bits 2*(j%4) of byte j//4."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 4 == 0 and c.max(initial=0) <= 3
    g = c.reshape(c.shape[:-1] + (c.shape[-1] // 4, 4)).astype(np.uint32)
    b = g[..., 0] | (g[..., 1] << 2) | (g[..., 2] << 4) | (g[..., 3] << 6)
    return b.astype(np.uint8)


def v_slot_word_bit(slot: int):
    """(word, bit) of token slot ``slot`` (0..63) in a dim's four V-code words."""
    b, w, r = slot // 16, (slot // 4) % 4, slot % 4
    return w, 16 * (r % 2) + 4 * b + 2 * (r // 2)


def pack2_vrow(codes) -> np.ndarray:
    """codes uint8 [..., 64] (token slots) -> bytes [..., 16] in the V-row word layout."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] == 64 and c.max(initial=0) <= 3
    words = np.zeros(c.shape[:-1] + (4,), dtype=np.uint32)
    for s in range(64):
        w, bit = v_slot_word_bit(s)
        words[..., w] |= c[..., s].astype(np.uint32) << np.uint32(bit)
    return np.ascontiguousarray(words).view(np.uint8).reshape(c.shape[:-1] + (16,))


def unpack2_vrow(packed) -> np.ndarray:
    p = np.ascontiguousarray(np.asarray(packed, dtype=np.uint8))
    words = p.view(np.uint32).reshape(p.shape[:-1] + (4,))
    out = np.empty(p.shape[:-1] + (64,), dtype=np.uint8)
    for s in range(64):
        w, bit = v_slot_word_bit(s)
        out[..., s] = (words[..., w] >> np.uint32(bit)) & 3
    return out


def unpack2(packed, n: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    assert p.shape[-1] * 4 == n
    out = np.empty(p.shape[:-1] + (n,), dtype=np.uint8)
    for j in range(4):
        out[..., j::4] = (p >> (2 * j)) & 3
    return out


def v_word_offset(D: int, d: int, w: int) -> int:
    """Byte offset, inside the V plane, of word w (slots 16w..16w+15) of dim d."""
    half, word = w // 2, w % 2
    return half * 8 * D + 16 * (16 * (d // 32) + d % 16) + 8 * ((d // 16) % 2) + 4 * word


def v_plane_index(D: int) -> np.ndarray:
    """[D][16] byte indices into the V plane: row d lists dim d's 16 bytes in slot order."""
    idx = np.empty((D, 16), dtype=np.int64)
    for d in range(D):
        for w in range(4):
            o = v_word_offset(D, d, w)
            idx[d, 4 * w:4 * w + 4] = np.arange(o, o + 4)
    return idx


class _VRows:
    """[D][16] view of a V plane: row d = dim d's four words in slot order (a gather/scatter)."""

    def __init__(self, plane: np.ndarray, D: int):
        self.plane, self.idx = plane, v_plane_index(D)

    def __getitem__(self, key):
        return self.plane[self.idx][key]

    def __setitem__(self, key, value):
        rows = self.plane[self.idx]
        rows[key] = value
        self.plane[self.idx] = rows

    def __array__(self, dtype=None, copy=None):
        a = self.plane[self.idx]
        return a if dtype is None else a.astype(dtype)


class Q2Block:
    """Views into one 2-bit (layer, head) block of a page (a uint8 array of block_bytes)."""

    def __init__(self, buf: np.ndarray, D: int):
        assert buf.dtype == np.uint8 and buf.size == q2_block_bytes(D)
        self.D = D
        self.k_codes = buf[0:16 * D].reshape(PAGE, D // 4)
        self.v_codes = _VRows(buf[16 * D:32 * D], D)
        self.k_meta = buf[32 * D:32 * D + 512].view(np.float32).reshape(PAGE, 2)
        self.v_meta = buf[32 * D + 512:32 * D + 1024].view(np.float32).reshape(PAGE, 2)

    def write_k(self, slot: int, codes_row, scale, mn):
        self.k_codes[slot] = pack2(codes_row)
        self.k_meta[slot] = (scale, mn)

    def write_v(self, slot: int, codes_row, scale, mn):
        """Set the 2 bits of token ``slot`` in every dim row, leaving other slots untouched."""
        w, bit = v_slot_word_bit(slot)
        byte, shift = 4 * w + bit // 8, bit % 8
        keep = np.uint8(0xFF ^ (3 << shift))
        col = self.v_codes[:, byte]
        self.v_codes[:, byte] = (col & keep) | (np.asarray(codes_row, np.uint8) << shift)
        self.v_meta[slot] = (scale, mn)

    def read_k(self, n: int):
        codes = unpack2(self.k_codes[:n], self.D)
        return codes, self.k_meta[:n, 0].copy(), self.k_meta[:n, 1].copy()

    def read_v(self, n: int):
        codes = unpack2_vrow(np.asarray(self.v_codes))[:, :n].T.copy()   # [n][D]
        return codes, self.v_meta[:n, 0].copy(), self.v_meta[:n, 1].copy()


class Q8Block:
    """Views into one 8-bit (layer, head) block of a page."""

    def __init__(self, buf: np.ndarray, D: int):
        assert buf.dtype == np.uint8 and buf.size == q8_block_bytes(D)
        self.D = D
        self.k_codes = buf[0:64 * D].view(np.int8).reshape(PAGE, D)
        self.v_codes = buf[64 * D:128 * D].view(np.int8).reshape(D, PAGE)
        self.k_scale = buf[128 * D:132 * D].view(np.float32)
        self.v_scale = buf[132 * D:132 * D + 256].view(np.float32)

    def read_k(self, n: int):
        return self.k_codes[:n].copy(), self.k_scale.copy()

    def read_v(self, n: int):
        return self.v_codes[:, :n].T.copy(), self.v_scale[:n].copy()


class Bf16Block:
    """Views into one bf16 (layer, head) block of a page: bit patterns, no metadata."""

    def __init__(self, buf: np.ndarray, D: int):
        assert buf.dtype == np.uint8 and buf.size == bf16_block_bytes(D)
        self.D = D
        self.k = buf[0:128 * D].view(np.uint16).reshape(PAGE, D)
        self.v = buf[128 * D:256 * D].view(np.uint16).reshape(D, PAGE)

    def read_k(self, n: int):
        return self.k[:n].copy()

    def read_v(self, n: int):
        return self.v[:, :n].T.copy()
