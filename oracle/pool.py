"""A byte image of the page pool on the host, with append and gather.

Follows "KV at 9 KB a token" (How it works: fixed-size 64-token pages, a pool
that is a byte budget) and "The KV cache and prompt reuse" (What a sequence is
made of: one pool shared by all lanes; the most recent keys, which the
compressed format holds unquantized).  A sequence owns a block table: logical page i of the
sequence lives in physical page ``bt[i]``; token t sits in slot t % 64 of page
``bt[t // 64]``.

append writes each new token's K and V rows quantized into its slot, leaving
every other slot of the pool untouched.  The bf16 format stores the rows as
they come (their bf16 bit patterns): the exact cache the pages measure the
compressed formats against, read through the same block tables.  For the 8-bit variant, K is scaled per
channel over the tokens present in the open page; the exact K rows of that page
are kept aside (the exact window), and each append re-derives the page's K codes
and scales from the exact rows present, so a full page equals the plain
per-channel quantization of its 64 tokens.

The rotated 2-bit variant ("q2r") stores the 2-bit rows of H k (H the
unnormalised Walsh-Hadamard matrix, applied in fp32 butterflies) and V as the
2-bit format does; its gather returns H k^_r / D in fp64, the dequantized K
rows back in the original basis, so attention over it is the plain attention
of the other formats.  Only K is rotated: its outliers are channels, which the
rotation spreads over the row, while V's are whole tokens, which a per-token
range already absorbs ("Half the Cache, Twice the Context", section "What the
cache loses when you round it": persistent key-channel outliers, value-token
outliers).

A fork gives a new sequence the first n tokens of another: the whole pages
of that prefix are shared (both block tables name them), the page it only
partly fills is copied whole into a page of the child's, with the exact rows
kept for it.

The 2-bit format with an exact window ("q2w") keeps, besides the 2-bit pages,
the exact rows of the last page a (sequence, layer) has appended to: the
recent keys that "The KV cache and prompt reuse" (What a sequence is made of)
has the compressed format hold unquantized, read here as one page.
With A tokens appended, every reader sees tokens 64 * floor((A - 1) / 64) ..
A - 1 exact and every earlier token through the 2-bit codec; the pages
themselves hold exactly what a plain 2-bit pool holds.  Appends are then
sequential per (sequence, layer), since only the last page's rows are kept.

Pins: append-then-gather returns exactly the codec's dequantized rows for any
block table (permutation invariance) and slots outside the appended range keep
their fill bytes (tests/test_oracle_pool_attention.py); the window format's
body equals a plain 2-bit pool byte for byte, its last page reads back as the
appended rows, a sequence within one page attends exactly as a loop over the
input rows does, and the window moves when a new page opens
(tests/test_oracle_window.py).
"""

from __future__ import annotations

import numpy as np

from . import bf16, codec, layout
from .accounting import page_bytes
from .layout import PAGE, Bf16Block, Q2Block, Q8Block, block_bytes, block_offset


class OraclePool:
    def __init__(self, fmt: str, n_layers: int, n_kv_heads: int, head_dim: int, n_pages: int, fill: int = 0xA5):
        assert fmt in ("q2", "q8", "bf16", "q2w", "q2r")
        self.fmt, self.L, self.H, self.D = fmt, n_layers, n_kv_heads, head_dim
        # the window and rotated formats' pages are 2-bit pages
        self.page_fmt = "q2" if fmt in ("q2w", "q2r") else fmt
        self.page_bytes = page_bytes(self.page_fmt, n_layers, n_kv_heads, head_dim)
        self.data = np.full((n_pages, self.page_bytes), fill, dtype=np.uint8)
        self._exact_k = {}  # (seq, layer) -> fp32 [64][H][D] exact K rows of the open page (8-bit only)
        # q2w: (seq, layer) -> (tokens appended A, exact K and V fp32 [64][H][D] of page (A - 1) // 64)
        self._window = {}

    def block(self, page: int, layer: int, head: int):
        off = block_offset(self.page_fmt, layer, head, self.H, self.D)
        buf = self.data[page, off:off + block_bytes(self.page_fmt, self.D)]
        return {"q2": Q2Block, "q8": Q8Block, "bf16": Bf16Block}[self.page_fmt](buf, self.D)

    # ------------------------------------------------------------ append --
    def append(self, layer: int, seq: int, bt, start: int, k_rows, v_rows):
        """Quantize-append rows k_rows/v_rows [n][H][D] (fp32 values of bf16) at positions start..start+n-1."""
        k = np.asarray(k_rows, np.float32)
        v = np.asarray(v_rows, np.float32)
        n = k.shape[0]
        if n == 0:
            return
        assert k.shape == (n, self.H, self.D) and v.shape == k.shape
        if self.fmt == "bf16":
            kb, vb = bf16.f32_to_bits(k), bf16.f32_to_bits(v)
            for i in range(n):
                pos = start + i
                page, slot = int(bt[pos // PAGE]), pos % PAGE
                for h in range(self.H):
                    blk = self.block(page, layer, h)
                    blk.k[slot] = kb[i, h]
                    blk.v[:, slot] = vb[i, h]
            return
        if self.fmt == "q2w":
            self._append_window(layer, seq, start, k, v)
        if self.fmt == "q2r":   # the rotated variant stores the 2-bit codes of H k (V as in 2-bit)
            bf16.f32_to_bits(k)
            k = codec.hadamard_rows(k)
        if self.page_fmt == "q2":
            ck, sk, mk = codec.q2_quantize(k)
            cv, sv, mv = codec.q2_quantize(v)
            for i in range(n):
                pos = start + i
                page, slot = int(bt[pos // PAGE]), pos % PAGE
                for h in range(self.H):
                    blk = self.block(page, layer, h)
                    blk.write_k(slot, ck[i, h], sk[i, h], mk[i, h])
                    blk.write_v(slot, cv[i, h], sv[i, h], mv[i, h])
            return
        # 8-bit: V per token; K per channel over the open page's exact rows
        cv, sv = codec.q8_quantize_v(v)
        for i in range(n):
            pos = start + i
            page, slot = int(bt[pos // PAGE]), pos % PAGE
            for h in range(self.H):
                blk = self.block(page, layer, h)
                blk.v_codes[:, slot] = cv[i, h]
                blk.v_scale[slot] = sv[i, h]
        pos, end = start, start + n
        while pos < end:
            lp = pos // PAGE
            page_end = min(end, (lp + 1) * PAGE)
            key = (seq, layer)
            if pos % PAGE == 0 or key not in self._exact_k:
                exact = np.zeros((PAGE, self.H, self.D), np.float32)
                if pos % PAGE != 0:
                    raise ValueError("8-bit append into a page whose exact rows were not kept")
            else:
                exact = self._exact_k[key]
            exact[pos % PAGE:page_end - lp * PAGE] = k[pos - start:page_end - start]
            present = page_end - lp * PAGE
            codes, scales = codec.q8_quantize_k_page(exact[:present])
            page = int(bt[lp])
            for h in range(self.H):
                blk = self.block(page, layer, h)
                blk.k_codes[:present] = codes[:, h]
                blk.k_scale[:] = scales[h]
            self._exact_k[key] = exact
            pos = page_end

    def _append_window(self, layer: int, seq: int, start: int, k, v):
        """Keep the exact rows of the last page this append reaches."""
        bf16.f32_to_bits(k), bf16.f32_to_bits(v)  # the rows must be bf16 numbers
        appended, wk, wv = self._window.get((seq, layer), (0, None, None))
        if start != appended:
            raise ValueError(f"window appends are sequential: {appended} tokens held, append starts at {start}")
        end = start + k.shape[0]
        last = (end - 1) // PAGE
        if appended == 0 or (appended - 1) // PAGE != last:
            wk = np.zeros((PAGE, self.H, self.D), np.float32)
            wv = np.zeros_like(wk)
        lo = max(start, last * PAGE)
        wk[lo - last * PAGE:end - last * PAGE] = k[lo - start:]
        wv[lo - last * PAGE:end - last * PAGE] = v[lo - start:]
        self._window[(seq, layer)] = (end, wk, wv)

    def window_start(self, layer: int, seq: int) -> int:
        """First position read exactly (q2w): 64 * floor((A - 1) / 64) with A tokens appended."""
        appended = self._window[(seq, layer)][0]
        return PAGE * ((appended - 1) // PAGE)

    # -------------------------------------------------------------- fork --
    def fork(self, parent: int, parent_bt, child: int, child_bt, n: int):
        """A child sequence that starts with the parent's first n tokens.

        Its whole pages (logical pages below n // 64) are the parent's pages,
        shared: child_bt must name the same physical pages there.  A page the
        prefix only partly fills is copied whole into the child's own page
        (copy on write), so the child can append into it; the tokens the copy
        holds past n are never read by the child before it overwrites them.
        The exact rows kept for the open page (8-bit K window, 2-bit window)
        are copied with it, as the child's, with n tokens appended.  Follows
        "The KV cache and prompt reuse" (What a sequence is made of: a lane is
        charged for the pages it holds; full pages of a shared prefix are
        reused, the page being written is not)."""
        full = n // PAGE
        if list(map(int, child_bt[:full])) != list(map(int, parent_bt[:full])):
            raise ValueError("the child's whole prefix pages must be the parent's pages")
        if n % PAGE:
            src, dst = int(parent_bt[full]), int(child_bt[full])
            if src == dst:
                raise ValueError("the partly filled page must be copied, not shared")
            self.data[dst] = self.data[src]
        for layer in range(self.L):
            if self.fmt == "q2w":
                appended, wk, wv = self._window[(parent, layer)]
                if (n - 1) // PAGE != (appended - 1) // PAGE or n > appended:
                    raise ValueError("a window fork must end in the parent's last page")
                self._window[(child, layer)] = (n, wk.copy(), wv.copy())
            elif self.fmt == "q8" and n % PAGE:
                if (parent, layer) not in self._exact_k:
                    raise ValueError("the parent's open page was not appended")
                self._exact_k[(child, layer)] = self._exact_k[(parent, layer)].copy()

    # ------------------------------------------------------------ gather --
    def gather(self, layer: int, bt, ctx_len: int, seq: int = None):
        """Dequantized K^ and V^ [ctx_len][H][D] (fp32) read through the block table.

        The window format also needs the sequence: its tokens from the window
        start up to ctx_len (at most the tokens appended) are the exact rows."""
        if self.fmt == "q2r":   # dequantized rotated K rows, back in the original basis (fp64)
            K, V = self._gather_pages(layer, bt, ctx_len)
            return codec.unrotate_rows(K), V
        if self.fmt == "q2w":
            appended, wk, wv = self._window[(seq, layer)]
            if ctx_len > appended:
                raise ValueError(f"ctx_len {ctx_len} beyond the {appended} tokens appended")
            K, V = self._gather_pages(layer, bt, ctx_len)
            w0 = self.window_start(layer, seq)
            if ctx_len > w0:
                K[w0:ctx_len] = wk[:ctx_len - w0]
                V[w0:ctx_len] = wv[:ctx_len - w0]
            return K, V
        return self._gather_pages(layer, bt, ctx_len)

    def _gather_pages(self, layer: int, bt, ctx_len: int):
        K = np.empty((ctx_len, self.H, self.D), np.float32)
        V = np.empty_like(K)
        for lp in range(-(-ctx_len // PAGE)):
            n = min(PAGE, ctx_len - lp * PAGE)
            page = int(bt[lp])
            for h in range(self.H):
                blk = self.block(page, layer, h)
                if self.fmt == "bf16":
                    K[lp * PAGE:lp * PAGE + n, h] = bf16.bits_to_f32(blk.read_k(n))
                    V[lp * PAGE:lp * PAGE + n, h] = bf16.bits_to_f32(blk.read_v(n))
                elif self.page_fmt == "q2":
                    c, s, m = blk.read_k(n)
                    K[lp * PAGE:lp * PAGE + n, h] = codec.q2_dequantize(c, s, m)
                    c, s, m = blk.read_v(n)
                    V[lp * PAGE:lp * PAGE + n, h] = codec.q2_dequantize(c, s, m)
                else:
                    c, s = blk.read_k(n)
                    K[lp * PAGE:lp * PAGE + n, h] = codec.q8_dequantize(c, s[None, :])
                    c, s = blk.read_v(n)
                    V[lp * PAGE:lp * PAGE + n, h] = codec.q8_dequantize(c, s[:, None])
        return K, V


def dequantized_rows(fmt: str, k_rows, v_rows):
    """K^, V^ of a whole sequence quantized page by page, without a pool image.

    Same arithmetic as append + gather for a sequence appended from position 0
    (used for the large workloads, where a full pool image does not fit).
    """
    k = np.asarray(k_rows, np.float32)
    v = np.asarray(v_rows, np.float32)
    if fmt == "bf16":
        bf16.f32_to_bits(k), bf16.f32_to_bits(v)  # the rows must be bf16 numbers
        return k.copy(), v.copy()
    if fmt == "q2r":
        bf16.f32_to_bits(k), bf16.f32_to_bits(v)
        K = codec.unrotate_rows(codec.q2_dequantize(*codec.q2_quantize(codec.hadamard_rows(k))))
        V = codec.q2_dequantize(*codec.q2_quantize(v))
        return K, V
    if fmt in ("q2", "q2w"):
        K = codec.q2_dequantize(*codec.q2_quantize(k))
        V = codec.q2_dequantize(*codec.q2_quantize(v))
        if fmt == "q2w":  # the last page holds the exact rows
            bf16.f32_to_bits(k), bf16.f32_to_bits(v)
            w0 = PAGE * ((k.shape[0] - 1) // PAGE)
            K[w0:] = k[w0:]
            V[w0:] = v[w0:]
        return K, V
    cv, sv = codec.q8_quantize_v(v)
    V = codec.q8_dequantize(cv, sv[..., None])
    K = np.empty_like(k)
    for p0 in range(0, k.shape[0], PAGE):
        c, s = codec.q8_quantize_k_page(k[p0:p0 + PAGE])
        K[p0:p0 + PAGE] = codec.q8_dequantize(c, s[None])
    return K, V


def sequence_blocks(fmt: str, k_rows, v_rows):
    """Byte images of the (layer, KV head) blocks of a sequence appended from
    position 0 in whole pages: [T / 64][H][block_bytes] uint8 for rows
    k_rows, v_rows [T][H][D] (fp32 values of bf16, T a multiple of 64).

    The same codec and layout as OraclePool.append (the 2-bit codec and its
    block layout; the 8-bit codec with K per channel over each page's 64
    tokens and V per token), applied to all pages at once, so that whole pools
    of the large workloads can be checked byte for byte.  Pinned against
    OraclePool's token-by-token image in tests/test_oracle_pool_attention.py.
    """
    k = np.asarray(k_rows, np.float32)
    v = np.asarray(v_rows, np.float32)
    T, H, D = k.shape
    assert T % PAGE == 0 and v.shape == k.shape
    P = T // PAGE
    out = np.empty((P, H, block_bytes(fmt, D)), np.uint8)
    if fmt == "q2":
        ck, sk, mk = codec.q2_quantize(k)
        cv, sv, mv = codec.q2_quantize(v)
        # K codes token-major: [P][H][64][D/4]
        kp = layout.pack2(ck).reshape(P, PAGE, H, D // 4).transpose(0, 2, 1, 3)
        out[:, :, :16 * D] = kp.reshape(P, H, 16 * D)
        # V codes: each dim's 64 slots packed in the V-row word layout, then
        # placed where the plane puts that dim's words
        vrows = layout.pack2_vrow(cv.reshape(P, PAGE, H, D).transpose(0, 2, 3, 1))   # [P][H][D][16]
        plane = np.empty((P, H, 16 * D), np.uint8)
        plane[:, :, layout.v_plane_index(D)] = vrows
        out[:, :, 16 * D:32 * D] = plane
        for off, sc, mn in ((32 * D, sk, mk), (32 * D + 512, sv, mv)):
            meta = np.stack([sc, mn], axis=-1).astype(np.float32)                  # [T][H][2]
            meta = meta.reshape(P, PAGE, H, 2).transpose(0, 2, 1, 3)              # [P][H][64][2]
            out[:, :, off:off + 512] = np.ascontiguousarray(meta).view(np.uint8).reshape(P, H, 512)
        return out
    if fmt == "q8":
        cv, sv = codec.q8_quantize_v(v)                                            # [T][H][D], [T][H]
        ck, skc = codec.sym_quantize(k.reshape(P, PAGE, H, D), 8, axis=1, dtype=np.float32)
        out[:, :, :64 * D] = ck.astype(np.int8).transpose(0, 2, 1, 3).reshape(P, H, 64 * D).view(np.uint8)
        vd = cv.reshape(P, PAGE, H, D).transpose(0, 2, 3, 1)                       # [P][H][D][64]
        out[:, :, 64 * D:128 * D] = np.ascontiguousarray(vd).reshape(P, H, 64 * D).view(np.uint8)
        out[:, :, 128 * D:132 * D] = np.ascontiguousarray(skc[:, 0].astype(np.float32)).view(np.uint8).reshape(P, H, 4 * D)
        vsc = sv.reshape(P, PAGE, H).transpose(0, 2, 1).astype(np.float32)          # [P][H][64]
        out[:, :, 132 * D:132 * D + 256] = np.ascontiguousarray(vsc).view(np.uint8).reshape(P, H, 256)
        return out
    raise ValueError(fmt)
