"""The CPU experiments of "Half the Cache, Twice the Context", re-implemented.

These exist to pin the oracle's pieces to numbers the page prints:

* ``sizing_row``: the cache-sizing arithmetic of section "Size the cache
  before you quantize it" (bytes per token, GiB at a 128k context, GiB at one
  byte per value, how many 8k-token requests fit a 24 GiB budget).
* ``block2``: section "What the cache loses when you round it".  With numpy's
  default_rng seeded 7, a 4096 x 128 K (every 16th channel x4) and V (every
  64th token x6) are drawn in that order and quantized per token and per
  channel at 8/4/2 bits with the symmetric absmax quantizer; then, for the bit
  pairs 8/8, 4/4, 3/3, 2/2, 200 needle trials each draw q, a fresh K (channel
  outliers) and a fresh V (no outliers), replace the middle key by q scaled to
  score 0.5 above the best haystack key, and compare softmax attention before
  and after quantizing K per channel and V per token.  It reports top-1
  flips, the mean of the largest weight error and the mean relative L2 error
  of the output.
* ``flat_sum``: section "The cliff is in the accumulator, not the storage".
  n equal weights 1/n are summed in a running register rounded after every
  addition to fp32, fp16 or bf16, or kept in fp32 throughout (two-level).

Each function is my own code written from the section's description; the
numbers it must reproduce are stored under tests/golden/ with their citation.
"""

from __future__ import annotations

import numpy as np

from .accounting import bytes_per_token
from .bf16 import round_f32_to_bf16
from .codec import sym_roundtrip

GIB = 1024 ** 3


# ------------------------------------------------------------- sizing ----

def sizing_row(layers: int, kv_heads: int, head_dim: int, ctx: int = 131072, budget_gib: float = 24.0):
    b16 = bytes_per_token(layers, kv_heads, head_dim, 2)
    b8 = bytes_per_token(layers, kv_heads, head_dim, 1)
    return {
        "kib_per_token": b16 / 1024,
        "ctx_gib_bf16": b16 * ctx / GIB,
        "ctx_gib_1byte": b8 * ctx / GIB,
        "requests_8k": int(budget_gib * GIB // (b16 * 8192)),
        "ratio_vs_128kib": b16 / 131072,
    }


# ------------------------------------------------------------- block 2 ----

def _rel_l2(approx, exact):
    return float(np.linalg.norm(approx - exact) / np.linalg.norm(exact))


def _softmax64(s):
    e = np.exp(s - s.max())
    return e / e.sum()


def block2(seed: int = 7, n: int = 4096, d: int = 128, trials: int = 200, margin: float = 0.5,
           widths=((8, 8), (4, 4), (3, 3), (2, 2)), recon_bits=(8, 4, 2)):
    rng = np.random.default_rng(seed)
    outlier_ch = np.arange(d) % 16 == 0
    outlier_tok = np.arange(n) % 64 == 0

    K = rng.normal(0.0, 1.0, (n, d))
    K[:, outlier_ch] *= 4.0
    V = rng.normal(0.0, 1.0, (n, d))
    V[outlier_tok, :] *= 6.0
    recon = {}
    for name, X in (("K", K), ("V", V)):
        for b in recon_bits:
            per_token = _rel_l2(sym_roundtrip(X, b, axis=1), X)
            per_channel = _rel_l2(sym_roundtrip(X, b, axis=0), X)
            recon[(name, b)] = (per_token, per_channel)

    needle_at = n // 2
    needle = {}
    for kb, vb in widths:
        flips, w_err, o_err = 0, [], []
        for _ in range(trials):
            q = rng.normal(0.0, 1.0, d)
            Kt = rng.normal(0.0, 1.0, (n, d))
            Kt[:, outlier_ch] *= 4.0
            Vt = rng.normal(0.0, 1.0, (n, d))
            target = (Kt @ q).max() + margin
            Kt[needle_at] = q * (target / (q @ q))
            w = _softmax64(Kt @ q)
            ref = w @ Vt
            sq = sym_roundtrip(Kt, kb, axis=0) @ q
            wq = _softmax64(sq)
            flips += int(np.argmax(sq) != needle_at)
            w_err.append(np.abs(wq - w).max())
            o_err.append(_rel_l2(wq @ sym_roundtrip(Vt, vb, axis=1), ref))
        needle[(kb, vb)] = (flips, float(np.mean(w_err)), float(np.mean(o_err)))
    return recon, needle


# ------------------------------------------------------------- block 3 ----

def _round_to(x32, kind: str):
    if kind == "fp32":
        return x32
    if kind == "fp16":
        return np.float32(np.float16(x32))
    if kind == "bf16":
        return round_f32_to_bf16(x32)[()]
    raise ValueError(kind)


def flat_sum(n: int, kind: str, two_level: bool = False) -> float:
    """Sum n copies of 1/n in a register rounded to ``kind`` after each add.

    Each add is done in fp32 (the term is an fp32 number), then rounded to the
    register's format; with ``two_level`` the register stays fp32.  Once an
    add leaves the register unchanged, every later add does too, so the loop
    stops there.
    """
    term = np.float32(1.0 / n)
    acc = np.float32(0.0)
    for _ in range(n):
        nxt = np.float32(acc + term)
        if not two_level:
            nxt = np.float32(_round_to(nxt, kind))
        if nxt == acc:
            break
        acc = nxt
    return float(acc)
