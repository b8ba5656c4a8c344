"""GPU codec edge rows, bit-exact against the oracle.

The codes and metadata are a pure function of the bf16 rows (the 2-bit
codebook read into "KV at 9 KB a token", section "How it works", 64 B of code
and an 8-byte [scale, min] row per head per token; the 8-bit symmetric
quantizer of "Half the Cache, Twice the Context", section "What the cache
loses when you round it").  These rows take the corner paths of that
function:
  * constant rows and all-zero rows (scale 0 -> 1.0, codes 0);
  * rows whose minimum or maximum is -0.0 (stored as +0.0);
  * rows whose scale is subnormal (values a few multiples of 2^-133, the
    smallest bf16 step) or just above 2^-126;
  * rows whose scale exceeds 2^120, up to values near the bf16 maximum (the
    append kernels take the correctly rounded division there instead of a
    reciprocal);
  * for the 8-bit K channels of a page: an all-zero channel, a channel of
    subnormal values, a channel of values near 3e38.
Every byte of the pool and every dequantized page value equals the oracle's.
"""

import numpy as np
import pytest
import torch

from oracle import pool as opool
from synth import Workload, kv_rows
from tests.gpu_helpers import make_pool, need_gpu, say

pytestmark = pytest.mark.gpu

TINY = 2.0 ** -133   # the smallest bf16 subnormal step


def edge_rows(n, H, D, seed):
    """bf16 rows [n][H][D]: the edge rows first (one kind per token), the
    rest N(0, 1)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, H, D)).astype(np.float32)
    kinds = [
        np.full(D, 1.5),                                          # constant
        np.zeros(D),                                              # all zero
        np.where(np.arange(D) % 3 == 0, -0.0, rng.uniform(0.1, 2.0, D)),   # minimum -0.0
        np.where(np.arange(D) % 5 == 0, -0.0, -rng.uniform(0.1, 2.0, D)),  # maximum -0.0
        np.where(np.arange(D) % 2 == 0, -0.0, 0.0),               # +-0 only: span 0
        rng.integers(0, 31, D) * TINY,                            # subnormal scale (span / 3 < 2^-126)
        rng.integers(0, 127, D) * TINY,                           # subnormal values, larger span
        rng.uniform(0.0, 3.0, D) * 2.0 ** -126,                   # scale just around 2^-126
        rng.uniform(0.0, 3.3e38, D),                              # scale near 1.1e38 (> 2^120)
        -rng.uniform(0.0, 3.3e38, D),
        rng.uniform(-1.0e38, 1.0e38, D),                          # span 2e38, finite
        np.where(np.arange(D) == 7, 3.0e38, rng.standard_normal(D)),  # one huge element
    ]
    for t, row in enumerate(kinds):
        if t < n:
            x[t, t % H] = row
    return torch.from_numpy(x).to(torch.bfloat16)


def k_channel_edges(k):
    """8-bit K: channel 3 all zero, channel 5 subnormal, channel 7 near 3e38,
    over every token of the first page."""
    kf = k.float()
    kf[:64, :, 3] = 0.0
    kf[:64, :, 5] = torch.from_numpy((np.arange(64) % 9 - 4) * TINY).float()[:, None]
    kf[:64, :, 7] = torch.from_numpy(np.linspace(-3.0e38, 3.0e38, 64)).float()[:, None]
    return kf.to(torch.bfloat16)


@pytest.mark.parametrize("fmt_name,D", [("q2", 256), ("q2", 128), ("q8", 128), ("q8", 256)])
def test_codec_edge_rows_bit_exact(fmt_name, D):
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    fmt = {"q2": kvq.FMT_Q2, "q8": kvq.FMT_Q8}[fmt_name]
    w = Workload(97, "codec edges", fmt_name, 1, 2, D, 8, 1, 100)
    n = 100
    k = edge_rows(n, 2, D, 5)
    v = edge_rows(n, 2, D, 6)
    if fmt_name == "q8":
        k = k_channel_edges(k)
    n_pages = 3
    pool, mem = make_pool(w, n_pages, fmt, fill=0x5A, max_seqs=1, max_seq_tokens=128)
    bt = [2, 0]
    seq = pool.reserve(128, pages=bt)
    op = opool.OraclePool(fmt_name, 1, 2, D, n_pages, fill=0x5A)
    for a, b in ((0, 37), (37, 64), (64, n)):       # a partial page, its completion, the next page
        pool.append(0, [seq], [a], [b - a], k[a:b].cuda(), v[a:b].cuda())
        op.append(0, 0, bt, a, k[a:b].float().numpy(), v[a:b].float().numpy())
        torch.cuda.synchronize()
        got = mem.cpu().numpy().reshape(n_pages, -1)
        bad = np.nonzero(got != op.data)
        assert bad[0].size == 0, f"{fmt_name} D={D} after tokens {a}..{b}: {bad[0].size} bytes differ, first at " \
                                 f"page {bad[0][0]} byte {bad[1][0]}"
    for page in bt:
        for head in range(2):
            for kv in (0, 1):
                got = pool.dequant_page(page, 0, head, kv).cpu().numpy()
                blk = op.block(page, 0, head)
                nt = 64 if page == bt[0] else n - 64
                if fmt_name == "q2":
                    from oracle import codec
                    c, s, m = blk.read_k(nt) if kv == 0 else blk.read_v(nt)
                    ref = codec.q2_dequantize(c, s, m)
                else:
                    from oracle import codec
                    if kv == 0:
                        c, s = blk.read_k(nt)
                        ref = codec.q8_dequantize(c, s[None, :])
                    else:
                        c, s = blk.read_v(nt)
                        ref = codec.q8_dequantize(c, s[:, None])
                assert np.array_equal(got[:nt].view(np.uint32), np.asarray(ref, np.float32).view(np.uint32)), \
                    f"{fmt_name} D={D} page {page} head {head} kv {kv}: dequantized values differ"
    say(f"codec edges {fmt_name} D={D}: pool bytes and dequantized pages bit-exact")
