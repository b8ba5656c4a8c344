"""GPU parity of the 27B-geometry workload at full size, whole layers.

16 layers x 4 KV heads x 256 dims, 16 query heads, 8 lanes x 40,960 tokens
in one 3,019,898,880-byte pool whose 5,120 pages are a seeded permutation
dealt 640 per lane (the workload bench.py times, in its launch
configuration).  For layers 0, 5, 10 and 15, every lane's 640 pages are
compared byte for byte with the oracle's image of the same rows (codes and
metadata, "KV at 9 KB a token", section "How it works": 72 B per head per
token), and the layer's whole decode output (8 lanes x 16 heads x 256 dims)
is held to max abs 2e-3 and relative L2 1e-3 against the fp64 oracle.
"""

import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

from oracle import attention, pool as opool
from synth import WORKLOADS, kv_rows, page_permutation, queries
from tests.gpu_helpers import assert_close, geom_of, make_pool, need_gpu, say

pytestmark = pytest.mark.gpu

WORKERS = max(1, min(8, len(os.sched_getaffinity(0))))


def layer_blocks(mem, page_bytes, pages, layer, n_heads, block):
    """The bytes of one layer's (layer, KV head) blocks in the given physical
    pages, read back from the device pool: [len(pages)][n_heads * block]."""
    rows = mem.view(-1, page_bytes).index_select(0, torch.as_tensor(np.asarray(pages, np.int64), device=mem.device))
    return rows[:, layer * n_heads * block:(layer + 1) * n_heads * block].cpu().numpy()


def q2_unit(k, v, q, sm):
    """Oracle image of one lane's pages of one layer, and its decode output."""
    blocks = opool.sequence_blocks("q2", k, v)
    K, V = opool.dequantized_rows("q2", k, v)
    return blocks, attention.decode(q, K, V, sm)


@pytest.mark.timeout(1200)
def test_27b_whole_layers_pool_image_and_outputs():
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    w = WORKLOADS["27b"]
    L, H, D, B, ctx = w.n_layers, w.n_kv_heads, w.head_dim, w.lanes, w.ctx
    ppl = ctx // 64
    n_pages = B * ppl
    _, pb = kvq.token_bytes(geom_of(w), kvq.FMT_Q2)
    assert n_pages * pb == 3_019_898_880
    pool, mem = make_pool(w, n_pages, kvq.FMT_Q2, fill=0xA5, max_seqs=B, max_seq_tokens=ctx)
    perm = page_permutation(w, n_pages)
    seqs = [pool.reserve(ctx, pages=perm[i * ppl:(i + 1) * ppl]) for i in range(B)]
    for layer in range(L):
        kv = [kv_rows(w, layer, lane, ctx, device="cuda") for lane in range(B)]
        pool.append(layer, seqs, [0] * B, [ctx] * B, torch.cat([a for a, _ in kv]), torch.cat([b for _, b in kv]))
        del kv
    st = pool.stats()
    assert st["used_pages"] == n_pages and st["free_pages"] == 0
    sp = pool.decode_splits([ctx] * B)
    block = 32 * D + 1024
    say(f"27B geometry: populated 16 layers, splits={sp}, oracle on {WORKERS} threads")
    with cf.ThreadPoolExecutor(WORKERS) as ex:
        for layer in range(L):
            q = queries(w, layer, B, device="cuda")
            out = pool.decode(layer, seqs, [ctx] * B, q, w.sm_scale, n_splits=sp).cpu().numpy()
            if layer not in (0, 5, 10, 15):
                continue
            qh = q.float().cpu().numpy()
            jobs = []
            for lane in range(B):
                k, v = kv_rows(w, layer, lane, ctx, device="cuda")
                jobs.append(ex.submit(q2_unit, k.float().cpu().numpy(), v.float().cpu().numpy(), qh[lane],
                                      w.sm_scale))
            refs = []
            for lane, job in enumerate(jobs):
                blocks, ref = job.result()
                got = layer_blocks(mem, pb, perm[lane * ppl:(lane + 1) * ppl], layer, H, block)
                bad = int(np.count_nonzero(got != blocks.reshape(ppl, H * block)))
                assert bad == 0, f"layer {layer} lane {lane}: {bad} pool bytes differ from the oracle"
                refs.append(ref)
            assert_close(out, np.stack(refs), f"27B layer {layer}, all 8 lanes")
            say(f"27B layer {layer}: 8 x 640 pages bit-exact ({B * ppl * H * block / 1e6:.1f} MB), whole output "
                "within tolerance")
