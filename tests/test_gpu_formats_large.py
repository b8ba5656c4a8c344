"""GPU parity at the 27B geometry for the window and rotated 2-bit formats,
and HIP-graph replays of decode in every format.

* 2 of the 16 layers x 8 lanes x 40,960 tokens (the per-layer shape bench.py
  times), each layer's whole output (8 lanes) against the oracle: the window
  format reads each lane's last page exact; the rotated format reads rotated
  rows.  The same lanes with 32 query heads (group 8), plain and window.
* A decode step (two layers) captured in a HIP graph and replayed three times,
  with eager work and synchronizations between the replays: every replay's
  outputs equal the eager outputs bit for bit.  Decode records no memset.
"""

import numpy as np
import pytest
import torch

from oracle import attention, pool as opool
from synth import WORKLOADS, Workload, kv_rows, page_permutation, queries
from tests.gpu_helpers import assert_close, make_pool, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["q2w", "q2r"])
def test_27b_geometry_whole_layers(name):
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    fmt = {"q2w": kvq.FMT_Q2_WINDOW, "q2r": kvq.FMT_Q2_ROT}[name]
    w = WORKLOADS["27b"]
    L, B, ctx = w.n_layers, w.lanes, w.ctx
    geom = (L, w.n_kv_heads, w.head_dim, w.n_q_heads)
    ppl = ctx // 64
    n_pages = B * ppl
    _, pb = kvq.token_bytes(geom, fmt)
    pool = kvq.Pool(n_pages * pb, geom, fmt, max_seqs=B, max_seq_tokens=ctx)
    perm = page_permutation(w, n_pages)
    seqs = [pool.reserve(ctx, pages=perm[i * ppl:(i + 1) * ppl]) for i in range(B)]
    layers = (0, 15)
    for layer in layers:
        kv = [kv_rows(w, layer, lane, ctx, device="cuda") for lane in range(B)]
        pool.append(layer, seqs, [0] * B, [ctx] * B, torch.cat([a for a, _ in kv]), torch.cat([b for _, b in kv]))
        del kv
    sp = pool.decode_splits([ctx] * B)
    say(f"27B geometry {name}: populated layers {layers}, splits={sp}")
    for layer in layers:
        q = queries(w, layer, B, device="cuda")
        out = pool.decode(layer, seqs, [ctx] * B, q, w.sm_scale, n_splits=sp).cpu().numpy()
        refs = []
        for lane in range(B):
            k, v = kv_rows(w, layer, lane, ctx, device="cuda")
            K, V = opool.dequantized_rows(name, k.float().cpu().numpy(), v.float().cpu().numpy())
            refs.append(attention.decode(q[lane].float().cpu().numpy(), K, V, w.sm_scale))
        assert_close(out, np.stack(refs), f"27B {name} layer {layer}, all 8 lanes")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["q2", "q2w"])
def test_27b_lanes_group8_whole_layer(name):
    # the 27B lanes with 32 query heads over the 4 KV heads: both four-head
    # halves of each group in one launch, at the library's split count
    need_gpu()
    import dataclasses

    import quantized_kv_attention_append_amd as kvq
    fmt = {"q2": kvq.FMT_Q2, "q2w": kvq.FMT_Q2_WINDOW}[name]
    w = dataclasses.replace(WORKLOADS["27b"], n_layers=2, n_q_heads=32)
    B, ctx = w.lanes, w.ctx
    geom = (w.n_layers, w.n_kv_heads, w.head_dim, w.n_q_heads)
    ppl = ctx // 64
    _, pb = kvq.token_bytes(geom, fmt)
    pool = kvq.Pool(B * ppl * pb, geom, fmt, max_seqs=B, max_seq_tokens=ctx)
    perm = page_permutation(w, B * ppl)
    seqs = [pool.reserve(ctx, pages=perm[i * ppl:(i + 1) * ppl]) for i in range(B)]
    layer = 1
    kv = [kv_rows(w, layer, lane, ctx, device="cuda") for lane in range(B)]
    pool.append(layer, seqs, [0] * B, [ctx] * B, torch.cat([a for a, _ in kv]), torch.cat([b for _, b in kv]))
    del kv
    sp = pool.decode_splits([ctx] * B)
    say(f"27B lanes, group 8, {name}: splits={sp}")
    q = queries(w, layer, B, device="cuda")
    out = pool.decode(layer, seqs, [ctx] * B, q, w.sm_scale, n_splits=sp).cpu().numpy()
    refs = []
    for lane in range(B):
        k, v = kv_rows(w, layer, lane, ctx, device="cuda")
        K, V = opool.dequantized_rows(name, k.float().cpu().numpy(), v.float().cpu().numpy())
        refs.append(attention.decode(q[lane].float().cpu().numpy(), K, V, w.sm_scale))
    assert_close(out, np.stack(refs), f"27B lanes group 8 {name} layer {layer}, all 8 lanes")


# 2 layers x 4 KV heads x 128 dims, 16 query heads: every format at group 4
GW = Workload(92, "graph replay", "q2", 2, 4, 128, 16, 3, 500)


@pytest.mark.parametrize("name", ["q2", "q8", "bf16", "q2w", "q2r"])
def test_decode_graph_replays_equal_eager(name):
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    fmt = {"q2": kvq.FMT_Q2, "q8": kvq.FMT_Q8, "bf16": kvq.FMT_BF16, "q2w": kvq.FMT_Q2_WINDOW,
           "q2r": kvq.FMT_Q2_ROT}[name]
    w = GW
    lens = [500, 130, 77]
    n_pages = sum(-(-n // 64) for n in lens)
    pool, _ = make_pool(w, n_pages, fmt)
    seqs = [pool.reserve(n) for n in lens]
    for layer in range(2):
        for i, n in enumerate(lens):
            k, v = kv_rows(w, layer, i, n)
            pool.append(layer, [seqs[i]], [0], [n], k.cuda(), v.cuda())
    sp = 3
    qs = [queries(w, layer, len(lens), device="cuda") for layer in range(2)]
    ws = torch.empty(pool.workspace_bytes(kvq.OP_DECODE, len(lens), sp), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((len(lens), w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda") for _ in range(2)]

    def step():
        for layer in range(2):
            pool.decode(layer, seqs, lens, qs[layer], w.sm_scale, n_splits=sp, ws=ws, out=outs[layer])

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()   # warm-up on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    scratch = torch.empty((len(lens), w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for layer in range(2):
            assert torch.equal(outs[layer], eager[layer]), f"{name}: replay {r} layer {layer} differs from eager"
        # eager work between replays: another decode into other memory, a torch op
        pool.decode(1, seqs, lens, qs[0], w.sm_scale, n_splits=sp, ws=ws, out=scratch)
        scratch.mul_(2.0)
        torch.cuda.synchronize()
    say(f"{name}: 3 graph replays equal the eager step")
