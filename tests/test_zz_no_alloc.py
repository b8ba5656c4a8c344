"""kv_attn_decode_static (the decode step with its workspace in the library's
static device array, for callers that cannot allocate) against
kv_attn_decode with a caller's workspace: the same outputs bit for bit, on two
calls in a row, the second with a smaller batch, through the C ABI; both
within the tolerance of the fp64 oracle.  A batch whose workspace exceeds the
array is refused before anything is written."""

import numpy as np
import pytest
import torch

from oracle import attention, pool as opool
from synth import Workload, kv_rows, queries
from tests.gpu_helpers import assert_close, make_pool, need_gpu, say

pytestmark = pytest.mark.gpu

# 1 layer x 4 KV heads x 256 dims, 16 query heads (the 27B head geometry)
W = Workload(93, "static workspace", "q2", 1, 4, 256, 16, 8, 3000)


def test_static_workspace_decode_equals_the_workspace_call():
    need_gpu()
    import quantized_kv_attention_append_amd as kvq
    lens = [3000, 1700, 2500, 64, 999, 2048, 130, 2901]
    n_pages = sum(-(-L // 64) for L in lens)
    pool, mem = make_pool(W, n_pages, kvq.FMT_Q2, max_seqs=len(lens), max_seq_tokens=max(lens))
    seqs = [pool.reserve(L) for L in lens]
    rows = [kv_rows(W, 0, i, L) for i, L in enumerate(lens)]
    pool.append(0, seqs, [0] * len(lens), lens, torch.cat([k for k, _ in rows]).cuda(),
                torch.cat([v for _, v in rows]).cuda())
    q = queries(W, 0, len(lens))
    refs = []
    for i in range(len(lens)):
        K, V = opool.dequantized_rows("q2", rows[i][0].float().numpy(), rows[i][1].float().numpy())
        refs.append(attention.decode(q[i].float().numpy(), K, V, W.sm_scale))
    # two calls in a row, the second with fewer and shorter sequences; the
    # library's split count (merged inside the split kernel) and 32 splits
    # (merged by a kernel of its own)
    for sp in (0, 32):
        for pick, cut in ((list(range(8)), 0), ([1, 4, 6], 37)):
            s_ = [seqs[i] for i in pick]
            ctx = [lens[i] - cut for i in pick]
            qq = q[pick].cuda()
            splits = sp or pool.decode_splits(ctx)
            ws = torch.full((pool.workspace_bytes(kvq.OP_DECODE, len(pick), splits),), 0xFF, dtype=torch.uint8,
                            device="cuda")
            a = pool.decode(0, s_, ctx, qq, W.sm_scale, n_splits=sp, ws=ws)
            b = torch.full_like(a, float("nan"))
            pool.decode_static(0, s_, ctx, qq, W.sm_scale, n_splits=sp, out=b)
            torch.cuda.synchronize()
            assert torch.equal(a, b), f"splits={splits}, {len(pick)} sequences: static and workspace calls differ"
            if cut == 0:
                assert_close(b.cpu().numpy(), np.stack(refs), f"static workspace, splits={splits}")
            say(f"static workspace: {len(pick)} sequences, splits={splits}: identical to the workspace call")
    # too large for the array: refused, nothing written
    big = torch.full((128, W.n_q_heads, W.head_dim), float("nan"), device="cuda")
    need = pool.workspace_bytes(kvq.OP_DECODE, 128, 256)
    assert need > (16 << 20)
    with pytest.raises(kvq.KvError) as ei:
        pool.decode_static(0, [seqs[0]] * 128, [lens[0]] * 128, q[:1].repeat(128, 1, 1).cuda(), W.sm_scale,
                           n_splits=256, out=big)
    assert ei.value.name == "KV_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert torch.isnan(big).all()
