#!/usr/bin/env python3
"""Decode attention over a 2-bit paged KV pool, one MI355X.

Workload (27B geometry): 16 attention layers x 4 KV heads x 256 dims, 16
query heads; 8 lanes, each at 40,960 context tokens (640 pages of 64 tokens
per lane, pages shuffled across lanes in one pool of 5,120 pages =
3,019,898,880 B).  K/V are bf16 N(0,1) with every 16th key channel x4 and
every 64th value token x6, drawn on the device from fixed seeds and
quantize-appended once (untimed set-up, reported separately).  One step =
one decode launch per layer for all 8 lanes (16 launches), one bf16 query per
lane per layer.

Prints one JSON line: KV tokens attended per second (lane x layer x token
triples), the per-launch roofline of the decode kernel against 8 TB/s HBM, and
the CPU oracle timed on a bounded sample of the same work.

    python bench.py [--steps K] [--warmup W] [--splits P] [--no-cpu] [--copy-mib M]
                    [--no-prefill] [--no-extra]

Besides the headline line's decode, the same JSON line holds the chunked
prefill (65,536 + 1,024 tokens), the 131,072-token split-K decode at 16..128
splits (cache-warm and after a 1 GiB flush) and the 8-bit 24-lane x 32-layer
decode, each with its own figures.

The roofline's "traffic" (HBM bytes a decode call really moves, from the
FETCH_SIZE and WRITE_SIZE counters scaled by a copy of known size) is read
from the committed counter summary in profiles/ and reported only while the
decode sources still hash to the version the counters were taken on;
otherwise it is null.  --copy-mib runs that calibration copy (int32 -> fp32,
M MiB each way) after the timed region, for the counter passes.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
MFMA_BF16_TFLOPS = 2500.0  # dense bf16 matrix-core peak
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "quantized_kv_attention_append_amd", "csrc")
# sources of the two kernels of a 2-bit decode call (split kernel + merge)
DECODE_SOURCES = ("decode_q2_mfma.hip", "merge_splits.hip", "decode_common.h", "kvq_device.h", "kvq_internal.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_q2_mfma_27b_geometry_traffic.md")
METRIC = "decode attention: KV tokens attended/s and achieved HBM GB/s (% of peak), 2-bit"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--splits", type=int, default=0, help="split-K partitions per (lane, KV head); 0 = library choice")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget for the oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--copy-mib", type=int, default=0, help="calibration copy size for counter passes (0 = none)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill leg")
    ap.add_argument("--no-extra", action="store_true", help="skip the long-context, 8-bit, bf16, window and rotated legs")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode call from the committed counter summary, or None
    when it is absent or was taken on other decode sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            fields = dict(line.split(":", 1) for line in f if line.startswith(("source_sha256:", "traffic_bytes_per_call:")))
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != decode_source_hash():
        log("traffic: counter summary is for other decode sources; reporting null")
        return None
    return int(fields["traffic_bytes_per_call"].strip())


def prefill_leg(steps: int, warmup: int):
    """Chunked prefill over the 2-bit pool: 65,536 prior tokens + a 1,024-token
    chunk (1 layer, 4 KV heads x 256, 16 query heads), timed with HIP events
    per call (prefill kernel + its merge).  Useful flops = 4 D Hq sum_i (p0 + i + 1)."""
    import torch

    import quantized_kv_attention_append_amd as kvq
    from synth import WORKLOADS, kv_rows, page_permutation, queries

    w = WORKLOADS["prefill"]
    prior, n_q = w.ctx, w.chunk
    total = prior + n_q
    geom = (w.n_layers, w.n_kv_heads, w.head_dim, w.n_q_heads)
    _, pb = kvq.token_bytes(geom, kvq.FMT_Q2)
    n_pages = total // 64
    pool = kvq.Pool(n_pages * pb, geom, kvq.FMT_Q2, max_seqs=1, max_seq_tokens=total)
    seq = pool.reserve(total, pages=page_permutation(w, n_pages))
    k, v = kv_rows(w, 0, 0, total, device="cuda")
    pool.append(0, [seq], [0], [prior], k[:prior], v[:prior])
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    pool.append(0, [seq], [prior], [n_q], k[prior:], v[prior:])
    e1.record(stream)
    e1.synchronize()
    chunk_append_ms = e0.elapsed_time(e1)
    del k, v
    q = queries(w, 0, n_q, device="cuda", stream=1)
    ws = torch.empty(pool.workspace_bytes(kvq.OP_PREFILL, n_q, 0), dtype=torch.uint8, device="cuda")
    out = torch.empty((n_q, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        pool.prefill(0, seq, prior, q, w.sm_scale, ws=ws, out=out)
    torch.cuda.synchronize()
    ms = []
    for _ in range(steps):
        e0.record(stream)
        pool.prefill(0, seq, prior, q, w.sm_scale, ws=ws, out=out)
        e1.record(stream)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    avg = sum(ms) / len(ms)
    flops = 4.0 * w.head_dim * w.n_q_heads * sum(prior + i + 1 for i in range(n_q))
    tflops = flops / (avg * 1e-3) / 1e12
    log(f"prefill: {avg:.3f} ms per call, {tflops:.0f} TFLOP/s useful ({100 * tflops / MFMA_BF16_TFLOPS:.1f}% of bf16 peak)")
    return {
        "workload": "chunked prefill, 2-bit: 65536 prior + 1024 chunk tokens, 1 layer x 4 KV heads x 256 dims, "
                    "16 query heads",
        "ms_per_call": avg,
        "ms_min": min(ms),
        "useful_flops": flops,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_TFLOPS, "traffic": None,
                     "kernel": "one kv_attn_prefill call: prefill_kernel<256, 1> then prefill_merge_kernel"},
        "chunk_append_ms": chunk_append_ms,
    }


def _call_ms(fn, reps: int, flush=None):
    """Average, minimum and median of HIP-event times of fn() on the current
    stream, the calls enqueued back to back (one synchronisation at the end,
    so host launch latency does not enter); flush() (untimed) is enqueued
    before each timed call when given."""
    import torch
    stream = torch.cuda.current_stream()
    ev = []
    for _ in range(reps):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    return sum(ms) / len(ms), ms[0], ms[len(ms) // 2]


def long_context_leg(reps: int):
    """Split-K decode of one 131,072-token sequence (1 layer, 4 KV heads x 256,
    16 query heads, 2-bit; a planted key) at 16, 32, 64 and 128 splits: each
    call timed with HIP events back to back, and again after writing a 1 GiB
    scratch buffer before every call, so that the 75.5 MB of codes come from
    HBM rather than the last-level cache."""
    import torch

    import quantized_kv_attention_append_amd as kvq
    from synth import WORKLOADS, kv_rows, page_permutation, planted_position, queries
    from synth.workloads import plant_key

    w = WORKLOADS["long"]
    ctx = w.ctx
    geom = (w.n_layers, w.n_kv_heads, w.head_dim, w.n_q_heads)
    _, pb = kvq.token_bytes(geom, kvq.FMT_Q2)
    n_pages = ctx // 64
    pool = kvq.Pool(n_pages * pb, geom, kvq.FMT_Q2, max_seqs=1, max_seq_tokens=ctx)
    seq = pool.reserve(ctx, pages=page_permutation(w, n_pages))
    k, v = kv_rows(w, 0, 0, ctx, device="cuda")
    q = queries(w, 0, 1, device="cuda")
    plant_key(k, q[0], planted_position(w, ctx), w.group)
    pool.append(0, [seq], [0], [ctx], k, v)
    del k, v
    out = torch.empty((1, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    alg = ctx * w.n_kv_heads * 2 * (w.head_dim // 4 + 8) + w.n_q_heads * w.head_dim * (2 + 4)
    res = []
    for sp in (16, 32, 64, 128):
        ws = torch.empty(pool.workspace_bytes(kvq.OP_DECODE, 1, sp), dtype=torch.uint8, device="cuda")
        call = lambda: pool.decode(0, [seq], [ctx], q, w.sm_scale, n_splits=sp, ws=ws, out=out)
        for _ in range(3):
            call()
        warm = _call_ms(call, reps)
        cold = _call_ms(call, reps, flush=lambda: scratch.fill_(sp))
        res.append({"splits": sp,
                    "us_mean": warm[0] * 1e3, "us_min": warm[1] * 1e3, "us_median": warm[2] * 1e3,
                    "gbs_mean": alg / (warm[0] * 1e-3) / 1e9,
                    "flushed_us_mean": cold[0] * 1e3, "flushed_us_min": cold[1] * 1e3,
                    "flushed_gbs_mean": alg / (cold[0] * 1e-3) / 1e9})
        log(f"long context, splits={sp}: {warm[0] * 1e3:.1f} us ({alg / (warm[0] * 1e-3) / 1e9:.0f} GB/s), "
            f"after a 1 GiB flush {cold[0] * 1e3:.1f} us ({alg / (cold[0] * 1e-3) / 1e9:.0f} GB/s)")
    del scratch
    return {"workload": "long split-K decode, 2-bit: 1 lane x 131072 tokens, 1 layer x 4 KV heads x 256 dims, "
                        "16 query heads, planted key",
            "bytes_per_call": alg, "per_splits": res}


def q8_leg(reps: int):
    """The 8-bit format: 24 lanes of 64 x U[16, 128] tokens, 32 layers x 8 KV
    heads x 128 dims, 32 query heads.  Populate every layer (timed, HBM bytes
    of bf16 rows read and codes written), then decode every layer (one call per
    layer for all lanes, HIP events); algorithmic bytes 268 per (token, KV
    head) plus q and out."""
    import torch

    import quantized_kv_attention_append_amd as kvq
    from synth import WORKLOADS, q8_batch_lengths, kv_rows, page_permutation, queries

    w = WORKLOADS["q8"]
    lens = [int(x) for x in q8_batch_lengths(w)]
    geom = (w.n_layers, w.n_kv_heads, w.head_dim, w.n_q_heads)
    _, pb = kvq.token_bytes(geom, kvq.FMT_Q8)
    n_pages = sum(-(-L // 64) for L in lens)
    pool = kvq.Pool(n_pages * pb, geom, kvq.FMT_Q8, max_seqs=w.lanes, max_seq_tokens=max(lens))
    perm = page_permutation(w, n_pages)
    seqs, off = [], 0
    for L in lens:
        npg = -(-L // 64)
        seqs.append(pool.reserve(L, pages=perm[off:off + npg]))
        off += npg
    B = w.lanes
    stream = torch.cuda.current_stream()
    app_ms = 0.0
    for layer in range(w.n_layers):
        kv = [kv_rows(w, layer, i, lens[i], device="cuda") for i in range(B)]
        k = torch.cat([a for a, _ in kv])
        v = torch.cat([b for _, b in kv])
        del kv
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pool.append(layer, seqs, [0] * B, lens, k, v)
        e1.record(stream)
        e1.synchronize()
        app_ms += e0.elapsed_time(e1)
        del k, v
    tokens = sum(lens)
    qs = [queries(w, layer, B, device="cuda") for layer in range(w.n_layers)]
    sp = pool.decode_splits(lens)
    ws = torch.empty(pool.workspace_bytes(kvq.OP_DECODE, B, sp), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((B, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda") for _ in range(w.n_layers)]
    for layer in range(w.n_layers):  # warm-up
        pool.decode(layer, seqs, lens, qs[layer], w.sm_scale, n_splits=sp, ws=ws, out=outs[layer])
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):  # steps of one call per layer, back to back, an event pair around each call
        for layer in range(w.n_layers):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pool.decode(layer, seqs, lens, qs[layer], w.sm_scale, n_splits=sp, ws=ws, out=outs[layer])
            e1.record(stream)
            ev.append((e0, e1))
    torch.cuda.synchronize()
    avg = sum(e0.elapsed_time(e1) for e0, e1 in ev) / len(ev)
    alg = tokens * w.n_kv_heads * 268 + B * w.n_q_heads * w.head_dim * (2 + 4)
    app_bytes = w.n_layers * tokens * w.n_kv_heads * 2 * (2 * w.head_dim) + w.n_layers * tokens * w.n_kv_heads * (
        2 * w.head_dim + 8)
    gbs = alg / (avg * 1e-3) / 1e9
    log(f"8-bit: populate {w.n_layers} layers x {tokens} tokens in {app_ms:.1f} ms; decode {avg * 1e3:.1f} us a layer "
        f"call, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s), splits={sp}")
    return {"workload": "8-bit decode, 24 lanes x 64*U[16,128] tokens, 32 layers x 8 KV heads x 128 dims, 32 query heads",
            "tokens_per_layer": tokens, "pool_bytes": n_pages * pb, "splits": sp,
            "decode_us_per_layer_call": avg * 1e3, "bytes_per_call": alg,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                         "kernel": "one kv_attn_decode call per layer: decode_q8_mfma_kernel<128, 4> then merge_splits8_kernel"},
            "kv_tokens_per_s": tokens * w.n_layers / (avg * 1e-3 * w.n_layers),
            "populate_ms": app_ms, "populate_gbs": app_bytes / app_ms / 1e6}


def bf16_leg(reps: int, window: bool = False, rotated: bool = False):
    """The exact bf16 cache of the same 27B-geometry batch (16 layers x 4 KV
    heads x 256 dims, 8 lanes x 40,960 tokens: 21.47 GB, the pages' 20.0 GiB),
    through the same calls: populate, then the 16-layer decode step (each call
    timed with HIP events, and the step replayed as a HIP graph), and the
    65,536 + 1,024 chunked prefill over a bf16 pool.

    window=True runs the same legs over 2-bit pools with the exact window of
    the last page: each lane's last 64 tokens are read as bf16 rows, the rest
    as 2-bit rows (the pool's pages are the 2-bit 3.02 GB).  rotated=True runs
    the decode legs over the 2-bit pool of Hadamard-rotated K rows (same pages; no
    prefill for that format)."""
    import torch

    import quantized_kv_attention_append_amd as kvq
    from synth import WORKLOADS, kv_rows, page_permutation, queries

    fmt = kvq.FMT_Q2_WINDOW if window else kvq.FMT_Q2_ROT if rotated else kvq.FMT_BF16
    name = "2-bit window" if window else "2-bit rotated" if rotated else "bf16"
    w = WORKLOADS["27b"]
    L, H, D, Hq, B, ctx = w.n_layers, w.n_kv_heads, w.head_dim, w.n_q_heads, w.lanes, w.ctx
    geom = (L, H, D, Hq)
    tb, pb = kvq.token_bytes(geom, fmt)
    ppl = ctx // 64
    n_pages = B * ppl
    pool = kvq.Pool(n_pages * pb, geom, fmt, max_seqs=B, max_seq_tokens=ctx)
    perm = page_permutation(w, n_pages)
    seqs = [pool.reserve(ctx, pages=perm[i * ppl:(i + 1) * ppl]) for i in range(B)]
    stream = torch.cuda.current_stream()
    app_ms = 0.0
    for layer in range(L):
        kv = [kv_rows(w, layer, lane, ctx, device="cuda") for lane in range(B)]
        k = torch.cat([a for a, _ in kv])
        v = torch.cat([b for _, b in kv])
        del kv
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pool.append(layer, seqs, [0] * B, [ctx] * B, k, v)
        e1.record(stream)
        e1.synchronize()
        app_ms += e0.elapsed_time(e1)
        del k, v
    # every row of every layer read once (bf16) and written once (tb covers all layers)
    app_bytes = B * ctx * (L * H * 4 * D + tb)
    qs = [queries(w, layer, B, device="cuda") for layer in range(L)]
    sp = pool.decode_splits([ctx] * B)
    ws = torch.empty(pool.workspace_bytes(kvq.OP_DECODE, B, sp), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((B, Hq, D), dtype=torch.float32, device="cuda") for _ in range(L)]

    def step():
        for layer in range(L):
            pool.decode(layer, seqs, [ctx] * B, qs[layer], w.sm_scale, n_splits=sp, ws=ws, out=outs[layer])

    step()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        for layer in range(L):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pool.decode(layer, seqs, [ctx] * B, qs[layer], w.sm_scale, n_splits=sp, ws=ws, out=outs[layer])
            e1.record(stream)
            ev.append((e0, e1))
    torch.cuda.synchronize()
    avg_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / len(ev)
    eager_outs = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(reps):
        g.replay()
    g1.record(stream)
    g1.synchronize()
    graph_ms = g0.elapsed_time(g1) / reps
    same = all(torch.equal(a, b) for a, b in zip(outs, eager_outs))
    del g
    if window:   # 2-bit K and V rows before the window, bf16 rows in it, q in, fp32 out
        alg = B * H * ((ctx - 64) * 2 * (D // 4 + 8) + 64 * 4 * D) + B * Hq * D * (2 + 4)
    elif rotated:  # 2-bit K and V rows, q in, fp32 out
        alg = B * H * ctx * 2 * (D // 4 + 8) + B * Hq * D * (2 + 4)
    else:        # bf16 K and V rows, q in, fp32 out
        alg = B * ppl * H * 64 * (4 * D) + B * Hq * D * (2 + 4)
    gbs = alg / (avg_ms * 1e-3) / 1e9
    log(f"{name}: populate {app_ms:.1f} ms ({app_bytes / app_ms / 1e6:.0f} GB/s); decode {avg_ms * 1e3:.1f} us a call, "
        f"{gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s), splits={sp}; graph step {graph_ms:.3f} ms "
        f"(identical to eager: {same})")
    del pool, ws, outs, qs, eager_outs
    torch.cuda.empty_cache()
    if rotated:
        return {"workload": f"27B-geometry batched decode, {name}: 16 layers x 4 KV heads x 256 dims, 16 query heads, "
                            "8 lanes x 40960 tokens", "pool_bytes": n_pages * pb, "splits": sp,
                "decode_us_per_call": avg_ms * 1e3, "bytes_per_call": alg,
                "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                             "kernel": "one kv_attn_decode call per layer: decode_q2_mfma_kernel<256, false, true> "
                                       "then merge_splits8_kernel"},
                "graph_ms_per_step": graph_ms, "graph_identical_to_eager": same,
                "kv_tokens_per_s": B * L * ctx / (graph_ms * 1e-3),
                "populate_ms": app_ms, "populate_gbs": app_bytes / app_ms / 1e6}

    # ---- chunked prefill over a bf16 pool: 65,536 prior + 1,024 chunk ----
    w3 = WORKLOADS["prefill"]
    prior, n_q = w3.ctx, w3.chunk
    total = prior + n_q
    geom3 = (w3.n_layers, w3.n_kv_heads, w3.head_dim, w3.n_q_heads)
    _, pb3 = kvq.token_bytes(geom3, fmt)
    n3 = total // 64
    pool3 = kvq.Pool(n3 * pb3, geom3, fmt, max_seqs=1, max_seq_tokens=total)
    seq3 = pool3.reserve(total, pages=page_permutation(w3, n3))
    k, v = kv_rows(w3, 0, 0, total, device="cuda")
    pool3.append(0, [seq3], [0], [prior], k[:prior], v[:prior])
    pool3.append(0, [seq3], [prior], [n_q], k[prior:], v[prior:])
    del k, v
    q = queries(w3, 0, n_q, device="cuda", stream=1)
    ws3 = torch.empty(pool3.workspace_bytes(kvq.OP_PREFILL, n_q, 0), dtype=torch.uint8, device="cuda")
    out3 = torch.empty((n_q, w3.n_q_heads, w3.head_dim), dtype=torch.float32, device="cuda")
    pf = _call_ms(lambda: pool3.prefill(0, seq3, prior, q, w3.sm_scale, ws=ws3, out=out3), reps)
    flops = 4.0 * w3.head_dim * w3.n_q_heads * sum(prior + i + 1 for i in range(n_q))
    pf_tflops = flops / (pf[0] * 1e-3) / 1e12
    log(f"{name} prefill: {pf[0]:.3f} ms per call, {pf_tflops:.0f} TFLOP/s useful")
    kernel = ("one kv_attn_decode call per layer: decode_q2_mfma_kernel<256> then decode_window_merge_kernel<256>"
              if window else "one kv_attn_decode call per layer: decode_bf16_kernel<256, 4> then merge_splits8_kernel")
    return {"workload": f"27B-geometry batched decode, {name}: 16 layers x 4 KV heads x 256 dims, 16 query heads, "
                        "8 lanes x 40960 tokens", "pool_bytes": n_pages * pb, "splits": sp,
            "decode_us_per_call": avg_ms * 1e3, "bytes_per_call": alg,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": kernel},
            "graph_ms_per_step": graph_ms, "graph_identical_to_eager": same,
            "kv_tokens_per_s": B * L * ctx / (graph_ms * 1e-3),
            "populate_ms": app_ms, "populate_gbs": app_bytes / app_ms / 1e6,
            "prefill_ms_per_call": pf[0], "prefill_ms_min": pf[1], "prefill_useful_tflops": pf_tflops}


def oracle_baseline(w, budget_s: float):
    """The oracle's decode (dequantize the lane's codes, fp64 softmax attention)
    timed on (layer, lane) units of the same workload until the budget is spent."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import attention, codec
    from synth import kv_rows, queries

    ctx = w.ctx
    done_tokens, spent, units = 0, 0.0, []
    # (layer, lane) units in an order that spreads the sample over layers and
    # lanes, until the budget of oracle time is spent
    order = [(layer, (layer + s) % w.lanes) for s in range(w.lanes) for layer in range(w.n_layers)]
    for layer, lane in order:
        k, v = kv_rows(w, layer, lane, ctx, device="cuda")
        kf, vf = k.float().cpu().numpy(), v.float().cpu().numpy()
        del k, v
        ck = codec.q2_quantize(kf)
        cv = codec.q2_quantize(vf)
        q = queries(w, layer, w.lanes, device="cuda")[lane].float().cpu().numpy()
        t0 = time.perf_counter()
        K = codec.q2_dequantize(*ck)
        V = codec.q2_dequantize(*cv)
        attention.decode(q, K, V, w.sm_scale)
        dt = time.perf_counter() - t0
        spent += dt
        done_tokens += ctx
        units.append((layer, lane))
        log(f"oracle unit layer={layer} lane={lane}: {dt:.2f} s")
        if spent >= budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": done_tokens / spent,
        "unit": "KV tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(units)} (layer, lane) units of {ctx} tokens x 4 KV heads x 16 query heads "
                  f"(dequantize + fp64 softmax attention), {spent:.1f} s",
    }


def platform_info() -> dict:
    """Device, runtime versions and the current DPM clock levels from sysfs
    (the files rocm-smi reads; None where unavailable)."""
    import glob

    import torch

    props = torch.cuda.get_device_properties(0)
    clocks = []
    for dev in sorted(glob.glob("/sys/class/drm/card*/device"))[:16]:
        cur = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(dev, name)) as f:
                    cur[name[-4:]] = next((l.split(":", 1)[1].replace("*", "").strip() for l in f if "*" in l), None)
            except OSError:
                pass
        if cur:
            clocks.append(cur)
    return {"device": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hip": torch.version.hip, "torch": torch.__version__,
            "clocks": clocks or None}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this library runs on one GPU only (no multi-GPU path is built); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_kv_attention_append_amd as kvq
    from synth import WORKLOADS, kv_rows, page_permutation, queries

    w = WORKLOADS["27b"]
    L, H, D, Hq, B, ctx = w.n_layers, w.n_kv_heads, w.head_dim, w.n_q_heads, w.lanes, w.ctx
    geom = (L, H, D, Hq)
    tb, pb = kvq.token_bytes(geom, kvq.FMT_Q2)
    pages_per_lane = ctx // 64
    n_pages = B * pages_per_lane
    pool = kvq.Pool(n_pages * pb, geom, kvq.FMT_Q2, max_seqs=B, max_seq_tokens=ctx)
    perm = page_permutation(w, n_pages)
    seqs = [pool.reserve(ctx, pages=perm[i * pages_per_lane:(i + 1) * pages_per_lane]) for i in range(B)]
    stream = torch.cuda.current_stream()

    # ---- populate (quantize-append of every token, untimed for the metric) --
    app_ms = 0.0
    for layer in range(L):
        ks, vs = [], []
        for lane in range(B):
            k, v = kv_rows(w, layer, lane, ctx, device="cuda")
            ks.append(k); vs.append(v)
        k, v = torch.cat(ks), torch.cat(vs)
        del ks, vs
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pool.append(layer, seqs, [0] * B, [ctx] * B, k, v)
        e1.record(stream)
        e1.synchronize()
        app_ms += e0.elapsed_time(e1)
        del k, v
    append_rows = L * B * ctx * H * 2
    append_bytes = append_rows * (2 * D) + L * B * ctx * tb // L  # bf16 rows read + codes/metadata written
    log(f"populate: {append_rows} rows in {app_ms:.2f} ms -> {append_bytes / app_ms / 1e6:.0f} GB/s")

    # ---- decode ----------------------------------------------------------
    qs = [queries(w, layer, B, device="cuda") for layer in range(L)]
    sp = args.splits if args.splits > 0 else pool.decode_splits([ctx] * B)
    ws = torch.empty(pool.workspace_bytes(kvq.OP_DECODE, B, sp), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((B, Hq, D), dtype=torch.float32, device="cuda") for _ in range(L)]
    ctxs = [ctx] * B

    def step(events=None):
        for layer in range(L):
            if events is not None:
                events[layer][0].record(stream)
            pool.decode(layer, seqs, ctxs, qs[layer], w.sm_scale, n_splits=sp, ws=ws, out=outs[layer])
            if events is not None:
                events[layer][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(L)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [ev[s][l][0].elapsed_time(ev[s][l][1]) for s in range(args.steps) for l in range(L)]
    region_ms = ev[0][0][0].elapsed_time(ev[-1][-1][1])
    ms_per_step = region_ms / args.steps
    avg_launch_ms = sum(launch_ms) / len(launch_ms)

    kv_bytes_per_launch = B * pages_per_lane * H * 64 * (2 * (D // 4 + 8))   # K and V rows read
    io_bytes_per_launch = B * Hq * D * 2 + B * Hq * D * 4                      # q in, fp32 out
    bytes_per_launch = kv_bytes_per_launch + io_bytes_per_launch
    achieved = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9
    tokens_per_step = B * L * ctx
    value = tokens_per_step / (ms_per_step * 1e-3)
    log(f"splits={sp} avg decode launch {avg_launch_ms * 1e3:.1f} us, step {ms_per_step:.3f} ms, "
        f"{achieved:.0f} GB/s ({100 * achieved / HBM_PEAK_GBS:.1f}% of 8 TB/s), wall {wall:.3f} s")

    # ---- the same step captured once as a HIP graph and replayed (no host
    # launch work, no dispatch gaps between calls); its outputs must equal the
    # eager step's bit for bit ----
    eager_outs = [o.clone() for o in outs]
    graph_step = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_step):
        step()
    for _ in range(3):
        graph_step.replay()
    torch.cuda.synchronize()
    ge0, ge1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ge0.record(stream)
    for _ in range(args.steps):
        graph_step.replay()
    ge1.record(stream)
    ge1.synchronize()
    graph_ms = ge0.elapsed_time(ge1) / args.steps
    graph_same = all(torch.equal(a, b) for a, b in zip(outs, eager_outs))
    log(f"graph replay: step {graph_ms:.3f} ms ({graph_ms / L * 1e3:.1f} us a call), "
        f"{bytes_per_launch * L / (graph_ms * 1e-3) / 1e9:.0f} GB/s, outputs identical to eager: {graph_same}")
    graph = {"ms_per_step": graph_ms, "value": tokens_per_step / (graph_ms * 1e-3), "us_per_call": graph_ms / L * 1e3,
             "gbs": bytes_per_launch * L / (graph_ms * 1e-3) / 1e9, "identical_to_eager": graph_same}
    del graph_step
    # The headline step is the graph replay when it reproduces the eager
    # outputs exactly (the way a serving loop issues a decode step); the
    # per-launch roofline figure stays the eager, event-bracketed one.
    eager = {"ms_per_step": ms_per_step, "value": value}
    step_mode = "eager"
    if graph_same:
        ms_per_step, value, step_mode = graph_ms, graph["value"], "hip_graph"

    if args.copy_mib > 0:
        # calibration for the FETCH_SIZE / WRITE_SIZE counter passes: a plain
        # elementwise copy that reads and writes copy_mib MiB
        n = args.copy_mib << 18
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty(n, dtype=torch.float32, device="cuda")
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: 3 x {args.copy_mib} MiB int32 -> fp32")
        del src, dst

    prefill = None if args.no_prefill else prefill_leg(max(3, args.steps // 4), 2)
    long_ctx = None if args.no_extra else long_context_leg(10)
    q8 = None if args.no_extra else q8_leg(5)
    bf16 = None if args.no_extra else bf16_leg(5)
    if bf16 is not None:
        # the pages' A/B: decode price of the 2-bit cache against the exact one, same batch and calls
        bf16["q2_step_speedup"] = bf16["graph_ms_per_step"] / ms_per_step
        if prefill is not None:
            bf16["q2_prefill_time_ratio"] = prefill["ms_per_call"] / bf16["prefill_ms_per_call"]
        log(f"2-bit against bf16: decode step {bf16['q2_step_speedup']:.2f}x faster"
            + (f", prefill {bf16['q2_prefill_time_ratio']:.2f}x the bf16 time" if prefill is not None else ""))

    win = None if args.no_extra else bf16_leg(5, window=True)
    if win is not None:
        # the price of reading each lane's last page exact, same batch and calls
        win["step_time_vs_q2"] = win["graph_ms_per_step"] / ms_per_step
        if prefill is not None:
            win["prefill_time_vs_q2"] = win["prefill_ms_per_call"] / prefill["ms_per_call"]
        log(f"2-bit window against 2-bit: decode step {win['step_time_vs_q2']:.3f}x the time"
            + (f", prefill {win['prefill_time_vs_q2']:.3f}x" if prefill is not None else ""))

    rot = None if args.no_extra else bf16_leg(5, rotated=True)
    if rot is not None:
        # the price of the rotation: the query transform, butterflies on the K rows of append
        rot["step_time_vs_q2"] = rot["graph_ms_per_step"] / ms_per_step
        rot["populate_time_vs_q2"] = rot["populate_ms"] / app_ms
        log(f"2-bit rotated against 2-bit: decode step {rot['step_time_vs_q2']:.3f}x the time, "
            f"populate {rot['populate_time_vs_q2']:.3f}x")

    cpu = None
    if not args.no_cpu:
        cpu = oracle_baseline(w, args.cpu_seconds)

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u2/f32",
        "data": "synthetic",
        "config": {
            "workload": "27B-geometry batched decode, 2-bit: 16 layers x 4 KV heads x 256 dims, 16 query heads, "
                        "8 lanes x 40960 tokens",
            "layers": L, "kv_heads": H, "head_dim": D, "q_heads": Hq, "lanes": B, "ctx_tokens": ctx,
            "splits": sp, "pool_bytes": n_pages * pb,
        },
        "hbm_gbs": achieved,
        "hbm_pct_of_peak": 100 * achieved / HBM_PEAK_GBS,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
            "kernel": "one kv_attn_decode call per layer: decode_q2_mfma_kernel<256> then merge_splits8_kernel",
            "bytes_per_launch": bytes_per_launch,
            "avg_launch_us": avg_launch_ms * 1e3,
        },
        "step_mode": step_mode,
        "eager": eager,
        "graph": graph,
        "append": {"rows": append_rows, "ms": app_ms, "gbs": append_bytes / app_ms / 1e6},
        "prefill": prefill,
        "long_context": long_ctx,
        "q8": q8,
        "bf16": bf16,
        "q2_window": win,
        "q2_rotated": rot,
        "cpu_baseline": cpu,
        "platform": platform_info(),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
