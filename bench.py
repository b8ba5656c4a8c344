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
triples), the per-launch roofline of the decode kernel against 8 TB/s HBM
and against a measured probe of the same reads, and the CPU oracle timed on a
bounded sample of the same work.

    python bench.py [--steps K] [--warmup W] [--splits P] [--no-cpu] [--cpu-units U]
                    [--copy-mib M] [--no-prefill] [--no-extra]

Besides the headline decode, the same JSON line holds: probes of the chip's
streaming read rate, of the decode's read pattern without arithmetic and of
the bf16 matrix cores; the chunked prefill (65,536 + 1,024 tokens); the
131,072-token split-K decode at 16..128 splits (cache-warm and after a 1 GiB
flush) with the planted key's rank; the 8-bit 24-lane x 32-layer decode and
its layer step (decode, then one appended token per lane); the bf16, exact-
window and rotated 2-bit formats over the 27B batch; and the oracle baseline
(a pool of worker processes, one BLAS thread each) for the 27B decode and
populate, the long context per split count, the prefill chunk and the 8-bit
layer step.

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
# sources of the kernel of a 2-bit decode call at 8 splits (split partials and their merge)
DECODE_SOURCES = ("decode_q2_mfma.hip", "decode_common.h", "kvq_device.h", "kvq_internal.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_q2_mfma_27b_geometry_traffic.md")
# sources of an 8-bit decode call's two kernels (split partials, merge) and of its split count
Q8_SOURCES = ("decode_q8.hip", "merge_splits.hip", "decode_common.h", "kvq_device.h", "kvq_internal.h", "kvq_host.cpp")
Q8_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_q8_mfma_24_lanes_32_layers.md")
METRIC = "decode attention: KV tokens attended/s and achieved HBM GB/s (% of peak), 2-bit"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--splits", type=int, default=0, help="split-K partitions per (lane, KV head); 0 = library choice")
    ap.add_argument("--cpu-units", type=int, default=32, help="27B (layer, lane) units in the oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--copy-mib", type=int, default=0, help="calibration copy size for counter passes (0 = none)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill leg")
    ap.add_argument("--no-extra", action="store_true", help="skip the long-context, 8-bit, bf16, window and rotated legs")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def decode_source_hash(names=DECODE_SOURCES) -> str:
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_FILE, names=DECODE_SOURCES):
    """HBM bytes per decode call from a committed counter summary, or None
    when it is absent or was taken on other sources."""
    try:
        with open(path) as f:
            fields = dict(line.split(":", 1) for line in f if line.startswith(("source_sha256:", "traffic_bytes_per_call:")))
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != decode_source_hash(names):
        log(f"traffic: {os.path.basename(path)} is for other sources; reporting null")
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
        _hold(4)
        e0.record(stream)
        pool.prefill(0, seq, prior, q, w.sm_scale, ws=ws, out=out)
        e1.record(stream)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    avg = sum(ms) / len(ms)
    med = sorted(ms)[len(ms) // 2]
    flops = 4.0 * w.head_dim * w.n_q_heads * sum(prior + i + 1 for i in range(n_q))
    tflops = flops / (avg * 1e-3) / 1e12
    log(f"prefill: {avg:.3f} ms per call, {tflops:.0f} TFLOP/s useful ({100 * tflops / MFMA_BF16_TFLOPS:.1f}% of bf16 peak)")
    return {
        "workload": "chunked prefill, 2-bit: 65536 prior + 1024 chunk tokens, 1 layer x 4 KV heads x 256 dims, "
                    "16 query heads",
        "ms_per_call": avg,
        "ms_median": med,
        "ms_min": min(ms),
        "median_tflops": flops / (med * 1e-3) / 1e12,
        "useful_flops": flops,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_TFLOPS, "traffic": None,
                     "kernel": "one kv_attn_prefill call: prefill_ws_kernel<256, false> then prefill_merge_kernel"},
        "chunk_append_ms": chunk_append_ms,
    }


def _stats_us(ms):
    """mean / median / min of a list of millisecond times, in microseconds."""
    ms = sorted(ms)
    return {"us_mean": 1e3 * sum(ms) / len(ms), "us_median": 1e3 * ms[len(ms) // 2], "us_min": 1e3 * ms[0]}


_SLEEP_CYCLES_PER_MS = None


def _hold(n_calls: int):
    """Keep the current stream busy (a spin kernel) for about 0.25 ms per call
    about to be queued, plus 5 ms, so that the host enqueues those calls before
    the GPU reaches them: event pairs around each call then time the GPU's work
    back to back, not the host's launch pace or a pause of the interpreter."""
    global _SLEEP_CYCLES_PER_MS
    import torch
    if _SLEEP_CYCLES_PER_MS is None:
        stream = torch.cuda.current_stream()
        torch.cuda._sleep(1000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        torch.cuda._sleep(2_000_000)
        e1.record(stream)
        e1.synchronize()
        _SLEEP_CYCLES_PER_MS = 2_000_000 / max(e0.elapsed_time(e1), 1e-3)
    torch.cuda._sleep(int((5.0 + 0.25 * n_calls) * _SLEEP_CYCLES_PER_MS))


def _call_ms(fn, reps: int, flush=None):
    """Average, minimum and median of HIP-event times of fn() on the current
    stream, the calls enqueued back to back (one synchronisation at the end,
    so host launch latency does not enter); flush() (untimed) is enqueued
    before each timed call when given."""
    import torch
    stream = torch.cuda.current_stream()
    ev = []
    _hold(reps * (2 if flush is not None else 1))
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
    # drawn on the host (as the parity test and the oracle baseline draw them),
    # so that the oracle's rank of the planted key is over the same rows
    k, v = kv_rows(w, 0, 0, ctx)
    q = queries(w, 0, 1)
    plant_key(k, q[0], planted_position(w, ctx), w.group)
    k, v, q = k.cuda(), v.cuda(), q.cuda()
    pool.append(0, [seq], [0], [ctx], k, v)
    del k, v
    pos = planted_position(w, ctx)
    # the planted key's rank among the raw logits of each group's first query
    # head (1 + keys scoring strictly higher), from the kernel's own scores
    scores = torch.empty((1, w.n_q_heads, ctx), dtype=torch.float32, device="cuda")
    pool.decode(0, [seq], [ctx], q, w.sm_scale, scores=scores)
    sc = scores[0, ::w.group]
    gpu_rank = [int(x) for x in (1 + (sc > sc[:, pos:pos + 1]).sum(dim=1)).cpu()]
    del scores, sc
    log(f"long context: planted key at {pos}, rank among the GPU's logits per KV head {gpu_rank}")
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
                    "gbs_mean": alg / (warm[0] * 1e-3) / 1e9, "gbs_median": alg / (warm[2] * 1e-3) / 1e9,
                    "flushed_us_mean": cold[0] * 1e3, "flushed_us_min": cold[1] * 1e3,
                    "flushed_us_median": cold[2] * 1e3,
                    "flushed_gbs_median": alg / (cold[2] * 1e-3) / 1e9})
        log(f"long context, splits={sp}: {warm[0] * 1e3:.1f} us ({alg / (warm[0] * 1e-3) / 1e9:.0f} GB/s), "
            f"after a 1 GiB flush {cold[0] * 1e3:.1f} us ({alg / (cold[0] * 1e-3) / 1e9:.0f} GB/s)")
    del scratch
    return {"workload": "long split-K decode, 2-bit: 1 lane x 131072 tokens, 1 layer x 4 KV heads x 256 dims, "
                        "16 query heads, planted key",
            "bytes_per_call": alg, "per_splits": res, "default_splits": pool.decode_splits([ctx]),
            "planted_position": pos,
            "planted_rank": {"gpu": gpu_rank, "heads": list(range(0, w.n_q_heads, w.group))}}


def group8_leg(reps: int):
    """2-bit decode at GQA group 8: the 27B lanes (8 x 40,960 tokens, 4 KV heads
    x 256 dims) with 32 query heads, 4 layers.  The library runs both four-head
    halves of each group in one launch, the second half reading the pages
    mostly from L2; calls are timed with HIP events back to back at the
    library's split count, cycling over the layers."""
    import dataclasses

    import torch

    import quantized_kv_attention_append_amd as kvq
    from synth import WORKLOADS, kv_rows, page_permutation, queries

    w = dataclasses.replace(WORKLOADS["27b"], n_layers=4, n_q_heads=32)
    L, H, D, Hq, B, ctx = w.n_layers, w.n_kv_heads, w.head_dim, w.n_q_heads, w.lanes, w.ctx
    geom = (L, H, D, Hq)
    _, pb = kvq.token_bytes(geom, kvq.FMT_Q2)
    ppl = ctx // 64
    pool = kvq.Pool(B * ppl * pb, geom, kvq.FMT_Q2, max_seqs=B, max_seq_tokens=ctx)
    perm = page_permutation(w, B * ppl)
    seqs = [pool.reserve(ctx, pages=perm[i * ppl:(i + 1) * ppl]) for i in range(B)]
    for layer in range(L):
        kv = [kv_rows(w, layer, i, ctx, device="cuda") for i in range(B)]
        pool.append(layer, seqs, [0] * B, [ctx] * B, torch.cat([k for k, _ in kv]), torch.cat([v for _, v in kv]))
        del kv
    ctxs = [ctx] * B
    sp = pool.decode_splits(ctxs)
    ws = torch.empty(pool.workspace_bytes(kvq.OP_DECODE, B, sp), dtype=torch.uint8, device="cuda")
    qs = [queries(w, layer, B, device="cuda") for layer in range(L)]
    outs = [torch.empty((B, Hq, D), dtype=torch.float32, device="cuda") for _ in range(L)]
    turn = [0]

    def call():
        layer = turn[0] % L
        turn[0] += 1
        pool.decode(layer, seqs, ctxs, qs[layer], w.sm_scale, n_splits=sp, ws=ws, out=outs[layer])

    for _ in range(L):
        call()
    avg, mn, med = _call_ms(call, reps * L)
    alg = B * ppl * H * 64 * 2 * (D // 4 + 8) + B * Hq * D * (2 + 4)
    log(f"group 8: {avg * 1e3:.1f} us a call (median {med * 1e3:.1f}), splits={sp}, "
        f"{alg / (avg * 1e-3) / 1e9:.0f} GB/s against one read of the pages")
    return {"workload": "2-bit decode, 8 lanes x 40960 tokens, 4 layers x 4 KV heads x 256 dims, 32 query heads",
            "bytes_per_call": alg, "splits": sp, "us_mean": avg * 1e3, "us_median": med * 1e3, "us_min": mn * 1e3,
            "gbs_mean": alg / (avg * 1e-3) / 1e9}


def q8_leg(reps: int):
    """The 8-bit format: 24 lanes of 64 x U[16, 128] tokens, 32 layers x 8 KV
    heads x 128 dims, 32 query heads.  Populate every layer (timed, HBM bytes
    of bf16 rows read and codes written), then decode every layer (one call per
    layer for all lanes, HIP events); algorithmic bytes 268 per (token, KV
    head) plus q and out.  Then the workload's own unit, a layer step: the
    layer's decode for all lanes followed by the quantize-append of one new
    token per lane (which re-derives the open page's channel scales and codes
    from its exact rows), steps of all 32 layers timed per layer."""
    import torch

    import quantized_kv_attention_append_amd as kvq
    from synth import WORKLOADS, q8_batch_lengths, kv_rows, page_permutation, queries

    w = WORKLOADS["q8"]
    lens = [int(x) for x in q8_batch_lengths(w)]
    extra = reps + 2                       # tokens appended by the timed layer steps
    geom = (w.n_layers, w.n_kv_heads, w.head_dim, w.n_q_heads)
    _, pb = kvq.token_bytes(geom, kvq.FMT_Q8)
    n_pages = sum(-(-(L + extra) // 64) for L in lens)
    pool = kvq.Pool(n_pages * pb, geom, kvq.FMT_Q8, max_seqs=w.lanes, max_seq_tokens=max(lens) + extra)
    perm = page_permutation(w, n_pages)
    seqs, off = [], 0
    for L in lens:
        npg = -(-(L + extra) // 64)
        seqs.append(pool.reserve(L + extra, pages=perm[off:off + npg]))
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
    _hold(reps * w.n_layers)
    for _ in range(reps):  # steps of one call per layer, back to back, an event pair around each call
        for layer in range(w.n_layers):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pool.decode(layer, seqs, lens, qs[layer], w.sm_scale, n_splits=sp, ws=ws, out=outs[layer])
            e1.record(stream)
            ev.append((e0, e1))
    torch.cuda.synchronize()
    dec = _stats_us([e0.elapsed_time(e1) for e0, e1 in ev])
    avg = dec["us_mean"] * 1e-3
    alg = tokens * w.n_kv_heads * 268 + B * w.n_q_heads * w.head_dim * (2 + 4)
    # ---- layer steps: decode at the current length, then one new token per lane ----
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    new_rows = torch.randn((extra, w.n_layers, 2, B, w.n_kv_heads, w.head_dim), generator=g, device="cuda",
                           dtype=torch.float32).to(torch.bfloat16)
    cur = list(lens)
    step_ms = []
    _hold(2 * (reps + 1) * w.n_layers)
    for r in range(reps + 1):              # the first round is a warm-up
        for layer in range(w.n_layers):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pool.decode(layer, seqs, cur, qs[layer], w.sm_scale, ws=ws, out=outs[layer])
            pool.append(layer, seqs, cur, [1] * B, new_rows[r, layer, 0], new_rows[r, layer, 1])
            e1.record(stream)
            step_ms.append((r, e0, e1))
        cur = [c + 1 for c in cur]
    torch.cuda.synchronize()
    layer_step = _stats_us([e0.elapsed_time(e1) for r, e0, e1 in step_ms if r > 0])
    app_bytes = w.n_layers * tokens * w.n_kv_heads * 2 * (2 * w.head_dim) + w.n_layers * tokens * w.n_kv_heads * (
        2 * w.head_dim + 8)
    gbs = alg / (avg * 1e-3) / 1e9
    log(f"8-bit: populate {w.n_layers} layers x {tokens} tokens in {app_ms:.1f} ms; decode {avg * 1e3:.1f} us a layer "
        f"call (median {dec['us_median']:.1f}), {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s), splits={sp}; "
        f"layer step (decode + 1-token append per lane) {layer_step['us_mean']:.1f} us")
    return {"workload": "8-bit decode, 24 lanes x 64*U[16,128] tokens, 32 layers x 8 KV heads x 128 dims, 32 query heads",
            "tokens_per_layer": tokens, "pool_bytes": n_pages * pb, "splits": sp,
            "decode_us_per_layer_call": avg * 1e3, "decode_us_median": dec["us_median"], "bytes_per_call": alg,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic(Q8_TRAFFIC_FILE, Q8_SOURCES),
                         "kernel": "one kv_attn_decode call per layer: decode_q8_mfma_kernel<128, 4> then merge_splits8_kernel"},
            "kv_tokens_per_s": tokens * w.n_layers / (avg * 1e-3 * w.n_layers),
            "layer_step": {"what": "per layer: decode of all 24 lanes, then quantize-append of 1 token per lane",
                           **layer_step,
                           "step_ms_32_layers": layer_step["us_mean"] * w.n_layers * 1e-3},
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
    them over the 2-bit pool of Hadamard-rotated K rows (same pages; the
    prefill rotates the chunk's queries first)."""
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
    _hold(reps * L)
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
    # ---- chunked prefill over a pool of the same format: 65,536 prior + 1,024 chunk ----
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
              if window else
              "one kv_attn_decode call per layer: decode_q2_mfma_kernel<256, false, true, true, 8, 1> (merge inside)"
              if rotated else "one kv_attn_decode call per layer: decode_bf16_kernel<256, 4> then merge_splits8_kernel")
    return {"workload": f"27B-geometry batched decode, {name}: 16 layers x 4 KV heads x 256 dims, 16 query heads, "
                        "8 lanes x 40960 tokens", "pool_bytes": n_pages * pb, "splits": sp,
            "decode_us_per_call": avg_ms * 1e3, "bytes_per_call": alg,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": kernel},
            "graph_ms_per_step": graph_ms, "graph_identical_to_eager": same,
            "kv_tokens_per_s": B * L * ctx / (graph_ms * 1e-3),
            "populate_ms": app_ms, "populate_gbs": app_bytes / app_ms / 1e6,
            "prefill_ms_per_call": pf[0], "prefill_ms_min": pf[1], "prefill_useful_tflops": pf_tflops}


def probe_leg(pool, perm, reps: int = 10):
    """Measured ceilings for the headline kernels (libkvq_probe.so):
      * read_stream: a plain streaming read of one layer's 188.7 MB worth of
        the pool, 16 windows rotated through the 3.02 GB pool so that the
        256 MB last-level cache does not serve it;
      * read_pattern: the 2-bit decode's reads without its arithmetic: the
        (layer, KV head) blocks of every lane's 640 pages through the same
        page permutation, the decode's grid (8 lanes x 4 KV heads x 8 splits
        of 4 waves), the 16 layers in turn;
      * mfma_bf16: back-to-back bf16 matrix-core products in every wave, no
        memory traffic.
    Each call timed with HIP events, calls back to back."""
    import ctypes as C

    import torch

    path = os.path.join(ROOT, "quantized_kv_attention_append_amd", "libkvq_probe.so")
    lib = C.CDLL(path)
    lib.kvq_probe_read_stream.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_void_p, C.c_void_p]
    lib.kvq_probe_read_blocks.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int64,
                                          C.c_int64, C.c_int, C.c_void_p, C.c_void_p]
    lib.kvq_probe_read_blocks_lds.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int64,
                                              C.c_int64, C.c_void_p, C.c_void_p]
    lib.kvq_probe_mfma_bf16.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    stream = torch.cuda.current_stream()
    sp = C.c_void_p(stream.cuda_stream)
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    base, pool_bytes = pool.device_ptr()
    L, H, D, B, PPL = 16, 4, 256, 8, 640
    block = 32 * D + 1024
    page_bytes = L * H * block
    layer_bytes = B * PPL * H * block                      # 188,743,680
    bt = torch.as_tensor(perm.astype("int32"), device="cuda")

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"probe launch failed: {rc}")

    def timed(fn):
        for layer in range(L):
            fn(layer)
        torch.cuda.synchronize()
        ev = []
        _hold(reps * L)
        for _ in range(reps):
            for layer in range(L):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn(layer)
                e1.record(stream)
                ev.append((e0, e1))
        torch.cuda.synchronize()
        return _stats_us([e0.elapsed_time(e1) for e0, e1 in ev])

    stream_t = timed(lambda layer: check(lib.kvq_probe_read_stream(C.c_void_p(base + layer * layer_bytes), layer_bytes,
                                                                   16384, C.c_void_p(sink.data_ptr()), sp)))
    pattern_t = timed(lambda layer: check(lib.kvq_probe_read_blocks(
        C.c_void_p(base), C.c_void_p(bt.data_ptr()), B, PPL, H, 8, page_bytes, layer * H * block, block,
        C.c_void_p(sink.data_ptr()), sp)))
    pattern_lds_t = timed(lambda layer: check(lib.kvq_probe_read_blocks_lds(
        C.c_void_p(base), C.c_void_p(bt.data_ptr()), B, PPL, H, 8, page_bytes, layer * H * block,
        C.c_void_p(sink.data_ptr()), sp)))
    grid, iters = 1024, 2000
    mfma = []
    for shape, chains in ((0, 4), (0, 8), (1, 2), (1, 4)):
        go = lambda: check(lib.kvq_probe_mfma_bf16(shape, chains, grid, iters, C.c_void_p(sink.data_ptr()), sp))
        go()
        t = _call_ms(go, 10)
        fl = grid * 4 * iters * chains * (16384 if shape == 0 else 32768)  # 2 M N K flops an instruction
        mfma.append((fl / (t[2] * 1e-3) / 1e12, shape, chains, fl, t[2]))
    best = max(mfma)
    best_pattern = min(pattern_t, pattern_lds_t, key=lambda t: t["us_median"])
    res = {
        "read_stream": {"bytes": layer_bytes, **stream_t, "gbs_median": layer_bytes / stream_t["us_median"] / 1e3},
        "read_pattern": {"bytes": layer_bytes, **best_pattern,
                         "gbs_median": layer_bytes / best_pattern["us_median"] / 1e3,
                         "what": "the 2-bit decode's block reads at its grid (8 lanes x 4 KV heads x 8 splits of 4 "
                                 "waves), no arithmetic: the faster of register loads (two blocks in flight a wave) "
                                 "and LDS DMA staging (two page pairs in flight a wave)",
                         "register_us_median": pattern_t["us_median"], "lds_dma_us_median": pattern_lds_t["us_median"]},
        "mfma_bf16": {"flops": best[3], "us_median": best[4] * 1e3, "tflops_median": best[0],
                      "what": f"the fastest of 16x16x32 and 32x32x16 bf16 products, 2 to 8 independent chains a "
                              f"wave, 1024 x 4 waves: {'16x16x32' if best[1] == 0 else '32x32x16'} x {best[2]} chains",
                      "all_tflops": {f"{'16x16x32' if m[1] == 0 else '32x32x16'} x {m[2]}": m[0] for m in mfma}},
    }
    log(f"probes: stream read {res['read_stream']['gbs_median']:.0f} GB/s, decode read pattern "
        f"{res['read_pattern']['gbs_median']:.0f} GB/s, bf16 matrix cores {res['mfma_bf16']['tflops_median']:.0f} TFLOP/s")
    return res


# ---------------------------------------------------------------------------
# The oracle baseline: the oracle as it stands, timed on the host's cores, over
# independent units of the same workloads in a pool of worker processes with
# one BLAS thread each.  Workers never touch the GPU: each draws its unit's
# rows on the host from the workload's seeded recipe (outside the timed
# region) and times only the oracle's step.

def _cpu_init():
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import torch
    torch.set_num_threads(1)
    from threadpoolctl import threadpool_limits
    globals()["_cpu_limits"] = threadpool_limits(1)


def _cpu_q2_unit(layer, lane):
    """27B workload, one (layer, lane): per KV head, the append (quantize and
    pack the head's K and V rows into page blocks) and the decode (dequantize,
    fp64 softmax attention of the group's 4 query heads)."""
    import numpy as np

    from oracle import attention, codec, pool as opool
    from synth import WORKLOADS, kv_rows, queries
    w = WORKLOADS["27b"]
    k, v = kv_rows(w, layer, lane, w.ctx)
    q = queries(w, layer, w.lanes)[lane].float().numpy()
    kf, vf = k.float().numpy(), v.float().numpy()
    t_app = t_dec = 0.0
    for g in range(w.n_kv_heads):
        kh, vh = np.ascontiguousarray(kf[:, g:g + 1]), np.ascontiguousarray(vf[:, g:g + 1])
        t0 = time.perf_counter()
        opool.sequence_blocks("q2", kh, vh)
        t1 = time.perf_counter()
        ck, cv = codec.q2_quantize(kh), codec.q2_quantize(vh)           # the codes the pages hold (untimed)
        t2 = time.perf_counter()
        K, V = codec.q2_dequantize(*ck), codec.q2_dequantize(*cv)
        attention.decode(q[g * w.group:(g + 1) * w.group], K, V, w.sm_scale)
        t3 = time.perf_counter()
        t_app += t1 - t0
        t_dec += t3 - t2
    return {"tokens": w.ctx, "rows": 2 * w.ctx * w.n_kv_heads, "append_s": t_app, "decode_s": t_dec}


def _cpu_long_head(g):
    """Long split-K workload, KV head g: the decode of its 4 query heads with
    the keys split as the GPU splits them (whole page pairs, the same count
    in every split) at 16, 32, 64 and 128 splits; and the planted key's rank
    among the logits of query head 4g over the dequantized keys (the oracle's)
    and over the exact bf16 keys."""
    import numpy as np

    from oracle import attention, codec
    from synth import WORKLOADS, kv_rows, planted_position, queries
    from synth.workloads import plant_key
    w = WORKLOADS["long"]
    ctx = w.ctx
    k, v = kv_rows(w, 0, 0, ctx)
    q = queries(w, 0, 1)
    pos = planted_position(w, ctx)
    plant_key(k, q[0], pos, w.group)
    kh, vh = k[:, g:g + 1].float().numpy(), v[:, g:g + 1].float().numpy()
    qh = q[0, g * w.group:(g + 1) * w.group].float().numpy()
    ck, cv = codec.q2_quantize(kh), codec.q2_quantize(vh)
    res = {}
    for sp in (16, 32, 64, 128):
        t0 = time.perf_counter()
        K, V = codec.q2_dequantize(*ck)[:, 0], codec.q2_dequantize(*cv)[:, 0]
        s = attention.scores(qh, K[:, None], w.sm_scale)
        per = -(-((ctx // 64 + 1) // 2) // sp)          # page pairs a split, as the library sizes them
        bounds = [(p * per * 128, min((p + 1) * per * 128, ctx)) for p in range(sp)]
        for h in range(w.group):
            attention.merge_partials(attention.split_partials(s[h], np.asarray(V, np.float64), bounds))
        res[sp] = time.perf_counter() - t0
    K = codec.q2_dequantize(*ck)
    s_o = attention.scores(qh[:1], K, w.sm_scale)[0]
    s_x = attention.scores(qh[:1], kh, w.sm_scale)[0]
    return {"seconds": res, "rank_oracle": attention.planted_rank(s_o, pos), "rank_exact": attention.planted_rank(s_x, pos)}


def _cpu_prefill_head(g, rows):
    """Chunked prefill workload, KV head g: the chunk's append (quantize the
    1,024 new K and V rows), the read of all 66,560 keys (dequantize) and the
    causal attention of `rows` chunk rows for the group's 4 query heads."""
    import numpy as np

    from oracle import attention, codec
    from synth import WORKLOADS, kv_rows, queries
    w = WORKLOADS["prefill"]
    prior, n_q = w.ctx, w.chunk
    k, v = kv_rows(w, 0, 0, prior + n_q)
    q = queries(w, 0, n_q, stream=1)
    kh, vh = k[:, g:g + 1].float().numpy(), v[:, g:g + 1].float().numpy()
    ck_p, cv_p = codec.q2_quantize(kh[:prior]), codec.q2_quantize(vh[:prior])
    t0 = time.perf_counter()
    ck_c, cv_c = codec.q2_quantize(kh[prior:]), codec.q2_quantize(vh[prior:])
    t1 = time.perf_counter()
    K = np.concatenate([codec.q2_dequantize(*ck_p), codec.q2_dequantize(*ck_c)])
    V = np.concatenate([codec.q2_dequantize(*cv_p), codec.q2_dequantize(*cv_c)])
    t2 = time.perf_counter()
    sample = list(range(0, n_q, n_q // rows))[:rows]
    attention.prefill(q[:, g * w.group:(g + 1) * w.group].float().numpy(), K, V, w.sm_scale, prior, rows=sample)
    t3 = time.perf_counter()
    return {"append_s": t1 - t0, "read_s": t2 - t1, "rows": len(sample), "attend_s": t3 - t2}


def _cpu_q8_lane(lane):
    """8-bit workload, layer 0, one lane: the decode (dequantize every page,
    fp64 attention of 32 query heads) and the append of one more token (its V
    row; the open page's K channels re-derived from its exact rows)."""
    import numpy as np

    from oracle import attention, codec, pool as opool
    from synth import WORKLOADS, kv_rows, q8_batch_lengths, queries
    w = WORKLOADS["q8"]
    L = int(q8_batch_lengths(w)[lane])
    k, v = kv_rows(w, 0, lane, L + 1)
    q = queries(w, 0, w.lanes)[lane].float().numpy()
    kf, vf = k.float().numpy(), v.float().numpy()
    t0 = time.perf_counter()
    K, V = opool.dequantized_rows("q8", kf[:L], vf[:L])
    attention.decode(q, K, V, w.sm_scale)
    t1 = time.perf_counter()
    codec.q8_quantize_v(vf[L:L + 1])
    codec.q8_quantize_k_page(kf[L - L % 64:L + 1])
    t2 = time.perf_counter()
    return {"tokens": L, "decode_s": t1 - t0, "append_s": t2 - t1}


def cpu_baseline(budget_units: int = 32):
    """The oracle on the host's cores (see the functions above), all units in
    one pool of worker processes, one BLAS thread each."""
    import multiprocessing as mp

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    t_start = time.perf_counter()
    with mp.get_context("spawn").Pool(workers, initializer=_cpu_init) as pool:
        # the 27B units: (layer, lane) pairs spread over layers and lanes
        units = [(layer, (layer + s) % 8) for s in range(8) for layer in range(16)][:budget_units]
        jobs27 = [pool.apply_async(_cpu_q2_unit, u) for u in units]
        jobs_long = [pool.apply_async(_cpu_long_head, (g,)) for g in range(4)]
        jobs_pf = [pool.apply_async(_cpu_prefill_head, (g, 16)) for g in range(4)]
        jobs_q8 = [pool.apply_async(_cpu_q8_lane, (i,)) for i in range(24)]
        r27 = [j.get() for j in jobs27]
        rl = [j.get() for j in jobs_long]
        rp = [j.get() for j in jobs_pf]
        r8 = [j.get() for j in jobs_q8]
    wall = time.perf_counter() - t_start
    dec_s = sum(r["decode_s"] for r in r27)
    app_s = sum(r["append_s"] for r in r27)
    tokens = sum(r["tokens"] for r in r27)
    rows = sum(r["rows"] for r in r27)
    value = tokens / dec_s * workers     # worker-seconds spread over the pool's cores
    ctx_long = 131072
    par = min(workers, 4)                 # the 4 KV-head units run side by side
    long = {f"splits_{sp}": {"seconds_per_call": sum(r["seconds"][sp] for r in rl) / par,
                             "kv_tokens_per_s": ctx_long / (sum(r["seconds"][sp] for r in rl) / par)}
            for sp in (16, 32, 64, 128)}
    pf_rows = 1024
    pf_attend = sum(r["attend_s"] / r["rows"] for r in rp) * pf_rows      # worker-seconds for the whole chunk
    pf_append = sum(r["append_s"] for r in rp)
    pf_read = sum(r["read_s"] for r in rp)
    q8_dec = sum(r["decode_s"] for r in r8)
    q8_app = sum(r["append_s"] for r in r8)
    q8_tokens = sum(r["tokens"] for r in r8)
    res = {
        "value": value,
        "unit": "KV tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"27B-geometry 2-bit decode: {len(units)} (layer, lane) units of 40960 tokens x 4 KV heads "
                   f"(dequantize + fp64 softmax attention of 16 query heads), {dec_s:.1f} worker-seconds on "
                   f"{workers} worker processes with one BLAS thread each; value = tokens / worker-seconds x "
                   f"workers; rows drawn on the host from the workload's seeds, outside the timed region"),
        "wall_s": wall,
        "populate": {"rows_per_s": rows / app_s * workers,
                     "what": "quantize + pack K and V rows into page blocks, the same units"},
        "long_context": {**long, "what": "131,072-token decode of 16 query heads split as the GPU splits it, "
                                         "4 KV-head units on 4 workers"},
        "prefill": {"chunk_s": (pf_append + pf_read + pf_attend) / min(workers, 4),
                    "what": "65,536 + 1,024 chunk: append, read and causal attention of all 1,024 rows "
                            "(extrapolated from 16 sampled rows a KV head), 4 KV-head units on 4 workers"},
        "q8": {"layer_step_s": (q8_dec + q8_app) / workers, "decode_kv_tokens_per_s": q8_tokens / q8_dec * workers,
               "what": "8-bit layer 0: decode of 24 lanes then one appended token each, on the pool"},
        "planted_rank": {"oracle": [r["rank_oracle"] for r in rl], "exact_bf16": [r["rank_exact"] for r in rl]},
    }
    log(f"oracle baseline on {workers} workers ({wall:.1f} s wall): decode {value:.3g} KV tokens/s, populate "
        f"{res['populate']['rows_per_s']:.3g} rows/s, planted rank oracle {res['planted_rank']['oracle']} "
        f"exact {res['planted_rank']['exact_bf16']}")
    return res


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
    _hold(args.steps * L)
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    launch_ms = [ev[s][l][0].elapsed_time(ev[s][l][1]) for s in range(args.steps) for l in range(L)]
    region_ms = ev[0][0][0].elapsed_time(ev[-1][-1][1])
    ms_per_step = region_ms / args.steps
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    launch_stats = _stats_us(launch_ms)

    kv_bytes_per_launch = B * pages_per_lane * H * 64 * (2 * (D // 4 + 8))   # K and V rows read
    io_bytes_per_launch = B * Hq * D * 2 + B * Hq * D * 4                      # q in, fp32 out
    bytes_per_launch = kv_bytes_per_launch + io_bytes_per_launch
    achieved = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9
    tokens_per_step = B * L * ctx
    value = tokens_per_step / (ms_per_step * 1e-3)
    log(f"splits={sp} avg decode launch {avg_launch_ms * 1e3:.1f} us, step {ms_per_step:.3f} ms, "
        f"{achieved:.0f} GB/s ({100 * achieved / HBM_PEAK_GBS:.1f}% of 8 TB/s)")

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

    probes = probe_leg(pool, perm)
    median_gbs = bytes_per_launch / (launch_stats["us_median"] * 1e-6) / 1e9

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

    g8 = None if args.no_extra else group8_leg(5)
    rot = None if args.no_extra else bf16_leg(5, rotated=True)
    if rot is not None:
        # the price of the rotation: the query transform, butterflies on the K rows of append
        rot["step_time_vs_q2"] = rot["graph_ms_per_step"] / ms_per_step
        rot["populate_time_vs_q2"] = rot["populate_ms"] / app_ms
        if prefill is not None:
            rot["prefill_time_vs_q2"] = rot["prefill_ms_per_call"] / prefill["ms_per_call"]
        log(f"2-bit rotated against 2-bit: decode step {rot['step_time_vs_q2']:.3f}x the time, "
            f"populate {rot['populate_time_vs_q2']:.3f}x"
            + (f", prefill {rot['prefill_time_vs_q2']:.3f}x" if prefill is not None else ""))

    if prefill is not None:
        pt = probes["mfma_bf16"]["tflops_median"]
        prefill["roofline"]["probe"] = pt
        prefill["roofline"]["frac_of_probe"] = prefill["roofline"]["achieved"] / pt

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(args.cpu_units)
        if long_ctx is not None:
            long_ctx["planted_rank"]["oracle"] = cpu["planted_rank"]["oracle"]
            long_ctx["planted_rank"]["exact_bf16"] = cpu["planted_rank"]["exact_bf16"]

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
            "kernel": "one kv_attn_decode call per layer: decode_q2_mfma_kernel<256, false, false, true, 8, 1> "
                      "(split-K partials and their merge in one launch)",
            "bytes_per_launch": bytes_per_launch,
            "avg_launch_us": avg_launch_ms * 1e3,
            "median_launch_us": launch_stats["us_median"],
            "min_launch_us": launch_stats["us_min"],
            "median_frac": median_gbs / HBM_PEAK_GBS,
            "probe": probes["read_pattern"]["gbs_median"],
            "frac_of_probe": achieved / probes["read_pattern"]["gbs_median"],
            "probe_what": "the decode's block reads at its grid without arithmetic, GB/s (median)",
        },
        "probes": probes,
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
        "q2_group8": g8,
        "cpu_baseline": cpu,
        "platform": platform_info(),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
