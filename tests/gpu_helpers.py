"""Shared helpers for the GPU parity tests (not a test module)."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

# Tolerances for attention outputs against the fp64 oracle: max abs 2e-3 and
# relative L2 1e-3 over each compared output.
MAX_ABS = 2e-3
REL_L2 = 1e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print("[gpu-test]", *a, file=sys.stderr, flush=True)


def geom_of(w):
    return (w.n_layers, w.n_kv_heads, w.head_dim, w.n_q_heads)


def make_pool(w, n_pages, fmt, fill=0xA5, max_seqs=8, max_seq_tokens=1 << 20):
    import quantized_kv_attention_append_amd as kvq
    _, pb = kvq.token_bytes(geom_of(w), fmt)
    mem = torch.full((n_pages * pb,), fill, dtype=torch.uint8, device="cuda")
    pool = kvq.Pool(n_pages * pb, geom_of(w), fmt, max_seqs=max_seqs, max_seq_tokens=max_seq_tokens, memory=mem)
    return pool, mem


def assert_close(got, ref, what, max_abs=MAX_ABS, rel_l2=REL_L2):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    say(f"{what}: max_abs={err.max():.3e} rel_l2={rel:.3e}")
    assert err.max() <= max_abs, f"{what}: max abs error {err.max():.3e} > {max_abs}"
    assert rel <= rel_l2, f"{what}: relative L2 error {rel:.3e} > {rel_l2}"
