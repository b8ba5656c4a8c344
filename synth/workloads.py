"""Workload shapes and seeded tensor draws (no quantize / attend arithmetic).

Every draw is keyed by ``seed_for(cfg, layer, lane, tensor_id)``: the root seed
7 (the seed of the experiments on "Half the Cache, Twice the Context", section
"What the cache loses when you round it") extended with the workload, layer,
lane and tensor number through numpy's SeedSequence.  Tensors are drawn with
torch on the requested device so that the multi-GiB workloads can be produced
directly in device memory; a test that needs the same numbers on the host
copies the tensor, it never redraws it elsewhere.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

PAGE = 64
ROOT_SEED = 7

# tensor ids inside a (cfg, layer, lane) stream
T_K, T_V, T_Q, T_PLANT, T_LEN, T_PERM = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    fmt: str            # "q2" (2-bit, hq-e8-2b-sized rows) or "q8" (int8 K per channel, V per token)
    n_layers: int
    n_kv_heads: int
    head_dim: int
    n_q_heads: int
    lanes: int
    ctx: int            # context tokens per lane (the 8-bit batch: upper bound; lengths are drawn)
    chunk: int = 0      # prefill chunk

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


# The five workloads; the first field numbers each one's seed stream.
WORKLOADS = {
    "tiny": Workload(0, "tiny decode, 1 layer, 1 lane x 256 tokens, 2-bit", "q2", 1, 4, 256, 16, 1, 256),
    "27b": Workload(1, "27B geometry decode, 16 layers, 8 lanes x 40960 tokens, 2-bit", "q2", 16, 4, 256, 16, 8, 40960),
    "long": Workload(2, "long split-K decode, 1 layer, 1 lane x 131072 tokens, 2-bit", "q2", 1, 4, 256, 16, 1, 131072),
    "prefill": Workload(3, "chunked prefill, 1 layer, 65536 prior + 1024 chunk, 2-bit", "q2", 1, 4, 256, 16, 1, 65536,
                        1024),
    "q8": Workload(4, "8-bit decode + append, 32 layers x 8 KV heads x 128, 24 lanes", "q8", 32, 8, 128, 32, 24, 8192),
}


def seed_for(cfg: int, layer: int, lane: int, tensor_id: int) -> int:
    ss = np.random.SeedSequence([ROOT_SEED, cfg, layer, lane, tensor_id])
    a, b = ss.generate_state(2, dtype=np.uint32)
    return int((int(a) << 31) ^ int(b)) & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def kv_rows(w: Workload, layer: int, lane: int, n_tokens: int, device="cpu", t0: int = 0):
    """K and V rows for logical positions [t0, t0+n_tokens) of one (layer, lane).

    Returns two bf16 tensors [n_tokens][Hkv][D].  N(0,1) draws; K channels
    with d % 16 == 0 are scaled by 4 and V tokens at logical position
    t % 64 == 0 by 6, in fp32, before rounding to bf16 (round to nearest even).
    The stream always starts at position 0, so a slice [t0, t0+n) equals the
    same rows of a longer draw.
    """
    H, D = w.n_kv_heads, w.head_dim
    total = t0 + n_tokens
    out = []
    for tid in (T_K, T_V):
        g = _gen(device, seed_for(w.cfg, layer, lane, tid))
        x = torch.randn((total, H, D), generator=g, device=device, dtype=torch.float32)
        x = x[t0:]
        if tid == T_K:
            x[:, :, ::16] *= 4.0
        else:
            pos = torch.arange(t0, total, device=device)
            x[pos % 64 == 0] *= 6.0
        out.append(x.to(torch.bfloat16).contiguous())
    return out[0], out[1]


def queries(w: Workload, layer: int, n_rows: int, device="cpu", stream: int = 0):
    """bf16 N(0,1) queries [n_rows][Hq][D] for one layer (``stream`` keys repeated steps)."""
    g = _gen(device, seed_for(w.cfg, layer, 1000 + stream, T_Q))
    x = torch.randn((n_rows, w.n_q_heads, w.head_dim), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16).contiguous()


def page_permutation(w: Workload, n_pages: int, salt: int = 0) -> np.ndarray:
    """Seeded permutation of physical page ids 0..n_pages-1 (int32)."""
    rng = np.random.default_rng(seed_for(w.cfg, salt, 0, T_PERM))
    return rng.permutation(n_pages).astype(np.int32)


def q8_batch_lengths(w: Workload) -> np.ndarray:
    """Context lengths for the 8-bit workload: 64 * UniformInt[16, 128] per lane."""
    rng = np.random.default_rng(seed_for(w.cfg, 0, 0, T_LEN))
    return (PAGE * rng.integers(16, 129, size=w.lanes)).astype(np.int64)


def planted_position(w: Workload, ctx: int) -> int:
    rng = np.random.default_rng(seed_for(w.cfg, 0, 0, T_PLANT))
    return int(rng.integers(0, ctx))


def plant_key(k: torch.Tensor, q: torch.Tensor, pos: int, group: int) -> None:
    """Overwrite key row ``pos`` of every KV head g with bf16(8 * q_{g*group} / |q_{g*group}|).

    ``k`` is [T][Hkv][D] bf16, ``q`` is [Hq][D] bf16; done in fp32 on the
    host copy of q, then rounded to bf16.
    """
    qf = q.float().cpu()
    for g in range(k.shape[1]):
        v = qf[g * group]
        row = (8.0 * v / torch.linalg.vector_norm(v)).to(torch.bfloat16)
        k[pos, g] = row.to(k.device)


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
