"""Python binding of libkvq: a paged, quantized KV cache with attention that
reads the compressed pages, for MI355X (gfx950).

Thin argument marshalling over the C ABI of include/kvq.h.  torch supplies
device memory and streams; every step of the path (quantize-append, split-K
decode and merge, prefill, page dequantization) runs in the library's HIP
kernels.  Errors surface as ``KvError`` carrying the C status name.
"""

from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence

import torch

from ._lib import Geom, KvError, PoolStats, check, lib

__all__ = ["Geom", "KvError", "Pool", "FMT_Q2", "FMT_Q8", "FMT_BF16", "FMT_Q2_WINDOW", "FMT_Q2_ROT", "OP_DECODE", "OP_PREFILL", "token_bytes",
           "pool_bytes_for_tokens", "lib"]

FMT_Q2, FMT_Q8, FMT_BF16, FMT_Q2_WINDOW, FMT_Q2_ROT = 1, 2, 3, 4, 5
OP_DECODE, OP_PREFILL = 0, 1
PAGE = 64
MAX_BATCH = 128


def _geom(g) -> Geom:
    if isinstance(g, Geom):
        return g
    return Geom(*[int(x) for x in g])


def token_bytes(geom, fmt: int):
    tb, pb = C.c_int64(), C.c_int64()
    check(lib.kv_token_bytes(C.byref(_geom(geom)), fmt, C.byref(tb), C.byref(pb)))
    return tb.value, pb.value


def pool_bytes_for_tokens(geom, fmt: int, tokens: int) -> int:
    b = C.c_int64()
    check(lib.kv_pool_bytes_for_tokens(C.byref(_geom(geom)), fmt, int(tokens), C.byref(b)))
    return b.value


def _i32(xs):
    a = (C.c_int32 * len(xs))(*[int(x) for x in xs])
    return a


def _i64(xs):
    return (C.c_int64 * len(xs))(*[int(x) for x in xs])


def _same_length(n: int, **lists):
    """The library reads one entry per sequence from each per-sequence array
    (it takes no length for them): a shorter list would be read past its end."""
    for name, xs in lists.items():
        if len(xs) != n:
            raise ValueError(f"{name} has {len(xs)} entries for {n} sequences")


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str, shape=None, device=None):
    """Device pointer of a contiguous tensor, after the checks that keep the
    kernels inside it: device, dtype, layout and (where the library takes no
    size for it) shape."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the pool on {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")
    return C.c_void_p(t.data_ptr())


# Pools released while the current stream is capturing a HIP graph: their
# destruction frees device memory, which would invalidate the capture, so it
# waits for the next release or pool creation outside a capture.
_deferred = []


def _capturing() -> bool:
    return torch.cuda.is_available() and torch.cuda.is_current_stream_capturing()


def _flush_deferred():
    while _deferred and not _capturing():
        h, _memory = _deferred.pop()
        check(lib.kv_pool_destroy(h))


class Pool:
    """A byte-budgeted pool of 64-token pages in one KV format."""

    def __init__(self, budget_bytes: int, geom, fmt: int = FMT_Q2, max_seqs: int = 64,
                 max_seq_tokens: int = 1 << 20, memory: Optional[torch.Tensor] = None):
        self.geom = _geom(geom)
        self.fmt = fmt
        _flush_deferred()
        self._memory = memory  # keeps caller memory alive
        self.device = torch.device("cuda", torch.cuda.current_device())  # the library allocates here
        h = C.c_void_p()
        d_mem = C.c_void_p(0)
        if memory is not None:
            if memory.dtype != torch.uint8 or not memory.is_cuda or not memory.is_contiguous():
                raise TypeError("memory must be a contiguous uint8 device tensor")
            if memory.device != self.device:
                raise ValueError(f"memory is on {memory.device}, the current device is {self.device}")
            if memory.numel() < budget_bytes:
                raise ValueError("memory is smaller than the budget")
            d_mem = C.c_void_p(memory.data_ptr())
        check(lib.kv_pool_create(int(budget_bytes), C.byref(self.geom), fmt, int(max_seqs), int(max_seq_tokens),
                                 d_mem, C.byref(h)))
        self._h = h

    # ---------------------------------------------------------- lifetime --
    def close(self):
        """Destroys the pool; inside a HIP graph capture on the current stream
        (for instance when the garbage collector drops a pool there) the
        destruction is deferred until a later release or pool creation."""
        h = getattr(self, "_h", None)
        if h:
            self._h = None
            if _capturing():
                _deferred.append((h, self._memory))
                return
            _flush_deferred()
            check(lib.kv_pool_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # ---------------------------------------------------------- metadata --
    def stats(self) -> dict:
        s = PoolStats()
        check(lib.kv_pool_stats(self._h, C.byref(s)))
        return {name: getattr(s, name) for name, _ in PoolStats._fields_}

    def device_ptr(self):
        p, n = C.c_void_p(), C.c_int64()
        check(lib.kv_pool_device_ptr(self._h, C.byref(p), C.byref(n)))
        return p.value, n.value

    def reserve(self, max_tokens: int, pages: Optional[Sequence[int]] = None) -> int:
        seq = C.c_int32()
        arr = None
        if pages is not None:
            need = -(-int(max_tokens) // PAGE)
            if len(pages) != need:
                # the library reads exactly ceil(max_tokens / 64) ids
                raise ValueError(f"pages must list {need} page ids for {max_tokens} tokens, got {len(pages)}")
            arr = _i32(pages)
        check(lib.kv_seq_reserve(self._h, int(max_tokens), arr, C.byref(seq)))
        return seq.value

    def fork(self, parent: int, n_tokens: int, max_tokens: int, stream=None) -> int:
        """A new sequence whose first n_tokens are the parent's: whole pages
        shared, the partly filled page copied; returns its id."""
        seq = C.c_int32()
        check(lib.kv_seq_fork(self._h, int(parent), int(n_tokens), int(max_tokens), _stream(stream), C.byref(seq)))
        return seq.value

    def release(self, seq: int):
        check(lib.kv_seq_release(self._h, int(seq)))

    def block_table(self, seq: int):
        """(device address, page count) of the sequence's block table: the
        int32 page ids the kernels walk, logical page i at element i."""
        p, n = C.c_void_p(), C.c_int32()
        check(lib.kv_seq_block_table(self._h, int(seq), C.byref(p), C.byref(n)))
        return p.value, n.value

    def pages(self, seq: int):
        n = C.c_int32()
        check(lib.kv_seq_pages(self._h, int(seq), None, 0, C.byref(n)))
        arr = (C.c_int32 * max(1, n.value))()
        check(lib.kv_seq_pages(self._h, int(seq), arr, n.value, C.byref(n)))
        return list(arr[:n.value])

    def workspace_bytes(self, op: int, n_rows: int, n_splits: int = 0) -> int:
        b = C.c_int64()
        check(lib.kv_workspace_bytes(self._h, op, int(n_rows), int(n_splits), C.byref(b)))
        return b.value

    def decode_splits(self, ctx_len: Sequence[int]) -> int:
        n = C.c_int32()
        check(lib.kv_decode_splits(self._h, len(ctx_len), _i64(ctx_len), C.byref(n)))
        return n.value

    # ------------------------------------------------------------- compute --
    def append(self, layer: int, seqs, start_pos, n_new, k: torch.Tensor, v: torch.Tensor, stream=None):
        """Quantize-append bf16 rows k, v [sum(n_new)][Hkv][D] for one layer."""
        n = len(seqs)
        g = self.geom
        _same_length(n, start_pos=start_pos, n_new=n_new)
        rows = sum(int(x) for x in n_new)
        for t, name in ((k, "k"), (v, "v")):
            if tuple(t.shape) != (rows, g.n_kv_heads, g.head_dim):
                raise ValueError(f"{name} must be [{rows}][{g.n_kv_heads}][{g.head_dim}], got {tuple(t.shape)}")
        check(lib.kv_append_quant(self._h, int(layer), n, _i32(seqs), _i64(start_pos), _i32(n_new),
                                  _dev(k, torch.bfloat16, "k", device=self.device),
                                  _dev(v, torch.bfloat16, "v", device=self.device), _stream(stream)))

    def decode(self, layer: int, seqs, ctx_len, q: torch.Tensor, sm_scale: float, n_splits: int = 0,
               ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               scores: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """One decode step; q bf16 [n][Hq][D] -> fp32 [n][Hq][D]."""
        n = len(seqs)
        g = self.geom
        _same_length(n, ctx_len=ctx_len)
        if tuple(q.shape) != (n, g.n_q_heads, g.head_dim):
            raise ValueError(f"q must be [{n}][{g.n_q_heads}][{g.head_dim}], got {tuple(q.shape)}")
        if out is None:
            out = torch.empty((n, g.n_q_heads, g.head_dim), dtype=torch.float32, device=q.device)
        if ws is None:
            sp = n_splits if n_splits > 0 else self.decode_splits(ctx_len)
            ws = torch.empty(self.workspace_bytes(OP_DECODE, n, sp), dtype=torch.uint8, device=q.device)
            n_splits = sp
        sc_ptr, sc_stride = C.c_void_p(0), 0
        if scores is not None:
            if scores.dim() != 3:
                raise ValueError("scores must be [n][Hq][stride]")
            sc_stride = scores.shape[-1]
            sc_ptr = _dev(scores, torch.float32, "scores", (n, g.n_q_heads, sc_stride), self.device)
        check(lib.kv_attn_decode(self._h, int(layer), n, _i32(seqs), _i64(ctx_len),
                                 _dev(q, torch.bfloat16, "q", device=self.device), float(sm_scale), int(n_splits),
                                 _dev(ws, None, "ws", device=self.device), ws.numel() * ws.element_size(),
                                 _dev(out, torch.float32, "out", (n, g.n_q_heads, g.head_dim), self.device), sc_ptr,
                                 int(sc_stride), _stream(stream)))
        return out

    def decode_static(self, layer: int, seqs, ctx_len, q: torch.Tensor, sm_scale: float, n_splits: int = 0,
                      out: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
        """decode() with the library's static device workspace instead of ws
        (kv_attn_decode_static): the library allocates nothing; out is
        allocated here only when not given."""
        n = len(seqs)
        g = self.geom
        _same_length(n, ctx_len=ctx_len)
        if tuple(q.shape) != (n, g.n_q_heads, g.head_dim):
            raise ValueError(f"q must be [{n}][{g.n_q_heads}][{g.head_dim}], got {tuple(q.shape)}")
        if out is None:
            out = torch.empty((n, g.n_q_heads, g.head_dim), dtype=torch.float32, device=q.device)
        sc_ptr, sc_stride = C.c_void_p(0), 0
        if scores is not None:
            if scores.dim() != 3:
                raise ValueError("scores must be [n][Hq][stride]")
            sc_stride = scores.shape[-1]
            sc_ptr = _dev(scores, torch.float32, "scores", (n, g.n_q_heads, sc_stride), self.device)
        check(lib.kv_attn_decode_static(self._h, int(layer), n, _i32(seqs), _i64(ctx_len),
                                        _dev(q, torch.bfloat16, "q", device=self.device), float(sm_scale),
                                        int(n_splits),
                                        _dev(out, torch.float32, "out", (n, g.n_q_heads, g.head_dim), self.device),
                                        sc_ptr, int(sc_stride), _stream(stream)))
        return out

    def prefill(self, layer: int, seq: int, q_start: int, q: torch.Tensor, sm_scale: float, n_splits: int = 0,
                ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """Causal prefill of a chunk q bf16 [n_q][Hq][D] at positions q_start.. -> fp32 [n_q][Hq][D]."""
        g = self.geom
        n_q = q.shape[0]
        if tuple(q.shape) != (n_q, g.n_q_heads, g.head_dim):
            raise ValueError(f"q must be [n_q][{g.n_q_heads}][{g.head_dim}], got {tuple(q.shape)}")
        if out is None:
            out = torch.empty((n_q, g.n_q_heads, g.head_dim), dtype=torch.float32, device=q.device)
        if ws is None:
            ws = torch.empty(self.workspace_bytes(OP_PREFILL, n_q, n_splits), dtype=torch.uint8, device=q.device)
        check(lib.kv_attn_prefill(self._h, int(layer), int(seq), int(q_start), int(n_q),
                                  _dev(q, torch.bfloat16, "q", device=self.device), float(sm_scale), int(n_splits),
                                  _dev(ws, None, "ws", device=self.device), ws.numel() * ws.element_size(),
                                  _dev(out, torch.float32, "out", (n_q, g.n_q_heads, g.head_dim), self.device),
                                  _stream(stream)))
        return out

    def dequant_page(self, page: int, layer: int, head: int, kv: int, out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
        if out is None:
            out = torch.empty((PAGE, self.geom.head_dim), dtype=torch.float32, device=self.device)
        check(lib.kv_dequant_page(self._h, int(page), int(layer), int(head), int(kv),
                                  _dev(out, torch.float32, "out", (PAGE, self.geom.head_dim), self.device),
                                  _stream(stream)))
        return out
