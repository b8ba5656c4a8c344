"""Byte accounting of the KV formats and the page pool.

Pinned by closed forms the pages print:
  * "Half the Cache, Twice the Context", section "Size the cache before you
    quantize it": bytes per token = 2 x layers x KV heads x head dim x bytes
    per value, and its Block 1 sizing table (tests/golden/block1_sizing.txt).
  * "KV at 9 KB a token", section "How it works" table: BF16 512 B per head per
    token, hq-e8-2b 64 B of 2-bit code + 8 B metadata = 72 B, x 128 at the
    27B geometry = 65,536 vs 9,216 B a token (7.11x, metadata +12.5%); section
    "The numbers": eight lanes at 40,960 tokens = 3.02 GB against 20.0 GiB.
"""

PAGE_TOKENS = 64  # "Pages hold 64 tokens" (KV at 9 KB a token, How it works)


def bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_value: float = 2) -> float:
    """K and V, one entry per KV head per layer per token."""
    return 2 * layers * kv_heads * head_dim * bytes_per_value


def q2_head_token_bytes(head_dim: int) -> int:
    """2-bit row: head_dim codes of 2 bits plus an 8-byte [fp32 scale, fp32 min] row."""
    assert head_dim % 4 == 0
    return head_dim // 4 + 8


def q2_token_bytes(layers: int, kv_heads: int, head_dim: int) -> int:
    return 2 * layers * kv_heads * q2_head_token_bytes(head_dim)


def q8_token_bytes(layers: int, kv_heads: int, head_dim: int) -> int:
    """int8 K and V codes, fp32 per-token V scale, fp32 per-channel K scales shared by a page."""
    per_head = 2 * head_dim + 4 + (4 * head_dim) // PAGE_TOKENS
    return layers * kv_heads * per_head


def token_bytes(fmt: str, layers: int, kv_heads: int, head_dim: int) -> int:
    """Page bytes per token.  The 2-bit format with an exact window ("q2w") has
    the 2-bit pages; its exact rows are one page per (sequence, layer, head)
    outside the page budget."""
    if fmt in ("q2", "q2w", "q2r"):
        return q2_token_bytes(layers, kv_heads, head_dim)
    if fmt == "q8":
        return q8_token_bytes(layers, kv_heads, head_dim)
    if fmt == "bf16":
        return int(bytes_per_token(layers, kv_heads, head_dim, 2))
    raise ValueError(fmt)


def page_bytes(fmt: str, layers: int, kv_heads: int, head_dim: int) -> int:
    return PAGE_TOKENS * token_bytes(fmt, layers, kv_heads, head_dim)


def pool_pages(budget_bytes: int, fmt: str, layers: int, kv_heads: int, head_dim: int) -> int:
    """A byte budget buys floor(budget / page bytes) whole pages."""
    return budget_bytes // page_bytes(fmt, layers, kv_heads, head_dim)


def pages_for_tokens(tokens: int) -> int:
    return -(-tokens // PAGE_TOKENS)


def pool_bytes_for_tokens(tokens: int, fmt: str, layers: int, kv_heads: int, head_dim: int) -> int:
    return pages_for_tokens(tokens) * page_bytes(fmt, layers, kv_heads, head_dim)
