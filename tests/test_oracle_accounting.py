"""Oracle pins: byte accounting against the pages' printed figures."""

from oracle import accounting as A
from oracle.experiments import sizing_row


def _kv(golden):
    return {k: float(v) for k, v in golden("kv_bytes.txt")}


def test_per_head_token_bytes(golden):
    g = _kv(golden)
    assert A.q2_head_token_bytes(256) == g["q2_head_token_bytes"] == g["q2_code_bytes"] + g["q2_meta_bytes"]
    assert A.bytes_per_token(1, 1, 256, 2) / 2 == g["bf16_head_token_bytes"]


def test_27b_token_bytes_and_ratio(golden):
    g = _kv(golden)
    q2 = A.q2_token_bytes(16, 4, 256)
    bf = A.bytes_per_token(16, 4, 256, 2)
    assert q2 == g["q2_token_bytes"] == 9216
    assert bf == g["bf16_token_bytes"] == 65536
    assert round(bf / q2, 2) == g["capacity_ratio"]
    # metadata adds 8 B on top of 64 B of code
    assert 100.0 * 8 / 64 == g["metadata_overhead_pct"]


def test_eight_lanes_at_40960(golden):
    g = _kv(golden)
    lanes, toks = int(g["lanes"]), int(g["lane_tokens"])
    pages = lanes * A.pages_for_tokens(toks)
    assert pages == 5120
    pb = A.page_bytes("q2", 16, 4, 256)
    assert pb == 589824
    q2_pool = pages * pb
    assert q2_pool == 3_019_898_880
    assert round(q2_pool / 1e9, 2) == g["q2_pool_gb"]          # decimal GB, as printed
    bf_pool = lanes * toks * A.bytes_per_token(16, 4, 256, 2)
    assert bf_pool == 21_474_836_480
    assert round(bf_pool / 1024 ** 3, 1) == g["bf16_pool_gib"]  # binary GiB, as printed
    # a pool created from that byte budget holds exactly those pages
    assert A.pool_pages(q2_pool, "q2", 16, 4, 256) == 5120
    assert A.pool_pages(q2_pool - 1, "q2", 16, 4, 256) == 5119


def test_block1_sizing_table(golden):
    for name, L, H, D, kib, gib, gib8, req in golden("block1_sizing.txt"):
        r = sizing_row(int(L), int(H), int(D))
        assert f"{r['kib_per_token']:.0f}" == kib, name
        assert f"{r['ctx_gib_bf16']:.1f}" == gib, name
        assert f"{r['ctx_gib_1byte']:.1f}" == gib8, name
        assert r["requests_8k"] == int(req), name


def test_q8_geometry_page_bytes():
    # 8-bit variant at 32 layers x 8 KV heads x 128: K 128 + 8 (page-shared scales), V 128 + 4
    assert A.q8_token_bytes(32, 8, 128) == 268 * 32 * 8
    assert A.page_bytes("q8", 32, 8, 128) == 4_390_912
    # the same geometry in bf16 is the 128 KiB/token row of the sizing table
    assert A.bytes_per_token(32, 8, 128, 2) == 128 * 1024


def test_single_layer_pools():
    assert A.page_bytes("q2", 1, 4, 256) == 36864
    assert 2048 * A.page_bytes("q2", 1, 4, 256) == 75_497_472
    assert A.pool_bytes_for_tokens(65536 + 1024, "q2", 1, 4, 256) == 1040 * 36864
