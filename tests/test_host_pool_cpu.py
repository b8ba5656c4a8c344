"""The host runtime's pool, reservation, fork, release and refusal paths on
the CPU, through the C ABI of include/kvq.h.

The library's host runtime (quantized_kv_attention_append_amd/csrc/
kvq_host.cpp) is linked by g++ with a host-memory backend
(tests/hostmem/rt_hostmem.cpp): pool memory and block tables are host memory,
and no kernel runs; each launch the library asks for is recorded (kind,
layer, batch, work items, splits), and a fork's page copy is done.  The
tests check the pool's accounting ("KV at 9 KB a token", sections "How it
works" and "See it, control it": a byte budget of 64-token pages, reserved
for a request's whole bound when it is admitted; "The KV cache and prompt
reuse", section "What a sequence is made of": a lane is charged for the
pages it holds, shared prefix pages once), that every refused call leaves
the pool's bytes and the launch log unchanged ("The KV cache and prompt
reuse", section "When reuse misses": a refusal copies nothing), and
the launch plans.  test_host_runtime_under_address_sanitizer runs this file
again with the library built with -fsanitize=address.
"""

import ctypes as C
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_kv_attention_append_amd", "csrc")
SOURCES = [os.path.join(CSRC, "kvq_host.cpp"), os.path.join(ROOT, "tests", "hostmem", "rt_hostmem.cpp")]

OK, ARG, NO_SPACE, BOUND, FORMAT, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3, -4, -5, -6
Q2, Q8, BF16, Q2W, Q2R = 1, 2, 3, 4, 5
PAGE = 64


def build(out, sanitize=False):
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    if sanitize:
        cmd += ["-fsanitize=address", "-fno-omit-frame-pointer"]
    subprocess.run(cmd + SOURCES + ["-o", out], check=True, capture_output=True, text=True)
    return out


class Geom(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("n_q_heads", C.c_int32)]


class Stats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in
                ("pages", "free_pages", "reserved_pages", "used_pages", "page_bytes", "token_bytes", "tokens", "n_seqs")]


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    path = os.environ.get("KVQ_HOSTMEM_LIB") or build(str(tmp_path_factory.mktemp("hostmem") / "libkvq_hostmem.so"))
    L = C.CDLL(path)
    P, I32, I64, F = C.c_void_p, C.c_int32, C.c_int64, C.c_float
    PI32, PI64 = C.POINTER(C.c_int32), C.POINTER(C.c_int64)
    sig = {
        "kv_token_bytes": [C.POINTER(Geom), C.c_int, PI64, PI64],
        "kv_pool_create": [I64, C.POINTER(Geom), C.c_int, I32, I64, P, C.POINTER(P)],
        "kv_pool_destroy": [P], "kv_pool_stats": [P, C.POINTER(Stats)],
        "kv_pool_device_ptr": [P, C.POINTER(P), PI64],
        "kv_seq_reserve": [P, I64, PI32, PI32], "kv_seq_fork": [P, I32, I64, I64, P, PI32],
        "kv_seq_release": [P, I32], "kv_seq_pages": [P, I32, PI32, I32, PI32],
        "kv_seq_block_table": [P, I32, C.POINTER(P), PI32],
        "kv_append_quant": [P, I32, I32, PI32, PI64, PI32, P, P, P],
        "kv_workspace_bytes": [P, I32, I32, I32, PI64], "kv_decode_splits": [P, I32, PI64, PI32],
        "kv_attn_decode": [P, I32, I32, PI32, PI64, P, F, I32, P, I64, P, P, I64, P],
        "kv_attn_prefill": [P, I32, I32, I64, I32, P, F, I32, P, I64, P, P],
        "kv_dequant_page": [P, I32, I32, I32, I32, P, P],
        "kvq_hostmem_launches": [], "kvq_hostmem_launch_kind": [C.c_int], "kvq_hostmem_launch_arg": [C.c_int, C.c_int],
        "kvq_hostmem_clear": [],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = C.c_char_p if name == "kvq_hostmem_launch_kind" else (None if name == "kvq_hostmem_clear" else C.c_int)
    L.kv_last_error.restype = C.c_char_p
    return L


def i32(xs):
    return (C.c_int32 * max(1, len(xs)))(*xs)


def i64(xs):
    return (C.c_int64 * max(1, len(xs)))(*xs)


class HostPool:
    def __init__(self, lib, geom, fmt, n_pages, max_seqs=8, max_seq_tokens=4096):
        self.lib, self.geom, self.fmt = lib, Geom(*geom), fmt
        tb, pb = C.c_int64(), C.c_int64()
        assert lib.kv_token_bytes(C.byref(self.geom), fmt, C.byref(tb), C.byref(pb)) == OK
        self.page_bytes = pb.value
        self.h = C.c_void_p()
        assert lib.kv_pool_create(n_pages * pb.value, C.byref(self.geom), fmt, max_seqs, max_seq_tokens, None,
                                  C.byref(self.h)) == OK, lib.kv_last_error()
        p, n = C.c_void_p(), C.c_int64()
        assert lib.kv_pool_device_ptr(self.h, C.byref(p), C.byref(n)) == OK
        self.mem, self.bytes = p.value, n.value

    def close(self):
        assert self.lib.kv_pool_destroy(self.h) == OK

    def image(self):
        return C.string_at(self.mem, self.bytes)

    def fill(self, page, byte):
        C.memset(self.mem + page * self.page_bytes, byte, self.page_bytes)

    def stats(self):
        s = Stats()
        assert self.lib.kv_pool_stats(self.h, C.byref(s)) == OK
        return {n: getattr(s, n) for n, _ in Stats._fields_}

    def reserve(self, tokens, pages=None):
        seq = C.c_int32()
        st = self.lib.kv_seq_reserve(self.h, tokens, i32(pages) if pages is not None else None, C.byref(seq))
        return st, seq.value

    def pages(self, seq):
        n = C.c_int32()
        assert self.lib.kv_seq_pages(self.h, seq, None, 0, C.byref(n)) == OK
        arr = (C.c_int32 * max(1, n.value))()
        assert self.lib.kv_seq_pages(self.h, seq, arr, n.value, C.byref(n)) == OK
        return list(arr[:n.value])

    def fork(self, parent, n, bound):
        child = C.c_int32()
        st = self.lib.kv_seq_fork(self.h, parent, n, bound, None, C.byref(child))
        return st, child.value

    def append(self, layer, seqs, starts, counts):
        rows = sum(counts)
        buf = (C.c_uint16 * max(1, rows * self.geom.n_kv_heads * self.geom.head_dim))()
        return self.lib.kv_append_quant(self.h, layer, len(seqs), i32(seqs), i64(starts), i32(counts), C.cast(buf, C.c_void_p),
                                        C.cast(buf, C.c_void_p), None)

    def decode(self, layer, seqs, ctx, splits=0, ws_bytes=None, sm=0.0625, n=None):
        n = len(seqs) if n is None else n
        need = C.c_int64()
        sp = C.c_int32()
        if splits == 0 and n <= 128:
            self.lib.kv_decode_splits(self.h, n, i64(ctx), C.byref(sp))
        self.lib.kv_workspace_bytes(self.h, 0, n, splits or max(sp.value, 1), C.byref(need))
        ws = (C.c_uint8 * max(1, need.value if ws_bytes is None else ws_bytes))()
        q = (C.c_uint16 * max(1, n * self.geom.n_q_heads * self.geom.head_dim))()
        out = (C.c_float * max(1, n * self.geom.n_q_heads * self.geom.head_dim))()
        return self.lib.kv_attn_decode(self.h, layer, n, i32(seqs), i64(ctx), C.cast(q, C.c_void_p), sm, splits,
                                       C.cast(ws, C.c_void_p), need.value if ws_bytes is None else ws_bytes,
                                       C.cast(out, C.c_void_p), None, 0, None)


G27 = (16, 4, 256, 16)
SMALL = (2, 2, 128, 8)


def launches(lib):
    return [(lib.kvq_hostmem_launch_kind(i).decode(), [lib.kvq_hostmem_launch_arg(i, w) for w in range(4)])
            for i in range(lib.kvq_hostmem_launches())]


def test_pool_accounting(lib):
    tb, pb = C.c_int64(), C.c_int64()
    assert lib.kv_token_bytes(C.byref(Geom(*G27)), Q2, C.byref(tb), C.byref(pb)) == OK
    assert (tb.value, pb.value) == (9216, 589824)
    p = HostPool(lib, SMALL, Q2, 10)
    st = p.stats()
    assert st["pages"] == 10 and st["free_pages"] == 10 and st["tokens"] == 640
    assert st["page_bytes"] == 64 * st["token_bytes"] == 64 * 2 * 2 * 2 * (128 // 4 + 8)
    s1, a = p.reserve(200)            # 4 pages
    s2, b = p.reserve(64)             # 1 page
    assert s1 == s2 == OK
    st = p.stats()
    assert st["reserved_pages"] == 5 and st["used_pages"] == 0 and st["n_seqs"] == 2
    assert p.append(0, [a, b], [0, 0], [70, 10]) == OK
    assert p.stats()["used_pages"] == 3   # a holds tokens on 2 pages, b on 1
    assert p.lib.kv_seq_release(p.h, a) == OK
    st = p.stats()
    assert st["reserved_pages"] == 1 and st["free_pages"] == 9 and st["n_seqs"] == 1
    p.close()


def test_explicit_ids_free_stack_and_fork_take_each_page_once(lib):
    """Pages reserved by explicit id, released, re-reserved and forked, then
    the whole pool taken from the free list: every page is handed out once
    (a page pushed on the free stack twice would be taken twice)."""
    n = 12
    p = HostPool(lib, SMALL, Q2, n)
    st, a = p.reserve(3 * PAGE, pages=[7, 2, 9])
    assert st == OK and p.pages(a) == [7, 2, 9]
    st, b = p.reserve(2 * PAGE)
    assert st == OK and not set(p.pages(b)) & {7, 2, 9}
    assert lib.kv_seq_release(p.h, a) == OK
    st, c = p.reserve(2 * PAGE, pages=[2, 7])
    assert st == OK
    assert lib.kv_seq_release(p.h, c) == OK
    assert p.append(0, [b], [0], [100]) == OK
    st, d = p.fork(b, 100, 3 * PAGE)              # shares b's first page, copies its second
    assert st == OK
    assert p.pages(d)[0] == p.pages(b)[0] and p.pages(d)[1] != p.pages(b)[1]
    held = p.pages(b) + p.pages(d)[1:]
    free = p.stats()["free_pages"]
    assert free == n - len(held)
    st, e = p.reserve(free * PAGE)
    assert st == OK
    everything = held + p.pages(e)
    assert sorted(everything) == list(range(n)), everything
    assert p.stats()["free_pages"] == 0
    st, _ = p.reserve(1)
    assert st == NO_SPACE
    for s in (b, d, e):
        assert lib.kv_seq_release(p.h, s) == OK
    assert p.stats()["free_pages"] == n
    p.close()


def test_fork_copies_the_partial_page_and_counts_shared_pages_once(lib):
    p = HostPool(lib, SMALL, Q2, 8)
    st, a = p.reserve(200)
    assert p.append(0, [a], [0], [150]) == OK
    for lp, page in enumerate(p.pages(a)):
        p.fill(page, 0x10 + lp)
    st, b = p.fork(a, 150, 300)                     # pages 0, 1 shared; page 2 copied; 2 more fresh
    assert st == OK
    pa, pbs = p.pages(a), p.pages(b)
    assert pbs[:2] == pa[:2] and pbs[2] not in pa
    img = p.image()
    pgb = p.page_bytes
    assert img[pbs[2] * pgb:(pbs[2] + 1) * pgb] == img[pa[2] * pgb:(pa[2] + 1) * pgb]
    st = p.stats()
    assert st["reserved_pages"] == 4 + 3 and st["used_pages"] == 3 + 1   # shared pages once
    # neither may append into a page both hold
    before = p.image()
    assert p.append(0, [b], [100], [1]) == ARG
    assert p.append(0, [a], [60], [1]) == ARG
    assert p.image() == before
    assert lib.kv_seq_release(p.h, a) == OK
    assert p.stats()["reserved_pages"] == 5           # the shared pages stay with b
    assert lib.kv_seq_release(p.h, b) == OK
    assert p.stats()["free_pages"] == 8
    p.close()


def test_refused_calls_change_nothing(lib):
    """Every refusal returns before any byte of the pool moves and before any
    launch is asked for."""
    p = HostPool(lib, SMALL, Q2, 6, max_seqs=2, max_seq_tokens=256)
    q8 = HostPool(lib, SMALL, Q8, 4, max_seqs=2, max_seq_tokens=256)
    st, a = p.reserve(200)
    assert p.append(0, [a], [0], [100]) == OK
    st, s8 = q8.reserve(128)
    assert q8.append(0, [s8], [0], [70]) == OK
    lib.kvq_hostmem_clear()
    img, img8, stats = p.image(), q8.image(), p.stats()
    buf = (C.c_uint8 * 4096)()
    refusals = [
        (p.append(0, [a], [180], [30]), BOUND),                   # past the reserved bound
        (p.append(2, [a], [100], [1]), ARG),                      # no layer 2
        (p.append(0, [a, a], [100, 101], [1, 1]), ARG),           # one sequence twice
        (p.append(0, [5], [0], [1]), ARG),                        # not a live sequence
        (q8.append(0, [s8], [80], [1]), ARG),                     # 8-bit appends are sequential
        (p.decode(0, [a], [100], ws_bytes=16), WORKSPACE),        # workspace too small
        (p.decode(0, [a], [300]), BOUND),                         # context past the bound
        (p.decode(0, [a], [0]), ARG),
        (p.decode(0, [a], [100], sm=0.0), ARG),                   # the scale must be finite and > 0
        (p.decode(0, [a], [100], sm=float("nan")), ARG),
        (p.decode(0, [a], [100], splits=300), ARG),
        (p.decode(0, [a] * 129, [100] * 129, n=129), UNSUPPORTED),   # more than KV_MAX_BATCH
        (lib.kv_attn_prefill(q8.h, 0, s8, 0, 8, C.cast(buf, C.c_void_p), 0.1, 0, C.cast(buf, C.c_void_p), 4096,
                             C.cast(buf, C.c_void_p), None), FORMAT),   # no prefill over 8-bit pools
        (lib.kv_attn_prefill(p.h, 0, a, 90, 8, C.cast(buf, C.c_void_p), 0.1, 0, C.cast(buf, C.c_void_p), 16,
                             C.cast(buf, C.c_void_p), None), WORKSPACE),
        (lib.kv_dequant_page(p.h, 6, 0, 0, 0, C.cast(buf, C.c_void_p), None), ARG),   # no page 6
        (lib.kv_dequant_page(p.h, 0, 0, 2, 0, C.cast(buf, C.c_void_p), None), ARG),   # no head 2
        (p.reserve(300)[0], BOUND),                               # above max_seq_tokens
        (p.reserve(3 * PAGE)[0], NO_SPACE),                       # 2 pages left
        (p.reserve(PAGE, pages=[p.pages(a)[0]])[0], NO_SPACE),     # a page another sequence holds
        (p.reserve(2 * PAGE, pages=[5, 5])[0], ARG),              # a free page listed twice
        (p.fork(a, 150, 200)[0], ARG),                            # beyond the tokens appended
    ]
    for got, want in refusals:
        assert got == want, (got, want, lib.kv_last_error())
    assert p.image() == img and q8.image() == img8
    assert launches(lib) == []
    st = p.stats()
    assert st["reserved_pages"] == stats["reserved_pages"] and st["n_seqs"] == stats["n_seqs"]
    # every slot live
    p2 = HostPool(lib, SMALL, Q2, 6, max_seqs=1, max_seq_tokens=256)
    assert p2.reserve(64)[0] == OK and p2.reserve(64)[0] == NO_SPACE
    # bad geometry and format, refused before a pool exists
    h = C.c_void_p()
    assert lib.kv_pool_create(1 << 20, C.byref(Geom(2, 2, 96, 8)), Q2, 2, 256, None, C.byref(h)) == UNSUPPORTED
    assert lib.kv_pool_create(1 << 20, C.byref(Geom(2, 2, 128, 8)), 9, 2, 256, None, C.byref(h)) == FORMAT
    assert lib.kv_pool_create(100, C.byref(Geom(2, 2, 128, 8)), Q2, 2, 256, None, C.byref(h)) == NO_SPACE
    for pool in (p, q8, p2):
        pool.close()


def test_launch_plans(lib):
    p = HostPool(lib, SMALL, Q2, 16, max_seq_tokens=1024)
    _, a = p.reserve(300)
    _, b = p.reserve(200)
    lib.kvq_hostmem_clear()
    assert p.append(1, [a, b], [0, 0], [130, 64]) == OK          # a touches 3 pages, b 1
    assert launches(lib) == [("append_q2", [1, 2, 4, 0])]
    lib.kvq_hostmem_clear()
    assert p.decode(1, [a, b], [130, 64], splits=2) == OK
    kind, (layer, n, per, splits) = launches(lib)[0]
    assert (kind, layer, n, splits) == ("decode_q2", 1, 2, 2) and per == 1   # 2 page pairs over 2 splits
    # 8-bit: an append that starts inside a page and runs past it goes in two launches
    q8 = HostPool(lib, SMALL, Q8, 8, max_seq_tokens=512)
    _, s = q8.reserve(400)
    assert q8.append(0, [s], [0], [40]) == OK
    lib.kvq_hostmem_clear()
    assert q8.append(0, [s], [40], [100]) == OK
    assert [k for k, _ in launches(lib)] == ["append_q8", "append_q8"]
    # window pools: the 2-bit pages, then the rows of the last page reached
    w = HostPool(lib, SMALL, Q2W, 8, max_seq_tokens=512)
    _, s = w.reserve(400)
    lib.kvq_hostmem_clear()
    assert w.append(0, [s], [0], [150]) == OK
    assert [k for k, _ in launches(lib)] == ["append_q2", "append_window"]
    # rotated pools: prefill takes the rotated path and a query-term workspace
    r = HostPool(lib, SMALL, Q2R, 8, max_seq_tokens=512)
    _, s = r.reserve(200)
    assert r.append(0, [s], [0], [200]) == OK
    plain, rot = C.c_int64(), C.c_int64()
    lib.kv_workspace_bytes(p.h, 1, 64, 2, C.byref(plain))
    lib.kv_workspace_bytes(r.h, 1, 64, 2, C.byref(rot))
    assert rot.value - plain.value == 4 * 64 * 8 * 128
    ws = (C.c_uint8 * rot.value)()
    qb = (C.c_uint16 * (64 * 8 * 128))()
    out = (C.c_float * (64 * 8 * 128))()
    lib.kvq_hostmem_clear()
    assert lib.kv_attn_prefill(r.h, 0, s, 136, 64, C.cast(qb, C.c_void_p), 0.1, 2, C.cast(ws, C.c_void_p), rot.value,
                               C.cast(out, C.c_void_p), None) == OK
    assert launches(lib) == [("prefill_rot", [0, 64, 0, 2])]
    # the library's split count for the 27B batch: one workgroup a compute unit
    g = HostPool(lib, G27, Q2, 8 * 640, max_seq_tokens=40960)
    seqs = [g.reserve(40960)[1] for _ in range(8)]
    sp = C.c_int32()
    assert lib.kv_decode_splits(g.h, 8, i64([40960] * 8), C.byref(sp)) == OK and sp.value == 8
    # at group 8 the 2-bit decode runs two workgroups a split, so half the splits
    g2 = HostPool(lib, (16, 4, 256, 32), Q2, 8 * 640, max_seq_tokens=40960)
    for _ in range(8):
        g2.reserve(40960)
    assert lib.kv_decode_splits(g2.h, 8, i64([40960] * 8), C.byref(sp)) == OK and sp.value == 4
    g2.close()
    # and for the 8-bit batch (24 lanes of 16..124 pages, 8 KV heads x 128 dims): the most splits whose
    # workgroups with pages fit two to each of 256 compute units (472 at 4 splits, 568 at 5)
    from synth import WORKLOADS, q8_batch_lengths
    g8 = HostPool(lib, (32, 8, 128, 32), Q8, 4, max_seqs=24, max_seq_tokens=8192)
    lens = [int(x) for x in q8_batch_lengths(WORKLOADS["q8"])]
    assert lib.kv_decode_splits(g8.h, 24, i64(lens), C.byref(sp)) == OK

    def live(splits):
        pairs = [((t + 63) // 64 + 1) // 2 for t in lens]
        per = -(-max(pairs) // splits)
        return 8 * sum(-(-x // per) for x in pairs)

    assert live(sp.value) <= 512 < live(sp.value + 1), (sp.value, live(sp.value), live(sp.value + 1))
    assert sp.value == 4
    g8.close()
    # at group 8 (here 4 KV heads, 32 query heads) the decode holds one workgroup a
    # compute unit, so the workgroups with pages must fit 256 slots
    g8 = HostPool(lib, (32, 4, 128, 32), Q8, 4, max_seqs=24, max_seq_tokens=8192)
    assert lib.kv_decode_splits(g8.h, 24, i64(lens), C.byref(sp)) == OK
    live4 = lambda s: live(s) // 2  # live() counts 8 KV heads
    assert live4(sp.value) <= 256 < live4(sp.value + 1), (sp.value, live4(sp.value), live4(sp.value + 1))
    assert sp.value == 4
    g8.close()
    ptr, npg = C.c_void_p(), C.c_int32()
    assert lib.kv_seq_block_table(g.h, seqs[3], C.byref(ptr), C.byref(npg)) == OK and npg.value == 640
    assert list((C.c_int32 * 640).from_address(ptr.value)) == g.pages(seqs[3])
    for pool in (p, q8, w, r, g):
        pool.close()


@pytest.mark.slow
def test_host_runtime_under_address_sanitizer(tmp_path):
    """The tests above again, with the host runtime built with
    -fsanitize=address (heap overflows, use after free, double free in the
    page lists and block tables abort the run)."""
    if os.environ.get("KVQ_HOSTMEM_LIB"):
        pytest.skip("already the sanitized run")
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not asan or not os.path.exists(asan):
        pytest.skip("no libasan")
    lib_path = build(str(tmp_path / "libkvq_hostmem_asan.so"), sanitize=True)
    env = dict(os.environ, KVQ_HOSTMEM_LIB=lib_path, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", __file__, "-k",
                        "not address_sanitizer"], env=env, capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
