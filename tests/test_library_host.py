"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and its host-only calls (page pool, block-table rows, split planner, argument
checks) behave as specified.  No device work is launched here."""
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from workloads import INT8_LONG, LLAMA3_70B_FULL, LLAMA3_8B_LAYER, SHARED_PREFIX_MQA, TINY, make_case

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvp.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvp_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def kvp():
    import paged_kv_cache_465_amd as m
    return m


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("kvp_pool_create", "kvp_pages_alloc", "kvp_pages_free", "kvp_kv_append",
                     "kvp_paged_attention_decode"):
        assert required in names


def test_library_exports_every_declared_symbol(kvp):
    from paged_kv_cache_465_amd import _lib
    lib = _lib.load()
    names = _declared_functions()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.PROTOTYPES), "binding prototypes drift from the header"
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                             text=True).stdout
        exported = set(re.findall(r"\bT (kvp_\w+)", out))
        assert set(names) <= exported


def test_pool_bytes_match_layout(kvp):
    d = kvp.make_desc(100, 16, 8, 128, "bf16")
    kv, meta = kvp.kvp_pool_bytes(d)
    assert kv == 100 * 8 * 16 * 128 * 2 and meta == 0
    d = kvp.make_desc(10, 32, 8, 128, "int8")
    kv, meta = kvp.kvp_pool_bytes(d)
    assert kv == 10 * 8 * 32 * 128 and meta == 10 * 8 * 32 * 4
    # per page per KV head the INT8 pool holds (D + 4) bytes per token
    assert (kv + meta) / (10 * 8 * 32) == 132


@pytest.mark.parametrize("bad", [(0, 16, 8, 128), (8, 24, 8, 128), (8, 16, 0, 128),
                                 (8, 16, 8, 96)])
def test_pool_create_rejects_bad_shapes(kvp, bad):
    with pytest.raises(kvp.KvpError) as e:
        kvp.kvp_pool_create(kvp.make_desc(*bad))
    assert e.value.status == kvp.KVP_E_INVAL


def test_allocator_against_model(kvp):
    """Random alloc/ref/free sequences: what is unique (which pages are in use,
    their counts, the free count, which calls fail) matches the oracle model."""
    rng = np.random.default_rng(5)
    pool = kvp.kvp_pool_create(kvp.make_desc(40, 16, 1, 64))
    model = oracle.PoolModel(40)
    held = []
    for _ in range(3000):
        op = rng.integers(0, 3)
        if op == 0:
            n = int(rng.integers(0, 7))
            if n > model.free_count:
                with pytest.raises(kvp.KvpError) as e:
                    kvp.kvp_pages_alloc(pool, n)
                assert e.value.status == kvp.KVP_E_NOPAGES
            else:
                ids = kvp.kvp_pages_alloc(pool, n).tolist()
                model.check_alloc(n, ids)
                held += ids
        elif op == 1 and held:
            ids = [held[i] for i in rng.integers(0, len(held), size=int(rng.integers(1, 4)))]
            kvp.kvp_pages_ref(pool, ids)
            model.share(ids)
            held += ids
        elif op == 2 and held:
            k = int(rng.integers(0, len(held)))
            ids = [held.pop(k)]
            kvp.kvp_pages_free(pool, ids)
            model.free(ids)
        assert kvp.kvp_pool_free_count(pool) == model.free_count
        for p in range(40):
            assert kvp.kvp_pool_refcount(pool, p) == model.refcount(p)
    pool.close()


def test_allocator_error_paths_leave_state(kvp):
    pool = kvp.kvp_pool_create(kvp.make_desc(4, 16, 1, 64))
    a = kvp.kvp_pages_alloc(pool, 3)
    with pytest.raises(kvp.KvpError):
        kvp.kvp_pages_alloc(pool, 2)                 # only one left: nothing taken
    assert kvp.kvp_pool_free_count(pool) == 1
    with pytest.raises(kvp.KvpError):
        kvp.kvp_pages_free(pool, [a[0], a[0]])       # freed twice, held once
    assert kvp.kvp_pool_refcount(pool, int(a[0])) == 1
    with pytest.raises(kvp.KvpError):
        kvp.kvp_pages_free(pool, [a[1], 4])          # out of range: nothing freed
    assert kvp.kvp_pool_refcount(pool, int(a[1])) == 1
    free_page = ({0, 1, 2, 3} - set(a.tolist())).pop()
    with pytest.raises(kvp.KvpError):
        kvp.kvp_pages_ref(pool, [free_page])         # cannot share a free page
    kvp.kvp_pages_free(pool, a)
    assert kvp.kvp_pool_free_count(pool) == 4
    assert kvp.kvp_pool_refcount(pool, 9) == -1
    pool.close()


def test_block_table_rows_shared_prefix(kvp):
    """The shared-prefix workload built with the library's row helpers: every
    sequence references the 125 prefix pages; unique pages = eq. 2's count."""
    cfg = SHARED_PREFIX_MQA
    case = make_case(cfg, with_data=False)
    P = cfg.page_size
    pool = kvp.kvp_pool_create(kvp.make_desc(case.num_pages, P, 1, 128))
    rows = np.full((cfg.batch, case.max_blocks), -1, dtype=np.int32)
    kvp.kvp_seq_grow(pool, rows[0], 0, int(case.ctx[0]))
    n_prefix = cfg.shared_prefix // P
    for b in range(1, cfg.batch):
        kvp.kvp_seq_share(pool, rows[0], rows[b], n_prefix)
        kvp.kvp_seq_grow(pool, rows[b], cfg.shared_prefix, int(case.ctx[b]))
    used = np.unique(rows[rows >= 0])
    assert used.size == 3325 == case.num_pages - kvp.kvp_pool_free_count(pool)
    assert all(kvp.kvp_pool_refcount(pool, int(p)) == cfg.batch for p in rows[0, :n_prefix])
    for b in range(cfg.batch):
        assert (rows[b, :n_prefix] == rows[0, :n_prefix]).all()
    for b in range(cfg.batch):
        kvp.kvp_seq_release(pool, rows[b], -(-int(case.ctx[b]) // P))
    assert kvp.kvp_pool_free_count(pool) == case.num_pages
    pool.close()


@pytest.mark.parametrize("cfg", [TINY, LLAMA3_8B_LAYER, LLAMA3_70B_FULL, INT8_LONG,
                                 SHARED_PREFIX_MQA], ids=lambda c: c.name)
@pytest.mark.parametrize("req", [0, 1, 3])
def test_planner_covers_every_block(kvp, cfg, req):
    case = make_case(cfg, with_data=False)
    d = kvp.make_desc(case.num_pages, cfg.page_size, cfg.num_kv_heads, cfg.head_dim, cfg.kv_dtype)
    mx = int(case.ctx.max())
    plan = kvp.kvp_decode_plan(d, cfg.batch, cfg.num_q_heads, mx, req, 256)
    nblk = -(-mx // cfg.page_size)
    S, pps = plan["num_splits"], plan["pages_per_split"]
    assert S >= 1 and S * pps >= nblk and (S - 1) * pps < nblk
    if req:
        assert S == min(req, nblk) or S <= req
    assert plan["use_mfma"] == (cfg.group >= 4)
    g = cfg.group
    hp = -(-g // 16) * 16 if plan["use_mfma"] else g
    lds = plan["waves_per_group"] * (g * cfg.head_dim + 2 * hp +
                                     (0 if plan["use_mfma"] else g * cfg.page_size)) * 4
    assert lds <= 65536
    parts = cfg.batch * cfg.num_q_heads * S
    if S == 1:
        assert plan["workspace_bytes"] == 0
    else:
        assert plan["workspace_bytes"] >= parts * (cfg.head_dim + 2) * 4


def test_planner_rejects_bad_groups(kvp):
    d = kvp.make_desc(16, 16, 8, 128)
    with pytest.raises(kvp.KvpError):
        kvp.kvp_decode_plan(d, 4, 12, 100)   # 12 q heads over 8 KV heads
    with pytest.raises(kvp.KvpError) as e:
        kvp.kvp_decode_plan(d, 4, 8 * 65, 100)
    assert e.value.status == kvp.KVP_E_UNSUPPORTED


def test_host_pool_under_sanitizers(tmp_path):
    """pool.cpp built alone with g++ -fsanitize=address,undefined and driven by
    random operation sequences checked against a shadow model."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "pool_check"
    src = os.path.join(ROOT, "paged_kv_cache_465_amd", "csrc", "pool.cpp")
    drv = os.path.join(ROOT, "tests", "native", "pool_check.cpp")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}", src, drv,
           "-o", str(exe)]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"


def test_merge_and_partials_argument_checks(kvp):
    """Argument errors of the two-phase entry points come back as
    KVP_E_INVAL before any device work."""
    from paged_kv_cache_465_amd import _lib
    lib = _lib.load()
    import ctypes
    dummy = ctypes.c_void_p(16)          # never dereferenced: every call below fails its checks
    assert lib.kvp_lse_merge(dummy, -1, 2, 128, dummy, None) == kvp.KVP_E_INVAL
    assert lib.kvp_lse_merge(dummy, 4, 0, 128, dummy, None) == kvp.KVP_E_INVAL
    assert lib.kvp_lse_merge(dummy, 4, 2, 96, dummy, None) == kvp.KVP_E_INVAL
    assert lib.kvp_lse_merge(None, 4, 2, 128, dummy, None) == kvp.KVP_E_INVAL
    assert lib.kvp_lse_merge(dummy, 4, 2, 128, None, None) == kvp.KVP_E_INVAL
    assert lib.kvp_lse_merge(None, 0, 2, 128, None, None) == kvp.KVP_OK  # nothing to do
    d = kvp.make_desc(64, 16, 8, 128, "bf16")
    pool = kvp.kvp_pool_create(d)
    ns = ctypes.c_int32()
    # H_q not a multiple of H_kv; negative batch; max_context_len beyond the table
    assert lib.kvp_paged_attention_decode_partials(
        pool.handle, dummy, dummy, dummy, None, None, dummy, 4, dummy, 2, 12, 64, 0.1, 0, dummy,
        1 << 20, ctypes.byref(ns), None) == kvp.KVP_E_INVAL
    assert lib.kvp_paged_attention_decode_partials(
        pool.handle, dummy, dummy, dummy, None, None, dummy, 4, dummy, -1, 64, 64, 0.1, 0, dummy,
        1 << 20, ctypes.byref(ns), None) == kvp.KVP_E_INVAL
    assert lib.kvp_paged_attention_decode_partials(
        pool.handle, dummy, dummy, dummy, None, None, dummy, 4, dummy, 2, 64, 65, 0.1, 0, dummy,
        1 << 20, ctypes.byref(ns), None) == kvp.KVP_E_INVAL
    # INT8 metadata given to a bf16 pool
    assert lib.kvp_paged_attention_decode_partials(
        pool.handle, dummy, dummy, dummy, dummy, dummy, dummy, 4, dummy, 2, 64, 64, 0.1, 0, dummy,
        1 << 20, ctypes.byref(ns), None) == kvp.KVP_E_INVAL
    pool.close()


@pytest.mark.parametrize("P,n,sink,window", [(16, 300, 4, 64), (16, 300, 0, 17), (32, 1000, 40, 100),
                                             (16, 100, 90, 20), (16, 33, 0, 1), (32, 65, 31, 2)])
def test_evict_window_frees_the_oracle_blocks(kvp, P, n, sink, window):
    """kvp_seq_evict_window releases exactly the blocks that hold no kept
    position (derived by the oracle from the kept set), leaves the others,
    and is idempotent; a shared page only loses one reference."""
    d = kvp.make_desc(64, P, 1, 64, "bf16")
    pool = kvp.kvp_pool_create(d)
    mb = -(-n // P)
    row = np.full(mb, -1, dtype=np.int32)
    kvp.kvp_seq_grow(pool, row, 0, n)
    other = np.full(mb, -1, dtype=np.int32)
    kvp.kvp_seq_share(pool, row, other, 1)              # block 0 shared by a second sequence
    before = row.copy()
    free0 = kvp.kvp_pool_free_count(pool)
    kvp.kvp_seq_evict_window(pool, row, n, sink, window)
    dropped = oracle.window_evicted_blocks(n, P, sink, window)
    for i in range(mb):
        if i in dropped:
            assert row[i] == -1
        else:
            assert row[i] == before[i]
    freed_pages = [before[i] for i in dropped if not (i == 0)]
    assert kvp.kvp_pool_free_count(pool) == free0 + len(freed_pages)
    if 0 in dropped:
        assert kvp.kvp_pool_refcount(pool, int(before[0])) == 1   # still held by `other`
    kvp.kvp_seq_evict_window(pool, row, n, sink, window)          # idempotent
    assert kvp.kvp_pool_free_count(pool) == free0 + len(freed_pages)
    with pytest.raises(kvp.KvpError):
        kvp.kvp_seq_evict_window(pool, row, n, sink, 0)
    pool.close()


# ---- prefix cache ("KV-Cache Optimization Techniques", section "Prefix Caching") ----
def _rand_requests(rng, n_req, P, vocab=3):
    """Token lists that share prefixes of random whole-block lengths."""
    seqs = []
    for _ in range(n_req):
        if seqs and rng.random() < 0.8:
            src = seqs[int(rng.integers(0, len(seqs)))]
            cut = int(rng.integers(0, len(src) // P + 1)) * P
            toks = src[:cut] + rng.integers(0, vocab, int(rng.integers(1, 4 * P))).tolist()
        else:
            toks = rng.integers(0, vocab, int(rng.integers(1, 6 * P))).tolist()
        seqs.append(toks)
    return seqs


def test_prefix_cache_matches_the_model(kvp):
    """Random requests with shared prefixes: every match returns the pages the
    oracle's prefix model names, and every page's reference count equals the
    sequences plus the cache holding it."""
    P = 16
    rng = np.random.default_rng(21)
    d = kvp.make_desc(4096, P, 1, 64, "bf16")
    pool = kvp.kvp_pool_create(d)
    cache = kvp.kvp_prefix_cache_create(pool)
    model = oracle.PrefixModel(P)
    holders = {}           # page -> references held by live sequences
    live = []
    for toks in _rand_requests(rng, 150, P):
        got = kvp.kvp_prefix_match(cache, toks)
        assert got.tolist() == model.match(toks)
        n_blocks = -(-len(toks) // P)
        row = np.full(n_blocks, -1, dtype=np.int32)
        row[:got.size] = got
        kvp.kvp_seq_grow(pool, row, got.size * P, len(toks))
        for p in row:
            holders[int(p)] = holders.get(int(p), 0) + 1
        kvp.kvp_prefix_insert(cache, toks, row)
        model.insert(toks, row)
        live.append(row)
        if rng.random() < 0.3:                       # a request completes
            done = live.pop(int(rng.integers(0, len(live))))
            pages = done.copy()
            kvp.kvp_seq_release(pool, done, done.size)     # sets the row to -1
            for p in pages:
                holders[int(p)] -= 1
        cached = set(model.blocks.values())
        assert kvp.kvp_prefix_cache_pages(cache) == len(cached)
        for p in set(holders) | cached:
            assert kvp.kvp_pool_refcount(pool, p) == holders.get(p, 0) + (p in cached), p
    # eviction releases only pages no sequence holds, and they go back to the free list
    free0 = kvp.kvp_pool_free_count(pool)
    only_cache = [p for p in model.blocks.values() if holders.get(p, 0) == 0]
    freed = kvp.kvp_prefix_evict(cache, 10**6)
    assert freed == len(only_cache)
    assert kvp.kvp_pool_free_count(pool) == free0 + freed
    for p in set(model.blocks.values()) - set(only_cache):
        assert kvp.kvp_pool_refcount(pool, p) == holders[p] + 1
    cache.close()                                    # drops the cache's remaining references
    for p in list(holders):
        assert kvp.kvp_pool_refcount(pool, p) == holders[p]
    for row in live:
        kvp.kvp_seq_release(pool, row, row.size)
    assert kvp.kvp_pool_free_count(pool) == 4096
    pool.close()


def test_prefix_cache_evicts_least_recently_used_first(kvp):
    """Three unrelated prompts cached at increasing times; the first is then
    matched again (most recent).  Evicting as many pages as the second prompt
    holds removes exactly the second prompt's pages."""
    P = 16
    d = kvp.make_desc(256, P, 1, 64, "bf16")
    pool = kvp.kvp_pool_create(d)
    cache = kvp.kvp_prefix_cache_create(pool)
    prompts = [[i] * (3 * P) for i in (1, 2, 3)]
    rows = []
    for toks in prompts:
        row = np.full(3, -1, dtype=np.int32)
        kvp.kvp_seq_grow(pool, row, 0, len(toks))
        kvp.kvp_prefix_insert(cache, toks, row)
        kvp.kvp_seq_release(pool, row.copy(), 3)     # the request completes; the cache keeps them
        rows.append(row)
    again = kvp.kvp_prefix_match(cache, prompts[0])
    kvp.kvp_pages_free(pool, again)
    assert kvp.kvp_prefix_evict(cache, 3) == 3
    for p in rows[1]:
        assert kvp.kvp_pool_refcount(pool, int(p)) == 0
    for p in np.concatenate([rows[0], rows[2]]):
        assert kvp.kvp_pool_refcount(pool, int(p)) == 1
    # a partly shared chain: a leaf goes before the node it hangs from
    assert kvp.kvp_prefix_evict(cache, 1) == 1
    assert kvp.kvp_prefix_cache_pages(cache) == 5
    cache.close()
    assert kvp.kvp_pool_free_count(pool) == 256
    pool.close()


def test_prepare_append_copies_shared_partial_page(kvp):
    """Forking a sequence mid-page shares its last page; the first append on
    either side gets a private copy of that page (and fresh pages beyond);
    whole shared pages are never copied."""
    P = 16
    d = kvp.make_desc(64, P, 1, 64, "bf16")
    pool = kvp.kvp_pool_create(d)
    a = np.full(8, -1, dtype=np.int32)
    kvp.kvp_seq_grow(pool, a, 0, 40)                 # 3 pages, last one holds 8 tokens
    b = np.full(8, -1, dtype=np.int32)
    kvp.kvp_seq_share(pool, a, b, 3)                 # fork: b shares all three
    before = a.copy()
    copies = kvp.kvp_seq_prepare_append(pool, b, 40, 60)  # 20 more: partial page + 1 new
    assert len(copies) == 1 and copies[0][0] == before[2]
    assert b[2] == copies[0][1] and b[2] != before[2] and b[3] >= 0
    assert (b[:2] == before[:2]).all() and (a == before).all()
    assert kvp.kvp_pool_refcount(pool, int(before[2])) == 1     # now a's alone
    assert kvp.kvp_pool_refcount(pool, int(b[2])) == 1
    assert kvp.kvp_seq_prepare_append(pool, a, 40, 41) == []  # a's last page is private again
    c = np.full(8, -1, dtype=np.int32)
    kvp.kvp_seq_share(pool, a, c, 2)                 # share two whole pages only
    assert kvp.kvp_seq_prepare_append(pool, c, 32, 50) == []  # appends land in fresh pages
    # not enough pages: nothing changes
    free = kvp.kvp_pool_free_count(pool)
    row = np.full(free + 2, -1, dtype=np.int32)
    with pytest.raises(kvp.KvpError) as e:
        kvp.kvp_seq_prepare_append(pool, row, 0, 16 * (free + 1))
    assert e.value.status == kvp.KVP_E_NOPAGES and (row == -1).all()
    assert kvp.kvp_pool_free_count(pool) == free
    pool.close()


def test_host_prefix_cache_under_sanitizers(tmp_path):
    """pool.cpp + prefix_cache.cpp built with g++ -fsanitize=address,undefined
    and driven by random match/insert/release/evict sequences (leaks are
    reported by the address sanitizer at exit)."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "prefix_check"
    csrc = os.path.join(ROOT, "paged_kv_cache_465_amd", "csrc")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(csrc, "pool.cpp"), os.path.join(csrc, "prefix_cache.cpp"),
           os.path.join(ROOT, "tests", "native", "prefix_check.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"


# ---- balanced decode schedule (host) ------------------------------------------------
def _parse_schedule(words):
    nb, ni, nm, ns, ioff, moff = (int(x) for x in words[:6])
    starts = words[8:8 + nb + 1]
    items = words[ioff:ioff + 8 * ni].reshape(ni, 8)
    merge = words[moff:moff + 4 * nm].reshape(nm, 4)
    return nb, ns, starts, items, merge


def _streamed_blocks(n, P, sink, window):
    nblk = -(-n // P)
    if window <= 0:
        return nblk
    return nblk - len(oracle.window_evicted_blocks(n, P, sink, window))


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("sink,window", [(0, 0), (4, 300), (0, 17)])
def test_decode_schedule_covers_every_block_once(kvp, seed, sink, window):
    """Every (sequence, KV head) pair's streamed blocks are covered exactly once,
    in order, by consecutive items; a pair cut across bins has consecutive
    partial slots and one merge entry naming them; bins differ by at most one
    block; a pair within one bin writes its output (slot -1)."""
    rng = np.random.default_rng(100 + seed)
    P = (16, 32)[seed % 2]
    H = (1, 2, 8)[seed % 3]
    B = int(rng.integers(1, 70))
    kind = seed % 3
    if kind == 0:
        ctx = rng.integers(0, 3000, B)
    elif kind == 1:
        ctx = np.full(B, int(rng.integers(1, 5000)))
    else:
        ctx = np.where(rng.random(B) < 0.3, 0, rng.integers(1, 40000, B))
    max_blocks = int(-(-max(int(ctx.max()), 1) // P))
    cus = int(rng.choice([8, 80, 256]))
    pool = kvp.kvp_pool_create(kvp.make_desc(16, P, H, 128, "bf16"))
    s = kvp.kvp_decode_schedule(pool, ctx.astype(np.int32), 4 * H, max_blocks, cus, sink, window)
    nb, ns, starts, items, merge = _parse_schedule(s.words)
    nv = np.array([_streamed_blocks(int(n), P, sink, window) for n in ctx])
    T = int(nv.sum()) * H
    assert nb == max(1, min(cus, -(-T // 8)))
    assert starts[0] == 0 and starts[-1] == len(items) and (np.diff(starts) >= 0).all()
    loads = [int((items[starts[k]:starts[k + 1], 3] - items[starts[k]:starts[k + 1], 2]).sum())
             for k in range(nb)]
    assert sum(loads) == T
    assert max(loads) - min(loads) <= 1 if T >= nb else True
    seen = {}
    for it in items:
        seen.setdefault((int(it[0]), int(it[1])), []).append(it)
    assert set(seen) == {(b, h) for b in range(B) for h in range(H)}
    merged = {(int(m[0]), int(m[1])): (int(m[2]), int(m[3])) for m in merge}
    for (b, h), its in seen.items():
        pos = 0
        for it in its:
            assert it[2] == pos and it[3] >= it[2]
            pos = int(it[3])
        assert pos == nv[b]
        if len(its) == 1:
            assert its[0][4] == -1 and (b, h) not in merged
        else:
            slots = [int(it[4]) for it in its]
            assert slots == list(range(slots[0], slots[0] + len(its)))
            assert merged[(b, h)] == (slots[0], len(its))
            assert all(it[3] > it[2] for it in its)
    assert s.info.num_slots == ns == sum(c for _, c in merged.values())
    assert ns <= 2 * nb
    pool.close()


def test_decode_schedule_equal_lengths_need_no_merge(kvp):
    """32 sequences of 8,192 tokens, 8 KV heads, P = 16 on 256 compute units:
    one pair per bin, no partials, no workspace."""
    pool = kvp.kvp_pool_create(kvp.make_desc(16, 16, 8, 128, "bf16"))
    s = kvp.kvp_decode_schedule(pool, np.full(32, 8192, np.int32), 64, 512, 256)
    assert (s.info.num_bins, s.info.num_items, s.info.num_merge, s.info.workspace_bytes) == \
        (256, 256, 0, 0)
    pool.close()


def test_schedule_bins_rejects_bad_arguments(kvp):
    import ctypes
    from paged_kv_cache_465_amd import _lib
    lib = _lib.load()
    pool = kvp.kvp_pool_create(kvp.make_desc(16, 16, 2, 64, "bf16"))
    n = ctypes.c_int32()
    assert lib.kvp_decode_schedule_bins(None, 4, ctypes.byref(n)) == kvp.KVP_E_INVAL
    assert lib.kvp_decode_schedule_bins(pool.handle, 0, ctypes.byref(n)) == kvp.KVP_E_INVAL
    assert lib.kvp_decode_schedule_bins(pool.handle, 3, ctypes.byref(n)) == kvp.KVP_E_INVAL
    assert lib.kvp_decode_schedule_bins(pool.handle, 4, None) == kvp.KVP_E_INVAL
    pool.close()


def test_decode_schedule_rejects_bad_arguments(kvp):
    pool = kvp.kvp_pool_create(kvp.make_desc(16, 16, 2, 64, "bf16"))
    for ctx, mb in (([5, -1], 4), ([5, 65], 4)):
        with pytest.raises(kvp.KvpError):
            kvp.kvp_decode_schedule(pool, np.array(ctx, np.int32), 4, mb, 8)
    from paged_kv_cache_465_amd import _lib
    L = _lib.load()
    info = _lib.ScheduleInfo()
    ctx = np.array([10, 20], np.int32)
    small = np.zeros(4, np.int32)
    import ctypes
    st = L.kvp_decode_schedule(pool.handle, ctx.ctypes.data_as(_lib.P_int32), 2, 4, 4, 0, 0, 8,
                               small.ctypes.data_as(_lib.P_int32), small.nbytes,
                               ctypes.byref(info))
    assert st == kvp.KVP_E_INVAL
    pool.close()


def test_scheduled_decode_rejects_inconsistent_schedule_info(kvp):
    """A schedule info with partial slots but no merge entries (or merge entries
    but no slots) is not one kvp_decode_schedule builds: the scheduled decode
    refuses it on the host, before any device work (the kernels would
    otherwise be handed slots with no partials buffer behind them)."""
    import ctypes
    from paged_kv_cache_465_amd import _lib
    L = _lib.load()
    pool = kvp.kvp_pool_create(kvp.make_desc(16, 16, 2, 64, "bf16"))
    ctx = np.array([50, 100], np.int32)
    good = kvp.kvp_decode_schedule(pool, ctx, 8, 8, 3)
    assert good.info.num_merge > 0 and good.info.num_slots > 0
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the call fails on the host
    for merge, slots in ((0, good.info.num_slots), (good.info.num_merge, 0)):
        info = _lib.ScheduleInfo.from_buffer_copy(good.info)
        info.num_merge, info.num_slots = merge, slots
        st = L.kvp_paged_attention_decode_scheduled(
            pool.handle, fake, fake, fake, None, None, fake, 8, fake, 2, 8, 100, 0.125, fake,
            ctypes.byref(info), fake, None, 0, None)
        assert st == kvp.KVP_E_INVAL, (merge, slots)
    pool.close()


def test_binding_checks_shapes_before_any_call(kvp):
    """The Python wrappers compare tensor shapes and byte sizes with the pool
    descriptor before they reach the C ABI (a tensor of the wrong shape would
    otherwise let a kernel read or write past it).  CPU tensors suffice: the
    shape checks come before the device-pointer checks."""
    import torch
    desc = kvp.make_desc(8, 16, 2, 64, "int8")
    pool = kvp.kvp_pool_create(desc)
    kv_bytes, meta_bytes = kvp.kvp_pool_bytes(desc)
    kp = torch.zeros(kv_bytes, dtype=torch.int8)
    km = torch.zeros(meta_bytes // 2, dtype=torch.int16)
    bt = torch.zeros((3, 4), dtype=torch.int32)
    ctx = torch.zeros(3, dtype=torch.int32)
    q = torch.zeros((3, 8, 64), dtype=torch.int16)

    def raises(match, fn, *a):
        with pytest.raises(ValueError, match=match):
            fn(*a)

    dec = kvp.kvp_paged_attention_decode
    raises("q must be", dec, pool, q[..., :32], kp, kp, km, km, bt, ctx, 16, 0.1, q[..., :32])
    raises("multiple", dec, pool, q[:, :3], kp, kp, km, km, bt, ctx, 16, 0.1, q[:, :3])
    raises("out must", dec, pool, q, kp, kp, km, km, bt, ctx, 16, 0.1, q[:2])
    raises("cover the batch", dec, pool, q, kp, kp, km, km, bt[:2], ctx, 16, 0.1, q)
    raises("k_pool must hold", dec, pool, q, kp[:-1], kp, km, km, bt, ctx, 16, 0.1, q)
    raises("v_meta must hold", dec, pool, q, kp, kp, km, km[:-1], bt, ctx, 16, 0.1, q)
    raises("device tensor", dec, pool, q, kp, kp, km, km, bt, ctx, 16, 0.1, q)
    app = kvp.kvp_kv_append
    rows = torch.zeros((5, 2, 64), dtype=torch.int16)
    idx = torch.zeros(5, dtype=torch.int32)
    raises("k_new and v_new", app, pool, kp, kp, km, km, rows[:, :1], rows, idx, idx, bt)
    raises("k_new and v_new", app, pool, kp, kp, km, km, rows, rows[..., :32], idx, idx, bt)
    raises("k_pool must hold", app, pool, kp[:10], kp, km, km, rows, rows, idx, idx, bt)
    part = torch.zeros(100, dtype=torch.float32)
    raises("partials must hold", kvp.kvp_lse_merge, part, 3, 2, 64, torch.zeros((3, 64)))
    bf = kvp.kvp_pool_create(kvp.make_desc(8, 16, 2, 64, "bf16"))
    kb = torch.zeros(kvp.kvp_pool_bytes(bf.desc)[0] // 2, dtype=torch.int16)
    raises("take no k_meta", dec, bf, q, kb, kb, km, None, bt, ctx, 16, 0.1, q)
    bf.close()
    pool.close()


def test_read_probe_argument_checks(kvp):
    """The streaming-read probe refuses chunk sizes and ring depths it has no
    instance for, and bad counts, on the host (nothing is launched)."""
    import ctypes
    from paged_kv_cache_465_amd import _lib
    L = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    call = lambda n, chunk, depth, waves: L.kvp_probe_read_chunks(  # noqa: E731
        fake, fake, 1 << 20, fake, n, chunk, depth, waves, fake, None)
    assert call(4, 3000, 2, 4) == kvp.KVP_E_UNSUPPORTED
    assert call(4, 4096, 3, 4) == kvp.KVP_E_UNSUPPORTED
    assert call(4, 8192, 8, 4) == kvp.KVP_E_UNSUPPORTED
    assert call(-1, 4096, 2, 4) == kvp.KVP_E_INVAL
    assert call(4, 4096, 2, 0) == kvp.KVP_E_INVAL
    assert call(0, 4096, 2, 4) == kvp.KVP_OK


# ---- longest-first order of the multi-query call -------------------------------------------
def _prefill_units(dtype, B, Hkv, Hq, max_q_len, q_start, ctx):
    """The multi-query call's natural grid, as its header states it: workgroups
    of 128 rows (bfloat16), 64 or 32 rows (quantized, by chunk size) or one
    per (sequence, KV head) when every chunk's rows fit 32; groups of eight
    items, tile-major.  Returns {unit: (item, cost)} for units with rows."""
    g = Hq // Hkv
    max_rows = max_q_len * g
    split = max_rows <= 32
    quant = dtype != "bf16"
    nt = (2 if max_rows > 16 else 1) if split else (2 if max_rows >= 128 or not quant else 1)
    rows_wg = 16 * nt if split else (64 * nt if quant else 128)
    tiles = -(-max_rows // rows_wg)
    items = B * Hkv
    wgs = -(-items // 8) * 8 * tiles
    units = {}
    for u in range(wgs):
        grp, within = divmod(u, 8 * tiles)
        tile, item = within >> 3, grp * 8 + (within & 7)
        if item >= items:
            continue
        b = item // Hkv
        qlen = int(q_start[b + 1] - q_start[b])
        rows, row0 = qlen * g, 0 if split else tile * rows_wg
        if qlen <= 0 or row0 >= rows:
            continue
        n = int(ctx[b])
        pos_last = min(n - qlen + (min(row0 + rows_wg, rows) - 1) // g, n - 1)
        units[u] = (item, (pos_last // 64 + 1 if pos_last >= 0 else 0) + 1)
    return units, wgs


@pytest.mark.parametrize("seed", range(12))
def test_prefill_schedule_is_a_longest_first_permutation(kvp, seed):
    """Every unit with rows appears once; the length is a multiple of 8 with
    -1 padding; each class (position mod 8) runs its units costliest first.
    When whole items share out within 1.2x of the mean cost, all units of an
    item sit in one class and class costs differ by at most the costliest
    item; otherwise units are shared out and class costs differ by at most
    the costliest unit (greedy assignment, costliest first)."""
    rng = np.random.default_rng(500 + seed)
    dtype = ("bf16", "int8", "int4", "fp8")[seed % 4]
    Hkv = (1, 2, 8)[seed % 3]
    Hq = Hkv * int(rng.choice([1, 4, 8]))
    B = int(rng.integers(1, 40))
    P = (16, 32)[seed % 2]
    qlen = rng.integers(0, (600, 40, 4)[seed % 3] + 1, B)
    ctx = qlen + rng.integers(0, 5000, B)
    q_start = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    max_q_len = max(int(qlen.max()), 1)
    max_blocks = int(-(-int(ctx.max()) // P)) + 1
    pool = kvp.kvp_pool_create(kvp.make_desc(16, P, Hkv, 128, dtype))
    order = kvp.kvp_prefill_schedule(pool, q_start, ctx.astype(np.int32), Hq, max_blocks,
                                     max_q_len, int(ctx.max()))
    units, wgs = _prefill_units(dtype, B, Hkv, Hq, max_q_len, q_start, ctx)
    assert order.size % 8 == 0
    assert order.size <= kvp.kvp_prefill_schedule_bound(pool, B, Hq, max_blocks, max_q_len,
                                                        int(ctx.max()))
    named = order[order >= 0]
    assert sorted(named.tolist()) == sorted(units)
    assert (order[order < 0] == -1).all()
    item_cost = {}
    for it, c in units.values():
        item_cost[it] = item_cost.get(it, 0) + c
    greedy = np.zeros(8, np.int64)
    for it in sorted(item_cost, key=lambda i: (-item_cost[i], i)):
        greedy[int(np.argmin(greedy))] += item_cost[it]
    by_item = 10 * 8 * int(greedy.max()) <= 12 * int(greedy.sum())
    if by_item:
        cls = {}
        for pos, u in enumerate(order.tolist()):
            if u >= 0:
                assert cls.setdefault(units[u][0], pos % 8) == pos % 8, "an item split over XCDs"
    load = np.zeros(8, np.int64)
    for x in range(8):
        col = order[x::8]
        col = col[col >= 0]
        costs = [units[u][1] for u in col.tolist()]
        assert costs == sorted(costs, reverse=True)
        # padding only after the class's last unit
        assert (order[x::8][: len(col)] >= 0).all()
        load[x] = sum(costs)
    if item_cost:
        spread = max(item_cost.values()) if by_item else max(c for _, c in units.values())
        assert load.max() - load.min() <= spread
    pool.close()


def test_prefill_schedule_shares_out_a_lone_item(kvp):
    """One sequence, one KV head: the item's 64 row tiles go to all eight
    XCD classes (the grid order would run them all on one XCD)."""
    pool = kvp.kvp_pool_create(kvp.make_desc(16, 16, 1, 128, "bf16"))
    q_start = np.array([0, 1024], np.int32)
    ctx = np.array([8192], np.int32)
    order = kvp.kvp_prefill_schedule(pool, q_start, ctx, 8, 512, 1024, 8192)
    units, _ = _prefill_units("bf16", 1, 1, 8, 1024, q_start, ctx)
    assert len(units) == 64 and sorted(order[order >= 0].tolist()) == sorted(units)
    per_class = [int(np.count_nonzero(order[x::8] >= 0)) for x in range(8)]
    assert per_class == [8] * 8
    pool.close()


def test_prefill_schedule_shortens_the_chunked_prefill_tail(kvp):
    """The chunked-prefill workload (8 sequences, 512-token chunks on 1.5k-7.5k
    cached tokens, Llama-3-8B-shaped layer): simulated as greedy list
    scheduling over 64 workgroup slots per XCD, the order finishes sooner than
    the grid order."""
    from workloads import CHUNKED_PREFILL
    cfg = CHUNKED_PREFILL
    case = make_case(cfg, with_data=False)
    mq = int(np.diff(case.q_start).max())
    mb = case.block_tables.shape[1]
    pool = kvp.kvp_pool_create(kvp.make_desc(16, cfg.page_size, cfg.num_kv_heads, cfg.head_dim,
                                             "bf16"))
    order = kvp.kvp_prefill_schedule(pool, case.q_start, case.ctx, cfg.num_q_heads, mb, mq,
                                     int(case.ctx.max()))
    units, wgs = _prefill_units("bf16", case.B, cfg.num_kv_heads, cfg.num_q_heads, mq,
                                case.q_start, case.ctx)

    def makespan(seq):
        import heapq
        h = [0] * 64
        for u in seq:
            if u in units:
                heapq.heappush(h, heapq.heappop(h) + units[u][1])
        return max(h)
    grid = max(makespan(range(x, wgs, 8)) for x in range(8))
    ordered = max(makespan(order[x::8].tolist()) for x in range(8))
    assert ordered < grid
    pool.close()


def test_prefill_schedule_rejects_bad_arguments(kvp):
    import ctypes
    from paged_kv_cache_465_amd import _lib
    lib = _lib.load()
    pool = kvp.kvp_pool_create(kvp.make_desc(16, 16, 2, 64, "bf16"))
    n = ctypes.c_int64()
    buf = np.zeros(1024, np.int32)
    P = lambda a: a.ctypes.data_as(_lib.P_int32)  # noqa: E731
    ok_qs, ok_ctx = np.array([0, 3, 5], np.int32), np.array([10, 20], np.int32)
    assert lib.kvp_prefill_schedule(pool.handle, P(ok_qs), P(ok_ctx), 2, 8, 4, 3, 20, P(buf),
                                    buf.size, ctypes.byref(n)) == kvp.KVP_OK
    assert n.value > 0 and n.value % 8 == 0
    for qs, ctx in (([1, 3, 5], [10, 20]), ([0, 3, 2], [10, 20]), ([0, 3, 5], [10, -1])):
        qs, ctx = np.array(qs, np.int32), np.array(ctx, np.int32)
        assert lib.kvp_prefill_schedule(pool.handle, P(qs), P(ctx), 2, 8, 4, 3, 20, P(buf),
                                        buf.size, ctypes.byref(n)) == kvp.KVP_E_INVAL
    # too small a buffer: KVP_E_INVAL with the needed length reported
    assert lib.kvp_prefill_schedule(pool.handle, P(ok_qs), P(ok_ctx), 2, 8, 4, 3, 20, P(buf), 1,
                                    ctypes.byref(n)) == kvp.KVP_E_INVAL
    assert n.value > 1
    # max_context_len beyond the table, heads not a multiple of the KV heads
    assert lib.kvp_prefill_schedule(pool.handle, P(ok_qs), P(ok_ctx), 2, 8, 1, 3, 20, P(buf),
                                    buf.size, ctypes.byref(n)) == kvp.KVP_E_INVAL
    assert lib.kvp_prefill_schedule(pool.handle, P(ok_qs), P(ok_ctx), 2, 3, 4, 3, 20, P(buf),
                                    buf.size, ctypes.byref(n)) == kvp.KVP_E_INVAL
    assert lib.kvp_prefill_schedule_bound(None, 2, 8, 4, 3, 20, ctypes.byref(n)) == \
        kvp.KVP_E_INVAL
    pool.close()
