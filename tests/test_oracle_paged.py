"""Pins of the paged-layout oracle ("AI 推理性能调优：KV Cache 优化与显存管理的工程实践",
bxzpzcl.cn/news/2871434, section 3.1 KVCacheManager and section 4).

The allocation policy is checked by hand on a sequence of requests that exercises the
free list's order, release to its end and the one-time eviction of the oldest request;
the row map by hand on a two-page table; the fragmentation and page-size closed forms
against the page's statements; gather / scatter as inverses over random tables.
"""
import numpy as np
import pytest

from oracle import paged


def test_allocation_policy_by_hand():
    m = paged.PageManager(page_size=16, max_pages=10)
    assert m.allocate("a", 33) == [0, 1, 2]          # ceil(33 / 16) = 3 pages, front first
    assert m.allocate("b", 16) == [3]
    m.release("a")                                     # back at the end of the list
    assert m.free_pages == [4, 5, 6, 7, 8, 9, 0, 1, 2]
    assert m.allocate("c", 100) == [4, 5, 6, 7, 8, 9, 0]   # 7 pages
    # 4 pages needed, 2 free: the oldest request ("b") is evicted, 3 free, still short
    with pytest.raises(MemoryError):
        m.allocate("d", 64)
    assert "b" not in m.request_pages and m.free_pages == [1, 2, 3]
    assert m.allocate("e", 48) == [1, 2, 3]


def test_page_row_by_hand():
    # P = 2, 2 KV heads, sequence table [3, 0]: positions 0, 1 in page 3, 2, 3 in page 0
    t = [3, 0]
    assert paged.page_row(t, 0, 0, 2, 2) == 12        # (3 * 2 + 0) * 2 + 0
    assert paged.page_row(t, 1, 1, 2, 2) == 15        # (3 * 2 + 1) * 2 + 1
    assert paged.page_row(t, 2, 0, 2, 2) == 0         # (0 * 2 + 0) * 2 + 0
    assert paged.page_row(t, 3, 1, 2, 2) == 3         # (0 * 2 + 1) * 2 + 1


def test_fragmentation_and_page_bytes():
    # the last page keeps page_size - (n mod page_size) empty slots (0 when it divides)
    assert paged.wasted_slots(33, 16) == 15
    assert paged.wasted_slots(32, 16) == 0
    assert paged.wasted_slots(1, 64) == 63
    for n in range(1, 300):
        for P in (16, 32, 64):
            w = paged.wasted_slots(n, P)
            assert 0 <= w < P and (n + w) % P == 0
    # smaller pages never waste more (section 4: smaller pages, less fragmentation)
    for n in range(1, 300):
        assert paged.wasted_slots(n, 16) <= paged.wasted_slots(n, 32) <= paged.wasted_slots(n, 64)
    # the page's fp16 accounting per page: 2 (K, V) * layers * kv heads * P * D * 2 bytes;
    # with a row of K + V fp16 (2 * D * 2 bytes) per position and head and 32 layers:
    # 8 KV heads, P = 16, D = 128 -> 2 MiB per page, 1024 pages -> 2 GiB
    per_layer = paged.page_bytes(8, 16, 2 * 128 * 2)
    assert 32 * per_layer == 2 * 32 * 8 * 16 * 128 * 2 == 2 << 20
    # the INT4 rows of this library (140 B per position and head at D = 128)
    assert paged.page_bytes(8, 16, 140) == 17920


@pytest.mark.parametrize("P", [16, 32, 64])
def test_gather_inverts_scatter_over_random_tables(P):
    rng = np.random.default_rng(P)
    B, H, D = 3, 2, 8
    lens = [5 * P + 3, 2 * P, 1]
    pps = 6
    pages = B * pps + 4
    table = rng.permutation(pages)[:B * pps].reshape(B, pps)
    rows = rng.standard_normal((B, H, max(lens), D))
    for b, ln in enumerate(lens):
        rows[b, :, ln:] = 0.0
    pool = paged.scatter(rows, table, lens, pages, P)
    assert pool.shape == (pages, H, P, D)
    back = paged.gather(pool, table, lens, P)
    assert np.array_equal(back, rows)
    # each used page holds positions of one sequence only, P of them for every head
    for b in range(B):
        used = (lens[b] + P - 1) // P
        for j in range(used):
            n = min(P, lens[b] - j * P)
            assert np.array_equal(pool[table[b][j], :, :n], rows[b, :, j * P:j * P + n])
