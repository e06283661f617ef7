"""Paged KV-cache layout (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Page cited
  [KV-opt]  "AI 推理性能调优：KV Cache 优化与显存管理的工程实践"
            (bxzpzcl.cn/news/2871434).  Section 3.1, ``KVCacheManager``: the cache is
            handed out in fixed pages of ``page_size`` tokens (16 by default) from a
            pool of ``max_pages`` (1024 by default) kept as a free list; a request of n
            tokens takes ceil(n / page_size) pages from the front of the list, evicting
            the oldest request once when the list is short and failing if it still is;
            a released request's pages go back at the end of the list.  Section 4: the
            last page of a sequence wastes the slots its tokens do not fill, and pages
            of 16-64 tokens are the usual compromise.

Layout read from the page's statement (its code manages page ids only, not the rows in
them): a page holds ``page_size`` consecutive positions of one sequence for every KV
head, so position p of sequence b, KV head h is row
``(table[b][p // P] * Hkv + h) * P + p % P`` of a pool shaped [pages, Hkv, P, ...]
(the [batch, heads, seq, head_dim] order of the same section, with the pool's pages in
place of the batch).
"""

import numpy as np


class PageManager:
    """The page's allocation policy ([KV-opt] §3.1), on page ids only."""

    def __init__(self, page_size=16, max_pages=1024):
        self.page_size = page_size
        self.max_pages = max_pages
        self.free_pages = list(range(max_pages))
        self.request_pages = {}                 # insertion order = age

    def pages_needed(self, num_tokens):
        return (num_tokens + self.page_size - 1) // self.page_size

    def allocate(self, request_id, num_tokens):
        need = self.pages_needed(num_tokens)
        if len(self.free_pages) < need:
            self.evict_oldest()
        if len(self.free_pages) < need:
            raise MemoryError(f"need {need} pages, {len(self.free_pages)} free")
        got = self.free_pages[:need]
        self.free_pages = self.free_pages[need:]
        self.request_pages[request_id] = got
        return got

    def release(self, request_id):
        if request_id in self.request_pages:
            self.free_pages.extend(self.request_pages.pop(request_id))

    def evict_oldest(self):
        if self.request_pages:
            self.release(next(iter(self.request_pages)))


def page_row(table_row, p, h, kv_heads, page_size):
    """Pool row of position p, KV head h of the sequence whose block table is table_row."""
    return (int(table_row[p // page_size]) * kv_heads + h) * page_size + p % page_size


def wasted_slots(num_tokens, page_size):
    """Slots of the last page a sequence of num_tokens leaves empty ([KV-opt] §4)."""
    pages = (num_tokens + page_size - 1) // page_size
    return pages * page_size - num_tokens


def page_bytes(kv_heads, page_size, row_bytes):
    """Bytes of one page of one layer: every KV head's page_size rows of K and V
    (row_bytes = the K + V bytes of one position and head)."""
    return kv_heads * page_size * row_bytes


def gather(pool, table, lens, page_size):
    """Logical rows [B, Hkv, N, ...] (N = max(lens)) of a pool [pages, Hkv, P, ...]
    through the block table [B, pages per sequence]; positions at or past len_b are
    left zero.  One row at a time, by ``page_row``."""
    pool = np.asarray(pool)
    pages, H, P = pool.shape[:3]
    if P != page_size:
        raise ValueError("pool page size differs from page_size")
    flat = pool.reshape((pages * H * P,) + pool.shape[3:])
    B, N = len(lens), int(max(lens))
    out = np.zeros((B, H, N) + pool.shape[3:], dtype=pool.dtype)
    for b in range(B):
        for h in range(H):
            for p in range(int(lens[b])):
                out[b, h, p] = flat[page_row(table[b], p, h, H, page_size)]
    return out


def scatter(rows, table, lens, pages, page_size):
    """The inverse of ``gather``: a pool [pages, Hkv, P, ...] holding the logical rows
    [B, Hkv, N, ...] of each sequence's first len_b positions (other rows zero)."""
    rows = np.asarray(rows)
    B, H = rows.shape[:2]
    flat = np.zeros((pages * H * page_size,) + rows.shape[3:], dtype=rows.dtype)
    for b in range(B):
        for h in range(H):
            for p in range(int(lens[b])):
                flat[page_row(table[b], p, h, H, page_size)] = rows[b, h, p]
    return flat.reshape((pages, H, page_size) + rows.shape[3:])
