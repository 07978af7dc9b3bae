"""CPU oracle for device-side page allocation -- TEST INFRASTRUCTURE
(imported only by the tests; the product library never uses it and shares
no code with it).

The pages describe the allocator only in outline ("Code Notes:
mini-sglang", Scheduler Layer table: the CacheManager row -- it manages
free_slots, the free token positions, and hands them out for new tokens;
the TableManager row -- one page_table row per request holds its KV
mapping).  The reading taken for one scheduling step:

  * the pool's free pages are the first ``num_free`` entries of a list of
    page ids; pages are taken from the tail of that list, in request order:
    the k-th page taken in the step (k = 0, 1, ...) is
    free_pages[num_free - 1 - k];
  * request r already holds ceil(P_r / page_size) pages in its page_table
    row (P_r tokens in the pool) and receives the pages its E_r new tokens
    need beyond those: ceil((P_r + E_r) / page_size) - ceil(P_r / page_size),
    written to the next entries of its row;
  * out_loc lists the slot of every new token, requests in order, token
    P_r + i of request r at page_table[row, (P_r + i) // page_size] *
    page_size + (P_r + i) % page_size;
  * a step that cannot be done -- more pages needed than are free, a row
    that would need more entries than the page table has, a negative
    length or a row index outside the table -- takes and writes nothing
    and is reported as failed.
"""

from __future__ import annotations

import numpy as np

__all__ = ["alloc_pages"]


def alloc_pages(free_pages: np.ndarray, num_free: int, page_table: np.ndarray,
                table_idx: np.ndarray, prefix_lens: np.ndarray, extend_lens: np.ndarray,
                page_size: int):
    """Returns (ok, new_num_free, new_page_table, out_loc)."""
    pt = np.array(page_table, dtype=np.int32, copy=True)
    P = np.asarray(prefix_lens, dtype=np.int64)
    E = np.asarray(extend_lens, dtype=np.int64)
    ps = int(page_size)
    rows = np.asarray(table_idx, dtype=np.int64)
    out_loc = np.zeros(max(int(E.clip(min=0).sum()), 0), dtype=np.int32)
    unchanged = (False, int(num_free), np.array(page_table, dtype=np.int32, copy=True), out_loc)
    if np.any(P < 0) or np.any(E < 0) or np.any(rows < 0) or np.any(rows >= pt.shape[0]):
        return unchanged
    have = (P + ps - 1) // ps
    need = (P + E + ps - 1) // ps - have
    if np.any(have + need > pt.shape[1]):
        return unchanged
    total = int(need.sum())
    if total > num_free:
        return unchanged
    k = 0
    t = 0
    for r in range(len(P)):
        row = int(table_idx[r])
        for j in range(int(need[r])):
            pt[row, int(have[r]) + j] = int(free_pages[num_free - 1 - k])
            k += 1
        for i in range(int(E[r])):
            pos = int(P[r]) + i
            out_loc[t] = pt[row, pos // ps] * ps + pos % ps
            t += 1
    return True, int(num_free) - total, pt, out_loc
