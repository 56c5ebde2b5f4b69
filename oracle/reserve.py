"""Cache-capacity reservation (TEST INFRASTRUCTURE ONLY).

Follows "Inside SGLang: DFlash and DFlash 2 Implementation", Step 2 (reserve
cache capacity before acceptance is known) and the overlap section (the next
step plans from the lengths the GPU published), with the Spec V2 PR's note
that the next step's preparation uses the prepared allocation watermark.

What the pages fix: the headroom is 2 x block_size tokens beyond the
committed prefix, page-aligned; allocating slots is not accepting tokens (the
reservation never shrinks and never changes which positions are valid); the
three lengths (committed prefix, verification extent = prefix + block,
reserved extent) are distinct.

Readings (not on the pages): a request's reservation is a list of pages in
logical order (its page-table row); physical pages come from a stack of free
pages; requests are served in batch order, each taking the pages it lacks
from the top of the stack (request 0 first); when the stack cannot cover a
request's shortfall, or the shortfall would overflow the row, that request
and every later one are left as they are and the shortage is reported;
released pages are pushed back in batch order, each request's pages in row
order.  Pinned by tests/test_oracle_reserve.py (the pages' example, the
invariants, conservation of pages).
"""
import numpy as np


def pages_needed(seq_len, block_size, page_size):
    """Pages that cover the committed prefix plus 2 x block_size tokens."""
    return -(-(int(seq_len) + 2 * int(block_size)) // int(page_size))


def reserve(seq_len, block_size, page_size, page_table, n_pages, free_pages, free_count):
    """Extend every request's reservation to pages_needed(); returns
    (page_table, n_pages, free_pages, free_count, status) as new arrays;
    status 0 = served, 1 = stopped for lack of free pages, 2 = a row too short."""
    pt = np.array(page_table, np.int64, copy=True)
    n = np.array(n_pages, np.int64, copy=True)
    stack = np.array(free_pages, np.int64, copy=True)
    top = int(free_count)
    status = 0
    for r in range(len(seq_len)):
        need = pages_needed(seq_len[r], block_size, page_size)
        short = max(0, need - int(n[r]))
        if need > pt.shape[1]:
            status = 2
            break
        if short > top:
            status = 1
            break
        for i in range(short):
            top -= 1
            pt[r, n[r] + i] = stack[top]
        n[r] += short
    return pt, n, stack, top, status


def release(mask, page_table, n_pages, free_pages, free_count):
    """Push the pages of every masked request back on the stack (batch order,
    row order) and empty its row."""
    pt = np.array(page_table, np.int64, copy=True)
    n = np.array(n_pages, np.int64, copy=True)
    stack = np.array(free_pages, np.int64, copy=True)
    top = int(free_count)
    for r in range(len(mask)):
        if mask[r]:
            for i in range(int(n[r])):
                stack[top] = pt[r, i]
                top += 1
            n[r] = 0
    return pt, n, stack, top
