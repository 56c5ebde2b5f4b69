"""Relay of per-request decode state through request-pool slots (TEST
INFRASTRUCTURE ONLY).

Follows "Inside SGLang: DFlash and DFlash 2 Implementation", section "Back in
the scheduler: GPU continuation and CPU output": with overlap, the step before
the worker gathers the previous iteration's anchor and lengths for the
current request rows, the worker publishes the lengths after acceptance, and
the next draft input's anchor is stashed after the worker; the relay is
indexed by request-pool slots, so the batch can be filtered or merged between
iterations without relying on the old row order.  Also the section "The state
objects crossing the boundaries": the useful payload between iterations is
the anchor and the length state (the context already sits in the draft K/V).

Readings (not on the pages): the pool holds, per slot, the next anchor, the
committed length and the request's page-table row with its page count (the
reservation of Step 2 travels with the request); a batch is a list of
distinct pool slots; resolve copies those slots' state into batch order and
stash copies batch-order results back to the same slots; every other slot is
left as it is.  A slot outside the pool resolves to anchor 0, length 0, no
pages and a row of -1, and is skipped by stash.  Pinned by
tests/test_oracle_relay.py.
"""
from dataclasses import dataclass

import numpy as np


@dataclass
class RequestPool:
    anchor: np.ndarray       # [capacity]
    seq_len: np.ndarray      # [capacity]
    page_table: np.ndarray   # [capacity, max_pages]
    n_pages: np.ndarray      # [capacity]

    @staticmethod
    def empty(capacity, max_pages):
        return RequestPool(np.zeros(capacity, np.int64), np.zeros(capacity, np.int64),
                           np.full((capacity, max_pages), -1, np.int64),
                           np.zeros(capacity, np.int64))

    def copy(self):
        return RequestPool(self.anchor.copy(), self.seq_len.copy(), self.page_table.copy(),
                           self.n_pages.copy())


def resolve(pool, req_slots):
    """Batch-order (anchor, prefix_len, page_table, n_pages) of the requests
    in pool slots req_slots."""
    cap, mp = pool.page_table.shape
    B = len(req_slots)
    anchor = np.zeros(B, np.int64)
    L = np.zeros(B, np.int64)
    pt = np.full((B, mp), -1, np.int64)
    n = np.zeros(B, np.int64)
    for b, s in enumerate(req_slots):
        s = int(s)
        if 0 <= s < cap:
            anchor[b] = pool.anchor[s]
            L[b] = pool.seq_len[s]
            pt[b] = pool.page_table[s]
            n[b] = pool.n_pages[s]
    return anchor, L, pt, n


def stash(pool, req_slots, next_anchor, new_seq_len, page_table, n_pages):
    """A new pool in which slot req_slots[b] holds batch row b's results."""
    out = pool.copy()
    cap = pool.page_table.shape[0]
    for b, s in enumerate(req_slots):
        s = int(s)
        if 0 <= s < cap:
            out.anchor[s] = next_anchor[b]
            out.seq_len[s] = new_seq_len[b]
            out.page_table[s] = page_table[b]
            out.n_pages[s] = n_pages[b]
    return out
