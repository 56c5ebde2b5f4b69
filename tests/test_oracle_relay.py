"""Pins of the oracle's request-pool relay ("Inside SGLang: DFlash and DFlash
2 Implementation", section "Back in the scheduler: GPU continuation and CPU
output": the relay is indexed by request-pool slots, so the batch can be
filtered or merged between iterations without relying on the old row order).

* resolve after stash returns what was stashed, for any order and subset of
  slots; slots outside the batch are untouched; slots outside the pool
  resolve to the documented defaults and are skipped by stash;
* the property the pages state: decode cycles over batches that drop, add
  and reorder requests between iterations give every request exactly the
  tokens, lengths and logits it gets when decoded alone in a batch of one.
"""
import numpy as np

import oracle
from oracle.relay import RequestPool, resolve, stash
from oracle.reserve import reserve
from workloads import synth
from workloads.configs import TINY
from tests.helpers import np_weights


def test_resolve_after_stash_any_order_and_subset():
    rng = np.random.default_rng(0)
    cap, mp = 9, 6
    pool = RequestPool(rng.integers(0, 1000, cap), rng.integers(0, 500, cap),
                       rng.integers(0, 99, (cap, mp)), rng.integers(0, mp + 1, cap))
    for trial in range(20):
        B = int(rng.integers(1, cap + 1))
        slots = rng.permutation(cap)[:B]
        a = rng.integers(0, 1000, B)
        L = rng.integers(0, 500, B)
        pt = rng.integers(0, 99, (B, mp))
        n = rng.integers(0, mp + 1, B)
        new = stash(pool, slots, a, L, pt, n)
        ra, rL, rpt, rn = resolve(new, slots)
        assert np.array_equal(ra, a) and np.array_equal(rL, L)
        assert np.array_equal(rpt, pt) and np.array_equal(rn, n)
        rest = np.setdiff1d(np.arange(cap), slots)
        assert np.array_equal(new.anchor[rest], pool.anchor[rest])
        assert np.array_equal(new.seq_len[rest], pool.seq_len[rest])
        assert np.array_equal(new.page_table[rest], pool.page_table[rest])
        assert np.array_equal(new.n_pages[rest], pool.n_pages[rest])
        # resolving a permutation of the slots permutes the rows
        perm = rng.permutation(B)
        pa, pL, ppt, pn = resolve(new, slots[perm])
        assert np.array_equal(pa, a[perm]) and np.array_equal(ppt, pt[perm])
        pool = new


def test_slots_outside_the_pool():
    pool = RequestPool(np.arange(4) + 10, np.arange(4) + 20, np.arange(12).reshape(4, 3),
                       np.array([1, 2, 3, 0]))
    a, L, pt, n = resolve(pool, [2, -1, 4, 0])
    assert a.tolist() == [12, 0, 0, 10] and L.tolist() == [22, 0, 0, 20]
    assert pt[1].tolist() == [-1, -1, -1] and pt[2].tolist() == [-1, -1, -1]
    assert n.tolist() == [3, 0, 0, 1]
    new = stash(pool, [5, 1, -2], [7, 8, 9], [1, 2, 3], np.zeros((3, 3)), [0, 0, 0])
    assert new.anchor.tolist() == [10, 8, 12, 13]
    assert new.seq_len.tolist() == [20, 2, 22, 23]


def _plant(cand, commit, rand_ids, V):
    """Target choices whose greedy commit length against cand is `commit`."""
    S = cand.shape[0]
    post = np.array(rand_ids, np.int64)
    post[:commit - 1] = cand[1:commit]
    if commit < S and post[commit - 1] == cand[commit]:
        post[commit - 1] = (cand[commit] + 1) % V
    return post


def _request_inputs(cfg, n_req, seed):
    rng = np.random.default_rng(seed)
    L0 = rng.integers(20, 60, n_req)
    anchor = rng.integers(0, cfg.vocab, n_req)
    return L0, anchor


def _commit(req, k, S):
    return int(np.random.default_rng([7, req, k]).integers(1, S + 1))


def _rand_post(req, k, S, V):
    return np.random.default_rng([8, req, k]).integers(0, V, S)


def _vfeat(cfg, req, k):
    return synth.features(cfg.block_size, cfg, 1000 + 16 * req + k).numpy()


def _prefix_feat(cfg, req, L):
    return synth.features(int(L), cfg, 500 + req).numpy()


def _alone(cfg, W, req, L0, a0, n_cycles):
    """Request `req` decoded by itself: batch of one, a linear page table."""
    S, P, V = cfg.block_size, cfg.page_size, cfg.vocab
    maxp = (int(L0) + (n_cycles + 2) * S) // P + 2
    pt = np.arange(maxp)[None]
    cache = oracle.OracleCache(cfg, maxp * P)
    pos = np.arange(L0)
    oracle.project_context(cfg, W, cache, _prefix_feat(cfg, req, L0), pos, pos)
    L, a = np.array([L0]), np.array([a0])
    rec = []
    for k in range(n_cycles):
        d = oracle.draft_block(cfg, W, cache, a, L, pt)
        cand = d["candidates"][0]
        post = _plant(cand, _commit(req, k, S), _rand_post(req, k, S, V), V)
        acc = oracle.accept(cand[None], post[None], L)
        oracle.project_context(cfg, W, cache, _vfeat(cfg, req, k), d["positions"][0],
                               d["slots"][0], valid_rows=acc["commit_len"], rows_per_req=S)
        rec.append((cand.copy(), acc["out_tokens"][0].copy(), int(acc["new_seq_len"][0]),
                    d["logits"][0].copy()))
        L, a = acc["new_seq_len"], acc["next_anchor"]
    return rec


# batches of pool slots per iteration: requests leave, join and change rows
SCHEDULE = [[0, 1, 2], [2, 0], [3, 2, 1, 4], [4, 0, 3], [1, 4], [2, 3, 0, 1, 4]]


def relay_cycles(cfg, W, L0, a0, schedule, num_pages, stack0):
    """The oracle's replay of decode cycles through the relay: every request's
    prefix injected once, pages reserved for the pool, then per iteration
    resolve -> draft -> accept -> inject committed rows -> reserve -> stash.
    Returns the per-(request, its cycle) records and the final pool."""
    S, P, V = cfg.block_size, cfg.page_size, cfg.vocab
    n_req = len(L0)
    maxp = num_pages
    pool = RequestPool.empty(n_req, maxp)
    stack, top = np.array(stack0, np.int64), len(stack0)
    pool.anchor[:] = a0
    pool.seq_len[:] = L0
    # prefix pages for every request (pool order), then its context
    pool.page_table, pool.n_pages, stack, top, st = reserve(pool.seq_len, S, P, pool.page_table,
                                                            pool.n_pages, stack, top)
    assert st == 0
    cache = oracle.OracleCache(cfg, num_pages * P)
    for r in range(n_req):
        pos = np.arange(L0[r])
        slots = pool.page_table[r, pos // P] * P + pos % P
        oracle.project_context(cfg, W, cache, _prefix_feat(cfg, r, L0[r]), pos, slots)
    cyc = np.zeros(n_req, np.int64)
    rec = {}
    for batch in schedule:
        slots = np.array(batch)
        a, L, pt, n = resolve(pool, slots)
        d = oracle.draft_block(cfg, W, cache, a, L, pt)
        post = np.stack([_plant(d["candidates"][b], _commit(r, cyc[r], S),
                                _rand_post(r, cyc[r], S, V), V) for b, r in enumerate(batch)])
        acc = oracle.accept(d["candidates"], post, L)
        vf = np.concatenate([_vfeat(cfg, r, cyc[r]) for r in batch])
        oracle.project_context(cfg, W, cache, vf, d["positions"].ravel(), d["slots"].ravel(),
                               valid_rows=acc["commit_len"], rows_per_req=S)
        pt, n, stack, top, st = reserve(acc["new_seq_len"], S, P, pt, n, stack, top)
        assert st == 0
        pool = stash(pool, slots, acc["next_anchor"], acc["new_seq_len"], pt, n)
        for b, r in enumerate(batch):
            rec[(r, int(cyc[r]))] = (d["candidates"][b], acc["out_tokens"][b],
                                     int(acc["new_seq_len"][b]), d["logits"][b])
            cyc[r] += 1
    return rec, pool, cyc


def test_filtered_and_merged_batches_equal_each_request_alone():
    cfg = TINY
    W = np_weights(synth.weights(cfg, 0, "cpu"))
    n_req = 5
    L0, a0 = _request_inputs(cfg, n_req, 3)
    num_pages = 64
    stack0 = np.random.default_rng(4).permutation(num_pages)
    rec, pool, cyc = relay_cycles(cfg, W, L0, a0, SCHEDULE, num_pages, stack0)
    for r in range(n_req):
        ref = _alone(cfg, W, r, L0[r], a0[r], int(cyc[r]))
        for k in range(int(cyc[r])):
            cand, out, newL, lg = rec[(r, k)]
            rc, ro, rL, rlg = ref[k]
            assert np.array_equal(cand, rc), (r, k)
            assert np.array_equal(out, ro), (r, k)
            assert newL == rL, (r, k)
            assert np.allclose(lg, rlg, rtol=1e-12, atol=1e-12), (r, k)
        assert pool.seq_len[r] == ref[-1][2]
