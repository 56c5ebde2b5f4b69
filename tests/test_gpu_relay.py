"""The request-pool relay on the GPU ("Inside SGLang ...", section "Back in
the scheduler: GPU continuation and CPU output": the relay is indexed by
request-pool slots so the batch can be filtered or merged between
iterations).

* dflash_relay_resolve / dflash_relay_stash bit-exact with oracle.relay on
  random pools, batches in any order, slots outside the pool, NULL fields;
* decode cycles resident on the device over batches that drop, add and
  reorder requests between iterations (resolve -> draft -> accept ->
  reserve -> stash -> inject committed rows), with no host synchronisation
  between iterations: candidates, emitted tokens, lengths, page tables, the
  free-page stack and the pool match the oracle's replay bit-exactly, logits
  within the fp32 tolerance (1e-4 of the row maximum).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle.relay import RequestPool, resolve as o_resolve, stash as o_stash
from oracle.reserve import reserve as o_reserve
from workloads import synth
from workloads.configs import get_workload
from tests.gpu_harness import Setup, logits_row_rel_err, dfl
from tests.helpers import paged_to_slots
from tests.test_gpu_cycle_loop import plant

pytestmark = pytest.mark.gpu


def _pool_t(p, dev):
    return [torch.from_numpy(a.astype(np.int32)).to(dev).contiguous()
            for a in (p.anchor, p.seq_len, p.page_table, p.n_pages)]


@pytest.mark.parametrize("cap,mp,B", [(9, 6, 5), (300, 37, 257), (4, 1, 4), (64, 600, 32)])
def test_relay_resolve_stash_bitexact(cap, mp, B):
    m = dfl()
    rng = np.random.default_rng(cap + mp + B)
    pool = RequestPool(rng.integers(0, 10**6, cap), rng.integers(0, 10**5, cap),
                       rng.integers(-1, 10**4, (cap, mp)), rng.integers(0, mp + 1, cap))
    slots = rng.permutation(cap)[:B].astype(np.int64)
    if B > 2:
        slots[1] = -3                     # outside the pool on both sides
        slots[2] = cap + 5
    dp = _pool_t(pool, "cuda")
    cp = m.make_request_pool(*dp)
    ds = torch.from_numpy(slots.astype(np.int32)).cuda()
    outs = [torch.full((B,), 77, dtype=torch.int32, device="cuda"),
            torch.full((B,), 77, dtype=torch.int32, device="cuda"),
            torch.full((B, mp), 77, dtype=torch.int32, device="cuda"),
            torch.full((B,), 77, dtype=torch.int32, device="cuda")]
    m.dflash_relay_resolve(cp, ds, *outs)
    torch.cuda.synchronize()
    ref = o_resolve(pool, slots)
    for g, r in zip(outs, ref):
        assert np.array_equal(g.cpu().numpy(), r)
    new = [rng.integers(0, 10**6, B), rng.integers(0, 10**5, B),
           rng.integers(-1, 10**4, (B, mp)), rng.integers(0, mp + 1, B)]
    dn = [torch.from_numpy(a.astype(np.int32)).cuda() for a in new]
    m.dflash_relay_stash(cp, ds, *dn)
    torch.cuda.synchronize()
    want = o_stash(pool, slots, *new)
    for g, r in zip(dp, (want.anchor, want.seq_len, want.page_table, want.n_pages)):
        assert np.array_equal(g.cpu().numpy(), r)
    # NULL page fields on both sides: only anchors and lengths move
    cp2 = m.make_request_pool(dp[0], dp[1])
    m.dflash_relay_stash(cp2, ds, dn[1], dn[0])
    torch.cuda.synchronize()
    w2 = o_stash(want, slots, new[1], new[0], want.page_table[np.clip(slots, 0, cap - 1)],
                 want.n_pages[np.clip(slots, 0, cap - 1)])
    assert np.array_equal(dp[0].cpu().numpy(), w2.anchor)
    assert np.array_equal(dp[2].cpu().numpy(), want.page_table)


# batches of pool slots per iteration: requests leave, join and change rows
SCHEDULE = [[0, 1, 2], [2, 0], [3, 2, 1, 4], [4, 0, 3], [1, 4], [2, 3, 0, 1, 4]]


def test_relay_cycles_filtered_and_merged_match_oracle():
    m = dfl()
    n_req = 5
    wl = dataclasses.replace(get_workload("tiny_f32"), batch=n_req, ctx=(40, 70))
    cfg = wl.cfg
    S, P, V = cfg.block_size, cfg.page_size, cfg.vocab
    st = Setup(wl, extra_tokens=2 * S, random_cache=False)
    n_cyc = {r: sum(r in b for b in SCHEDULE) for r in range(n_req)}
    L0 = st.L.numpy().astype(np.int64)
    a0 = st.anchor.numpy().astype(np.int64)
    maxp = int((L0.max() + max(n_cyc.values()) * S + 2 * S) // P) + 2
    need = -(-(L0 + 2 * S) // P)
    total = st.num_pages + 64
    pool0 = RequestPool.empty(n_req, maxp)
    pool0.anchor[:], pool0.seq_len[:] = a0, L0
    for r in range(n_req):
        pool0.page_table[r, :need[r]] = st.pt[r, :need[r]].numpy()
        pool0.n_pages[r] = need[r]
    used = set(pool0.page_table[pool0.page_table >= 0].tolist())
    stack0 = np.random.default_rng(9).permutation(
        np.array([p for p in range(total) if p not in used], np.int64))
    K, Vv = synth.kv_pool_random(cfg, total, st.seed, "cuda")
    cache = m.KVCache(K, Vv, total)
    oc = oracle.OracleCache.__new__(oracle.OracleCache)
    oc.k = [paged_to_slots(k.cpu().double().numpy(), P) for k in K]
    oc.v = [paged_to_slots(v.cpu().double().numpy(), P, transposed=True) for v in Vv]

    # per-iteration inputs, keyed by (request, its cycle), in batch order
    cyc = {r: 0 for r in range(n_req)}
    plan = []
    for batch in SCHEDULE:
        ks = [cyc[r] for r in batch]
        commit = torch.tensor([int(np.random.default_rng([7, r, k]).integers(1, S + 1))
                               for r, k in zip(batch, ks)], dtype=torch.int32)
        rand = torch.stack([synth.randint(0, V - 1, (S,), 1000 + 16 * r + k, "relay_post")
                            for r, k in zip(batch, ks)]).to(torch.int32)
        feats = torch.cat([synth.features(S, cfg, 2000 + 16 * r + k) for r, k in zip(batch, ks)])
        plan.append((torch.tensor(batch, dtype=torch.int32), commit, rand, feats))
        for r in batch:
            cyc[r] += 1
    max_prefix = int(L0.max()) + max(n_cyc.values()) * S

    # ---------------------------------------------------------------- GPU
    dev = "cuda"
    dp = _pool_t(pool0, dev)
    cp = m.make_request_pool(*dp)
    stack = torch.from_numpy(stack0.astype(np.int32)).to(dev)
    top = torch.tensor([len(stack0)], dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    dplan = [tuple(t.to(dev) for t in p) for p in plan]
    cw = st.c_weights()
    dws = m.workspace(m.draft_workspace_bytes(cfg, n_req, max_prefix))
    cws = m.workspace(m.context_workspace_bytes(cfg, n_req * S))
    rec = []
    print(f"[relay] {len(SCHEDULE)} iterations over {n_req} requests", flush=True)
    for slots, commit, rand, feats in dplan:
        B = slots.shape[0]
        anc = torch.empty(B, dtype=torch.int32, device=dev)
        Ld, npg = torch.empty_like(anc), torch.empty_like(anc)
        pt = torch.empty((B, maxp), dtype=torch.int32, device=dev)
        m.dflash_relay_resolve(cp, slots, anc, Ld, pt, npg)
        pos = torch.empty((B, S), dtype=torch.int32, device=dev)
        sl, cand = torch.empty_like(pos), torch.empty_like(pos)
        lg = torch.empty((B, S - 1, V), dtype=torch.float32, device=dev)
        m.dflash_draft_block(cfg, cw, cache, anc, Ld, pt, max_prefix, pos, sl, cand, dws,
                             logits=lg)
        post = plant(cand, commit, rand, V)
        acc = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(4)]
        out = torch.empty((B, S), dtype=torch.int32, device=dev)
        m.dflash_accept(cand, post, Ld, acc[0], acc[1], out, acc[2], acc[3])
        m.dflash_reserve_pages(acc[3], S, P, pt, npg, stack, top, status)
        m.dflash_relay_stash(cp, slots, acc[2], acc[3], pt, npg)
        m.dflash_project_context(cfg, cw, cache, feats, pos.view(-1), sl.view(-1), acc[1], B, S,
                                 cws)
        rec.append((cand, out, acc[3], lg))
    torch.cuda.synchronize()
    assert int(status.item()) == 0

    # ---------------------------------------------------------------- oracle
    W = st.np_W()
    opool = pool0.copy()
    ost, otop = stack0.copy(), len(stack0)
    for it, (slots, commit, rand, feats) in enumerate(plan):
        sl_np = slots.numpy()
        a, L, pt, n = o_resolve(opool, sl_np)
        d = oracle.draft_block(cfg, W, oc, a, L, pt)
        gcand, gout, gL, glg = (t.cpu().numpy() for t in rec[it])
        assert np.array_equal(gcand, d["candidates"]), it
        rel = logits_row_rel_err(glg, d["logits"])
        assert rel.max() < 1e-4, (it, rel.max())
        post = plant(torch.from_numpy(d["candidates"]), commit, rand, V).numpy()
        acc = oracle.accept(d["candidates"], post, L)
        assert np.array_equal(gout, acc["out_tokens"]), it
        assert np.array_equal(gL, acc["new_seq_len"]), it
        pt, n, ost, otop, s = o_reserve(acc["new_seq_len"], S, P, pt, n, ost, otop)
        assert s == 0
        opool = o_stash(opool, sl_np, acc["next_anchor"], acc["new_seq_len"], pt, n)
        oracle.project_context(cfg, W, oc, feats.numpy(), d["positions"].ravel(),
                               d["slots"].ravel(), valid_rows=acc["commit_len"], rows_per_req=S)
    for g, r in zip(dp, (opool.anchor, opool.seq_len, opool.page_table, opool.n_pages)):
        assert np.array_equal(g.cpu().numpy(), r)
    assert int(top.item()) == otop
    assert np.array_equal(stack.cpu().numpy()[:otop], ost[:otop])
