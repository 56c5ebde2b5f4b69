"""Checked mode: dflash_check_{draft,context,accept}_inputs report, per rule of
include/dflash.h, the number of violations and the smallest offending index,
bit-exactly against the rules written out below in plain Python; the calls'
`checked=True` flags raise before launching on bad inputs and run normally on
good ones.  The bad inputs go only to the check kernels (which read every
array inside its bounds) or are refused by the flag before any other kernel
runs."""
import dataclasses

import numpy as np
import pytest
import torch

from workloads.configs import get_workload
from tests.gpu_harness import Setup, dfl

pytestmark = pytest.mark.gpu

NONE = 2**31 - 1


def _print(*a):
    print(*a, flush=True)


def _pairs(found_by_rule, n):
    """[(count, first)] for rules 0..n-1 from {rule: [indices]}."""
    return [(len(found_by_rule.get(k, [])), min(found_by_rule[k]) if found_by_rule.get(k) else NONE)
            for k in range(n)]


def expected_draft(anchor, prefix_len, pt, max_prefix, S, P, vocab, num_pages, cwin):
    bad = {}
    max_pages = pt.shape[1]
    for r in range(len(anchor)):
        L_raw = int(prefix_len[r])
        if not 0 <= int(anchor[r]) < vocab:
            bad.setdefault(0, []).append(r)
        if not 0 <= L_raw <= max_prefix:
            bad.setdefault(1, []).append(r)
        if cwin == 0 and L_raw + S > max_pages * P:
            bad.setdefault(2, []).append(r)
        L = min(max(L_raw, 0), max_prefix)
        lo = max(0, L - cwin) if cwin > 0 else 0
        entries = set()
        for p in range(lo // P, (L + S - 1) // P + 1):
            if cwin > 0:
                entries.add(p % max_pages)
            elif p < max_pages:
                entries.add(p)
        for e in entries:
            if not 0 <= int(pt[r, e]) < num_pages:
                bad.setdefault(3, []).append(r * max_pages + e)
    return _pairs(bad, 4)


def expected_context(positions, slots, valid, n_req, rpr, num_slots):
    bad = {}
    for t in range(n_req * rpr):
        if valid is not None and t % rpr >= int(valid[t // rpr]):
            continue
        if not 0 <= int(slots[t]) < num_slots:
            bad.setdefault(0, []).append(t)
        if int(positions[t]) < 0:
            bad.setdefault(1, []).append(t)
    if valid is not None:
        for r in range(n_req):
            if not 0 <= int(valid[r]) <= rpr:
                bad.setdefault(2, []).append(r)
    return _pairs(bad, 4)


def expected_accept(cand, post, prefix_len, vocab):
    bad = {}
    flat_c, flat_p = cand.reshape(-1), post.reshape(-1)
    for i in range(len(flat_c)):
        if not 0 <= int(flat_c[i]) < vocab:
            bad.setdefault(0, []).append(i)
        if not 0 <= int(flat_p[i]) < vocab:
            bad.setdefault(1, []).append(i)
    for r in range(len(prefix_len)):
        if int(prefix_len[r]) < 0:
            bad.setdefault(2, []).append(r)
    return _pairs(bad, 4)


def _raw_report(fn, *args):
    """Call a dflash_check_* entry point through the C ABI; the raw report."""
    import ctypes
    m = dfl()
    rep = torch.empty(2 * m.CHECKS, dtype=torch.int32, device="cuda")
    st = fn(*args, ctypes.c_void_p(rep.data_ptr()), None)
    assert st == 0, m.raw_lib().dflash_last_error()
    torch.cuda.synchronize()
    return [tuple(x) for x in rep.view(-1, 2).cpu().tolist()]


def _draft_report(st, cfg, anchor, L, pt, max_prefix):
    import ctypes
    m = dfl()
    c_cfg, c_cache = m.make_config(cfg), st.cache.c_struct()
    d = "cuda"
    a, l, p = anchor.to(d), L.to(d), pt.to(d)
    return _raw_report(m.raw_lib().dflash_check_draft_inputs, ctypes.byref(c_cfg),
                       ctypes.byref(c_cache), ctypes.c_void_p(a.data_ptr()),
                       ctypes.c_void_p(l.data_ptr()), ctypes.c_void_p(p.data_ptr()),
                       int(pt.shape[1]), int(anchor.shape[0]), int(max_prefix))


@pytest.mark.parametrize("name,cwin", [("small_bf16", 0), ("small_swa_fp8", 0),
                                       ("small_bf16", 40), ("small_swa_fp8", 24)])
def test_check_draft_inputs(name, cwin):
    wl = get_workload(name)
    cfg = dataclasses.replace(wl.cfg, context_window=cwin)
    st = Setup(dataclasses.replace(wl, cfg=cfg))
    S, P, V = cfg.block_size, cfg.page_size, cfg.vocab
    max_prefix = int(st.L.max())
    _print(f"[checked draft] {name} window {cwin}: batch {st.B}, max prefix {max_prefix}")
    good = _draft_report(st, cfg, st.anchor, st.L, st.pt, max_prefix)
    assert good == [(0, NONE)] * 4, good
    # plant violations of every rule
    anchor, L, pt = st.anchor.clone(), st.L.clone(), st.pt.clone()
    B = st.B
    anchor[min(1, B - 1)] = V
    anchor[B - 1] = -2
    L[0] = max_prefix + 1
    if B > 2:
        L[2] = -5
    if cwin == 0:
        L[B - 1] = pt.shape[1] * P  # no room for the block in its row
    r = min(1, B - 1)
    e = min(int(st.L[r]) // P, pt.shape[1] - 1)
    pt[r, e] = st.num_pages
    pt[B - 1, 0] = -1
    got = _draft_report(st, cfg, anchor, L, pt, max_prefix)
    want = expected_draft(anchor.numpy(), L.numpy(), pt.numpy(), max_prefix, S, P, V,
                          st.num_pages, cwin)
    _print(f"  report {got}")
    assert got == want, (got, want)
    assert all(c > 0 for c, _ in got[:2]) and got[3][0] > 0


def test_check_context_inputs():
    m = dfl()
    wl = get_workload("small_bf16")
    cfg = wl.cfg
    st = Setup(wl, extra_tokens=64)
    n_slots = st.num_pages * cfg.page_size
    n_req, rpr = 4, 16
    T = n_req * rpr
    g = torch.Generator().manual_seed(3)
    slots = torch.randperm(n_slots, generator=g)[:T].to(torch.int32)
    pos = torch.randint(0, 5000, (T,), generator=g, dtype=torch.int32)
    valid = torch.tensor([16, 5, 0, 9], dtype=torch.int32)
    d = "cuda"
    assert m.check_context_inputs(cfg, st.cache, pos.to(d), slots.to(d), valid.to(d), n_req,
                                  rpr) == {}
    slots[3] = -1                      # live
    slots[16 + 7] = n_slots            # dead (row 7 of request 1, valid 5): not reported
    slots[48 + 2] = n_slots + 9        # live
    pos[16 + 1] = -4                   # live
    pos[32 + 0] = -1                   # dead (request 2 has no live rows)
    for vv in (valid, torch.tensor([17, 5, -1, 9], dtype=torch.int32)):
        import ctypes
        c_cfg, c_cache = m.make_config(cfg), st.cache.c_struct()
        p_d, s_d, v_d = pos.to(d), slots.to(d), vv.to(d)
        got = _raw_report(m.raw_lib().dflash_check_context_inputs, ctypes.byref(c_cfg),
                          ctypes.byref(c_cache), ctypes.c_void_p(p_d.data_ptr()),
                          ctypes.c_void_p(s_d.data_ptr()), ctypes.c_void_p(v_d.data_ptr()),
                          n_req, rpr)
        want = expected_context(pos.numpy(), slots.numpy(), vv.numpy(), n_req, rpr, n_slots)
        _print(f"[checked context] valid {vv.tolist()}: {got}")
        assert got == want, (got, want)
    # every row live when valid_rows is NULL
    found = m.check_context_inputs(cfg, st.cache, pos.to(d), slots.to(d), None, n_req, rpr)
    want = expected_context(pos.numpy(), slots.numpy(), None, n_req, rpr, n_slots)
    assert {k: v for k, v in found.items()} == {
        m.CHECK_RULES["context"][k]: want[k] for k in range(3) if want[k][0] > 0}


def test_check_accept_inputs():
    m = dfl()
    B, S, V = 5, 8, 1000
    g = torch.Generator().manual_seed(11)
    cand = torch.randint(0, V, (B, S), generator=g, dtype=torch.int32)
    post = torch.randint(0, V, (B, S), generator=g, dtype=torch.int32)
    L = torch.randint(0, 100, (B,), generator=g, dtype=torch.int32)
    d = "cuda"
    assert m.check_accept_inputs(cand.to(d), post.to(d), L.to(d), V) == {}
    cand[2, 3], cand[4, 0], post[0, 7], L[3] = V, -1, V + 5, -2
    found = m.check_accept_inputs(cand.to(d), post.to(d), L.to(d), V)
    want = expected_accept(cand.numpy(), post.numpy(), L.numpy(), V)
    _print(f"[checked accept] {found}")
    assert found == {m.CHECK_RULES["accept"][k]: want[k] for k in range(3) if want[k][0] > 0}
    assert want[0] == (2, 2 * S + 3) and want[1] == (1, 7) and want[2] == (1, 3)


def test_checked_flag_raises_before_launch_and_passes_good_inputs():
    m = dfl()
    wl = get_workload("small_bf16")
    cfg = wl.cfg
    st = Setup(wl)
    d = "cuda"
    out = st.draft()  # the plain call
    max_prefix = int(st.L.max())
    pos = torch.empty((st.B, st.S), dtype=torch.int32, device=d)
    sl, cand = torch.empty_like(pos), torch.empty_like(pos)
    ws = m.workspace(m.draft_workspace_bytes(cfg, st.B, max_prefix))
    m.dflash_draft_block(cfg, st.c_weights(), st.cache, st.anchor.to(d), st.L.to(d),
                         st.pt.to(d), max_prefix, pos, sl, cand, ws, checked=True)
    torch.cuda.synchronize()
    assert torch.equal(cand.cpu(), out["candidates"].cpu())
    bad_anchor = st.anchor.clone()
    bad_anchor[0] = cfg.vocab + 3
    before = cand.clone()
    with pytest.raises(ValueError, match="anchor id outside"):
        m.dflash_draft_block(cfg, st.c_weights(), st.cache, bad_anchor.to(d), st.L.to(d),
                             st.pt.to(d), max_prefix, pos, sl, cand, ws, checked=True)
    torch.cuda.synchronize()
    assert torch.equal(cand, before)  # nothing launched
    B, S = st.B, st.S
    acc = [torch.empty(B, dtype=torch.int32, device=d) for _ in range(4)]
    ot = torch.empty((B, S), dtype=torch.int32, device=d)
    post = torch.zeros((B, S), dtype=torch.int32, device=d)
    post[0, 1] = -7
    with pytest.raises(ValueError, match="posterior id outside"):
        m.dflash_accept(cand, post, st.L.to(d), acc[0], acc[1], ot, acc[2], acc[3],
                        checked_vocab=cfg.vocab)
    with pytest.raises(ValueError, match="slot outside the pool"):
        m.dflash_project_context(cfg, st.c_weights(), st.cache,
                                 torch.zeros((2, cfg.feat_dim), dtype=torch.bfloat16, device=d),
                                 torch.zeros(2, dtype=torch.int32, device=d),
                                 torch.tensor([0, -1], dtype=torch.int32, device=d), None, 1, 2,
                                 m.workspace(m.context_workspace_bytes(cfg, 2)), checked=True)
