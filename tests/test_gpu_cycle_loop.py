"""Decode cycles resident on the device: draft -> accept -> inject the
committed rows -> reserve the next block's pages, three times, with no host
synchronisation between cycles (each cycle's prefix lengths and anchors are
the device tensors the previous accept wrote; the reservation reads them on
the stream, "Inside SGLang ...", the overlap section).  The oracle replays the
same cycles; candidates, emitted tokens, lengths, page tables and the logits
of a final pass must match (fp32 model: argmax decisions agree)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle.reserve import reserve as o_reserve
from workloads import synth
from workloads.configs import get_workload
from tests.gpu_harness import Setup, logits_row_rel_err

pytestmark = pytest.mark.gpu


def plant(cand, commit, rand_ids, V):
    """Target choices whose greedy commit length against cand is `commit`
    (test plumbing on either device: the same rule for GPU and oracle)."""
    B, S = cand.shape
    cand = cand.to(torch.int64)
    j = torch.arange(S, device=cand.device)[None, :]
    c = commit.to(torch.int64)[:, None].to(cand.device)
    post = torch.where(j < c - 1, torch.roll(cand, -1, 1), rand_ids.to(cand.device).long())
    cnext = torch.gather(cand, 1, torch.clamp(c, max=S - 1))
    fix = (j == c - 1) & (c < S) & (post == cnext)
    return torch.where(fix, (cnext + 1) % V, post).to(torch.int32)


def logits_for(post, noise):
    """Target logits whose greedy choice is `post`: seeded values below 0 and
    1.0 at the planted id of every position (test plumbing, either device)."""
    x = noise.to(post.device).clone()
    x.scatter_(2, post.long()[..., None], 1.0)
    return x


@pytest.mark.parametrize("via_logits", [False, True])
def test_device_resident_cycles_match_oracle(via_logits):
    """via_logits: the accept reads the target's logits [B, S, V]
    (dflash_accept_logits / oracle.accept_logits) instead of its greedy ids."""
    import block_diffusion_drafter_rmsnorm_amd as m
    wl = dataclasses.replace(get_workload("tiny_f32"), batch=3, ctx=(40, 70))
    cfg = wl.cfg
    S, P, V, H = cfg.block_size, cfg.page_size, cfg.vocab, cfg.hidden
    st = Setup(wl, extra_tokens=64)
    B, cycles = st.B, 3
    L0 = st.L.clone()
    maxp = int((L0.max() + cycles * S + 2 * S) // P) + 2
    rng = np.random.default_rng(0)
    stack0 = rng.permutation(st.num_pages).astype(np.int32)
    commits = [torch.tensor(rng.integers(1, S + 1, B), dtype=torch.int32) for _ in range(cycles)]
    rand_ids = [synth.randint(0, V - 1, (B, S), c, "loop_post") for c in range(cycles)]
    feats = [synth.features(B * S, cfg, 100 + c) for c in range(cycles)]
    noise = [-torch.rand((B, S, V), generator=torch.Generator().manual_seed(50 + c)) - 0.01
             for c in range(cycles)]
    max_prefix = int(L0.max()) + cycles * S

    # ---------------------------------------------------------------- GPU
    dev = "cuda"
    pt = torch.full((B, maxp), -1, dtype=torch.int32, device=dev)
    npg = torch.zeros(B, dtype=torch.int32, device=dev)
    stack = torch.from_numpy(stack0).to(dev)
    top = torch.tensor([st.num_pages], dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    Ld, anc = L0.to(dev), st.anchor.to(dev)
    m.dflash_reserve_pages(Ld, S, P, pt, npg, stack, top, status)
    cw = st.c_weights()
    dws = m.workspace(m.draft_workspace_bytes(cfg, B, max_prefix))
    cws = m.workspace(m.context_workspace_bytes(cfg, B * S))
    aws = m.workspace(m.accept_logits_workspace_bytes(B, S, V))
    rec = []
    for c in range(cycles):
        pos = torch.empty((B, S), dtype=torch.int32, device=dev)
        slots, cand = torch.empty_like(pos), torch.empty_like(pos)
        m.dflash_draft_block(cfg, cw, st.cache, anc, Ld, pt, max_prefix, pos, slots, cand, dws)
        post = plant(cand, commits[c], rand_ids[c], V)
        acc = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(4)]
        out = torch.empty((B, S), dtype=torch.int32, device=dev)
        if via_logits:
            m.dflash_accept_logits(cand, logits_for(post, noise[c]), Ld, acc[0], acc[1], out,
                                   acc[2], acc[3], aws)
        else:
            m.dflash_accept(cand, post, Ld, acc[0], acc[1], out, acc[2], acc[3])
        m.dflash_project_context(cfg, cw, st.cache, feats[c].to(dev), pos.view(-1),
                                 slots.view(-1), acc[1], B, S, cws)
        m.dflash_reserve_pages(acc[3], S, P, pt, npg, stack, top, status)
        rec.append((cand, out, acc[1], acc[3]))
        Ld, anc = acc[3], acc[2]
    lg = torch.empty((B, S - 1, V), dtype=torch.float32, device=dev)
    pos = torch.empty((B, S), dtype=torch.int32, device=dev)
    fin = [torch.empty_like(pos) for _ in range(2)]
    m.dflash_draft_block(cfg, cw, st.cache, anc, Ld, pt, max_prefix, pos, fin[0], fin[1], dws,
                         logits=lg)
    torch.cuda.synchronize()
    assert int(status.item()) == 0

    # ---------------------------------------------------------------- oracle
    W = st.np_W()
    oc = st.oracle_cache()
    opt = np.full((B, maxp), -1, np.int64)
    on = np.zeros(B, np.int64)
    ost, otop = stack0.astype(np.int64), st.num_pages
    L, a0 = L0.numpy().astype(np.int64), st.anchor.numpy().astype(np.int64)
    opt, on, ost, otop, s0 = o_reserve(L, S, P, opt, on, ost, otop)
    for c in range(cycles):
        d = oracle.draft_block(cfg, W, oc, a0, L, opt)
        gcand, gout, gcommit, gL = (t.cpu().numpy() for t in rec[c])
        assert np.array_equal(gcand, d["candidates"]), c
        post = plant(torch.from_numpy(d["candidates"]), commits[c], rand_ids[c], V).numpy()
        if via_logits:
            a = oracle.accept_logits(d["candidates"],
                                     logits_for(torch.from_numpy(post), noise[c]).numpy(), L)
        else:
            a = oracle.accept(d["candidates"], post, L)
        assert np.array_equal(gout, a["out_tokens"]) and np.array_equal(gL, a["new_seq_len"])
        assert np.array_equal(gcommit, commits[c].numpy())
        oracle.project_context(cfg, W, oc, feats[c].numpy(), d["positions"].ravel(),
                               d["slots"].ravel(), valid_rows=a["commit_len"], rows_per_req=S)
        L, a0 = a["new_seq_len"], a["next_anchor"]
        opt, on, ost, otop, s = o_reserve(L, S, P, opt, on, ost, otop)
        assert s == 0
    assert np.array_equal(pt.cpu().numpy(), opt) and np.array_equal(npg.cpu().numpy(), on)
    d = oracle.draft_block(cfg, W, oc, a0, L, opt)
    rel = logits_row_rel_err(lg.cpu().numpy(), d["logits"])
    assert rel.max() < 1e-4, rel.max()
