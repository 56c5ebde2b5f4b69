"""GPU parity of the DFlash 2 candidate selector (dflash_draft_block_selector)
against the fp64 oracle, through the C ABI.

The oracle's selector reads the logits the GPU wrote (identical unary logits,
so the candidate ids must match bit for bit) and its own fp64 final-normed
rows for the compatibility term.  The GPU forms W_h y from the bf16 pass, so a
lattice score differs from the oracle's by the bf16 error of the pass (the
same ~1e-2 of scale as the logits); the walk is compared along the GPU's own
path: wherever the oracle's row for the same predecessor has a top-2 gap above
GAP, the GPU's choice must be the oracle's; the greedy walk's q_rows must be
one-hot on the GPU's own choice, bit for bit (the proposal of a greedy walk
is a point mass), and the sampled walk's must match the softmax of the row
walked within QTOL.  With the compatibility switched off the selector must
reproduce the plain draft pass exactly (same logits, same tie rule).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.selector import select, top_k
from workloads import synth
from workloads.configs import get_workload
from tests.gpu_harness import Setup

pytestmark = pytest.mark.gpu

GAP = 0.05
QTOL = 2e-2


def dfl():
    import block_diffusion_drafter_rmsnorm_amd as m
    return m


def _selector(cfg, r, K, seed, zero_a=False):
    dt = synth._DT[cfg.act_dtype]
    A = synth.normal((cfg.vocab, r), 0.3, seed, "sel_a", dt, "cuda")
    if zero_a:
        A.zero_()
    Bt = synth.normal((cfg.vocab, r), 0.3, seed, "sel_b", dt, "cuda")
    Wh = synth.normal((r, cfg.hidden), 0.02, seed, "sel_wh", dt, "cuda")
    return A, Bt, Wh, dfl().Selector(A, Bt, Wh, K)


def _run(st, sel, K, uniforms=None, T=1.0):
    m = dfl()
    cfg, B, S = st.cfg, st.B, st.S
    mp = int(st.L.max())
    ws = m.workspace(m.selector_workspace_bytes(cfg, sel, B, mp))
    out = dict(positions=torch.empty((B, S), dtype=torch.int32, device="cuda"),
               slots=torch.empty((B, S), dtype=torch.int32, device="cuda"),
               candidates=torch.empty((B, S), dtype=torch.int32, device="cuda"),
               cand_ids=torch.full((B, S - 1, K), -1, dtype=torch.int32, device="cuda"),
               q_rows=torch.empty((B, S - 1, K), dtype=torch.float32, device="cuda"),
               logits=torch.empty((B, S - 1, cfg.vocab), dtype=synth._DT[cfg.act_dtype],
                                  device="cuda"))
    m.dflash_draft_block_selector(cfg, st.c_weights(), st.cache, sel, st.anchor.cuda(),
                                  st.L.cuda(), st.pt.cuda(), mp, out["positions"], out["slots"],
                                  out["candidates"], out["cand_ids"], out["q_rows"], ws,
                                  uniforms=uniforms, temperature=T, logits=out["logits"])
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in out.items()}


@pytest.mark.parametrize("name,K", [(n, k) for n in ("small_bf16", "tiny_f32", "small_bf16_wide")
                                     for k in (8, 4)] +
                         [("small_bf16", 1), ("small_bf16", 2), ("small_bf16", 16),
                          ("tiny_f32", 16)])
def test_selector_parity(name, K):
    wl = get_workload(name)
    st = Setup(wl)
    cfg, B, S = st.cfg, st.B, st.S
    r = 64
    A, Bt, Wh, sel = _selector(cfg, r, K, 7)
    g = _run(st, sel, K)
    d = oracle.draft_block(cfg, st.np_W(), st.oracle_cache(), st.anchor.numpy(), st.L.numpy(),
                           st.pt.numpy())
    f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    o = select(f(g["logits"]), d["hidden"], st.anchor.numpy(), f(A), f(Bt), f(Wh), k=K)
    cand = g["cand_ids"].numpy()
    assert np.array_equal(cand, o["cand_ids"])            # identical logits -> identical ids
    gc = g["candidates"].numpy()
    assert np.array_equal(gc[:, 0], st.anchor.numpy())
    n_clear = n_all = 0
    for b in range(B):
        p = 0
        for j in range(S - 1):
            row = o["score"][b, j, p]
            k = int(np.nonzero(cand[b, j] == gc[b, 1 + j])[0][0])   # the GPU's choice
            srt = np.sort(row)[::-1]
            n_all += 1
            if K == 1 or srt[0] - srt[1] > GAP:
                n_clear += 1
                assert k == int(np.argmax(row)), (b, j, k, row)
            assert np.array_equal(g["q_rows"].numpy()[b, j], np.eye(K, dtype=np.float32)[k]), \
                (b, j)
            p = k
    assert n_clear >= 0.7 * n_all, (n_clear, n_all)


def test_selector_without_compatibility_is_the_plain_draft():
    st = Setup(get_workload("small_bf16"))
    K = 8
    _, _, _, sel = _selector(st.cfg, 64, K, 3, zero_a=True)
    g = _run(st, sel, K)
    plain = st.draft()
    assert np.array_equal(g["candidates"].numpy(), plain["candidates"].cpu().numpy())
    assert torch.equal(g["logits"], plain["logits"].cpu())
    assert np.array_equal(g["cand_ids"].numpy()[:, :, 0], plain["candidates"].cpu().numpy()[:, 1:])


def test_selector_sampled_walk_draws_from_its_q_rows():
    st = Setup(get_workload("small_bf16_wide"))
    K, T = 8, 0.8
    A, Bt, Wh, sel = _selector(st.cfg, 64, K, 5)
    B, S = st.B, st.S
    u = torch.rand(B, S - 1, generator=torch.Generator("cuda").manual_seed(4), device="cuda")
    g = _run(st, sel, K, uniforms=u, T=T)
    u = u.cpu().numpy().astype(np.float64)
    cand, gc, q = g["cand_ids"].numpy(), g["candidates"].numpy(), g["q_rows"].numpy()
    assert np.allclose(q.sum(-1), 1.0, atol=1e-5)
    # q_rows are the softmax of the row walked, rows taken from the oracle's
    # lattice on the GPU's logits along the GPU's path
    d = oracle.draft_block(st.cfg, st.np_W(), st.oracle_cache(), st.anchor.numpy(),
                           st.L.numpy(), st.pt.numpy())
    f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    o = select(f(g["logits"]), d["hidden"], st.anchor.numpy(), f(A), f(Bt), f(Wh), k=K)
    for b in range(B):
        p = 0
        for j in range(S - 1):
            k = int(np.nonzero(cand[b, j] == gc[b, 1 + j])[0][0])
            e = np.exp((o["score"][b, j, p] - o["score"][b, j, p].max()) / T)
            # a score error ds moves a softmax entry by at most ds / (4 T)
            assert np.allclose(q[b, j], e / e.sum(), atol=QTOL / T), (b, j)
            p = k
            c = np.cumsum(q[b, j].astype(np.float64))
            lo = c[k - 1] if k > 0 else 0.0
            assert lo - 1e-5 <= u[b, j] and (u[b, j] < c[k] + 1e-5 or k == K - 1), (b, j, k)


@pytest.mark.parametrize("name,K", [("small_bf16_vocab", 16), ("small_bf16", 4)])
def test_selector_topk_ties_across_tiles(name, K):
    """lm_head rows repeat with period 7, so every 128-column tile holds the same
    maximum and each logit value recurs across the whole vocabulary: every tile
    qualifies for the search, and the candidates must be the lowest ids of the
    largest values, in the oracle's (value, lower id) order."""
    st = Setup(get_workload(name))
    W = st.W["lm_head"]
    V = st.cfg.vocab
    W.copy_(W[:7].repeat((V + 6) // 7, 1)[:V])
    _, _, _, sel = _selector(st.cfg, 32, K, 9)
    g = _run(st, sel, K)
    f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    lg = f(g["logits"])
    ids = top_k(lg, K)[0]
    assert np.array_equal(g["cand_ids"].numpy(), ids)
    # the case is what it claims: the K-th candidate ties the first in most rows
    top = np.take_along_axis(lg, ids, -1)
    assert np.mean(top[..., 0] == top[..., K - 1]) > 0.5


def test_selector_parity_wide_vocab():
    """A vocabulary of 257 tiles with a ragged last tile, K = 16."""
    st = Setup(get_workload("small_bf16_vocab"))
    K = 16
    A, Bt, Wh, sel = _selector(st.cfg, 32, K, 11)
    g = _run(st, sel, K)
    f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    ids, _ = top_k(f(g["logits"]), K)
    assert np.array_equal(g["cand_ids"].numpy(), ids)


def test_selector_topk_many_ties_in_few_tiles():
    """lm_head rows 0..255 (two tiles) all equal one row, the rest scaled by
    0.01: in every drafted row whose shared logit is positive, few tiles
    qualify but they hold 256 logits tied at the top, more than one ranking
    pass takes; the candidates must still be the oracle's (the lowest ids)."""
    st = Setup(get_workload("small_bf16_vocab"))
    W = st.W["lm_head"]
    row0 = W[0].clone()
    W.mul_(0.01)
    W[:256] = row0
    K = 16
    _, _, _, sel = _selector(st.cfg, 32, K, 13)
    g = _run(st, sel, K)
    f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    lg = f(g["logits"])
    ids = top_k(lg, K)[0]
    assert np.array_equal(g["cand_ids"].numpy(), ids)
    tied = (lg == lg.max(-1, keepdims=True)).sum(-1)
    assert (tied >= 256).sum() >= 5, tied      # the case occurs in several rows
