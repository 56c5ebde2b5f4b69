"""GPU parity of the rejection-sampling verify (dflash_accept_sampling) against
the fp64 oracle, through the C ABI.

Floating point decides integers here (each acceptance test and the inverse-CDF
draw), and the kernels decide in fp32 while the oracle works in fp64, so the
comparison is in two tiers:
* requests whose decisions all clear the fp32 error bound (relative gap
  |u q(y) - p(y)| / max(u q(y), p(y)) above DEC_TOL, from the oracle) must
  match the oracle exactly in accept_len, commit_len, new_seq_len and every
  surviving draft in out_tokens; at most 1/32 of the requests (none below
  batch 32) may fall inside the bound, and those are checked only for
  well-formed outputs;
* the drawn token (correction or bonus) must be a valid inverse-CDF result
  under the oracle's fp64 weights up to CDF_TOL (running sum before it at most
  the draw + CDF_TOL, running sum through it at least the draw - CDF_TOL),
  and must equal the oracle's token whenever the draw lies farther than
  CDF_TOL from both ends of the oracle's interval.
The tolerances: fp32 exp2 and the row sums carry a relative error of a few
1e-6 per probability (the exponent (l - max) / T is rounded once; exp2 is
within a few ulp; sums of <= 300 terms per thread, then fixed-order
merges), so a probability or a running sum over the weights (total <= 1) is
off by well under 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import synth

pytestmark = pytest.mark.gpu

DEC_TOL = 1e-4
CDF_TOL = 1e-4


def dfl():
    import block_diffusion_drafter_rmsnorm_amd as m
    return m


def run_gpu(cand, tl, u, L, Tt=1.0, dl=None, Td=1.0):
    m = dfl()
    B, S = cand.shape
    V = tl.shape[-1]
    outs = [torch.full((B,), -7, dtype=torch.int32, device="cuda") for _ in range(4)]
    out_tok = torch.full((B, S), -7, dtype=torch.int32, device="cuda")
    ws = m.workspace(max(m.accept_sampling_workspace_bytes(B, S, V, dl is not None), 16))
    m.dflash_accept_sampling(cand, tl, u, L, outs[0], outs[1], out_tok, outs[2], outs[3], ws,
                             target_temperature=Tt, draft_logits=dl, draft_temperature=Td)
    torch.cuda.synchronize()
    names = ["accept_len", "commit_len", "next_anchor", "new_seq_len"]
    r = {n: o.cpu().numpy().astype(np.int64) for n, o in zip(names, outs)}
    r["out_tokens"] = out_tok.cpu().numpy().astype(np.int64)
    return r


def run_oracle(cand, tl, u, L, Tt=1.0, dl=None, Td=1.0):
    f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    return oracle.accept_sampling(cand.cpu().numpy(), f(tl), L.cpu().numpy(), f(u), Tt,
                                  None if dl is None else f(dl), Td)


def check(g, o, cand, L, max_ambiguous=0.01):
    """The two-tier comparison described in the module docstring."""
    cand = cand.cpu().numpy().astype(np.int64)
    L = L.cpu().numpy().astype(np.int64)
    B, S = cand.shape
    a = g["accept_len"]
    # well-formed outputs for every request
    assert np.all((a >= 0) & (a <= S - 1))
    assert np.array_equal(g["commit_len"], a + 1)
    assert np.array_equal(g["new_seq_len"], L + a + 1)
    for r in range(B):
        assert np.array_equal(g["out_tokens"][r, :a[r]], cand[r, 1:a[r] + 1])
        assert g["out_tokens"][r, a[r]] == g["next_anchor"][r]
        assert np.all(g["out_tokens"][r, a[r] + 1:] == 0)
    clear = o["margin"] > DEC_TOL
    print(f"  {int(np.sum(~clear))} of {B} requests with a decision within {DEC_TOL:g}", flush=True)
    assert np.mean(~clear) <= max_ambiguous, f"{np.sum(~clear)} of {B} decisions within tolerance"
    for k in ("accept_len", "commit_len", "new_seq_len"):
        assert np.array_equal(g[k][clear], o[k][clear]), k
    n_exact = n_unique = 0
    for r in np.nonzero(clear)[0]:
        w = np.asarray(o["weights"][r], np.float64)
        cum = np.cumsum(w)
        x = o["draw"][r]
        t = int(g["next_anchor"][r])
        assert 0 <= t < len(w)
        lo = cum[t - 1] if t > 0 else 0.0
        assert lo <= x + CDF_TOL and cum[t] >= x - CDF_TOL and w[t] >= 0, (r, t, lo, cum[t], x)
        to = int(o["next_anchor"][r])
        olo = cum[to - 1] if to > 0 else 0.0
        if x - olo > CDF_TOL and cum[to] - x > CDF_TOL:
            n_unique += 1
            assert t == to, (r, t, to)
        n_exact += int(t == to)
    return {"clear": int(clear.sum()), "unique_draws": n_unique, "equal_draws": n_exact}


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("with_draft", [False, True])
@pytest.mark.parametrize("shape", [(7, 4, 1000), (3, 16, 4096), (5, 2, 1003), (2, 64, 256)])
def test_sampling_parity_small(dtype, with_draft, shape):
    B, S, V = shape
    cand, tl, dl, u = synth.verify_inputs(B, S, V, seed=B * 131 + S, dtype=dtype, device="cuda")
    L = synth.randint(0, 9000, (B,), 3, "verify_L", "cuda").to(torch.int32)
    dl = dl if with_draft else None
    Tt, Td = (0.8, 1.2) if with_draft else (1.0, 1.0)
    g = run_gpu(cand, tl, u, L, Tt, dl, Td)
    o = run_oracle(cand, tl, u, L, Tt, dl, Td)
    check(g, o, cand, L, max_ambiguous=1 / 32)


@pytest.mark.parametrize("with_draft", [False, True])
def test_sampling_parity_batch32_full_vocab(with_draft):
    """The batch-32 Qwen3-8B verify shape: S = 16, V = 151936, bf16 logits (the
    draft's logit is raised by U(13, 22) so that p(draft) spans (0.2, 1) over the
    larger vocabulary and accept lengths spread over the block)."""
    B, S, V = 32, 16, 151936
    cand, tl, dl, u = synth.verify_inputs(B, S, V, seed=32, dtype=torch.bfloat16, device="cuda",
                                          bump=22.0, bump_lo=13.0)
    L = synth.randint(512, 8192, (B,), 32, "verify_L", "cuda").to(torch.int32)
    dl = dl if with_draft else None
    g = run_gpu(cand, tl, u, L, 1.0, dl, 1.0)
    o = run_oracle(cand, tl, u, L, 1.0, dl, 1.0)
    stats = check(g, o, cand, L, max_ambiguous=1 / 32)
    assert len(set(g["accept_len"].tolist())) > 3          # a spread of accept lengths
    # fp32 rounding moves a running sum by ~1e-6, far below most token masses:
    # nearly every draw equals the oracle's even where CDF_TOL cannot decide it
    assert stats["equal_draws"] >= 0.9 * stats["clear"], stats
    print(stats)


def test_sampling_parity_many_requests_capped_chunks():
    """Batch 200 at V = 151936: the pick chunks hit their 8192-logit cap (19
    chunks per row instead of one per ~1024 / batch)."""
    B, S, V = 200, 2, 151936
    cand, tl, dl, u = synth.verify_inputs(B, S, V, seed=200, dtype=torch.bfloat16, device="cuda",
                                          bump=22.0, bump_lo=13.0)
    L = torch.zeros(B, dtype=torch.int32, device="cuda")
    for d in (None, dl):
        g = run_gpu(cand, tl, u, L, 1.0, d, 1.0)
        stats = check(g, run_oracle(cand, tl, u, L, 1.0, d, 1.0), cand, L)
        assert stats["equal_draws"] >= 0.9 * stats["clear"], stats


def test_sampling_misaligned_rows_take_scalar_path():
    """Logits that start 2 bytes past a 16-byte boundary run the scalar loads."""
    B, S, V = 4, 8, 2048
    cand, tl, dl, u = synth.verify_inputs(B, S, V, seed=9, dtype=torch.bfloat16, device="cuda")
    buf = torch.empty(B * S * V + 1, dtype=torch.bfloat16, device="cuda")
    tl_mis = buf[1:].view(B, S, V)
    tl_mis.copy_(tl)
    L = torch.zeros(B, dtype=torch.int32, device="cuda")
    g1 = run_gpu(cand, tl_mis, u, L)
    g2 = run_gpu(cand, tl, u, L)
    o = run_oracle(cand, tl, u, L)
    check(g1, o, cand, L, max_ambiguous=1 / 32)
    for k in g1:
        assert np.array_equal(g1[k][o["margin"] > DEC_TOL], g2[k][o["margin"] > DEC_TOL]), k


def test_sampling_special_cases():
    B, S, V = 16, 8, 512
    cand, tl, dl, u = synth.verify_inputs(B, S, V, seed=5, dtype=torch.float32, device="cuda")
    L = torch.full((B,), 100, dtype=torch.int32, device="cuda")
    # draft == target: every draft survives, the bonus comes from p_{S-1}
    g = run_gpu(cand, tl, u, L, 0.9, tl[:, :S - 1].contiguous(), 0.9)
    assert np.all(g["accept_len"] == S - 1) and np.all(g["new_seq_len"] == 100 + S)
    o = run_oracle(cand, tl, u, L, 0.9, tl[:, :S - 1].contiguous(), 0.9)
    check(g, o, cand, L)
    # p(d_1) = 0: every request rejects at the first draft, never re-emitting it
    tl0 = tl.clone()
    tl0[torch.arange(B), 0, cand[:, 1].long()] = float("-inf")
    g = run_gpu(cand, tl0, u, L)
    assert np.all(g["accept_len"] == 0)
    assert np.all(g["out_tokens"][:, 0] != cand[:, 1].cpu().numpy())
    check(g, run_oracle(cand, tl0, u, L), cand, L)
    # the greedy limit: a tiny temperature equals the greedy accept on argmax posteriors
    post = torch.argmax(tl, dim=-1).to(torch.int32)
    cand2 = cand.clone()
    cand2[:, 1:5] = post[:, 0:4]
    ug = torch.rand(B, S, generator=torch.Generator("cuda").manual_seed(1), device="cuda")
    ug = ug * 0.998 + 0.001
    g = run_gpu(cand2, tl, ug, L, 1e-4)
    m = dfl()
    outs = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(4)]
    ot = torch.empty((B, S), dtype=torch.int32, device="cuda")
    m.dflash_accept(cand2, post, L, outs[0], outs[1], ot, outs[2], outs[3])
    torch.cuda.synchronize()
    assert np.array_equal(g["accept_len"], outs[0].cpu().numpy())
    assert np.array_equal(g["out_tokens"], ot.cpu().numpy())
    assert np.all(g["accept_len"] >= 4)


def test_sampling_deterministic_and_batch_zero():
    B, S, V = 32, 16, 151936
    cand, tl, dl, u = synth.verify_inputs(B, S, V, seed=77, dtype=torch.bfloat16, device="cuda")
    L = torch.zeros(B, dtype=torch.int32, device="cuda")
    g1 = run_gpu(cand, tl, u, L, 1.0, dl, 1.0)
    g2 = run_gpu(cand, tl, u, L, 1.0, dl, 1.0)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k
    m = dfl()
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    m.dflash_accept_sampling(cand[:0], tl[:0], u[:0], e, e, e, cand[:0], e, e,
                             torch.empty(16, dtype=torch.uint8, device="cuda"))


def test_sampling_is_lossless_on_gpu():
    """Every emitted first token follows the target's p (chi-square over many
    requests with a tiny vocabulary), drafts drawn from q by the test."""
    B, S, V = 20000, 2, 5
    gen = torch.Generator().manual_seed(11)
    zt = torch.tensor([0.3, -0.8, 1.1, 0.0, -0.2])
    zd = torch.tensor([-0.5, 0.9, 0.2, 1.0, -1.0])
    p = torch.softmax(zt.double(), 0).numpy()
    q = torch.softmax(zd.double(), 0)
    cand = torch.zeros(B, S, dtype=torch.int32)
    cand[:, 1] = torch.multinomial(q, B, replacement=True, generator=gen).to(torch.int32)
    tl = zt.expand(B, S, V).contiguous()
    dl = zd.expand(B, S - 1, V).contiguous()
    u = torch.rand(B, S, generator=gen)
    L = torch.zeros(B, dtype=torch.int32)
    g = run_gpu(cand.cuda(), tl.cuda(), u.cuda(), L.cuda(), 1.0, dl.cuda(), 1.0)
    counts = np.bincount(g["out_tokens"][:, 0], minlength=V)
    chi2 = float(np.sum((counts - B * p) ** 2 / (B * p)))
    assert chi2 < 23.51, (counts, B * p)     # 4 degrees of freedom, p = 1e-4


def _sparse_q(cand, V, K, seed):
    """Per drafted row K distinct ids (the drafted token among them) with
    Dirichlet probabilities: a stand-in for the selector's q rows."""
    rng = np.random.default_rng(seed)
    c = cand.cpu().numpy()
    B, S = c.shape
    ids = np.zeros((B, S - 1, K), np.int32)
    probs = rng.dirichlet(np.ones(K), size=(B, S - 1)).astype(np.float32)
    for b in range(B):
        for j in range(S - 1):
            others = rng.choice(np.setdiff1d(np.arange(V), [c[b, j + 1]]), K - 1, replace=False)
            row = np.concatenate([[c[b, j + 1]], others])
            ids[b, j] = rng.permutation(row)
    dense = np.zeros((B, S - 1, V))
    np.put_along_axis(dense, ids.astype(np.int64), probs.astype(np.float64), axis=-1)
    return torch.from_numpy(ids).cuda(), torch.from_numpy(probs).cuda(), dense


def _run_sparse(cand, tl, qi, qp, u, L, Tt=1.0):
    m = dfl()
    B, S = cand.shape
    V = tl.shape[-1]
    outs = [torch.full((B,), -7, dtype=torch.int32, device="cuda") for _ in range(4)]
    out_tok = torch.full((B, S), -7, dtype=torch.int32, device="cuda")
    ws = m.workspace(m.accept_sampling_workspace_bytes(B, S, V, False))
    m.dflash_accept_sampling_sparse(cand, tl, qi, qp, u, L, outs[0], outs[1], out_tok, outs[2],
                                    outs[3], ws, target_temperature=Tt)
    torch.cuda.synchronize()
    names = ["accept_len", "commit_len", "next_anchor", "new_seq_len"]
    r = {n: o.cpu().numpy().astype(np.int64) for n, o in zip(names, outs)}
    r["out_tokens"] = out_tok.cpu().numpy().astype(np.int64)
    return r


@pytest.mark.parametrize("shape,dtype", [((9, 8, 1000), torch.float32), ((6, 16, 4096), torch.bfloat16),
                                         ((4, 16, 151936), torch.bfloat16)])
def test_sampling_sparse_q_parity(shape, dtype):
    B, S, V = shape
    cand, tl, _, u = synth.verify_inputs(B, S, V, seed=B + S, dtype=dtype, device="cuda",
                                         bump=22.0 if V > 10000 else 12.0,
                                         bump_lo=13.0 if V > 10000 else 0.0)
    L = synth.randint(0, 5000, (B,), 5, "verify_L", "cuda").to(torch.int32)
    qi, qp, dense = _sparse_q(cand, V, 8, B * S)
    g = _run_sparse(cand, tl, qi, qp, u, L, 0.9)
    f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    o = oracle.accept_sampling(cand.cpu().numpy(), f(tl), L.cpu().numpy(), f(u), 0.9,
                               draft_probs=dense)
    check(g, o, cand, L, max_ambiguous=1 / 32)


def test_selector_then_sparse_verify():
    """The DFlash 2 path end to end on the GPU: the selector's candidates and
    q rows feed the sparse sampled verify; the oracle verifies the same
    candidates with the q rows scattered over the vocabulary."""
    from tests.gpu_harness import Setup
    from workloads.configs import get_workload
    m = dfl()
    st = Setup(get_workload("small_bf16"))
    cfg, B, S, K = st.cfg, st.B, st.S, 8
    dt = synth._DT[cfg.act_dtype]
    sel = m.Selector(synth.normal((cfg.vocab, 64), 0.3, 1, "sel_a", dt, "cuda"),
                     synth.normal((cfg.vocab, 64), 0.3, 1, "sel_b", dt, "cuda"),
                     synth.normal((64, cfg.hidden), 0.02, 1, "sel_wh", dt, "cuda"), K)
    mp = int(st.L.max())
    ws = m.workspace(m.selector_workspace_bytes(cfg, sel, B, mp))
    pos = torch.empty((B, S), dtype=torch.int32, device="cuda")
    slots, cand = torch.empty_like(pos), torch.empty_like(pos)
    cids = torch.empty((B, S - 1, K), dtype=torch.int32, device="cuda")
    q = torch.empty((B, S - 1, K), dtype=torch.float32, device="cuda")
    u_sel = torch.rand(B, S - 1, generator=torch.Generator("cuda").manual_seed(2), device="cuda")
    m.dflash_draft_block_selector(cfg, st.c_weights(), st.cache, sel, st.anchor.cuda(),
                                  st.L.cuda(), st.pt.cuda(), mp, pos, slots, cand, cids, q, ws,
                                  uniforms=u_sel, temperature=1.0)
    tl = synth.normal((B, S, cfg.vocab), 2.0, 9, "sel_target", torch.float32, "cuda")
    u = torch.rand(B, S, generator=torch.Generator("cuda").manual_seed(3), device="cuda")
    L = st.L.cuda()
    g = _run_sparse(cand, tl, cids, q, u, L)
    dense = np.zeros((B, S - 1, cfg.vocab))
    np.put_along_axis(dense, cids.cpu().numpy().astype(np.int64),
                      q.cpu().numpy().astype(np.float64), axis=-1)
    o = oracle.accept_sampling(cand.cpu().numpy(), tl.cpu().numpy().astype(np.float64),
                               st.L.numpy(), u.cpu().numpy().astype(np.float64), 1.0,
                               draft_probs=dense)
    check(g, o, cand, L, max_ambiguous=1 / 32)


def test_greedy_selector_q_rows_give_the_point_mass_verify():
    """After a greedy walk the selector's q rows are one-hot on the drafted
    token, so the sparse verify fed with them takes the decisions of the
    point-mass verify (the argmax drafter's case; section on sampling with the
    proposal distribution the walk actually used)."""
    from tests.gpu_harness import Setup
    from workloads.configs import get_workload
    m = dfl()
    st = Setup(get_workload("small_bf16"))
    cfg, B, S, K = st.cfg, st.B, st.S, 8
    dt = synth._DT[cfg.act_dtype]
    sel = m.Selector(synth.normal((cfg.vocab, 64), 0.3, 2, "sel_a", dt, "cuda"),
                     synth.normal((cfg.vocab, 64), 0.3, 2, "sel_b", dt, "cuda"),
                     synth.normal((64, cfg.hidden), 0.02, 2, "sel_wh", dt, "cuda"), K)
    mp = int(st.L.max())
    ws = m.workspace(m.selector_workspace_bytes(cfg, sel, B, mp))
    pos = torch.empty((B, S), dtype=torch.int32, device="cuda")
    slots, cand = torch.empty_like(pos), torch.empty_like(pos)
    cids = torch.empty((B, S - 1, K), dtype=torch.int32, device="cuda")
    q = torch.empty((B, S - 1, K), dtype=torch.float32, device="cuda")
    m.dflash_draft_block_selector(cfg, st.c_weights(), st.cache, sel, st.anchor.cuda(),
                                  st.L.cuda(), st.pt.cuda(), mp, pos, slots, cand, cids, q, ws)
    tl = synth.normal((B, S, cfg.vocab), 2.0, 8, "sel_target", torch.float32, "cuda")
    u = torch.rand(B, S, generator=torch.Generator("cuda").manual_seed(5), device="cuda")
    L = st.L.cuda()
    g = _run_sparse(cand, tl, cids, q, u, L, 0.9)
    o = oracle.accept_sampling(cand.cpu().numpy(), tl.cpu().numpy().astype(np.float64),
                               st.L.numpy(), u.cpu().numpy().astype(np.float64), 0.9)
    check(g, o, cand, L, max_ambiguous=1 / 32)
