"""Pins of the oracle's rejection-sampling verify ("Inside SGLang: DFlash and
DFlash 2 Implementation", section on sampling and the proposal distribution;
Step 6 for the emitted tokens and the commit).

The method's defining property is that rejection sampling is lossless: every
emitted token is distributed exactly as the target's p, whatever proposal
distribution q produced the drafts.  It is checked by a chi-square test on
many seeded draws, for a point-mass q (argmax drafts), for a sampled q, for
the token after an accepted draft and for the bonus token.  A dropped clip of
[p - q]_+, a ratio taken the wrong way round, a missing exclusion of the
rejected token or the wrong row for the bonus each move some probability by
more than 0.05 and fail it.  Special cases: the greedy limit (T -> 0) equals
the greedy accept, q == p accepts every draft, p(y) = 0 always rejects.
"""
import numpy as np
import pytest

import oracle
from oracle.sampling import _inverse_cdf

# chi-square critical value for 4 degrees of freedom at p = 1e-4
CHI2_4DF_1EM4 = 23.51


def _chi2(counts, p):
    n = counts.sum()
    e = n * p
    return float(np.sum((counts - e) ** 2 / e))


def _softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


P_LOGITS = np.array([0.3, -0.8, 1.1, 0.0, -0.2])     # p = softmax: all entries > 0.05
Q_LOGITS = np.array([-0.5, 0.9, 0.2, 1.0, -1.0])      # q differs from p everywhere


def _draw_candidates(rng, qs, n):
    """Drafts d_{j+1} ~ q_j (test input generation)."""
    return np.stack([rng.choice(len(q), size=n, p=q) for q in qs], axis=1)


def test_first_token_is_target_distributed_point_mass_q():
    rng = np.random.default_rng(1)
    n, V = 30000, 5
    p = _softmax(P_LOGITS)
    cand = np.zeros((n, 2), np.int64)
    cand[:, 1] = 2                                    # argmax draft: q = point mass on 2
    tl = np.broadcast_to(P_LOGITS, (n, 2, V))
    u = rng.random((n, 2))
    r = oracle.accept_sampling(cand, tl, np.zeros(n), u, 1.0)
    counts = np.bincount(r["out_tokens"][:, 0], minlength=V)
    assert _chi2(counts, p) < CHI2_4DF_1EM4
    # acceptance rate of the point-mass draft is p(y)
    assert abs(np.mean(r["accept_len"] == 1) - p[2]) < 4 * np.sqrt(p[2] * (1 - p[2]) / n)


@pytest.mark.parametrize("temps", [(1.0, 1.0), (0.7, 1.3)])
def test_first_token_is_target_distributed_sampled_q(temps):
    Tt, Td = temps
    rng = np.random.default_rng(2)
    n, V = 30000, 5
    p = _softmax(P_LOGITS / Tt)
    q = _softmax(Q_LOGITS / Td)
    cand = np.zeros((n, 2), np.int64)
    cand[:, 1:] = _draw_candidates(rng, [q], n)
    tl = np.broadcast_to(P_LOGITS, (n, 2, V))
    dl = np.broadcast_to(Q_LOGITS, (n, 1, V))
    u = rng.random((n, 2))
    r = oracle.accept_sampling(cand, tl, np.zeros(n), u, Tt, dl, Td)
    counts = np.bincount(r["out_tokens"][:, 0], minlength=V)
    assert _chi2(counts, p) < CHI2_4DF_1EM4
    # overall acceptance probability is sum_y min(p(y), q(y))
    acc = float(np.sum(np.minimum(p, q)))
    assert abs(np.mean(r["accept_len"] >= 1) - acc) < 4 * np.sqrt(acc * (1 - acc) / n)


def test_later_and_bonus_tokens_are_target_distributed():
    """S = 3 with a different target row per position: the token emitted after
    an accepted d_1 follows p_1, the bonus after two accepted drafts p_2."""
    rng = np.random.default_rng(3)
    n, V = 40000, 5
    rows = np.stack([P_LOGITS, Q_LOGITS[::-1], np.array([0.5, 0.4, -0.3, 0.2, 0.9])])
    drows = np.stack([Q_LOGITS, P_LOGITS[::-1]])
    ps = [_softmax(z) for z in rows]
    qs = [_softmax(z) for z in drows]
    cand = np.zeros((n, 3), np.int64)
    cand[:, 1:] = _draw_candidates(rng, qs, n)
    u = rng.random((n, 3))
    r = oracle.accept_sampling(cand, np.broadcast_to(rows, (n, 3, V)), np.zeros(n), u, 1.0,
                               np.broadcast_to(drows, (n, 2, V)), 1.0)
    a = r["accept_len"]
    out = r["out_tokens"]
    assert _chi2(np.bincount(out[:, 0], minlength=V), ps[0]) < CHI2_4DF_1EM4
    sel = a >= 1
    assert sel.sum() > 5000
    assert _chi2(np.bincount(out[sel, 1], minlength=V), ps[1]) < CHI2_4DF_1EM4
    sel = a == 2
    assert sel.sum() > 2000
    assert _chi2(np.bincount(out[sel, 2], minlength=V), ps[2]) < CHI2_4DF_1EM4


def test_greedy_limit_equals_greedy_accept():
    """T_t -> 0 with argmax drafts: p is the point mass on the target's argmax,
    so the result is the greedy accept against posterior = argmax."""
    rng = np.random.default_rng(4)
    B, S, V = 64, 8, 50
    tl = rng.permutation(np.arange(V))[None, None, :] * 0.01 + rng.normal(0, 1, (B, S, 1))
    tl = tl + rng.permutation(B * S * V).reshape(B, S, V) * 1e-3   # distinct values per row
    post = np.argmax(tl, axis=-1)
    cand = rng.integers(0, V, (B, S))
    commit = rng.integers(1, S + 1, B)
    for r in range(B):                       # plant surviving prefixes of every length
        c = commit[r]
        cand[r, 1:c] = post[r, :c - 1]
        if c < S and cand[r, c] == post[r, c - 1]:
            cand[r, c] = (post[r, c - 1] + 1) % V
    u = rng.uniform(0.001, 0.999, (B, S))
    L = rng.integers(0, 1000, B)
    rs = oracle.accept_sampling(cand, tl, L, u, 1e-4)
    rg = oracle.accept(cand, post, L)
    for k in ("accept_len", "commit_len", "out_tokens", "next_anchor", "new_seq_len"):
        assert np.array_equal(rs[k], rg[k]), k
    assert np.array_equal(rg["commit_len"], commit)


def test_draft_equal_to_target_accepts_everything():
    rng = np.random.default_rng(5)
    B, S, V = 32, 6, 40
    tl = rng.normal(0, 2, (B, S, V))
    cand = rng.integers(0, V, (B, S))
    u = rng.random((B, S))
    r = oracle.accept_sampling(cand, tl, np.full(B, 9), u, 0.8, tl[:, :S - 1], 0.8)
    assert np.all(r["accept_len"] == S - 1)
    assert np.all(r["commit_len"] == S)
    assert np.array_equal(r["out_tokens"][:, :S - 1], cand[:, 1:])
    assert np.all(r["new_seq_len"] == 9 + S)


def test_zero_target_probability_always_rejects():
    rng = np.random.default_rng(6)
    B, S, V = 32, 4, 16
    tl = rng.normal(0, 1, (B, S, V))
    cand = rng.integers(0, V, (B, S))
    tl[np.arange(B), 0, cand[:, 1]] = -np.inf
    u = rng.random((B, S))
    for dl in (None, rng.normal(0, 1, (B, S - 1, V))):
        r = oracle.accept_sampling(cand, tl, np.zeros(B), u, 1.0, dl, 1.0)
        assert np.all(r["accept_len"] == 0)
        assert np.all(r["out_tokens"][:, 0] != cand[:, 1])   # the residual excludes y
        assert np.all(r["out_tokens"][:, 1:] == 0)


def test_inverse_cdf_boundaries():
    """Smallest t with running sum > u * total: exact dyadic cases."""
    w = np.array([0.0, 1.0, 1.0, 2.0, 0.0])
    assert _inverse_cdf(w, 0.0)[0] == 1          # zero-weight tokens are never drawn
    assert _inverse_cdf(w, 0.2499)[0] == 1
    assert _inverse_cdf(w, 0.25)[0] == 2         # a draw on a boundary goes up
    assert _inverse_cdf(w, 0.5)[0] == 3
    assert _inverse_cdf(w, 0.999)[0] == 3
    assert _inverse_cdf(w, 1.0)[0] == 3          # u rounded to 1: last positive weight


def test_output_invariants():
    rng = np.random.default_rng(7)
    B, S, V = 200, 16, 30
    tl = rng.normal(0, 1.5, (B, S, V))
    dl = tl[:, :S - 1] + rng.normal(0, 0.3, (B, S - 1, V))
    cand = np.concatenate([rng.integers(0, V, (B, 1)), np.argmax(dl, -1)], axis=1)
    L = rng.integers(0, 5000, B)
    r = oracle.accept_sampling(cand, tl, L, rng.random((B, S)), 1.0, dl, 1.0)
    a, c = r["accept_len"], r["commit_len"]
    assert np.all((1 <= c) & (c <= S)) and np.array_equal(c, a + 1)
    assert np.array_equal(r["new_seq_len"], L + c)
    for i in range(B):
        assert np.array_equal(r["out_tokens"][i, :a[i]], cand[i, 1:a[i] + 1])
        assert r["out_tokens"][i, a[i]] == r["next_anchor"][i]
        assert np.all(r["out_tokens"][i, c[i]:] == 0)
    assert len(set(a.tolist())) > 3              # a spread of accept lengths


def test_sparse_proposal_is_lossless_and_matches_dense_forms():
    """q given directly as a distribution over a few candidates (the DFlash 2
    selector's q rows scattered over the vocabulary): the first emitted token
    still follows p; a point-mass q given this way equals the argmax-draft
    mode; q == p given this way accepts every draft."""
    rng = np.random.default_rng(8)
    n, V = 30000, 5
    p = _softmax(P_LOGITS)
    qs = np.array([0.0, 0.6, 0.0, 0.4, 0.0])          # support on two candidates
    cand = np.zeros((n, 2), np.int64)
    cand[:, 1] = rng.choice(V, size=n, p=qs)
    tl = np.broadcast_to(P_LOGITS, (n, 2, V))
    dq = np.broadcast_to(qs, (n, 1, V))
    u = rng.random((n, 2))
    r = oracle.accept_sampling(cand, tl, np.zeros(n), u, 1.0, draft_probs=dq)
    assert _chi2(np.bincount(r["out_tokens"][:, 0], minlength=V), p) < CHI2_4DF_1EM4
    B, S = 40, 5
    tl2 = rng.normal(0, 1.5, (B, S, V))
    c2 = rng.integers(0, V, (B, S))
    u2 = rng.random((B, S))
    pm = np.zeros((B, S - 1, V))
    pm[np.arange(B)[:, None], np.arange(S - 1)[None, :], c2[:, 1:]] = 1.0
    a = oracle.accept_sampling(c2, tl2, np.zeros(B), u2, 1.0, draft_probs=pm)
    b = oracle.accept_sampling(c2, tl2, np.zeros(B), u2, 1.0)
    for k in ("accept_len", "out_tokens"):
        assert np.array_equal(a[k], b[k])
    pe = np.exp(tl2[:, :S - 1] - tl2[:, :S - 1].max(-1, keepdims=True))
    pe /= pe.sum(-1, keepdims=True)
    full = oracle.accept_sampling(c2, tl2, np.zeros(B), u2, 1.0, draft_probs=pe)
    assert np.all(full["accept_len"] == S - 1)
