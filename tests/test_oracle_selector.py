"""Pins of the oracle's DFlash 2 candidate selector ("Inside SGLang: DFlash
and DFlash 2 Implementation", section on DFlash 2: candidates, lattice, walk).

With the learned compatibility switched off the selector must reduce to the
plain draft (top-1 candidate = the argmax the draft pass already pins); a
planted compatibility must steer the walk; the walk is greedy, not a best-path
search; top-k orders by value with ties to the lower id; the sampled walk
draws from q_rows, the softmax of the row actually used.  q_rows are the
proposal the walk drew from (section on sampling with the distribution the
walk actually used): after a greedy walk they are one-hot, and fed to the
sampled verify they keep it lossless, which softmax rows would not.
"""
import numpy as np

import oracle
from oracle.selector import top_k, walk, build_lattice, select
from workloads import synth
from workloads.configs import TINY
from tests.helpers import np_weights


def _pass(seed=0):
    cfg = TINY
    W = np_weights(synth.weights(cfg, seed))
    L = np.array([40])
    pt, npages = synth.page_table(__import__("torch").tensor(L), cfg, seed, 32)
    pt = pt.numpy()
    cache = oracle.OracleCache(cfg, npages * 16)
    f = synth.features(40, cfg, 5).numpy()
    pos = np.arange(40)
    oracle.project_context(cfg, W, cache, f, pos, pt[0, pos // 16] * 16 + pos % 16)
    return cfg, W, oracle.draft_block(cfg, W, cache, [17], L, pt)


def test_top_k_order_and_ties():
    x = np.array([[0.5, 2.0, 2.0, -1.0, 2.0, 0.5, 3.0]])
    ids, vals = top_k(x, 5)
    assert ids.tolist() == [[6, 1, 2, 4, 0]]
    assert vals.tolist() == [[3.0, 2.0, 2.0, 2.0, 0.5]]
    rng = np.random.default_rng(0)
    y = rng.integers(0, 20, (50, 300)).astype(float)          # many ties
    ids, vals = top_k(y, 8)
    for r in range(50):
        ref = sorted(range(300), key=lambda i: (-y[r, i], i))[:8]
        assert ids[r].tolist() == ref


def test_without_compatibility_the_selector_is_the_plain_draft():
    cfg, W, d = _pass()
    r = 64
    rng = np.random.default_rng(1)
    A = np.zeros((cfg.vocab, r))
    Bt = rng.standard_normal((cfg.vocab, r))
    Wh = rng.standard_normal((r, cfg.hidden))
    s = select(d["logits"], d["hidden"], [17], A, Bt, Wh, k=8)
    assert np.array_equal(s["draft_ids"], d["draft_ids"])
    assert np.all(s["chosen"] == 0)
    assert np.allclose(s["q_rows"].sum(-1), 1.0)


def test_planted_compatibility_steers_the_walk():
    """A[p] * w_j aligned with B[c] for one (predecessor, candidate) pair per
    position: the walk must follow the planted chain."""
    cfg, W, d = _pass()
    r, K = 64, 8
    s0 = select(d["logits"], d["hidden"], [17], np.zeros((cfg.vocab, r)),
                np.zeros((cfg.vocab, r)), np.zeros((r, cfg.hidden)), k=K)
    cand = s0["cand_ids"][0]
    J = cand.shape[0]
    y = d["hidden"][0]
    Wh = np.zeros((r, cfg.hidden))
    for j in range(J):                      # w_j[j] = 1 at component j (rows are independent)
        Wh[j] = y[j] / (y[j] @ y[j])
    A = np.zeros((cfg.vocab, r))
    Bt = np.zeros((cfg.vocab, r))
    want = [(j * 3 + 5) % (K - 1) + 1 for j in range(J)]  # planted slots, never the unary top
    prev = 17
    for j in range(J):
        c = int(cand[j, want[j]])
        A[prev, j] += 100.0
        Bt[c, j] += 1.0
        prev = c
    s = select(d["logits"], d["hidden"], [17], A, Bt, Wh, k=K)
    assert s["chosen"][0].tolist() == want
    assert np.array_equal(s["draft_ids"][0], cand[np.arange(J), want])
    # q_rows is the softmax of the row actually walked: its argmax is the choice
    assert np.array_equal(np.argmax(s["q_rows"][0], -1), want)


def test_walk_is_greedy_not_best_path():
    cand = np.array([[[10, 11], [20, 21]]])
    score = np.full((1, 2, 2, 2), -np.inf)
    score[0, 0, 0] = [1.0, 0.9]              # from the anchor: greedy takes slot 0
    score[0, 1, 0] = [0.0, 0.0]              # after slot 0: tie, first maximum
    score[0, 1, 1] = [5.0, 0.0]              # the best full path would go 1 -> 0
    draft, q, chosen = walk(cand, score)
    assert chosen.tolist() == [[0, 0]] and draft.tolist() == [[10, 20]]
    assert q[0].tolist() == [[1.0, 0.0], [1.0, 0.0]]   # a tie still puts all mass on the choice


def _scatter(cand_ids, q_rows, V):
    """q_rows over the candidate slots -> [B, J, V] over the vocabulary."""
    B, J, K = cand_ids.shape
    dense = np.zeros((B, J, V))
    for b in range(B):
        for j in range(J):
            np.add.at(dense[b, j], cand_ids[b, j], q_rows[b, j])
    return dense


def test_greedy_q_rows_are_the_point_mass_the_verify_assumes():
    """Greedy q_rows scattered over the vocabulary are exactly the point mass
    on the drafted token, so the sampled verify takes the same decisions with
    them as with no proposal given (the argmax drafter's case)."""
    rng = np.random.default_rng(5)
    B, J, K, V = 6, 7, 4, 23
    cand = np.stack([np.stack([rng.permutation(V)[:K] for _ in range(J)]) for _ in range(B)])
    score = rng.standard_normal((B, J, K, K))
    score[:, 0, 1:] = -np.inf
    draft, q, chosen = walk(cand, score)
    dense = _scatter(cand, q, V)
    assert np.array_equal(dense, np.eye(V)[draft])
    candidates = np.concatenate([rng.integers(0, V, (B, 1)), draft], 1)
    tl = rng.standard_normal((B, J + 1, V)) * 1.5
    L = rng.integers(0, 100, B)
    for trial in range(20):
        u = rng.random((B, J + 1))
        a = oracle.accept_sampling(candidates, tl, L, u, 0.9, draft_probs=dense)
        b = oracle.accept_sampling(candidates, tl, L, u, 0.9)
        assert np.array_equal(a["out_tokens"], b["out_tokens"])
        assert np.array_equal(a["accept_len"], b["accept_len"])


def test_greedy_walk_with_its_q_rows_emits_target_distributed_tokens():
    """The first emitted token of a greedily drafted block, verified with the
    walk's q_rows, follows the target's p (chi-square on seeded draws); the
    same block verified with softmax rows in their place does not."""
    rng = np.random.default_rng(6)
    n, K, V = 20000, 4, 5
    cand = np.array([[[3, 1, 4, 0]]])
    score = np.full((1, 1, K, K), -np.inf)
    score[0, 0, 0] = [1.0, 0.6, 0.2, -0.3]
    draft, q, _ = walk(cand, score)
    assert draft.tolist() == [[3]]
    p_logits = np.array([0.1, 0.9, -0.2, 0.3, 0.5])
    p = np.exp(p_logits) / np.exp(p_logits).sum()
    candidates = np.tile([[2, 3]], (n, 1))
    tl = np.tile(np.stack([p_logits, np.zeros(V)])[None], (n, 1, 1))
    u = rng.random((n, 2))
    soft = np.exp(score[0, 0, 0]) / np.exp(score[0, 0, 0]).sum()

    def first_tokens(qk):
        dense = np.tile(_scatter(cand, qk, V), (n, 1, 1))
        return oracle.accept_sampling(candidates, tl, np.zeros(n, np.int64), u, 1.0,
                                      draft_probs=dense)["out_tokens"][:, 0]

    def chi2(tok):
        counts = np.bincount(tok, minlength=V)
        return np.sum((counts - n * p) ** 2 / (n * p))

    assert chi2(first_tokens(q)) < 23.5                  # 4 degrees of freedom, p = 1e-4
    assert chi2(first_tokens(soft[None, None])) > 100.0  # the unrealised proposal is biased


def test_lattice_rows_use_the_previous_candidates():
    rng = np.random.default_rng(2)
    V, r, H, K = 30, 4, 6, 3
    cand = np.array([[[1, 2, 3], [4, 5, 6]]])
    unary = rng.standard_normal((1, 2, K))
    A, Bt = rng.standard_normal((V, r)), rng.standard_normal((V, r))
    Wh = rng.standard_normal((r, H))
    hid = rng.standard_normal((1, 2, H))
    sc = build_lattice(cand, unary, [9], hid, A, Bt, Wh)
    w1 = Wh @ hid[0, 1]
    # position 1, predecessor slot 2 (token 3), candidate slot 1 (token 5)
    assert np.isclose(sc[0, 1, 2, 1], unary[0, 1, 1] + np.sum(A[3] * w1 * Bt[5]))
    w0 = Wh @ hid[0, 0]
    assert np.isclose(sc[0, 0, 0, 2], unary[0, 0, 2] + np.sum(A[9] * w0 * Bt[3]))
    assert np.all(np.isinf(sc[0, 0, 1:]))  # the first position has one predecessor


def test_sampled_walk_draws_from_q_rows():
    rng = np.random.default_rng(3)
    n, K = 20000, 4
    cand = np.tile(np.arange(K)[None, None, :], (n, 1, 1))
    score = np.full((n, 1, K, K), -np.inf)
    score[:, 0, 0] = [0.2, -0.5, 1.0, 0.0]
    u = rng.random((n, 1))
    draft, q, chosen = walk(cand, score, u, temperature=0.7)
    p = np.exp(np.array([0.2, -0.5, 1.0, 0.0]) / 0.7)
    p /= p.sum()
    assert np.allclose(q[0, 0], p)
    counts = np.bincount(chosen[:, 0], minlength=K)
    chi2 = np.sum((counts - n * p) ** 2 / (n * p))
    assert chi2 < 21.1                       # 3 degrees of freedom, p = 1e-4
