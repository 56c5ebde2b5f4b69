"""Pins of the oracle's accept and block preparation against the pages'
worked examples (tests/golden/accept_examples.json), brute force and
invariants."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "accept_examples.json")))


def _ids(symbols, table):
    out = []
    for s in symbols:
        if isinstance(s, int):
            out.append(s)
            continue
        if s not in table:
            table[s] = 100 + len(table)
        out.append(table[s])
    return out


@pytest.mark.parametrize("ex", GOLD["examples"], ids=["sglang_step6", "csdn_step8"])
def test_worked_examples(ex):
    table = {}
    cand = _ids(ex["candidates"], table)
    # "<any>" rows are never compared; give them a fresh symbol each.
    post = []
    for i, s in enumerate(ex["posterior"]):
        post.append(_ids([f"<any{i}>" if s == "<any>" else s], table)[0])
    r = oracle.accept(np.array([cand]), np.array([post]), [ex["prefix_len"]])
    assert r["accept_len"][0] == ex["accept_len"]
    assert r["commit_len"][0] == ex["commit_len"]
    assert r["next_anchor"][0] == table[ex["bonus"]]
    c = ex["commit_len"]
    if "out_tokens_valid" in ex:
        assert list(r["out_tokens"][0, :c]) == _ids(ex["out_tokens_valid"], table)
        assert r["new_seq_len"][0] == ex["new_seq_len"]
        # computed inputs are the anchor and the surviving drafts at L..L+a
        L = ex["prefix_len"]
        assert list(range(L, L + c)) == ex["committed_input_positions"]
        assert list(range(L + 1, L + 1 + c)) == ex["emitted_positions"]
        assert r["new_seq_len"][0] == ex["next_anchor_position"]
    if "out_tokens" in ex:
        assert list(r["out_tokens"][0]) == _ids(ex["out_tokens"], table)


@pytest.mark.parametrize("S", [2, 4, 8, 16])
def test_edge_cases(S):
    rng = np.random.default_rng(S)
    cand = rng.integers(0, 50, (1, S))
    # none survive
    post = cand[:, 1:].copy()
    post = np.concatenate([post + 1, rng.integers(0, 50, (1, 1))], axis=1)
    r = oracle.accept(cand, post, [7])
    assert r["commit_len"][0] == GOLD["edge_cases"]["none_survive_commit"]
    assert r["out_tokens"][0, 0] == post[0, 0] and (r["out_tokens"][0, 1:] == 0).all()
    assert r["new_seq_len"][0] == 8
    # all survive
    post = np.concatenate([cand[:, 1:], [[999]]], axis=1)
    r = oracle.accept(cand, post, [7])
    assert r["commit_len"][0] == S and r["accept_len"][0] == S - 1
    assert list(r["out_tokens"][0]) == list(cand[0, 1:]) + [999]
    assert r["next_anchor"][0] == 999


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5])
def test_bruteforce_small_alphabet(S):
    """Every (candidates, posterior) over the alphabet {0,1,2} against the
    cumulative-product form of the acceptance length printed in the CSDN
    article's z-lab verify step, plus the invariants of the commit."""
    rows = list(itertools.product(range(3), repeat=S))
    pairs = [(c, p) for c in rows for p in rows]
    cand = np.array([c for c, _ in pairs])
    post = np.array([p for _, p in pairs])
    L = np.arange(len(pairs)) % 37
    r = oracle.accept(cand, post, L)
    cum = np.cumprod((cand[:, 1:] == post[:, :-1]).astype(np.int64), axis=1).sum(axis=1) \
        if S > 1 else np.zeros(len(pairs), np.int64)
    assert (r["accept_len"] == cum).all()
    a = r["accept_len"]
    idx = np.arange(len(pairs))
    assert (r["commit_len"] == a + 1).all()
    assert ((1 <= r["commit_len"]) & (r["commit_len"] <= S)).all()
    assert (r["out_tokens"][idx, a] == post[idx, a]).all()
    assert (r["next_anchor"] == post[idx, a]).all()
    assert (r["new_seq_len"] - L == r["commit_len"]).all()
    for j in range(S):
        tail = j > a
        assert (r["out_tokens"][tail, j] == 0).all()
        if j < S - 1:
            head = j < a
            assert (r["out_tokens"][head, j] == cand[head, j + 1]).all()


def test_block_prep_worked_example():
    g = GOLD["block_prep"]
    S, P = g["block_size"], 16
    pt = np.array([[5, 2, 9]])       # physical pages: slots differ from positions
    ids, pos, slots = oracle.block_prep([77], [g["prefix_len"]], pt, S, 1000, P)
    assert list(pos[0]) == g["positions"]
    assert list(ids[0]) == [77, 1000, 1000, 1000]
    assert list(slots[0]) == [5 * 16 + p for p in g["positions"]]
    assert all(s != p for s, p in zip(slots[0], pos[0]))
    # crossing a page boundary
    ids, pos, slots = oracle.block_prep([1], [14], pt, 4, 0, P)
    assert list(slots[0]) == [5 * 16 + 14, 5 * 16 + 15, 2 * 16 + 0, 2 * 16 + 1]


def test_kv_bytes_per_token_kimi():
    from workloads.configs import KIMI_DRAFT
    g = GOLD["kv_bytes_per_token"]
    assert KIMI_DRAFT.n_layers == g["layers"] and KIMI_DRAFT.n_kv_heads == g["kv_heads"]
    assert KIMI_DRAFT.kv_bytes_per_token == g["bytes"]


def test_greedy_posterior_ties_and_nan():
    """First index among equal maxima; NaN never wins; a row of only NaN and
    -inf gives index 0."""
    x = np.array([[0.5, 2.0, 2.0, -1.0],
                  [np.nan, 0.0, np.nan, 0.0],
                  [np.nan, np.nan, np.nan, np.nan],
                  [-np.inf, np.nan, -np.inf, -np.inf],
                  [-3.0, -2.0, -2.5, np.inf]])
    assert oracle.greedy_posterior(x).tolist() == [1, 1, 0, 0, 3]


@pytest.mark.parametrize("S", [2, 5, 16])
def test_accept_logits_reproduces_planted_posteriors(S):
    """Logits that put one clear maximum on a planted posterior id per position
    (every other logit below it) give that posterior, so the commit lengths
    planted through the candidates come back exactly."""
    rng = np.random.default_rng(S)
    B, V = 40, 97
    post = rng.integers(0, V, (B, S))
    commit = rng.integers(1, S + 1, B)
    cand = rng.integers(0, V, (B, S))
    for r in range(B):
        c = commit[r]
        cand[r, 1:c] = post[r, :c - 1]
        if c < S and cand[r, c] == post[r, c - 1]:
            cand[r, c] = (post[r, c - 1] + 1) % V
    logits = -np.abs(rng.normal(0, 1, (B, S, V))) - 0.01
    logits[np.arange(B)[:, None], np.arange(S)[None, :], post] = rng.uniform(0, 3, (B, S))
    L = rng.integers(0, 1000, B)
    out = oracle.accept_logits(cand, logits, L)
    assert np.array_equal(out["commit_len"], commit)
    assert np.array_equal(out["next_anchor"], post[np.arange(B), commit - 1])
    assert np.array_equal(out["new_seq_len"], L + commit)
