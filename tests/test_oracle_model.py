"""Pins of the oracle's primitives, context injection and draft pass:
library routines (torch CPU) for the special cases they cover, closed forms,
invariants and a pure-Python brute force on the tiny shape."""
import dataclasses
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import oracle
from oracle.primitives import rms_norm, rope_neox, silu, block_attention
from workloads import synth
from workloads.configs import TINY, SMALL_F32_D64
from tests.helpers import np_weights


def _hf_window_visible(q_pos, k_pos, window):
    """Visibility of key positions to query positions under transformers' own
    sliding-window rule (masking_utils.sliding_window_overlay, the overlay its
    sliding-window causal masks are built from), evaluated elementwise: an
    independent statement of the window boundary, not the oracle's."""
    from transformers.masking_utils import sliding_window_overlay
    keep = sliding_window_overlay(int(window))
    qp = torch.as_tensor(np.asarray(q_pos, np.int64))[:, None]
    kp = torch.as_tensor(np.asarray(k_pos, np.int64))[None, :]
    return keep(0, 0, qp, kp)


# ---------------------------------------------------------------- primitives
def test_rms_norm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 96))
    g = 1 + 0.1 * rng.standard_normal(96)
    ref = Fnn.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(rms_norm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-13)


def test_silu_matches_torch():
    x = np.linspace(-20, 20, 1001)
    assert np.allclose(silu(x), Fnn.silu(torch.from_numpy(x)).numpy(), rtol=1e-13, atol=1e-15)


def test_rope_identity_norm_and_complex_form():
    rng = np.random.default_rng(1)
    D = 128
    x = rng.standard_normal((5, 3, D))
    assert np.array_equal(rope_neox(x, np.zeros((5, 1)), 1e6), x)
    p = rng.integers(0, 40000, (5, 1))
    y = rope_neox(x, p, 1e6)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # neox layout as a complex rotation: z_i = x_i + i x_{i+D/2}, z_i * exp(i p w_i)
    w = np.array([1e6 ** (-2 * i / D) for i in range(D // 2)])
    z = (x[..., :D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * p[..., None] * w)
    assert np.allclose(y, np.concatenate([z.real, z.imag], axis=-1), rtol=1e-10, atol=1e-10)


def test_rope_relative_positions():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((2, 64))
    a = rope_neox(q, 1000, 1e4) @ rope_neox(k, 990, 1e4)
    b = rope_neox(q, 20, 1e4) @ rope_neox(k, 10, 1e4)
    assert abs(a - b) < 1e-9


@pytest.mark.parametrize("window", [0, 7])
def test_block_attention_matches_torch_sdpa(window):
    rng = np.random.default_rng(3)
    S, nq, nkv, D, n = 6, 8, 2, 32, 23
    q = rng.standard_normal((S, nq, D))
    kc, vc = rng.standard_normal((2, n, nkv, D))
    kb, vb = rng.standard_normal((2, S, nkv, D))
    cpos = np.arange(n) + 4
    qpos = np.arange(S) + n + 4
    o = block_attention(q, kc, vc, cpos, kb, vb, qpos, window)
    keys = torch.from_numpy(np.concatenate([kc, kb])).permute(1, 0, 2)     # [nkv, n+S, D]
    vals = torch.from_numpy(np.concatenate([vc, vb])).permute(1, 0, 2)
    keys = keys.repeat_interleave(nq // nkv, 0)
    vals = vals.repeat_interleave(nq // nkv, 0)
    mask = torch.ones(S, n + S, dtype=torch.bool)
    if window:
        mask[:, :n] = _hf_window_visible(qpos, cpos, window)
    ref = Fnn.scaled_dot_product_attention(torch.from_numpy(q).permute(1, 0, 2), keys, vals,
                                           attn_mask=mask, is_causal=False)
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_block_attention_bruteforce_loops():
    """Pure-Python loops over (query, head, key) on the tiny shape."""
    rng = np.random.default_rng(4)
    S, nq, nkv, D, n, W = 4, 4, 2, 8, 9, 5
    q = rng.standard_normal((S, nq, D))
    kc, vc = rng.standard_normal((2, n, nkv, D))
    kb, vb = rng.standard_normal((2, S, nkv, D))
    cpos, qpos = list(range(n)), [n + j for j in range(S)]
    o = block_attention(q, kc, vc, np.array(cpos), kb, vb, np.array(qpos), W)
    for j in range(S):
        for h in range(nq):
            g = h // (nq // nkv)
            sc, vs = [], []
            for i in range(n):
                if qpos[j] - cpos[i] < W:
                    sc.append(sum(q[j, h, d] * kc[i, g, d] for d in range(D)) / math.sqrt(D))
                    vs.append(vc[i, g])
            for i in range(S):
                sc.append(sum(q[j, h, d] * kb[i, g, d] for d in range(D)) / math.sqrt(D))
                vs.append(vb[i, g])
            m = max(sc)
            e = [math.exp(s - m) for s in sc]
            tot = sum(e)
            ref = sum((ei / tot) * v for ei, v in zip(e, vs))
            assert np.allclose(o[j, h], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window", [1, 5, 12])
def test_block_attention_window_boundary_keys(window):
    """The window boundary itself: with zero queries every visible key gets
    the same weight, and one-hot values read back which keys were visible.
    For the query at position p the context key at p - W must be invisible and
    the one at p - W + 1 visible (transformers' sliding_window_overlay); every
    other key agrees with that overlay too."""
    S, nq, nkv, D, n = 3, 2, 1, 40, 30
    cpos = np.arange(n) + 7
    qpos = np.arange(S) + n + 7
    q = np.zeros((S, nq, D))
    kc = np.zeros((n, nkv, D))
    kb = np.zeros((S, nkv, D))
    vc = np.zeros((n, nkv, D))
    vb = np.zeros((S, nkv, D))
    for i in range(n):
        vc[i, 0, i] = 1.0
    for j in range(S):
        vb[j, 0, n + j] = 1.0
    o = block_attention(q, kc, vc, cpos, kb, vb, qpos, window)
    hf = _hf_window_visible(qpos, cpos, window).numpy()
    for j in range(S):
        seen = o[j, 0, :n] > 0
        assert np.array_equal(seen, hf[j])
        assert np.all(o[j, 0, n:n + S] > 0)          # every block key, always
        p = qpos[j]
        i_out, i_in = p - window - cpos[0], p - window + 1 - cpos[0]
        if 0 <= i_out < n:
            assert not seen[i_out]
        if 0 <= i_in < n:
            assert seen[i_in]
        assert np.isclose(o[j, 0].sum(), 1.0, rtol=1e-12)


def test_draft_window_boundary_rows():
    """At the draft-pass level, on a sliding layer placed first (so that what
    the anchor row sees there reaches every drafted row through the block keys
    of the next layer): the cached rows before position L - W + 1 are never
    read (NaN there leaves the logits unchanged), and the row at L - W + 1 is
    read (changing it changes the logits)."""
    Wwin = 33
    cfg = dataclasses.replace(SMALL_F32_D64, sliding_window=(Wwin, 0))
    Lr = 61
    W, pt, npages = _setup(cfg, L=(Lr,))
    cache = _ctx_cache(cfg, W, pt, npages, [Lr])
    base = oracle.draft_block(cfg, W, cache, [5], [Lr], pt)["logits"]
    P = cfg.page_size

    def slot(i):
        return pt[0, i // P] * P + i % P

    first = Lr - Wwin + 1
    poisoned = oracle.OracleCache(cfg, npages * P)
    for l in range(cfg.n_layers):
        poisoned.k[l][:] = cache.k[l]
        poisoned.v[l][:] = cache.v[l]
    for i in range(first):
        poisoned.k[0][slot(i)] = np.nan
        poisoned.v[0][slot(i)] = np.nan
    got = oracle.draft_block(cfg, W, poisoned, [5], [Lr], pt)["logits"]
    assert np.array_equal(got, base)
    poisoned.v[0][slot(first)] *= -3.0
    moved = oracle.draft_block(cfg, W, poisoned, [5], [Lr], pt)["logits"]
    assert np.max(np.abs(moved - base)) > 1e-9


# ---------------------------------------------------------------- fixtures
def _setup(cfg, seed=0, B=1, L=(40,), extra=32):
    W = np_weights(synth.weights(cfg, seed))
    L = np.array(L)
    pt, npages = synth.page_table(__import__("torch").tensor(L), cfg, seed, extra)
    return W, pt.numpy(), npages


def _inject_prefix(cfg, W, cache, pt, L, seed=5):
    for r, l in enumerate(L):
        f = synth.features(l, cfg, seed + r).numpy()
        pos = np.arange(l)
        oracle.project_context(cfg, W, cache, f, pos, pt[r, pos // 16] * 16 + pos % 16)


# ---------------------------------------------------------------- injection
def test_injection_matches_torch_composition():
    cfg = TINY
    W, pt, npages = _setup(cfg)
    cache = oracle.OracleCache(cfg, npages * 16)
    f = synth.features(10, cfg, 9).numpy()
    pos = np.arange(10) * 3 + 1
    slots = np.arange(10) + 50
    oracle.project_context(cfg, W, cache, f, pos, slots)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    c = Fnn.rms_norm(Fnn.linear(t(f), t(W["fc"])), (cfg.hidden,), t(W["hidden_norm"]), eps=cfg.rms_eps)
    L0 = W["layers"][0]
    nq, nkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    wk = t(L0["w_qkv"][nq * D:(nq + nkv) * D])
    wv = t(L0["w_qkv"][(nq + nkv) * D:])
    k = Fnn.rms_norm(Fnn.linear(c, wk).view(10, nkv, D), (D,), t(L0["k_norm"]), eps=cfg.rms_eps)
    v = Fnn.linear(c, wv).view(10, nkv, D)
    # RoPE as a complex rotation (torch.polar), neox halves
    inv = cfg.rope_theta ** (-torch.arange(D // 2, dtype=torch.float64) * 2 / D)
    rot = torch.polar(torch.ones(10, D // 2, dtype=torch.float64), t(pos)[:, None] * inv)
    z = torch.complex(k[..., :D // 2], k[..., D // 2:]) * rot[:, None, :]
    k = torch.cat([z.real, z.imag], -1)
    assert np.allclose(cache.k[0][slots], k.float().double().numpy(), rtol=1e-6, atol=1e-6)
    assert np.allclose(cache.v[0][slots], v.float().double().numpy(), rtol=1e-6, atol=1e-6)


def test_injection_closed_form_head_norm():
    """With k_norm gain 1, each stored K head has |k|^2 = D ms / (ms + eps)."""
    cfg = dataclasses.replace(TINY, kv_dtype="f32")
    W, pt, npages = _setup(cfg)
    W["layers"][0]["k_norm"] = np.ones(cfg.head_dim, np.float32)
    cache = oracle.OracleCache(cfg, npages * 16)
    f = synth.features(6, cfg, 11).numpy().astype(np.float64)
    slots = np.arange(6)
    oracle.project_context(cfg, W, cache, f, np.arange(6) * 1000, slots)
    c = rms_norm(f @ W["fc"].astype(np.float64).T, W["hidden_norm"], cfg.rms_eps)
    nq, nkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    kraw = (c @ W["layers"][0]["w_qkv"][nq * D:(nq + nkv) * D].astype(np.float64).T).reshape(6, nkv, D)
    ms = np.mean(kraw ** 2, -1)
    got = np.sum(cache.k[0][slots] ** 2, -1)
    assert np.allclose(got, D * ms / (ms + cfg.rms_eps), rtol=1e-6)


def test_injection_scale_invariance_without_eps():
    cfg = dataclasses.replace(TINY, rms_eps=0.0)
    W, pt, npages = _setup(cfg)
    f = synth.features(8, cfg, 12).numpy().astype(np.float64)
    a = oracle.OracleCache(cfg, 64)
    b = oracle.OracleCache(cfg, 64)
    oracle.project_context(cfg, W, a, f, np.arange(8), np.arange(8))
    oracle.project_context(cfg, W, b, 3.5 * f, np.arange(8), np.arange(8))
    assert np.allclose(a.k[0][:8], b.k[0][:8], rtol=1e-6) and np.allclose(a.v[0][:8], b.v[0][:8], rtol=1e-6)


def test_injection_once_equals_chunked_and_prefix_valid():
    cfg = TINY
    W, pt, npages = _setup(cfg)
    f = synth.features(64, cfg, 13).numpy()
    pos = np.arange(64)
    slots = pt[0, pos // 16] * 16 + pos % 16
    a = oracle.OracleCache(cfg, npages * 16)
    b = oracle.OracleCache(cfg, npages * 16)
    oracle.project_context(cfg, W, a, f, pos, slots)
    for lo, hi in [(0, 5), (5, 33), (33, 64)]:
        oracle.project_context(cfg, W, b, f[lo:hi], pos[lo:hi], slots[lo:hi])
    for l in range(cfg.n_layers):
        assert np.allclose(a.k[l], b.k[l], rtol=1e-12, atol=1e-12, equal_nan=True)
    # prefix-valid writes over a dense [4, 16] grid: rows j >= valid stay untouched (NaN)
    c = oracle.OracleCache(cfg, npages * 16)
    valid = np.array([3, 0, 16, 1])
    live = oracle.project_context(cfg, W, c, f, pos, slots, valid_rows=valid, rows_per_req=16)
    assert live.sum() == valid.sum()
    assert np.isnan(c.k[0][slots[~live]]).all() and not np.isnan(c.k[0][slots[live]]).any()
    assert np.allclose(c.k[0][slots[live]], a.k[0][slots[live]], rtol=1e-12)
    # crop then re-append: writing the same rows again leaves the cache bit-identical
    d = c.copy()
    oracle.project_context(cfg, W, d, f, pos, slots, valid_rows=valid, rows_per_req=16)
    for l in range(cfg.n_layers):
        assert np.array_equal(np.nan_to_num(c.k[l], nan=7.0), np.nan_to_num(d.k[l], nan=7.0))


# ---------------------------------------------------------------- draft pass
def _ctx_cache(cfg, W, pt, npages, L, shift=0, seed=5):
    cache = oracle.OracleCache(cfg, npages * 16)
    for r, l in enumerate(L):
        f = synth.features(l, cfg, seed + r).numpy()
        pos = np.arange(l)
        oracle.project_context(cfg, W, cache, f, pos + shift, pt[r, pos // 16] * 16 + pos % 16)
    return cache


def test_draft_zero_residual_branches_closed_form():
    """With W_o = W_down = 0 the residual stream is the embedding, so every
    logits row is rms(E[id]; final_norm) W_lm^T."""
    cfg = TINY
    W, pt, npages = _setup(cfg)
    W["layers"][0]["w_o"] = np.zeros_like(W["layers"][0]["w_o"])
    W["layers"][0]["w_down"] = np.zeros_like(W["layers"][0]["w_down"])
    cache = _ctx_cache(cfg, W, pt, npages, [40])
    d = oracle.draft_block(cfg, W, cache, [17], [40], pt)
    y = rms_norm(W["embed"][cfg.mask_token_id].astype(np.float64), W["final_norm"], cfg.rms_eps)
    ref = y @ W["lm_head"].astype(np.float64).T
    for j in range(cfg.block_size - 1):
        assert np.allclose(d["logits"][0, j], ref, rtol=1e-10, atol=1e-12)


def test_draft_mask_rows_equivariant_without_rope():
    """Without RoPE, non-causal attention treats the MASK rows symmetrically:
    they share one embedding, so their logits are identical.  With RoPE (and
    with any causal mask) they differ.  (No sliding window here: the window
    bound depends on each row's position.)"""
    cfg = dataclasses.replace(SMALL_F32_D64, sliding_window=())
    W, pt, npages = _setup(cfg, L=(30, 55))
    cache = _ctx_cache(cfg, W, pt, npages, [30, 55])
    d = oracle.draft_block(cfg, W, cache, [3, 9], [30, 55], pt, rope=False)
    for r in range(2):
        for j in range(1, cfg.block_size - 1):
            assert np.allclose(d["logits"][r, j], d["logits"][r, 0], rtol=1e-11, atol=1e-11)
    d2 = oracle.draft_block(cfg, W, cache, [3, 9], [30, 55], pt)
    assert not np.allclose(d2["logits"][0, 1], d2["logits"][0, 0], rtol=1e-6)
    # the anchor is visible to the MASK rows: changing it changes their logits
    d3 = oracle.draft_block(cfg, W, cache, [4, 9], [30, 55], pt, rope=False)
    assert not np.allclose(d3["logits"][0, 0], d["logits"][0, 0], rtol=1e-6)


def test_draft_translation_invariance():
    """Shifting every logical position (context and block) by the same amount
    leaves the logits unchanged: RoPE only sees position differences, and so
    does the sliding window.  Every layer is a sliding layer here so that the
    shifted run reads only context it was given."""
    cfg = dataclasses.replace(SMALL_F32_D64, sliding_window=(20, 17))
    W, pt, npages = _setup(cfg, L=(45, 61))
    a = oracle.draft_block(cfg, W, _ctx_cache(cfg, W, pt, npages, [45, 61]), [5, 6], [45, 61], pt)
    k = 771                                   # shift by whole pages; roll the page table
    sh = 16 * k
    cache = _ctx_cache(cfg, W, pt, npages, [45, 61], shift=sh)
    pt3 = np.zeros((2, pt.shape[1] + k), np.int64)
    pt3[:, k:] = pt
    b = oracle.draft_block(cfg, W, cache, [5, 6], [45 + sh, 61 + sh], pt3)
    # the fp32 cache rounds the rotated keys differently at different positions
    assert np.allclose(a["logits"], b["logits"], rtol=1e-5, atol=1e-5)
    assert np.array_equal(a["slots"], b["slots"])


def test_select_draft_tokens_brute_force():
    """Selection step on rows spanning the oracle's 16384-row weight chunks:
    every logit against a pure-Python dot product, each id against a scan
    that keeps the first maximum, and a planted tie that the lower index wins."""
    rng = np.random.default_rng(5)
    V, H = 16384 + 37, 3
    y = rng.standard_normal((2, H))
    lm = rng.standard_normal((V, H)).astype(np.float32)
    # row 1: a tie between columns on both sides of the chunk edge
    lm[16390] = lm[100] = 10.0 * np.sign(y[1]).astype(np.float32)
    logits, ids = oracle.select_draft_tokens(y, lm)
    assert logits.shape == (2, V) and ids.shape == (2,)
    for r in range(2):
        ref = [sum(float(y[r, h]) * float(lm[v, h]) for h in range(H)) for v in range(V)]
        assert np.allclose(logits[r], ref, rtol=1e-13, atol=1e-13)
        best = 0
        for v in range(1, V):
            if ref[v] > ref[best]:
                best = v
        assert int(ids[r]) == best
    assert int(ids[1]) == 100


def test_select_draft_tokens_one_hot_rows():
    """A one-hot hidden row e_h reads column h of the lm_head: logits equal it
    exactly and the id is that column's argmax; a batch shape carries through."""
    rng = np.random.default_rng(6)
    V, H = 501, 8
    lm = rng.standard_normal((V, H))
    y = np.zeros((2, 4, H))
    for i in range(8):
        y[i // 4, i % 4, i] = 1.0
    logits, ids = oracle.select_draft_tokens(y, lm)
    assert logits.shape == (2, 4, V)
    for i in range(8):
        assert np.array_equal(logits[i // 4, i % 4], lm[:, i])
        assert int(ids[i // 4, i % 4]) == int(np.argmax(lm[:, i]))


def test_draft_planted_argmax():
    cfg = TINY
    W, pt, npages = _setup(cfg)
    cache = _ctx_cache(cfg, W, pt, npages, [40])
    d = oracle.draft_block(cfg, W, cache, [17], [40], pt)
    # plant token t's lm_head row as 4x the row of the current argmax (whose
    # logit is positive): t's logit becomes 4x the maximum, so argmax moves to t.
    t = 321
    W2 = dict(W)
    lm = W["lm_head"].copy()
    j = 1
    am = int(d["draft_ids"][0, j])
    lm[t] = 4.0 * lm[am]
    W2["lm_head"] = lm
    d2 = oracle.draft_block(cfg, W2, cache, [17], [40], pt)
    assert d2["draft_ids"][0, j] == t
    assert np.allclose(d2["logits"][0, j, t], 4.0 * d["logits"][0, j, am], rtol=1e-12)


def test_draft_reads_only_committed_context():
    """Slots at or beyond the prefix stay NaN in the cache; a finite result
    shows the pass never reads them (and never reads other requests' pages)."""
    cfg = SMALL_F32_D64
    W, pt, npages = _setup(cfg, L=(1, 33))
    cache = _ctx_cache(cfg, W, pt, npages, [1, 33])
    d = oracle.draft_block(cfg, W, cache, [0, 1], [1, 33], pt)
    assert np.isfinite(d["logits"]).all()


def test_speculative_decode_equals_greedy_target():
    """Greedy speculative decoding must emit exactly the target's own greedy
    continuation, whatever the draft proposes ("Inside SGLang ...", Step 5-7:
    the target verifies every block and supplies the correction/bonus)."""
    cfg = TINY
    W = np_weights(synth.weights(cfg, 0))
    V = cfg.vocab
    rng = np.random.default_rng(7)
    feat_tab = rng.standard_normal((64, cfg.feat_dim)) * 0.02

    def target_next(tok, pos):        # a Markov stand-in for the target model
        return int((tok * 7 + pos * 3 + 11) % 13)

    def target_feat(tok, pos):
        return feat_tab[(tok * 5 + pos) % 64]

    prompt = [5, 3, 8, 1, 2, 9, 4]
    pt = np.arange(8)[None, :]
    em, commits, L, cache = oracle.speculative_decode(cfg, W, 8 * 16, pt, prompt, 30,
                                                      target_next, target_feat)
    ref = [target_next(prompt[-1], len(prompt) - 1)]
    while len(ref) < len(em):
        ref.append(target_next(ref[-1], len(prompt) + len(ref) - 1))
    assert em == ref
    assert L == len(prompt) + sum(commits)
    assert len(em) == 1 + sum(commits)
    assert all(1 <= c <= cfg.block_size for c in commits)


# ---------------------------------------------------------------- library cross-check
@pytest.mark.parametrize("windowed", [False, True])
def test_draft_pass_matches_transformers_qwen3_layers(windowed):
    """The draft backbone is a stack of Qwen3 decoder layers whose attention
    reads the injected context K/V as a pre-filled cache, with no causal mask
    inside the block.  transformers' own Qwen3DecoderLayer (an independent
    implementation of the pre-norm layer, per-head q/k RMSNorm, neox RoPE, GQA
    and SwiGLU) must give the oracle's logits."""
    from transformers import Qwen3Config
    from transformers.cache_utils import DynamicCache
    from transformers.models.qwen3 import modeling_qwen3 as q3

    cfg = SMALL_F32_D64 if windowed else dataclasses.replace(SMALL_F32_D64, sliding_window=())
    W, pt, npages = _setup(cfg, L=(45, 61))
    L = [45, 61]
    cache = _ctx_cache(cfg, W, pt, npages, L)
    anchors = [5, 6]
    o = oracle.draft_block(cfg, W, cache, anchors, L, pt)

    hc = Qwen3Config(hidden_size=cfg.hidden, intermediate_size=cfg.inter,
                     num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_q_heads,
                     num_key_value_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                     rms_norm_eps=cfg.rms_eps, vocab_size=cfg.vocab, attention_bias=False,
                     rope_theta=cfg.rope_theta, max_position_embeddings=1 << 20)
    hc._attn_implementation = "eager"
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    nq, nkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    layers = []
    for l in range(cfg.n_layers):
        lay = q3.Qwen3DecoderLayer(hc, l).double()
        Lw = W["layers"][l]
        wqkv = t(Lw["w_qkv"])
        with torch.no_grad():
            lay.self_attn.q_proj.weight.copy_(wqkv[:nq * D])
            lay.self_attn.k_proj.weight.copy_(wqkv[nq * D:(nq + nkv) * D])
            lay.self_attn.v_proj.weight.copy_(wqkv[(nq + nkv) * D:])
            lay.self_attn.o_proj.weight.copy_(t(Lw["w_o"]))
            lay.self_attn.q_norm.weight.copy_(t(Lw["q_norm"]))
            lay.self_attn.k_norm.weight.copy_(t(Lw["k_norm"]))
            lay.input_layernorm.weight.copy_(t(Lw["in_norm"]))
            lay.post_attention_layernorm.weight.copy_(t(Lw["post_norm"]))
            lay.mlp.gate_proj.weight.copy_(t(Lw["w_gate"]))
            lay.mlp.up_proj.weight.copy_(t(Lw["w_up"]))
            lay.mlp.down_proj.weight.copy_(t(Lw["w_down"]))
        layers.append(lay)
    rope = q3.Qwen3RotaryEmbedding(hc).double()
    final = q3.Qwen3RMSNorm(cfg.hidden, eps=cfg.rms_eps).double()
    with torch.no_grad():
        final.weight.copy_(t(W["final_norm"]))
    S, P = cfg.block_size, cfg.page_size
    for r in range(2):
        ids = [anchors[r]] + [cfg.mask_token_id] * (S - 1)
        x = t(W["embed"][ids])[None]                                 # [1, S, H]
        pos = torch.arange(L[r], L[r] + S)[None]
        pe = rope(x, pos)
        kv = DynamicCache()
        cpos = np.arange(L[r])
        cslot = pt[r, cpos // P] * P + cpos % P
        for l in range(cfg.n_layers):
            kv.update(t(cache.k[l][cslot]).permute(1, 0, 2)[None],
                      t(cache.v[l][cslot]).permute(1, 0, 2)[None], l)
        with torch.no_grad():
            for l, lay in enumerate(layers):
                mask = torch.zeros(1, 1, S, L[r] + S, dtype=torch.float64)
                Wl = cfg.window(l)
                if Wl:
                    vis = _hf_window_visible(np.arange(L[r], L[r] + S), np.arange(L[r]), Wl)
                    mask[0, 0, :, :L[r]] = torch.where(vis, 0.0, float("-inf"))
                out = lay(x, attention_mask=mask, position_ids=pos, past_key_values=kv,
                          use_cache=True, position_embeddings=pe)
                x = out[0] if isinstance(out, tuple) else out
            logits = final(x[:, 1:]) @ t(W["lm_head"]).T
        # transformers builds its RoPE frequency table in fp32 (relative error
        # ~1e-7); any structural difference would show at the 1e-1 scale
        assert np.allclose(logits[0].numpy(), o["logits"][r], rtol=1e-5, atol=1e-5)


# ---------------------------------------------------------------- draft window
def _windowed(cfg, n):
    return dataclasses.replace(cfg, context_window=n)


def test_draft_window_covering_the_context_changes_nothing():
    cfg = SMALL_F32_D64
    W, pt, npages = _setup(cfg, L=(45, 61))
    cache = _ctx_cache(cfg, W, pt, npages, [45, 61])
    a = oracle.draft_block(cfg, W, cache, [5, 6], [45, 61], pt)
    b = oracle.draft_block(_windowed(cfg, 61), W, cache, [5, 6], [45, 61], pt)
    assert np.array_equal(a["logits"], b["logits"])


def test_draft_window_ring_table_equals_linear_table():
    """A ring of R pages holding only the window's rows (logical page q in
    physical page table[q mod R]) gives bit-identical logits to the full
    linear table; rows before the window are NaN in the linear cache, so a
    finite result also shows they are never read."""
    N, L = 20, [45, 61]
    cfg = _windowed(SMALL_F32_D64, N)
    W, pt, npages = _setup(cfg, L=tuple(L))
    lin = _ctx_cache(cfg, W, pt, npages, L)
    S, P = cfg.block_size, cfg.page_size
    R = (N + S - 1 + P - 1) // P + 1                  # pages spanned by window + block
    rng = np.random.default_rng(0)
    ring_pt = rng.permutation(2 * R)[:2 * R].reshape(2, R)
    ring = oracle.OracleCache(cfg, 2 * R * P)
    for r, l in enumerate(L):
        for p in range(l - N, l):
            src = pt[r, p // P] * P + p % P
            dst = ring_pt[r, (p // P) % R] * P + p % P
            for layer in range(cfg.n_layers):
                ring.k[layer][dst] = lin.k[layer][src]
                ring.v[layer][dst] = lin.v[layer][src]
        for p in range(0, l - N):                    # poison what the window excludes
            src = pt[r, p // P] * P + p % P
            for layer in range(cfg.n_layers):
                lin.k[layer][src] = np.nan
                lin.v[layer][src] = np.nan
    a = oracle.draft_block(cfg, W, lin, [5, 6], L, pt)
    b = oracle.draft_block(cfg, W, ring, [5, 6], L, ring_pt)
    assert np.isfinite(a["logits"]).all()
    assert np.array_equal(a["logits"], b["logits"])
    pos = np.array(L)[:, None] + np.arange(S)
    assert np.array_equal(b["slots"], ring_pt[np.arange(2)[:, None], (pos // P) % R] * P + pos % P)


def test_draft_window_equals_shifted_short_context():
    """Attending to the last N rows of an L-row context equals attending to a
    context of exactly those N rows re-injected at positions shifted by L - N
    (RoPE sees only differences): the window means what it says."""
    N, L = 24, 61
    base = dataclasses.replace(SMALL_F32_D64, sliding_window=())
    cfg = _windowed(base, N)
    W, pt, npages = _setup(cfg, L=(L,))
    f = synth.features(L, cfg, 5).numpy()
    full = oracle.OracleCache(cfg, npages * 16)
    pos = np.arange(L)
    oracle.project_context(cfg, W, full, f, pos, pt[0, pos // 16] * 16 + pos % 16)
    a = oracle.draft_block(cfg, W, full, [7], [L], pt)
    short = oracle.OracleCache(base, npages * 16)
    sp = np.arange(N)
    oracle.project_context(base, W, short, f[L - N:], sp, pt[0, sp // 16] * 16 + sp % 16)
    b = oracle.draft_block(base, W, short, [7], [N], pt)
    assert np.allclose(a["logits"], b["logits"], rtol=1e-5, atol=1e-5)
    c = oracle.draft_block(base, W, full, [7], [L], pt)
    assert not np.allclose(a["logits"], c["logits"], rtol=1e-3, atol=1e-3)
