"""The three operations of the DFlash draft-and-accept path, fp64 (fp32 under
the timing setting of oracle.precision).

Notation: H hidden, nq / nkv query / kv heads, D head_dim, G = nq / nkv,
S block size (anchor included), B requests, L_r committed prefix of request r,
P page size.  Matrices are [out, in]; y = x @ W.T.
"""
from __future__ import annotations

import numpy as np

from .formats import round_kv
from .precision import real
from .primitives import rms_norm, rope_neox, silu, block_attention


def _f64(a):
    """a in the working precision (fp64 unless the timing setting is on)."""
    return np.asarray(a, dtype=real())


def _qkv_split(w_qkv, cfg):
    nq, nkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    w = np.asarray(w_qkv)
    return w[:nq * D], w[nq * D:(nq + nkv) * D], w[(nq + nkv) * D:]


def _linear_chunked(x, w, chunk=16384):
    """x @ w.T with w converted to the working precision one block of output
    rows at a time."""
    w = np.asarray(w)
    out = np.empty(x.shape[:-1] + (w.shape[0],), dtype=real())
    for n0 in range(0, w.shape[0], chunk):
        out[..., n0:n0 + chunk] = x @ _f64(w[n0:n0 + chunk]).T
    return out


class OracleCache:
    """Draft K/V cache indexed by physical slot: K[l][slot] is [nkv, D].

    Unwritten slots hold NaN so that reading one poisons the result.
    """

    def __init__(self, cfg, num_slots):
        shp = (num_slots, cfg.n_kv_heads, cfg.head_dim)
        self.k = [np.full(shp, np.nan, dtype=real()) for _ in range(cfg.n_layers)]
        self.v = [np.full(shp, np.nan, dtype=real()) for _ in range(cfg.n_layers)]

    def copy(self):
        c = OracleCache.__new__(OracleCache)
        c.k = [a.copy() for a in self.k]
        c.v = [a.copy() for a in self.v]
        return c


def block_prep(anchor, prefix_len, page_table, block_size, mask_token_id, page_size):
    """Block preparation ("Inside SGLang ...", Step 3; CSDN article, step 7).

    For request r and block offset j: input id = anchor_r if j == 0 else the
    mask id; logical position = L_r + j; physical slot = the request's
    position-to-slot mapping at that position, here a page table read as a
    ring: page_table[r][(pos // P) mod width] * P + pos % P (the identity
    when the table covers every position; with a draft window the table
    only needs the pages of the window and the block, which is the private
    compact mapping windowed drafting uses: "Inside SGLang ...", section
    "Who owns what?" of the startup walk-through).
    """
    anchor = np.asarray(anchor, np.int64)
    L = np.asarray(prefix_len, np.int64)
    B, S = anchor.shape[0], block_size
    ids = np.full((B, S), mask_token_id, dtype=np.int64)
    ids[:, 0] = anchor
    pos = L[:, None] + np.arange(S)[None, :]
    pt = np.asarray(page_table, np.int64)
    slots = pt[np.arange(B)[:, None], (pos // page_size) % pt.shape[1]] * page_size + \
        pos % page_size
    return ids, pos, slots


def project_context(cfg, W, cache, feats, positions, slots, valid_rows=None,
                    rows_per_req=None):
    """Context injection ("Inside SGLang ...", Step 1 and Step 7; CSDN article,
    draft model input and the fused K/V materialisation section).

    The concatenated target features f [T, F] become c = hidden_norm(fc(f)),
    an RMSNorm over the fc output.  The same c feeds every draft layer l: its
    K/V projection, the layer's k-norm (per head) and RoPE at the row's
    logical position give the context K; V is the plain projection.  Both are
    rounded to the cache dtype and stored at the row's physical slot.  The
    context does not pass through the layer's input norm or the rest of the
    layer.  Only live rows are written: with valid_rows given, the rows form a
    dense [n_req, rows_per_req] grid and row j of request r is live iff
    j < valid_rows[r] (prefix-valid writes of the committed verify rows).
    Returns the boolean live mask.
    """
    feats = _f64(feats)
    T = feats.shape[0]
    positions = np.asarray(positions, np.int64).reshape(-1)
    slots = np.asarray(slots, np.int64).reshape(-1)
    live = np.ones(T, dtype=bool)
    if valid_rows is not None:
        j = np.arange(T) % rows_per_req
        r = np.arange(T) // rows_per_req
        live = j < np.asarray(valid_rows, np.int64)[r]
    if not live.any():
        return live
    nkv, D = cfg.n_kv_heads, cfg.head_dim
    c = rms_norm(feats[live] @ _f64(W["fc"]).T, _f64(W["hidden_norm"]), cfg.rms_eps)
    pos, sl = positions[live], slots[live]
    for l in range(cfg.n_layers):
        Lw = W["layers"][l]
        _, wk, wv = _qkv_split(Lw["w_qkv"], cfg)
        k = (c @ _f64(wk).T).reshape(-1, nkv, D)
        v = (c @ _f64(wv).T).reshape(-1, nkv, D)
        k = rms_norm(k, _f64(Lw["k_norm"]), cfg.rms_eps)
        k = rope_neox(k, pos[:, None], cfg.rope_theta)
        cache.k[l][sl] = round_kv(k, cfg.kv_dtype)
        cache.v[l][sl] = round_kv(v, cfg.kv_dtype)
    return live


def draft_block(cfg, W, cache, anchor, prefix_len, page_table, rope=True, requests=None):
    """One non-causal draft pass over [anchor, MASK x (S-1)] per request
    ("Inside SGLang ...", Step 3 and Step 4; CSDN article, draft model predict
    and SGLang flow step 7).

    x = E[ids] (the target's embedding; the drafter has none of its own).
    Each decoder layer (Qwen3-style pre-norm):
        h = rms(x; in_norm); q, k, v = h Wq^T, h Wk^T, h Wv^T
        q, k per head <- RoPE(rms(.; q_norm / k_norm), pos)
        o = attention of the block queries over the cached context keys at
            logical positions [0, L_r) (window-limited on sliding layers; with
            a draft window N only positions [L_r - N, L_r), on every layer)
            and all S block keys, non-causal
        x += o Wo^T;  h2 = rms(x; post_norm);  x += (silu(h2 Wg^T) * h2 Wu^T) Wd^T
    Final: y = rms(x; final_norm) on rows 1..S-1 (the anchor row is not a
    prediction), logits = y W_lm^T with the target's lm_head, draft id =
    argmax (first index among equal maxima).  The block's own K/V are not
    stored (the draft cache is cropped back to the prefix).

    rope=False skips RoPE everywhere (used by the permutation pin).
    requests: optional subset of request indices to evaluate (others skipped).
    Returns a dict: block_ids, positions, slots [B, S]; logits [b, S-1, V];
    draft_ids [b, S-1]; candidates [b, S] for the evaluated requests.
    """
    S, P = cfg.block_size, cfg.page_size
    ids, pos, slots = block_prep(anchor, prefix_len, page_table, S, cfg.mask_token_id, P)
    L = np.asarray(prefix_len, np.int64)
    pt = np.asarray(page_table, np.int64)
    reqs = list(range(ids.shape[0])) if requests is None else list(requests)
    nq, nkv, D, H = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.hidden
    emb = np.asarray(W["embed"])
    x = np.stack([_f64(emb[ids[r]]) for r in reqs])          # [b, S, H]
    b = len(reqs)
    for l in range(cfg.n_layers):
        Lw = W["layers"][l]
        wq, wk, wv = _qkv_split(Lw["w_qkv"], cfg)
        h = rms_norm(x, _f64(Lw["in_norm"]), cfg.rms_eps)
        q = (h @ _f64(wq).T).reshape(b, S, nq, D)
        k = (h @ _f64(wk).T).reshape(b, S, nkv, D)
        v = (h @ _f64(wv).T).reshape(b, S, nkv, D)
        q = rms_norm(q, _f64(Lw["q_norm"]), cfg.rms_eps)
        k = rms_norm(k, _f64(Lw["k_norm"]), cfg.rms_eps)
        if rope:
            q = rope_neox(q, pos[reqs][:, :, None], cfg.rope_theta)
            k = rope_neox(k, pos[reqs][:, :, None], cfg.rope_theta)
        o = np.empty((b, S, nq, D), dtype=real())
        W_l = cfg.window(l)
        for i, r in enumerate(reqs):
            lo = 0
            if W_l:
                lo = max(0, int(L[r]) - W_l + 1)
            if cfg.context_window:
                lo = max(lo, int(L[r]) - cfg.context_window)
            cpos = np.arange(lo, int(L[r]), dtype=np.int64)
            cslot = pt[r, (cpos // P) % pt.shape[1]] * P + cpos % P
            o[i] = block_attention(q[i], cache.k[l][cslot], cache.v[l][cslot], cpos,
                                   k[i], v[i], pos[r], W_l)
        x = x + o.reshape(b, S, nq * D) @ _f64(Lw["w_o"]).T
        h2 = rms_norm(x, _f64(Lw["post_norm"]), cfg.rms_eps)
        act = silu(h2 @ _f64(Lw["w_gate"]).T) * (h2 @ _f64(Lw["w_up"]).T)
        x = x + act @ _f64(Lw["w_down"]).T
    y = rms_norm(x[:, 1:, :], _f64(W["final_norm"]), cfg.rms_eps)
    logits, draft = select_draft_tokens(y, W["lm_head"])
    cand = np.concatenate([np.asarray(anchor, np.int64)[reqs][:, None], draft], axis=1)
    return {"block_ids": ids, "positions": pos, "slots": slots, "logits": logits,
            "draft_ids": draft, "candidates": cand, "requests": reqs, "hidden": y}


def select_draft_tokens(y, lm_head):
    """The selection step on final draft hidden rows ("Inside SGLang ...",
    Step 4: the target's lm_head turns each normalised row into logits, the
    greedy draft token is their argmax).  y [..., H] (already through the final
    RMSNorm), lm_head [V, H]; returns logits = y lm_head^T [..., V] and the
    first index among equal maxima [...]."""
    logits = _linear_chunked(_f64(y), lm_head)
    return logits, np.argmax(logits, axis=-1)


def accept(candidates, posterior, prefix_len):
    """Greedy verify-accept and commit ("Inside SGLang ...", Step 6 and Step 7;
    CSDN article, the z-lab verify step and SGLang flow steps 7-9).

    candidates[r] = [anchor, d_1, ..., d_{S-1}]; posterior[r, j] is the
    target's greedy choice after reading candidates[r, j].  Draft d_{j+1}
    survives while it equals posterior[r, j]; the walk stops at the first
    mismatch.  accept_len a = number of surviving drafts (0..S-1);
    commit = a + 1 (surviving drafts plus one target token: the correction at
    the first mismatch, or the bonus after full acceptance); out_tokens =
    d_1..d_a, posterior[a], then zero padding; next anchor = posterior[a];
    new prefix = L + commit (the cache is cropped logically to it).
    """
    cand = np.asarray(candidates, np.int64)
    post = np.asarray(posterior, np.int64)
    L = np.asarray(prefix_len, np.int64)
    B, S = cand.shape
    acc = np.zeros(B, np.int64)
    out = np.zeros((B, S), np.int64)
    for r in range(B):
        a = 0
        while a < S - 1 and cand[r, a + 1] == post[r, a]:
            a += 1
        acc[r] = a
        out[r, :a] = cand[r, 1:a + 1]
        out[r, a] = post[r, a]
    commit = acc + 1
    bonus = post[np.arange(B), acc]
    return {"accept_len": acc, "commit_len": commit, "out_tokens": out,
            "next_anchor": bonus, "new_seq_len": L + commit}


def greedy_posterior(target_logits):
    """The target's greedy token at every verified position ("Inside SGLang
    ...", Step 6: the verify forward's logits give the target's choice after
    each block position): the first index among equal maxima over the
    vocabulary.  Reading: a NaN logit never wins (it counts as -inf, so a row
    of only NaN and -inf gives index 0).  target_logits [..., V] -> [...]."""
    x = np.asarray(target_logits, np.float64)
    x = np.where(np.isnan(x), -np.inf, x)
    return np.argmax(x, axis=-1)


def accept_logits(candidates, target_logits, prefix_len):
    """Greedy verify-accept reading the target's logits [B, S, V] instead of
    its greedy ids: accept() against greedy_posterior(target_logits)."""
    return accept(candidates, greedy_posterior(target_logits), prefix_len)


def speculative_decode(cfg, W, num_slots, page_table, prompt_tokens, max_new,
                       target_next, target_feat):
    """The decode loop for one request with a stand-in target (CSDN article,
    the z-lab loop; "Inside SGLang ...", the whole loop and Step 7).

    target_next(token, pos): the target's greedy next token after reading
    `token` at logical position `pos`; target_feat(token, pos): the target's
    concatenated layer features [F] for that input.  Prefill injects the
    prompt's features and samples the first anchor; each cycle drafts a
    block, verifies it, emits out_tokens[:commit] and injects the features of
    the committed verify rows [anchor, d_1..d_a].
    Returns (emitted tokens, list of commit lengths, final prefix length, cache).
    """
    cache = OracleCache(cfg, num_slots)
    P, S = cfg.page_size, cfg.block_size
    pt = np.asarray(page_table, np.int64)[None] if np.ndim(page_table) == 1 else \
        np.asarray(page_table, np.int64)
    L0 = len(prompt_tokens)
    pos = np.arange(L0)
    feats = np.stack([target_feat(t, p) for t, p in zip(prompt_tokens, pos)])
    project_context(cfg, W, cache, feats, pos, pt[0, pos // P] * P + pos % P)
    anchor = target_next(prompt_tokens[-1], L0 - 1)
    emitted = [anchor]
    L = L0
    commits = []
    while len(emitted) < max_new:
        d = draft_block(cfg, W, cache, [anchor], [L], pt)
        cand = d["candidates"][0]
        post = np.array([target_next(int(cand[j]), L + j) for j in range(S)])
        a = accept(cand[None], post[None], [L])
        c = int(a["commit_len"][0])
        emitted.extend(int(t) for t in a["out_tokens"][0, :c])
        commits.append(c)
        vfeat = np.stack([target_feat(int(cand[j]), L + j) for j in range(S)])
        project_context(cfg, W, cache, vfeat, d["positions"][0], d["slots"][0],
                        valid_rows=[c], rows_per_req=S)
        L = int(a["new_seq_len"][0])
        anchor = int(a["next_anchor"][0])
    return emitted, commits, L, cache
