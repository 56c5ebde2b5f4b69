"""Primitive operations of the draft model, fp64 (fp32 under the timing
setting of oracle.precision).

* rms_norm: RMSNorm with a learned gain, used by hidden_norm (the fc +
  hidden_norm projection of the fused target features), the per-head Q/K
  normalisation and the decoder-layer / final norms ("Inside SGLang ...",
  Step 1 and Step 4; CSDN article, the K RMSNorm of the fused K/V path).
* rope_neox: rotary position embedding in the neox / rotate-half layout over
  the full head dimension, driven by absolute token positions (CSDN article,
  fused_kv_materialize enabling conditions: neox-style RoPE, uniform rotary
  dim; "Inside SGLang ...", Step 3: positions drive RoPE).
* block_attention: non-causal attention of the block queries over the cached
  context keys plus every key of the block ("Inside SGLang ...", Step 4: query
  positions interact within the block; CSDN article, draft predict called
  with is_causal=False), with an optional sliding window over the context
  (Kimi-K2.6-DFlash config sample: sliding_attention layers, window 2048).
"""
import numpy as np

from .precision import real


def rms_norm(x, g, eps):
    """g * x / sqrt(mean(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=real())
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=real())


def rope_neox(x, pos, theta):
    """Rotate pairs (x[i], x[i + D/2]) by angle pos * theta^(-2i/D)."""
    x = np.asarray(x, dtype=real())
    D = x.shape[-1]
    half = D // 2
    inv_freq = float(theta) ** (-2.0 * np.arange(half, dtype=real()) / D)
    ang = np.asarray(pos, dtype=real())[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z):
    z = np.asarray(z, dtype=real())
    return z / (1.0 + np.exp(-z))


def softmax(s, axis=-1):
    s = np.asarray(s, dtype=real())
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def block_attention(q, k_ctx, v_ctx, ctx_pos, k_blk, v_blk, q_pos, window):
    """One request, one layer.

    q      [S, nq, D]   block queries (after q-norm and RoPE)
    k_ctx  [n, nkv, D]  cached context keys (as stored), v_ctx likewise
    ctx_pos[n]          logical positions of the context keys
    k_blk  [S, nkv, D]  the block's own keys (after k-norm and RoPE), v_blk likewise
    q_pos  [S]          logical positions of the block rows
    window 0 for full attention, else W: context key i is visible to query
           position p iff p - i < W.  Block keys are always visible (non-causal).
    Query head h reads kv head h // (nq / nkv).  Scale 1/sqrt(D).
    Returns o [S, nq, D].
    """
    q = np.asarray(q, real())
    S, nq, D = q.shape
    nkv = k_blk.shape[1]
    G = nq // nkv
    keys = np.concatenate([np.asarray(k_ctx, real()), np.asarray(k_blk, real())], 0)
    vals = np.concatenate([np.asarray(v_ctx, real()), np.asarray(v_blk, real())], 0)
    n = k_ctx.shape[0]
    visible = np.ones((S, n + S), dtype=bool)
    if window and n:
        visible[:, :n] = (np.asarray(q_pos)[:, None] - np.asarray(ctx_pos)[None, :]) < window
    o = np.empty_like(q)
    for h in range(nq):
        g = h // G
        s = q[:, h, :] @ keys[:, g, :].T / np.sqrt(D)
        s = np.where(visible, s, -np.inf)
        p = softmax(s, axis=-1)
        o[:, h, :] = p @ vals[:, g, :]
    return o
