"""Rejection-sampling verify-accept, fp64 (TEST INFRASTRUCTURE ONLY).

Follows "Inside SGLang: DFlash and DFlash 2 Implementation" (himanshu-arora.com),
section "Sampling: preserve the proposal distribution the walk actually used",
together with Step 6 (acceptance, output and computed state) for what the
cycle emits and commits.  The CSDN DFlash article (SGLang flow, the target
verify step) notes that non-greedy requests take a separate speculative-
sampling verify that yields the surviving drafts and the bonus token.

What the section fixes: a drafted token y survives with probability
min(1, p(y) / q(y)), where p is the target's distribution and q the one the
drafter drew from; the first rejected position is replaced by a draw from
[p - q]_+ rescaled to sum to one; when every draft survives, one more token
is drawn from the target's distribution at the last row.  The plain DFlash
drafter takes argmax tokens, so its q puts all mass on the drafted token.

Readings where the section is silent (each also applied by the GPU path):
* p_j = softmax(target_logits[j] / T_t): row j is the target's distribution
  after reading candidates[j], i.e. the one that verifies d_{j+1} (the same
  one-position shift as the greedy verify of Step 6).
* q_j = softmax(draft_logits[j] / T_d) when draft logits are given (row j
  proposed d_{j+1}); q_j = draft_probs[j] when a proposal distribution is
  given directly (the DFlash 2 selector's realised q rows, scattered over the
  vocabulary as the section describes); otherwise the point mass on d_{j+1}.
* The random draws are inputs: uniforms[r, j] in [0, 1) for j < S - 1 is the
  acceptance draw of d_{j+1} ("accept iff u * q(y) < p(y)", the event
  u < min(1, p/q) written without a division); uniforms[r, S - 1] is the one
  draw that picks the correction or bonus token by inverse CDF: the smallest
  token t whose running sum of weights exceeds u * (sum of all weights).
* If the residual [p - q]_+ has no mass (only possible when p == q, where a
  rejection cannot happen for u < 1), the token is drawn from p instead.
* If u * total is not below any running sum (u rounded up to 1), the last
  token with positive weight is taken.

Pins (tests/test_oracle_sampling.py): the theorem the method rests on (every
emitted token is distributed as the target's p, checked by chi-square on many
seeded draws, conditional on the earlier tokens being accepted), the greedy
limit T_t -> 0 against the greedy accept, q == p accepting every draft, and
p(y) == 0 rejecting.
"""
import numpy as np


def _softmax(z):
    z = np.asarray(z, np.float64)
    e = np.exp(z - np.max(z))
    return e / e.sum()


def _inverse_cdf(w, u):
    """Smallest t with cumsum(w)[t] > u * sum(w); the last positive-weight
    token when none is (u at the top of [0, 1) after rounding)."""
    c = np.cumsum(w)
    x = u * c[-1]
    hit = np.nonzero(c > x)[0]
    if hit.size:
        return int(hit[0]), x
    return int(np.nonzero(w > 0)[0][-1]), x


def accept_sampling(candidates, target_logits, prefix_len, uniforms, target_temperature,
                    draft_logits=None, draft_temperature=1.0, draft_probs=None):
    """Rejection-sampling verify and commit for a batch of blocks.

    candidates    [B, S]     [anchor, d_1 .. d_{S-1}]
    target_logits [B, S, V]  row j: the target's logits after reading candidates[j]
    draft_logits  [B, S-1, V] or None (argmax proposals: q is a point mass)
    draft_probs   [B, S-1, V] or None: q itself (takes precedence over draft_logits)
    uniforms      [B, S]     draws in [0, 1): acceptance draws, then the token draw
    Returns the greedy accept's outputs (accept_len, commit_len, out_tokens,
    next_anchor, new_seq_len) plus, per request, what a comparison with a
    computation done in another precision needs: `margin` (the smallest relative
    gap |u q(y) - p(y)| / max(u q(y), p(y)) over the decisions taken; inf when
    both sides are exactly 0), `weights` (the unnormalised
    weights the final token was drawn from) and `draw` (u * their sum).
    """
    cand = np.asarray(candidates, np.int64)
    tl = np.asarray(target_logits, np.float64)
    u = np.asarray(uniforms, np.float64)
    L = np.asarray(prefix_len, np.int64)
    B, S = cand.shape
    Tt = float(target_temperature)
    dl = None if draft_logits is None else np.asarray(draft_logits, np.float64)
    dq = None if draft_probs is None else np.asarray(draft_probs, np.float64)
    Td = float(draft_temperature)

    acc = np.zeros(B, np.int64)
    out = np.zeros((B, S), np.int64)
    bonus = np.zeros(B, np.int64)
    margin = np.full(B, np.inf)
    weights, draws = [], np.zeros(B)
    for r in range(B):
        a = 0
        w = None
        while a < S - 1:
            y = cand[r, a + 1]
            p = _softmax(tl[r, a] / Tt)
            if dq is not None:
                q = dq[r, a]
            elif dl is None:
                q = np.zeros_like(p)
                q[y] = 1.0
            else:
                q = _softmax(dl[r, a] / Td)
            lhs, rhs = u[r, a] * q[y], p[y]
            if max(lhs, rhs) > 0:
                margin[r] = min(margin[r], abs(lhs - rhs) / max(lhs, rhs))
            if lhs < rhs:
                a += 1
                continue
            w = np.maximum(p - q, 0.0)
            if not np.any(w > 0):
                w = p
            break
        if w is None:                       # every draft survived: bonus from p_{S-1}
            w = _softmax(tl[r, S - 1] / Tt)
        t, x = _inverse_cdf(w, u[r, S - 1])
        acc[r] = a
        out[r, :a] = cand[r, 1:a + 1]
        out[r, a] = t
        bonus[r] = t
        weights.append(w)
        draws[r] = x
    commit = acc + 1
    return {"accept_len": acc, "commit_len": commit, "out_tokens": out,
            "next_anchor": bonus, "new_seq_len": L + commit,
            "margin": margin, "weights": weights, "draw": draws}
