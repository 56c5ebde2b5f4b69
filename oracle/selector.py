"""DFlash 2 candidate selector, fp64 (TEST INFRASTRUCTURE ONLY).

Follows "Inside SGLang: DFlash and DFlash 2 Implementation" (himanshu-arora.com),
section "DFlash 2: replace selection, retain the serving loop", in the order it
gives: candidates, then the lattice, then the walk.

* Candidates: per drafted position j (rows 1..S-1 of the block, the rows the
  lm_head reads) the K tokens with the largest unary logits U_j = y_j W_lm^T,
  in descending order of logit, ties to the lower token id.
* Lattice: for every position the score of each (predecessor p, candidate c)
  pair, score(p, c) = U_j(c) + <A[p] * (W_h y_j), B[c]>, with A and B learned
  per-token tables of rank r and W_h a learned [r, H] projection of the
  position's hidden row.  The predecessor of the first drafted position is
  the anchor; later positions take the K candidates of the position before.
  All scores are built before the walk.
* Walk: position by position, the row of the predecessor actually chosen;
  greedy takes the first maximum (in candidate order), sampling draws from
  softmax(row / T) by inverse CDF at a caller-supplied uniform.  q_rows[j] is
  the realised proposal distribution the sampled verify needs (the section on
  sampling asks the verify to use the distribution the walk actually drew
  from): softmax(row / T) of the chosen predecessor's row when sampling, the
  point mass on the chosen slot when greedy.  The walk does not search for
  the best full path.

Readings (the section leaves them open): y_j is the final-normed hidden row
(the lm_head's input); U is the unary logit as the lm_head computes it (the
act-dtype logits); K = 8 and r = 64 by default; the same softmax temperature
T is used for sampling and for q_rows.

Pins (tests/test_oracle_selector.py): with the compatibility term switched
off (A = 0) the greedy walk returns the plain argmax drafts of the draft pass;
a planted compatibility that favours one successor after a given
predecessor is followed; a lattice where greedy and the best full path differ
shows the walk is greedy; greedy q_rows are one-hot on the choice, and fed
to the sampled verify they give the point-mass verify's decisions and
target-distributed tokens (softmax rows there would not).
"""
import numpy as np


def _softmax(z):
    z = np.asarray(z, np.float64)
    e = np.exp(z - np.max(z))
    return e / e.sum()


def top_k(logits, k):
    """Indices of the k largest values per row: descending value, ties to the
    lower index.  logits [..., V] -> (ids [..., k], values [..., k])."""
    x = np.asarray(logits, np.float64)
    V = x.shape[-1]
    # sort by (-value, index): a stable sort on -value keeps lower indices first
    order = np.argsort(-x, axis=-1, kind="stable")[..., :k]
    return order, np.take_along_axis(x, order, axis=-1)


def build_lattice(cand, unary, anchor, hidden, A, Bt, Wh):
    """score[b, j, p, c] for drafted position j (0-based over rows 1..S-1),
    predecessor slot p (j = 0: only p = 0, the anchor) and candidate slot c."""
    cand = np.asarray(cand, np.int64)
    B, J, K = cand.shape
    A = np.asarray(A, np.float64)
    Bt = np.asarray(Bt, np.float64)
    w = np.asarray(hidden, np.float64) @ np.asarray(Wh, np.float64).T      # [B, J, r]
    score = np.full((B, J, K, K), -np.inf)
    for b in range(B):
        for j in range(J):
            preds = [int(anchor[b])] if j == 0 else list(cand[b, j - 1])
            for pi, p in enumerate(preds):
                compat = (A[p] * w[b, j]) @ Bt[cand[b, j]].T                   # [K]
                score[b, j, pi] = unary[b, j] + compat
    return score


def walk(cand, score, uniforms=None, temperature=1.0):
    """Greedy (uniforms None) or sampled walk through the lattice."""
    cand = np.asarray(cand, np.int64)
    B, J, K = cand.shape
    draft = np.zeros((B, J), np.int64)
    q_rows = np.zeros((B, J, K))
    chosen = np.zeros((B, J), np.int64)
    T = float(temperature)
    for b in range(B):
        p = 0
        for j in range(J):
            row = score[b, j, p]
            if uniforms is None:
                k = int(np.argmax(row))                    # first maximum
                q = np.zeros(K)
                q[k] = 1.0                                 # a point mass: nothing was drawn
            else:
                q = _softmax(row / T)
                c = np.cumsum(q)
                hit = np.nonzero(c > float(uniforms[b, j]) * c[-1])[0]
                k = int(hit[0]) if hit.size else K - 1
            q_rows[b, j] = q
            chosen[b, j] = k
            draft[b, j] = cand[b, j, k]
            p = k
    return draft, q_rows, chosen


def select(logits, hidden, anchor, A, Bt, Wh, k=8, uniforms=None, temperature=1.0):
    """The selector over one draft pass: logits [B, S-1, V] (unary), hidden
    [B, S-1, H] (final-normed rows 1..S-1), anchor [B].  Returns candidate ids
    [B, S-1, K], draft tokens [B, S-1], q_rows [B, S-1, K], the lattice and the
    chosen slots."""
    cand, unary = top_k(logits, k)
    score = build_lattice(cand, unary, anchor, hidden, A, Bt, Wh)
    draft, q_rows, chosen = walk(cand, score, uniforms, temperature)
    return {"cand_ids": cand, "unary": unary, "score": score, "draft_ids": draft,
            "q_rows": q_rows, "chosen": chosen}
