"""Seeded synthetic inputs for the DFlash path.

Every tensor has its own torch.Generator seeded from (workload seed, tensor
name), so any subset can be regenerated alone and in any order.  Matrices and
features are N(0, 0.02^2) drawn in fp32 and rounded once to the activation
dtype; norm gains are 1 + N(0, 0.02^2) (a literal N(0, 0.02) gain would shrink
every logit towards zero and make argmax agreement vacuous); token ids are
uniform.  Physical cache pages are a seeded random permutation, so a cache
slot is never equal to a logical position.

Values drawn on a CUDA device differ from values drawn on the CPU (different
generators); each test draws all of its inputs on one device.
"""
from __future__ import annotations

import math
import zlib
from typing import Dict, List, Optional

import torch

from .configs import DFlashConfig, Workload

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + zlib.crc32(name.encode())) & 0x7FFF_FFFF_FFFF)
    return g


def normal(shape, std: float, seed: int, name: str, dtype, device="cpu", mean: float = 0.0):
    g = _gen(seed, name, device)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    if mean:
        t.add_(mean)
    return t.to(dtype)


def randint(lo: int, hi: int, shape, seed: int, name: str, device="cpu"):
    """Uniform integers in [lo, hi] (inclusive)."""
    g = _gen(seed, name, device)
    return torch.randint(lo, hi + 1, shape, generator=g, device=device, dtype=torch.int64)


def weights(cfg: DFlashConfig, seed: int = 0, device="cpu", std: float = 0.02,
            layers: Optional[List[int]] = None, skip=()) -> Dict:
    """Random-init draft weights plus the target's embedding and lm_head.

    All matrices are [out, in] row-major.  W_qkv stacks the q, k and v rows of
    one layer: [(nq + 2 nkv) * D, H].
    """
    dt = _DT[cfg.act_dtype]
    H, D, F = cfg.hidden, cfg.head_dim, cfg.feat_dim
    nq, nkv, I, V = cfg.n_q_heads, cfg.n_kv_heads, cfg.inter, cfg.vocab
    W = {}

    def mat(name, shape):
        if name in skip:
            return None
        return normal(shape, std, seed, name, dt, device)

    def gain(name, n):
        return normal((n,), std, seed, name, dt, device, mean=1.0)

    W["embed"] = mat("embed", (V, H))
    W["lm_head"] = mat("lm_head", (V, H))
    W["fc"] = mat("fc", (H, F))
    W["hidden_norm"] = gain("hidden_norm", H)
    W["final_norm"] = gain("final_norm", H)
    W["layers"] = []
    for l in range(cfg.n_layers):
        if layers is not None and l not in layers:
            W["layers"].append(None)
            continue
        W["layers"].append({
            "in_norm": gain(f"l{l}.in_norm", H),
            "w_qkv": mat(f"l{l}.w_qkv", ((nq + 2 * nkv) * D, H)),
            "q_norm": gain(f"l{l}.q_norm", D),
            "k_norm": gain(f"l{l}.k_norm", D),
            "w_o": mat(f"l{l}.w_o", (H, nq * D)),
            "post_norm": gain(f"l{l}.post_norm", H),
            "w_gate": mat(f"l{l}.w_gate", (I, H)),
            "w_up": mat(f"l{l}.w_up", (I, H)),
            "w_down": mat(f"l{l}.w_down", (H, I)),
        })
    return W


def prefix_lengths(wl: Workload, device="cpu", seed: Optional[int] = None):
    lo, hi = wl.ctx
    s = wl.seed if seed is None else seed
    if lo == hi:
        return torch.full((wl.batch,), lo, dtype=torch.int64, device=device)
    return randint(lo, hi, (wl.batch,), s, "prefix_len", device)


def page_table(prefix_len: torch.Tensor, cfg: DFlashConfig, seed: int, extra_tokens: int,
               spare_pages: int = 3):
    """Per-request page tables over a shared pool of physical pages.

    Request r owns ceil((L_r + extra_tokens) / page) pages, drawn without
    replacement from a random permutation of the pool.  Returns
    (page_table [B, max_pages] int32, num_pages).  Unused entries hold page 0.
    """
    P = cfg.page_size
    L = prefix_len.cpu().tolist()
    need = [math.ceil((l + extra_tokens) / P) for l in L]
    total = sum(need) + spare_pages
    g = _gen(seed, "page_perm", "cpu")
    perm = torch.randperm(total, generator=g)
    maxp = max(need)
    pt = torch.zeros((len(L), maxp), dtype=torch.int32)
    o = 0
    for r, n in enumerate(need):
        pt[r, :n] = perm[o:o + n].to(torch.int32)
        o += n
    return pt, total


def slots_for(page_tab: torch.Tensor, positions: torch.Tensor, page_size: int):
    """Logical position -> physical cache slot through a page table (host helper)."""
    pt = page_tab.to(torch.int64).cpu()
    pos = positions.to(torch.int64).cpu()
    rows = torch.arange(pt.shape[0]).view(-1, *([1] * (pos.dim() - 1))).expand_as(pos)
    return pt[rows, pos // page_size] * page_size + pos % page_size


def features(rows: int, cfg: DFlashConfig, seed: int, name: str = "feats", device="cpu"):
    return normal((rows, cfg.feat_dim), 0.02, seed, name, _DT[cfg.act_dtype], device)


def kv_pool_random(cfg: DFlashConfig, num_pages: int, seed: int, device="cpu"):
    """Random cache contents in the cache layout: K pages [pages, nkv, page, D],
    V pages transposed [pages, nkv, D, page].

    f32/bf16 pools hold N(0, 1) values rounded to the pool dtype.  fp8 pools
    hold raw e4m3 byte codes drawn field by field: a random sign, an exponent
    field uniform in 3..8 and a random 3-bit mantissa, i.e. magnitudes
    between 1/16 and 3.75 (no zero, subnormal or NaN codes)."""
    kshp = (num_pages, cfg.n_kv_heads, cfg.page_size, cfg.head_dim)
    vshp = (num_pages, cfg.n_kv_heads, cfg.head_dim, cfg.page_size)
    K, Vv = [], []
    for l in range(cfg.n_layers):
        if cfg.kv_dtype == "fp8_e4m3":
            pools = []
            for kv, shp in (("k", kshp), ("v", vshp)):
                sign = randint(0, 1, shp, seed, f"kv.{kv}{l}.sign", device)
                expo = randint(3, 8, shp, seed, f"kv.{kv}{l}.exp", device)
                mant = randint(0, 7, shp, seed, f"kv.{kv}{l}.mant", device)
                pools.append((sign * 128 + expo * 8 + mant).to(torch.uint8))
            K.append(pools[0])
            Vv.append(pools[1])
        else:
            dt = _DT[cfg.kv_dtype]
            K.append(normal(kshp, 1.0, seed, f"kv.k{l}", dt, device))
            Vv.append(normal(vshp, 1.0, seed, f"kv.v{l}", dt, device))
    return K, Vv


def plant_posterior(cand: torch.Tensor, commit: torch.Tensor, vocab: int, seed: int):
    """Target posterior ids [B, S] whose greedy commit length against `cand`
    is exactly `commit` (1..S): post[j] = cand[j+1] for j < commit-1 and
    post[commit-1] != cand[commit] when commit < S; the rest is random."""
    cand = cand.to(torch.int64).cpu()
    B, S = cand.shape
    post = randint(0, vocab - 1, (B, S), seed, "posterior", "cpu")
    for r in range(B):
        c = int(commit[r])
        assert 1 <= c <= S
        post[r, :c - 1] = cand[r, 1:c]
        if c < S and post[r, c - 1] == cand[r, c]:
            post[r, c - 1] = (cand[r, c] + 1) % vocab
    return post.to(torch.int32)


def verify_inputs(B: int, S: int, V: int, seed: int, dtype=torch.bfloat16, device="cpu",
                  spread: float = 2.0, bump: float = 12.0, draft_noise: float = 0.5,
                  bump_lo: float = 0.0):
    """Synthetic inputs of a sampled verify step.

    candidates [B, S]: anchor and drafts uniform in [0, V); target logits
    [B, S, V]: N(0, spread^2), with the logit of the draft each row verifies
    (row j, token candidates[j + 1]) raised by U(bump_lo, bump) so that acceptance
    probabilities spread over (0, 1); draft logits [B, S-1, V]: the target's
    rows 0..S-2 plus N(0, draft_noise^2) (a drafter close to the target);
    uniforms [B, S] in [0, 1).  Logits are rounded once to `dtype`.
    """
    cand = randint(0, V - 1, (B, S), seed, "verify_cand", device).to(torch.int32)
    tl = normal((B, S, V), spread, seed, "verify_target", torch.float32, device)
    up = torch.rand(B, S - 1, generator=_gen(seed, "verify_bump", device), device=device)
    up = bump_lo + up * (bump - bump_lo)
    rows = torch.arange(S - 1, device=device)
    for r in range(B):
        tl[r, rows, cand[r, 1:].long()] += up[r]
    dl = tl[:, :S - 1] + normal((B, S - 1, V), draft_noise, seed, "verify_draft",
                                torch.float32, device)
    u = torch.rand(B, S, generator=_gen(seed, "verify_uniform", device), device=device)
    return cand, tl.to(dtype), dl.to(dtype), u
