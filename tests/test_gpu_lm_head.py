"""Parity of dflash_lm_head_argmax (the selection step alone) with the oracle's
select_draft_tokens, through the C ABI, at row counts that take each GEMM path
of the lm_head: the narrow streaming kernel (1..64 rows, one and two row
blocks), the 128-row tiles (65..192 rows), the tall tiles (65..128 rows over a
wide vocabulary) and the 256 x 256 tiles beyond, each with a ragged last tile;
fp32 and bf16; and the full Qwen3-8B-shaped lm_head on sampled rows.

Tolerances are those of the draft pass (the same kernels): logits max|gpu -
oracle| / max|oracle| per row <= 2e-2 (bf16) or 1e-4 (fp32); ids equal the
oracle's wherever its top-2 margin exceeds 5e-2 (1e-3) of that scale; every id
is the first-index argmax of the GPU's own logits; a call without logits
returns the same ids.  Some rows are planted: the hidden row is a multiple of
lm_head row t, so t wins by a wide margin and the id must be t."""
import numpy as np
import pytest
import torch

import oracle
from workloads import synth
from workloads.configs import get_workload
from tests.gpu_harness import logits_row_rel_err, argmax_checked_rows, dfl

pytestmark = pytest.mark.gpu

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _print(*a):
    print(*a, flush=True)


def tol(cfg):
    return (1e-4, 1e-3) if cfg.act_dtype == "f32" else (2e-2, 5e-2)


def _inputs(cfg, rows, seed, lm_std=0.02, device="cuda"):
    """lm_head [V, H] and hidden [rows, H] in act_dtype; every third row
    planted on a token (returned as {row: token})."""
    dt = _DT[cfg.act_dtype]
    lm = synth.normal((cfg.vocab, cfg.hidden), lm_std, seed, "lm_head_only", dt, device)
    hid = synth.normal((rows, cfg.hidden), 1.0, seed, "lm_hidden", dt, device)
    tok = synth.randint(0, cfg.vocab - 1, (rows,), seed, "lm_planted", "cpu")
    planted = {}
    for r in range(0, rows, 3):
        t = int(tok[r])
        row = lm[t].float()
        hid[r] = (row * (cfg.hidden ** 0.5 / row.norm())).to(dt)
        planted[r] = t
    return lm, hid, planted


def _run(cfg, lm_packed, hid, want_logits=True):
    m = dfl()
    rows = hid.shape[0]
    ws = m.workspace(m.lm_head_workspace_bytes(cfg, rows))
    ids = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    logits = (torch.empty((rows, cfg.vocab), dtype=hid.dtype, device="cuda")
              if want_logits else None)
    m.dflash_lm_head_argmax(cfg, lm_packed, hid, ids, ws, logits=logits)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), (None if logits is None else logits.float().cpu().numpy())


def _check(cfg, ids, gl, ids_only, o_logits, o_ids, planted, rows_idx):
    rel_tol, m_tol = tol(cfg)
    rel = logits_row_rel_err(gl[rows_idx], o_logits)
    _print(f"  logits max rel err {rel.max():.3e}")
    assert rel.max() <= rel_tol
    sure = argmax_checked_rows(o_logits, m_tol)
    assert np.array_equal(ids[rows_idx][sure], o_ids[sure])
    assert np.array_equal(ids, np.argmax(gl, axis=-1))
    assert np.array_equal(ids_only, ids)
    for r, t in planted.items():
        assert int(ids[r]) == t, (r, t, int(ids[r]))


CASES = [("tiny_f32", 3), ("tiny_f32", 100),
         ("small_bf16", 1), ("small_bf16", 15), ("small_bf16", 17), ("small_bf16", 33),
         ("small_bf16", 64), ("small_bf16", 65), ("small_bf16", 100), ("small_bf16", 192),
         ("small_bf16", 193), ("small_bf16", 480),
         ("small_bf16_vocab_tall", 1), ("small_bf16_vocab_tall", 65),
         ("small_bf16_vocab_tall", 120), ("small_bf16_vocab_tall", 129),
         ("small_bf16_vocab_tall", 300)]


@pytest.mark.parametrize("name,rows", CASES)
def test_lm_head_argmax_parity(name, rows):
    m = dfl()
    cfg = get_workload(name).cfg
    _print(f"[lm_head parity] {name} rows {rows} V {cfg.vocab} H {cfg.hidden}")
    lm, hid, planted = _inputs(cfg, rows, seed=rows)
    packed = m.dflash_pack_matrix(lm)
    ids, gl = _run(cfg, packed, hid)
    ids_only, _ = _run(cfg, packed, hid, want_logits=False)
    o_logits, o_ids = oracle.select_draft_tokens(hid.double().cpu().numpy(),
                                                 lm.double().cpu().numpy())
    _check(cfg, ids, gl, ids_only, o_logits, o_ids, planted, np.arange(rows))


@pytest.mark.parametrize("rows", [15, 120, 480])
def test_lm_head_argmax_qwen3_8b_sampled_rows(rows):
    """The Qwen3-8B-shaped lm_head (151936 x 4096): a batch-1 block (15 rows),
    eight blocks (120 rows) and 32 blocks (480 rows), the launch shapes of the
    draft pass; the oracle on eight sampled rows (first, last, planted and
    random), the id rules on every row."""
    m = dfl()
    cfg = get_workload("qwen3_8b_b16").cfg
    _print(f"[lm_head full size] rows {rows} V {cfg.vocab} H {cfg.hidden}")
    lm, hid, planted = _inputs(cfg, rows, seed=1000 + rows)
    packed = m.dflash_pack_matrix(lm)
    ids, gl = _run(cfg, packed, hid)
    ids_only, _ = _run(cfg, packed, hid, want_logits=False)
    g = np.random.default_rng(rows)
    sample = np.unique(np.concatenate([[0, 1, rows - 1], g.integers(0, rows, 5)]))
    # the oracle takes the weights in fp32 (exact for bf16) and widens them
    # to fp64 one block of rows at a time
    o_logits, o_ids = oracle.select_draft_tokens(hid[sample].double().cpu().numpy(),
                                                 lm.cpu().float().numpy())
    _check(cfg, ids, gl, ids_only, o_logits, o_ids, planted, sample)


@pytest.mark.parametrize("hidden", [4096, 4128])
def test_lm_head_argmax_lds_image_boundary(hidden):
    """At up to 16 rows the narrow lm_head reads A from an LDS image when the
    hidden size is at most 4096 and from global memory above it: 7 rows at
    hidden 4096 (the largest image) and 4128 (the first size past it)."""
    import dataclasses
    m = dfl()
    cfg = dataclasses.replace(get_workload("small_bf16").cfg, hidden=hidden)
    rows = 7
    _print(f"[lm_head image boundary] hidden {hidden} rows {rows} V {cfg.vocab}")
    lm, hid, planted = _inputs(cfg, rows, seed=hidden)
    packed = m.dflash_pack_matrix(lm)
    ids, gl = _run(cfg, packed, hid)
    ids_only, _ = _run(cfg, packed, hid, want_logits=False)
    o_logits, o_ids = oracle.select_draft_tokens(hid.double().cpu().numpy(),
                                                 lm.double().cpu().numpy())
    _check(cfg, ids, gl, ids_only, o_logits, o_ids, planted, np.arange(rows))
