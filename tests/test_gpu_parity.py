"""Parity of the HIP path (through the C ABI) with the CPU oracle on seeded
inputs, at sizes the oracle finishes in seconds: several tiles in every
dimension, ragged vocabularies / prefixes / pages, sliding windows, fp8 and
fp32 caches.  Integers bit-exact; floating point within the tolerances below.

Tolerances (floating point):
* bf16 models: logits max|gpu - oracle| / max|oracle| per row <= 2e-2, and the
  draft id must equal the oracle's argmax wherever the oracle's top-2 margin
  exceeds 5e-2 on the same scale (5e-2 x max|oracle| of the row: within the
  2e-2 bound two logits can swap only if they are closer than 4e-2 of it);
  injected K/V per (slot, head) max|gpu - oracle| / max|oracle| <= 2e-2.
* fp32 models: 1e-4 relative, argmax agreement where the margin exceeds 1e-3
  of the row's max |oracle logit|.
* every row: the draft id is the argmax (first index among equal maxima) of
  the GPU's own stored logits, bit-exactly -- the integer decision taken in
  the kernel's precision.
* fp8 caches: every stored value within one E4M3 step (at that magnitude)
  plus the bf16-class allowance 2e-2 * max|oracle| of its head, and at least
  90% of codes identical: the two sides round slightly different values (the
  GPU's fp32 result of bf16 operands, the oracle's exact fp64 one) to a 3-bit
  mantissa, so a value near a rounding boundary may land one code away, and
  near zero, where codes are only 2^-9 apart, a few codes away.
* a cycle in which each side injects its own fp8 cache: logits 5e-2 (the
  draft pass then reads caches that differ by those single-code roundings;
  with identical caches the bf16 bound above holds).
"""
import dataclasses
import numpy as np
import pytest
import torch

import oracle
from workloads import synth
from workloads.configs import get_workload
from tests.gpu_harness import Setup, logits_row_rel_err, argmax_checked_rows, e4m3_spacing, dfl

pytestmark = pytest.mark.gpu

SMALL = ["tiny_f32", "small_bf16", "small_swa_fp8", "small_f32_d64", "small_bf16_wide",
         "small_bf16_vocab", "small_bf16_tall", "small_bf16_vocab_tall"]


def tol(cfg):
    return (1e-4, 1e-3) if cfg.act_dtype == "f32" else (2e-2, 5e-2)


def _print(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------- accept
@pytest.mark.parametrize("S", [2, 4, 8, 16])
def test_accept_bitexact(S):
    m = dfl()
    B = 2000
    g = torch.Generator().manual_seed(S)
    cand = torch.randint(0, 5, (B, S), generator=g, dtype=torch.int32)
    commit = torch.randint(1, S + 1, (B,), generator=g)
    post = synth.plant_posterior(cand, commit, 5, seed=S)
    post[: B // 4] = torch.randint(0, 5, (B // 4, S), generator=g, dtype=torch.int32)
    L = torch.randint(0, 100000, (B,), generator=g, dtype=torch.int32)
    outs = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(4)]
    out_tok = torch.full((B, S), -7, dtype=torch.int32, device="cuda")
    m.dflash_accept(cand.cuda(), post.cuda(), L.cuda(), outs[0], outs[1], out_tok, outs[2], outs[3])
    torch.cuda.synchronize()
    o = oracle.accept(cand.numpy(), post.numpy(), L.numpy())
    assert np.array_equal(outs[0].cpu().numpy(), o["accept_len"])
    assert np.array_equal(outs[1].cpu().numpy(), o["commit_len"])
    assert np.array_equal(out_tok.cpu().numpy(), o["out_tokens"])
    assert np.array_equal(outs[2].cpu().numpy(), o["next_anchor"])
    assert np.array_equal(outs[3].cpu().numpy(), o["new_seq_len"])
    assert np.array_equal(o["commit_len"][B // 4:], commit[B // 4:].numpy())


def _accept_logits_case(B, S, V, dtype, seed, ties=False, nan_rows=0, offset=0):
    """Seeded target logits (torch generator on the host), candidates planted
    from the oracle's posterior so every commit length 1..S occurs, and the
    GPU's five outputs compared with oracle.accept_logits element by element."""
    m = dfl()
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((B, S, V), generator=g) * 3.0
    if ties:                                   # few distinct values: ties across chunks
        x = torch.round(x)
    if nan_rows:
        x.view(B * S, V)[:nan_rows, ::3] = float("nan")
        x.view(B * S, V)[nan_rows:2 * nan_rows] = float("nan")   # rows of NaN only
    x = x.to(dtype)
    post = oracle.greedy_posterior(x.float().numpy())
    commit = torch.randint(1, S + 1, (B,), generator=g).numpy()
    cand = torch.randint(0, V, (B, S), generator=g, dtype=torch.int32).numpy()
    for r in range(B):
        c = commit[r]
        cand[r, 1:c] = post[r, :c - 1]
        if c < S and cand[r, c] == post[r, c - 1]:
            cand[r, c] = (post[r, c - 1] + 1) % V
    L = torch.randint(0, 100000, (B,), generator=g, dtype=torch.int32)
    # an offset view makes the rows start off a 16-byte boundary
    buf = torch.empty(B * S * V + offset, dtype=dtype, device="cuda")
    xd = buf[offset:].view(B, S, V)
    xd.copy_(x.cuda())
    outs = [torch.full((B,), -7, dtype=torch.int32, device="cuda") for _ in range(4)]
    out_tok = torch.full((B, S), -7, dtype=torch.int32, device="cuda")
    ws = m.workspace(m.accept_logits_workspace_bytes(B, S, V))
    m.dflash_accept_logits(torch.from_numpy(cand).cuda(), xd, L.cuda(), outs[0], outs[1], out_tok,
                           outs[2], outs[3], ws)
    torch.cuda.synchronize()
    o = oracle.accept_logits(cand, x.float().numpy(), L.numpy())
    assert np.array_equal(outs[0].cpu().numpy(), o["accept_len"])
    assert np.array_equal(outs[1].cpu().numpy(), o["commit_len"])
    assert np.array_equal(out_tok.cpu().numpy(), o["out_tokens"])
    assert np.array_equal(outs[2].cpu().numpy(), o["next_anchor"])
    assert np.array_equal(outs[3].cpu().numpy(), o["new_seq_len"])
    assert np.array_equal(o["commit_len"], commit)
    return o


@pytest.mark.parametrize("B,S,V,dtype", [(7, 4, 1000, torch.float32), (3, 16, 4096, torch.bfloat16),
                                         (5, 2, 1003, torch.bfloat16), (2, 64, 20000, torch.float32),
                                         (4, 8, 40001, torch.bfloat16)])
def test_accept_logits_bitexact(B, S, V, dtype):
    _accept_logits_case(B, S, V, dtype, seed=B * 1000 + S)


def test_accept_logits_ties_nan_and_misaligned_rows():
    # rounded logits tie within and across 16384-column chunks; NaN never wins
    _accept_logits_case(6, 8, 50000, torch.bfloat16, seed=5, ties=True, nan_rows=4)
    # rows that start off a 16-byte boundary take the element-wise loads
    _accept_logits_case(5, 4, 8192, torch.bfloat16, seed=6, offset=3)
    _accept_logits_case(5, 4, 8192, torch.float32, seed=7, offset=1, ties=True)


def test_accept_logits_full_size():
    """The batch-32, block-16, vocabulary-151936 shape in bf16."""
    _accept_logits_case(32, 16, 151936, torch.bfloat16, seed=11)


# ---------------------------------------------------------------- weight packing
def _packed_reference(w):
    """The packed layout written out from its definition: record l of chunk c
    of slab s holds w[16 s + l % 16, 32 c + 8 (l // 16) + e], e = 0..7, zero
    past the last row."""
    rows, cols = w.shape
    n_slab = (rows + 15) // 16
    wp = np.zeros((n_slab * 16, cols), w.dtype)
    wp[:rows] = w
    out = np.zeros((n_slab, cols // 32, 64, 8), w.dtype)
    for lane in range(64):
        for e in range(8):
            out[:, :, lane, e] = wp[lane % 16::16][:, 8 * (lane // 16) + e::32]
    return out.reshape(-1)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(37, 96), (16, 32), (160, 512)])
def test_pack_matrix_layout(dtype, shape):
    m = dfl()
    g = torch.Generator().manual_seed(shape[0] * 1000 + shape[1])
    w = torch.randn(shape, generator=g).to(dtype)
    got = m.dflash_pack_matrix(w.cuda())
    torch.cuda.synchronize()
    want = _packed_reference(w.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy())
    gi = got.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy()
    assert np.array_equal(gi, want)


# ---------------------------------------------------------------- draft pass
# (name, batch): besides each workload's own batch, block-row counts that are
# not multiples of 16 (3 x 8 = 24, 5 x 8 = 40, 3 x 5 = 15 rows), where the
# activations of a pass of at most 64 rows fill their last 16-row block partly
DRAFT_CASES = [(n, None) for n in SMALL] + [("small_swa_fp8", 3), ("small_swa_fp8", 5),
                                            ("small_f32_d64", 3)]


@pytest.mark.parametrize("name,batch", DRAFT_CASES)
def test_draft_block_parity(name, batch):
    wl = get_workload(name)
    if batch is not None:
        wl = dataclasses.replace(wl, batch=batch)
    cfg = wl.cfg
    _print(f"[draft parity] {name} B={wl.batch} S={cfg.block_size}")
    st = Setup(wl)
    out = st.draft()
    o = oracle.draft_block(cfg, st.np_W(), st.oracle_cache(), st.anchor.numpy(), st.L.numpy(),
                           st.pt.numpy())
    assert np.array_equal(out["positions"].cpu().numpy(), o["positions"])
    assert np.array_equal(out["slots"].cpu().numpy(), o["slots"])
    assert np.array_equal(out["block_ids"].cpu().numpy(), o["block_ids"])
    cand = out["candidates"].cpu().numpy()
    assert np.array_equal(cand[:, 0], st.anchor.numpy())
    rel_tol, m_tol = tol(cfg)
    gl = out["logits"].float().cpu().numpy()
    rel = logits_row_rel_err(gl, o["logits"])
    _print(f"  logits max rel err {rel.max():.3e}")
    assert rel.max() <= rel_tol
    sure = argmax_checked_rows(o["logits"], m_tol)
    # coverage of the id check (the wider the vocabulary, the more rows have
    # a close runner-up): at least a quarter of the rows
    assert sure.mean() >= 0.25
    assert np.array_equal(cand[:, 1:][sure], o["draft_ids"][sure])
    # the GPU's ids are the argmax of its own logits (first index on ties)
    assert np.array_equal(cand[:, 1:], np.argmax(gl, axis=-1))


EDGE_LENGTHS = [
    ("small_bf16", [0, 0]),                                          # no context at all
    ("small_bf16", [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 150]),  # byte partition
    ("small_swa_fp8", [0, 1, 23, 24, 25, 39, 40, 41]),               # window edges, aligned
    ("small_swa_fp8", [0, 2, 5, 8, 13, 21, 24, 31, 32, 33, 40, 41, 47, 48, 64, 65, 80, 95,
                       96, 97]),                                     # E4M3, byte partition
    ("tiny_f32", [0, 3, 4, 5]),
    ("small_f32_d64", [0, 1, 31, 32, 33]),
]


@pytest.mark.parametrize("name,lengths", EDGE_LENGTHS)
def test_draft_block_edge_lengths(name, lengths):
    """Context lengths at the edges: none, one key, one short of / at / past a
    page and a 32-key step, at the sliding windows' edges; every attention
    path (aligned and byte partitions, bf16 / E4M3 / fp32 caches, head_dim 64
    and 128)."""
    wl = dataclasses.replace(get_workload(name), batch=len(lengths))
    cfg = wl.cfg
    _print(f"[draft edge lengths] {name} L={lengths}")
    st = Setup(wl, random_cache=False)
    st.L = torch.tensor(lengths, dtype=torch.int32)
    st.pt, st.num_pages = synth.page_table(st.L, cfg, st.seed, 2 * cfg.block_size)
    K, V = synth.kv_pool_random(cfg, st.num_pages, st.seed, st.device)
    st.cache = dfl().KVCache(K, V, st.num_pages)
    out = st.draft()
    o = oracle.draft_block(cfg, st.np_W(), st.oracle_cache(), st.anchor.numpy(), st.L.numpy(),
                           st.pt.numpy())
    assert np.array_equal(out["positions"].cpu().numpy(), o["positions"])
    assert np.array_equal(out["slots"].cpu().numpy(), o["slots"])
    rel_tol, m_tol = tol(cfg)
    gl = out["logits"].float().cpu().numpy()
    rel = logits_row_rel_err(gl, o["logits"])
    _print(f"  logits max rel err {rel.max():.3e}")
    assert rel.max() <= rel_tol
    cand = out["candidates"].cpu().numpy()
    sure = argmax_checked_rows(o["logits"], m_tol)
    assert np.array_equal(cand[:, 1:][sure], o["draft_ids"][sure])
    assert np.array_equal(cand[:, 1:], np.argmax(gl, axis=-1))


@pytest.mark.parametrize("name", ["small_bf16", "tiny_f32"])
def test_draft_block_deterministic(name):
    st = Setup(get_workload(name))
    a = st.draft()
    b = st.draft()
    assert torch.equal(a["logits"], b["logits"])
    assert torch.equal(a["candidates"], b["candidates"])


# ---------------------------------------------------------------- injection
def _inject_case(st, T, seed, grid=None):
    cfg = st.cfg
    feats = synth.features(T, cfg, seed, "inj_feats", "cpu")
    g = torch.Generator().manual_seed(seed)
    pos = torch.randint(0, 200000, (T,), generator=g, dtype=torch.int32)
    slots = torch.randperm(st.num_pages * cfg.page_size, generator=g)[:T].to(torch.int32)
    valid = None
    if grid is not None:
        n_req, rpr = grid
        valid = torch.randint(0, rpr + 1, (n_req,), generator=g, dtype=torch.int32)
        valid[0], valid[-1] = 0, rpr
    return feats, pos, slots, valid


def _compare_pools(st, before, o_cache, written):
    cfg = st.cfg
    rel_tol, _ = tol(cfg)
    for l in range(cfg.n_layers):
        for kind, pool, opool, bpool in (("k", st.cache.k[l], o_cache.k[l], before.k[l]),
                                         ("v", st.cache.v[l], o_cache.v[l], before.v[l])):
            got = st._pool_values(pool, transposed=(kind == "v"))
            untouched = np.ones(got.shape[0], bool)
            untouched[written] = False
            assert np.array_equal(np.nan_to_num(got[untouched], nan=1e9),
                                  np.nan_to_num(bpool[untouched], nan=1e9)), (l, kind)
            g, o = got[written], opool[written]
            if cfg.kv_dtype == "fp8_e4m3":
                d = np.abs(g - o)
                allow = e4m3_spacing(np.maximum(np.abs(g), np.abs(o))) + \
                    rel_tol * np.max(np.abs(o), axis=-1, keepdims=True)
                assert (d <= allow).all(), (l, kind, float((d - allow).max()))
                frac = (g == o).mean()
                _print(f"  layer {l} {kind}: fp8 identical codes {frac:.4f}")
                assert frac >= 0.9
            else:
                err = np.max(np.abs(g - o), axis=-1) / np.max(np.abs(o), axis=-1)
                _print(f"  layer {l} {kind}: max rel err {err.max():.3e}")
                assert err.max() <= rel_tol, (l, kind)


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("grid", [None, (3, 16), (4, 16), 23, (3, 7), 65, (5, 16), (19, 16), 300])
def test_project_context_parity(name, grid):
    """Rows 77 and 5 x 16 (one 128-row tile), 19 x 16 and 300 (256-row tiles,
    ragged last tile), with and without a prefix-valid request grid; 3 x 16
    and 4 x 16 (48 and 64 rows: the narrow K/V store and its norm/RoPE/write
    kernel, the second at its largest size), 23 and 3 x 7 rows (the fc output
    in 16 x 32 blocks with a partly filled last block) and 65 rows (the first
    size the tiled GEMMs take, with the row scales computed ahead of them)."""
    wl = get_workload(name)
    cfg = wl.cfg
    _print(f"[inject parity] {name} grid={grid}")
    if isinstance(grid, int):
        T, grid = grid, None
    else:
        T = 77 if grid is None else grid[0] * grid[1]
    st = Setup(wl, extra_tokens=max(2 * cfg.block_size, T))  # a pool of >= T slots
    feats, pos, slots, valid = _inject_case(st, T, 100 + wl.seed, grid)
    before = st.oracle_cache()
    o_cache = before.copy()
    n_req, rpr = (1, T) if grid is None else grid
    st.inject(feats, pos, slots, valid, n_req, rpr)
    live = oracle.project_context(cfg, st.np_W(), o_cache, feats.float().numpy(), pos.numpy(),
                                  slots.numpy(), None if valid is None else valid.numpy(), rpr)
    _compare_pools(st, before, o_cache, slots.numpy()[live])


@pytest.mark.parametrize("name", ["small_bf16", "small_swa_fp8", "tiny_f32"])
@pytest.mark.parametrize("T", [48, 77, 300])
def test_project_context_slots_outside_the_pool(name, T):
    """Rows whose slot lies outside the pool (negative, or at or past
    num_pages * page_size) are skipped by every K/V path (the narrow store's
    write kernel at 48 rows, the tiled epilogues at 77 and 300 rows): the
    other rows match the oracle and no other slot changes."""
    wl = get_workload(name)
    cfg = wl.cfg
    _print(f"[inject outside pool] {name} T={T}")
    st = Setup(wl, extra_tokens=max(2 * cfg.block_size, T))
    feats, pos, slots, _ = _inject_case(st, T, 900 + T)
    n_slots = st.num_pages * cfg.page_size
    g = torch.Generator().manual_seed(T)
    bad = torch.randperm(T, generator=g)[: max(T // 8, 3)]
    for i, b in enumerate(bad.tolist()):
        slots[b] = -1 - i if i % 2 == 0 else n_slots + i
    before = st.oracle_cache()
    o_cache = before.copy()
    st.inject(feats, pos, slots)
    keep = (slots >= 0) & (slots < n_slots)
    oracle.project_context(cfg, st.np_W(), o_cache, feats[keep].float().numpy(),
                           pos[keep].numpy(), slots[keep].numpy())
    _compare_pools(st, before, o_cache, slots[keep].numpy())


def test_empty_calls_change_nothing():
    """Zero rows to inject (no requests, or requests of no rows) and a draft
    pass over an empty batch return OK and leave the cache bit-identical;
    the checked-mode calls on them report nothing."""
    m = dfl()
    wl = get_workload("small_bf16")
    cfg = wl.cfg
    st = Setup(wl)
    before = [t.clone() for t in st.cache.k + st.cache.v]
    d = st.device
    ws = m.workspace(m.context_workspace_bytes(cfg, 1), d)
    e_feats = torch.empty((0, cfg.feat_dim), dtype=torch.bfloat16, device=d)
    e_i = torch.empty(0, dtype=torch.int32, device=d)
    for n_req, rpr in ((0, 16), (3, 0)):
        m.dflash_project_context(cfg, st.c_weights(), st.cache, e_feats, e_i, e_i,
                                 torch.zeros(max(n_req, 1), dtype=torch.int32, device=d), n_req,
                                 rpr, ws, checked=True)
    e2 = torch.empty((0, cfg.block_size), dtype=torch.int32, device=d)
    m.dflash_draft_block(cfg, st.c_weights(), st.cache, e_i, e_i,
                         torch.zeros((0, 4), dtype=torch.int32, device=d), 0, e2, e2.clone(),
                         e2.clone(), m.workspace(m.draft_workspace_bytes(cfg, 0, 0), d),
                         checked=True)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(before, st.cache.k + st.cache.v))


def test_project_context_large_tiles():
    """8192 rows of the hidden-2048 model: the fc GEMM takes the 256 x 256-tile
    path.  The oracle recomputes a sample of rows (injection is row-local)."""
    wl = get_workload("small_bf16_wide")
    cfg = wl.cfg
    T = 8192
    st = Setup(wl, extra_tokens=T)
    feats, pos, slots, _ = _inject_case(st, T, 321)
    st.inject(feats, pos, slots)
    rows = np.arange(0, T, 37)
    o_cache = oracle.OracleCache(cfg, st.num_pages * cfg.page_size)
    oracle.project_context(cfg, st.np_W(), o_cache, feats[rows].float().numpy(),
                           pos.numpy()[rows], slots.numpy()[rows])
    sl = slots.numpy()[rows]
    for l in range(cfg.n_layers):
        for kind, pool, opool in (("k", st.cache.k[l], o_cache.k[l]),
                                  ("v", st.cache.v[l], o_cache.v[l])):
            g = st._pool_values(pool, transposed=(kind == "v"))[sl]
            o = opool[sl]
            err = np.max(np.abs(g - o), axis=-1) / np.max(np.abs(o), axis=-1)
            _print(f"  layer {l} {kind}: {len(rows)} sampled rows, max rel err {err.max():.3e}")
            assert err.max() <= 2e-2


def test_project_context_prefix_valid_longer_than_a_chunk():
    """A prefix-valid grid whose requests are longer than the 8192-row
    injection chunk (3 x 9000 rows, valid 8193 / 0 / 9000), with the workspace
    the query returns for all rows: chunks start and end inside requests.
    Rows past a request's valid prefix keep their old cache values; sampled
    live rows (around every chunk boundary too) match the oracle."""
    wl = get_workload("small_bf16")
    cfg = wl.cfg
    n_req, rpr = 3, 9000
    T = n_req * rpr
    _print(f"[inject prefix-valid long] {n_req} x {rpr}")
    st = Setup(wl, extra_tokens=T)
    feats, pos, slots, _ = _inject_case(st, T, 555)
    valid = torch.tensor([8193, 0, 9000], dtype=torch.int32)
    before = st.oracle_cache()
    st.inject(feats, pos, slots, valid, n_req, rpr)
    live = (np.arange(T) % rpr) < np.repeat(valid.numpy(), rpr)
    dead = slots.numpy()[~live]
    rows = np.arange(0, T, 53)
    edges = np.array([8190, 8191, 8192, 8193, 9000 + 8191, 18000 + 8191, 18000 + 8192, T - 1])
    rows = np.unique(np.concatenate([rows, edges]))
    rows = rows[live[rows]]
    o_cache = oracle.OracleCache(cfg, st.num_pages * cfg.page_size)
    oracle.project_context(cfg, st.np_W(), o_cache, feats[rows].float().numpy(),
                           pos.numpy()[rows], slots.numpy()[rows])
    sl = slots.numpy()[rows]
    for l in range(cfg.n_layers):
        for kind, pool, opool, bpool in (("k", st.cache.k[l], o_cache.k[l], before.k[l]),
                                         ("v", st.cache.v[l], o_cache.v[l], before.v[l])):
            got = st._pool_values(pool, transposed=(kind == "v"))
            assert np.array_equal(got[dead], bpool[dead]), (l, kind)
            g, o = got[sl], opool[sl]
            err = np.max(np.abs(g - o), axis=-1) / np.max(np.abs(o), axis=-1)
            _print(f"  layer {l} {kind}: {len(rows)} sampled rows, max rel err {err.max():.3e}")
            assert err.max() <= 2e-2


@pytest.mark.parametrize("name", ["small_bf16", "small_swa_fp8", "tiny_f32"])
def test_project_context_chunked_equals_once_and_idempotent(name):
    """Injecting rows in several calls of at most 64 rows gives the same bits
    as one such call (in the weight-streaming GEMM the K split of a row does
    not depend on how many rows share the call), and re-injecting the same
    rows leaves the cache bit-identical."""
    wl = get_workload(name)
    st = Setup(wl)
    T = 60
    feats, pos, slots, _ = _inject_case(st, T, 7)
    st.inject(feats, pos, slots)
    once = [t.clone() for t in st.cache.k + st.cache.v]
    st.inject(feats, pos, slots)
    assert all(torch.equal(a, b) for a, b in zip(once, st.cache.k + st.cache.v))
    st2 = Setup(wl)
    for lo, hi in [(0, 9), (9, 40), (40, 60)]:
        st2.inject(feats[lo:hi], pos[lo:hi], slots[lo:hi])
    assert all(torch.equal(a, b) for a, b in zip(once, st2.cache.k + st2.cache.v))


# ---------------------------------------------------------------- one cycle
@pytest.mark.parametrize("name", ["small_bf16", "small_swa_fp8", "small_f32_d64"])
def test_cycle_inject_draft_accept(name):
    """Prefill injection -> draft -> accept -> injection of the committed
    verify rows -> second draft, GPU and oracle each on their own state."""
    wl = get_workload(name)
    cfg = wl.cfg
    _print(f"[cycle] {name}")
    st = Setup(wl, random_cache=False)
    m = dfl()
    st.cache = m.KVCache.allocate(cfg, st.num_pages, "cuda", fill=0)
    o_cache = oracle.OracleCache(cfg, st.num_pages * cfg.page_size)
    Wn = st.np_W()
    P = cfg.page_size
    for r in range(st.B):
        Lr = int(st.L[r])
        if Lr == 0:
            continue
        f = synth.features(Lr, cfg, 500 + r, "prefill", "cpu")
        pos = torch.arange(Lr, dtype=torch.int32)
        sl = (st.pt[r, pos.long() // P] * P + pos % P).to(torch.int32)
        st.inject(f, pos, sl)
        oracle.project_context(cfg, Wn, o_cache, f.float().numpy(), pos.numpy(), sl.numpy())
    rel_tol, m_tol = tol(cfg)
    if cfg.kv_dtype == "fp8_e4m3":
        rel_tol = 5e-2
    out = st.draft()
    o = oracle.draft_block(cfg, Wn, o_cache, st.anchor.numpy(), st.L.numpy(), st.pt.numpy())
    rel = logits_row_rel_err(out["logits"].float().cpu().numpy(), o["logits"])
    _print(f"  cycle-1 logits max rel err {rel.max():.3e}")
    assert rel.max() <= rel_tol
    # target posterior planted on the oracle's candidates (commit drawn per request)
    commit = synth.randint(1, cfg.block_size, (st.B,), wl.seed, "commit")
    post = synth.plant_posterior(torch.from_numpy(o["candidates"]), commit, cfg.vocab, wl.seed)
    B, S = st.B, cfg.block_size
    res = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(4)]
    out_tok = torch.empty((B, S), dtype=torch.int32, device="cuda")
    m.dflash_accept(out["candidates"], post.cuda(), st.L.cuda(), res[0], res[1], out_tok, res[2],
                    res[3])
    torch.cuda.synchronize()
    oa = oracle.accept(o["candidates"], post.numpy(), st.L.numpy())
    same = (out["candidates"].cpu().numpy() == o["candidates"]).all(axis=1)
    assert same.any()
    assert np.array_equal(res[1].cpu().numpy()[same], oa["commit_len"][same])
    assert np.array_equal(out_tok.cpu().numpy()[same], oa["out_tokens"][same])
    # inject the committed verify rows at the block's slots, then draft again
    vf = synth.features(B * S, cfg, 900, "verify", "cpu")
    commit_used = torch.from_numpy(oa["commit_len"]).to(torch.int32)
    st.inject(vf, out["positions"].reshape(-1).cpu(), out["slots"].reshape(-1).cpu(),
              commit_used, B, S)
    oracle.project_context(cfg, Wn, o_cache, vf.float().numpy(), o["positions"].reshape(-1),
                           o["slots"].reshape(-1), oa["commit_len"], S)
    st.L = torch.from_numpy(oa["new_seq_len"]).to(torch.int32)
    st.anchor = torch.from_numpy(oa["next_anchor"]).to(torch.int32)
    out2 = st.draft()
    o2 = oracle.draft_block(cfg, Wn, o_cache, st.anchor.numpy(), st.L.numpy(), st.pt.numpy())
    rel = logits_row_rel_err(out2["logits"].float().cpu().numpy(), o2["logits"])
    _print(f"  cycle-2 logits max rel err {rel.max():.3e}")
    assert rel.max() <= rel_tol
    sure = argmax_checked_rows(o2["logits"], m_tol)
    assert np.array_equal(out2["candidates"].cpu().numpy()[:, 1:][sure], o2["draft_ids"][sure])


# ---------------------------------------------------------------- draft window
@pytest.mark.parametrize("name,window", [("small_bf16", 48), ("small_swa_fp8", 30),
                                         ("small_f32_d64", 20)])
def test_draft_block_window_ring_parity(name, window):
    """Draft window N with the page table read as a ring of R pages per
    request (prefixes up to several rings long, so positions wrap): every
    layer reads only the last N context rows."""
    wl = get_workload(name)
    cfg = dataclasses.replace(wl.cfg, context_window=window)
    wl = dataclasses.replace(wl, cfg=cfg)
    S, P = cfg.block_size, cfg.page_size
    R = (window + S - 1 + P - 1) // P + 1
    _print(f"[draft window parity] {name} N={window} ring of {R} pages")
    st = Setup(wl)
    assert st.B * R <= st.num_pages and int(st.L.max()) > R * P
    perm = torch.randperm(st.num_pages, generator=torch.Generator().manual_seed(window))
    st.pt = perm[:st.B * R].view(st.B, R).to(torch.int32)
    out = st.draft()
    o = oracle.draft_block(cfg, st.np_W(), st.oracle_cache(), st.anchor.numpy(), st.L.numpy(),
                           st.pt.numpy())
    assert np.array_equal(out["positions"].cpu().numpy(), o["positions"])
    assert np.array_equal(out["slots"].cpu().numpy(), o["slots"])
    rel_tol, m_tol = tol(cfg)
    gl = out["logits"].float().cpu().numpy()
    rel = logits_row_rel_err(gl, o["logits"])
    _print(f"  logits max rel err {rel.max():.3e}")
    assert rel.max() <= rel_tol
    sure = argmax_checked_rows(o["logits"], m_tol)
    cand = out["candidates"].cpu().numpy()
    assert np.array_equal(cand[:, 1:][sure], o["draft_ids"][sure])


# ---------------------------------------------------------------- page sizes
@pytest.mark.parametrize("name,P,batch", [("small_bf16", 32, 3), ("small_bf16", 48, 12),
                                          ("small_swa_fp8", 32, 4), ("small_swa_fp8", 48, 20),
                                          ("small_swa_fp8", 64, 9)])
def test_draft_block_page_sizes(name, P, batch):
    """Pages of 32, 48 and 64 keys: a 32-key step's two 16-key halves may sit
    in one page or straddle two, and the page-list index advances per step.
    Up to 16 (request, kv head) segments take the aligned partition, 12 x 2
    and 20 x 1 segments the byte partition; the E4M3 cache (head_dim 128)
    runs its direct-to-LDS path on both."""
    wl = get_workload(name)
    cfg = dataclasses.replace(wl.cfg, page_size=P)
    wl = dataclasses.replace(wl, cfg=cfg, batch=batch)
    _print(f"[page size parity] {name} P={P} B={batch} segments={batch * cfg.n_kv_heads}")
    st = Setup(wl)
    out = st.draft()
    o = oracle.draft_block(cfg, st.np_W(), st.oracle_cache(), st.anchor.numpy(), st.L.numpy(),
                           st.pt.numpy())
    assert np.array_equal(out["slots"].cpu().numpy(), o["slots"])
    rel_tol, m_tol = tol(cfg)
    gl = out["logits"].float().cpu().numpy()
    rel = logits_row_rel_err(gl, o["logits"])
    _print(f"  logits max rel err {rel.max():.3e}")
    assert rel.max() <= rel_tol
    sure = argmax_checked_rows(o["logits"], m_tol)
    cand = out["candidates"].cpu().numpy()
    assert np.array_equal(cand[:, 1:][sure], o["draft_ids"][sure])
    assert np.array_equal(cand[:, 1:], np.argmax(gl, axis=-1))
