"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, the header compiles as plain C, and host-visible argument
errors come back as status codes before any HIP call."""
import ctypes
import dataclasses
import os
import re
import subprocess

import pytest

from workloads.configs import TINY, QWEN3_8B_DRAFT, KIMI_DRAFT

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "dflash.h")

dfl = pytest.importorskip("block_diffusion_drafter_rmsnorm_amd")


def declared_functions():
    txt = open(HDR).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_\w+)\s*\(", txt)))


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HDR],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"dflash_project_context", "dflash_draft_block", "dflash_accept"} <= set(names)
    lib = dfl.raw_lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", dfl.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (dflash_\w+)", out))
    assert set(names) <= exported


def test_struct_layout_matches_header():
    # 11 int32, 16 windows, 2 floats, 3 int32
    assert ctypes.sizeof(dfl.CConfig) == 4 * (11 + 16 + 2 + 3)
    assert ctypes.sizeof(dfl.CWeights) == 8 * (5 + 9 * dfl.MAX_LAYERS)
    assert ctypes.sizeof(dfl.CKVCache) == 8 * (2 * dfl.MAX_LAYERS + 1)


def test_workspace_sizes():
    assert dfl.context_workspace_bytes(TINY, 64) > 0
    assert dfl.draft_workspace_bytes(QWEN3_8B_DRAFT, 1, 4096) > 0
    assert dfl.draft_workspace_bytes(KIMI_DRAFT, 16, 32768) > 0
    bad = dataclasses.replace(TINY, head_dim=96)
    assert dfl.context_workspace_bytes(bad, 10) == 0
    assert dfl.draft_workspace_bytes(TINY, 0, 10) == 0


def _status(fn, *args):
    return fn(*args)


def test_config_errors():
    lib = dfl.raw_lib()
    fake = ctypes.c_void_p(0x100000)
    for field, val, want in [("head_dim", 96, -2), ("block_size", 17, -2), ("n_kv_heads", 3, -2),
                             ("hidden", 100, -2), ("mask_token_id", 5000, -1), ("n_layers", 0, -2)]:
        c = dfl.make_config(dataclasses.replace(TINY, **{field: val}))
        w = dfl.CWeights()
        kv = dfl.CKVCache()
        st = lib.dflash_draft_block(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), fake, fake,
                                    fake, 4, 1, 64, None, fake, fake, fake, None, fake, 1 << 20,
                                    None)
        assert st == want, (field, st, lib.dflash_last_error())


def test_null_and_workspace_errors():
    lib = dfl.raw_lib()
    cfg = dfl.make_config(TINY)
    fake = 0x100000
    w = dfl.CWeights()
    for n in ("embed", "lm_head", "fc", "hidden_norm", "final_norm"):
        setattr(w, n, fake)
    for n in dfl._LAYER_FIELDS:
        setattr(w.layer[0], n, fake)
    kv = dfl.CKVCache()
    kv.k[0] = kv.v[0] = fake
    kv.num_pages = 8
    F = ctypes.c_void_p(fake)
    # missing cache page count
    kv0 = dfl.CKVCache()
    assert lib.dflash_project_context(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv0), F,
                                      512, F, F, None, 1, 4, F, 1 << 30, None) == -1
    # misaligned feats
    assert lib.dflash_project_context(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv),
                                      ctypes.c_void_p(fake + 2), 512, F, F, None, 1, 4, F, 1 << 30,
                                      None) == -1
    # stride smaller than feat_dim
    assert lib.dflash_project_context(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), F,
                                      100, F, F, None, 1, 4, F, 1 << 30, None) == -1
    # workspace too small
    st = lib.dflash_project_context(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), F, 512,
                                    F, F, None, 1, 4, F, 16, None)
    assert st == -3 and b"workspace" in lib.dflash_last_error()
    st = lib.dflash_draft_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), F, F, F, 4,
                                1, 64, None, F, F, F, None, F, 16, None)
    assert st == -3
    # a workspace off a 16-byte boundary
    st = lib.dflash_project_context(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), F, 512,
                                    F, F, None, 1, 4, ctypes.c_void_p(fake + 8), 1 << 30, None)
    assert st == -1 and b"aligned" in lib.dflash_last_error()
    st = lib.dflash_draft_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), F, F, F, 4,
                                1, 64, None, F, F, F, None, ctypes.c_void_p(fake + 4), 1 << 30,
                                None)
    assert st == -1 and b"aligned" in lib.dflash_last_error()
    # zero rows / zero batch: nothing to do, no launch
    assert lib.dflash_project_context(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), F, 512,
                                      F, F, None, 0, 4, F, 16, None) == 0
    assert lib.dflash_accept(F, F, F, 0, 4, F, F, F, F, F, None) == 0
    assert lib.dflash_accept(F, F, F, -1, 4, F, F, F, F, F, None) == -1
    assert lib.dflash_accept(None, F, F, 3, 4, F, F, F, F, F, None) == -1
    assert lib.dflash_status_string(-3) == b"workspace too small"


def test_packed_matrix_sizes_and_errors():
    """Packed size = ceil(rows / 16) * 16 * cols * element size; invalid shapes
    and dtypes, NULL, misaligned or overlapping buffers fail before any launch."""
    lib = dfl.raw_lib()
    assert lib.dflash_packed_matrix_bytes(15, 64, dfl.BF16) == 16 * 64 * 2
    assert lib.dflash_packed_matrix_bytes(16, 64, dfl.F32) == 16 * 64 * 4
    assert lib.dflash_packed_matrix_bytes(151936, 4096, dfl.BF16) == 151936 * 4096 * 2
    assert lib.dflash_packed_matrix_bytes(5003, 512, dfl.BF16) == 5008 * 512 * 2
    assert lib.dflash_packed_matrix_bytes(16, 40, dfl.BF16) == 0
    assert lib.dflash_packed_matrix_bytes(16, 64, dfl.FP8_E4M3) == 0
    assert lib.dflash_packed_matrix_bytes(0, 64, dfl.BF16) == 0
    a, b = 0x100000, 0x900000
    assert lib.dflash_pack_matrix(a, b, 16, 40, dfl.BF16, None) == -2
    assert lib.dflash_pack_matrix(a, b, 16, 64, dfl.FP8_E4M3, None) == -2
    assert lib.dflash_pack_matrix(None, b, 16, 64, dfl.BF16, None) == -1
    assert lib.dflash_pack_matrix(a, a + 8, 16, 64, dfl.BF16, None) == -1
    assert lib.dflash_pack_matrix(a, a + 1024, 16, 64, dfl.BF16, None) == -1  # overlap
    assert lib.dflash_pack_matrix(a, b, -1, 64, dfl.BF16, None) == -1


def test_accept_sampling_argument_errors():
    """Host-visible errors of dflash_accept_sampling come back before any launch."""
    lib = dfl.raw_lib()
    F = ctypes.c_void_p(0x100000)
    big = 1 << 30

    def call(B=2, S=4, V=1000, dt=dfl.BF16, Tt=1.0, Td=1.0, draft=F, cand=F, ws=F, wsb=big):
        return lib.dflash_accept_sampling(cand, F, draft, dt, V, Tt, Td, F, F, B, S, F, F, F, F, F,
                                          ws, wsb, None)

    assert call(B=0) == 0                       # nothing to do, no launch
    assert call(B=-1) == -1
    assert call(S=1) == -2 and call(S=65) == -2
    assert call(V=0) == -1 and call(V=524289) == -2
    assert call(dt=dfl.FP8_E4M3) == -2
    assert call(Tt=0.0) == -1 and call(Tt=float("nan")) == -1
    assert call(Td=-1.0) == -1
    assert call(cand=None) == -1
    assert call(wsb=16) == -3 and b"workspace" in lib.dflash_last_error()
    assert call(ws=ctypes.c_void_p(0x100004)) == -1
    assert dfl.accept_sampling_workspace_bytes(32, 16, 151936, True) > 0
    assert dfl.accept_sampling_workspace_bytes(32, 16, 151936, False) < \
        dfl.accept_sampling_workspace_bytes(32, 16, 151936, True)
    assert dfl.accept_sampling_workspace_bytes(0, 16, 151936, True) == 0
    assert dfl.accept_sampling_workspace_bytes(4, 1, 100, True) == 0


def test_selector_argument_errors():
    """dflash_draft_block_selector rejects a missing or unsupported selector
    before any launch (the draft arguments here pass their own checks)."""
    lib = dfl.raw_lib()
    cfg = dfl.make_config(TINY)
    fake = 0x100000
    w = dfl.CWeights()
    for n in ("embed", "lm_head", "fc", "hidden_norm", "final_norm"):
        setattr(w, n, fake)
    for n in dfl._LAYER_FIELDS:
        setattr(w.layer[0], n, fake)
    kv = dfl.CKVCache()
    kv.k[0] = kv.v[0] = fake
    kv.num_pages = 8
    F = ctypes.c_void_p(fake)

    def call(sel, cand_ids=F):
        return lib.dflash_draft_block_selector(
            ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv),
            ctypes.byref(sel) if sel is not None else None, F, F, F, 4, 1, 64, None, F, F, F,
            cand_ids, F, None, 1.0, None, F, 1 << 30, None)

    assert call(None) == -1
    assert call(dfl.CSelector(fake, fake, fake, 64, 3)) == -2
    assert call(dfl.CSelector(fake, fake, fake, 0, 8)) == -2
    assert call(dfl.CSelector(None, fake, fake, 64, 8)) == -1
    assert call(dfl.CSelector(fake, fake, fake, 64, 8), cand_ids=None) == -1
    assert dfl.selector_workspace_bytes(TINY, type("S", (), {"c": dfl.CSelector(
        fake, fake, fake, 64, 8)})(), 1, 64) > dfl.draft_workspace_bytes(TINY, 1, 64)


def test_accept_logits_argument_errors():
    """Host-visible errors of dflash_accept_logits come back before any launch
    (every call below fails a check, or has nothing to do)."""
    lib = dfl.raw_lib()
    F = ctypes.c_void_p(0x100000)

    def call(B=2, S=4, V=1000, dt=dfl.BF16, cand=F, ws=F, wsb=1 << 30):
        return lib.dflash_accept_logits(cand, F, dt, V, F, B, S, F, F, F, F, F, ws, wsb, None)

    assert call(B=0) == 0
    assert call(B=-1) == -1
    assert call(S=1) == -2 and call(S=65) == -2
    assert call(V=0) == -1 and call(V=524289) == -2
    assert call(dt=dfl.FP8_E4M3) == -2
    assert call(cand=None) == -1
    assert call(wsb=16) == -3 and b"workspace" in lib.dflash_last_error()
    assert call(ws=ctypes.c_void_p(0x100004)) == -1
    # one (max, index) partial per row and 16384-column chunk
    assert dfl.accept_logits_workspace_bytes(32, 16, 151936) == 8 * 32 * 16 * 10
    assert dfl.accept_logits_workspace_bytes(0, 16, 151936) == 0


def test_accept_sampling_sparse_argument_errors():
    lib = dfl.raw_lib()
    F = ctypes.c_void_p(0x100000)

    def call(B=2, S=4, V=1000, k=8, T=1.0, qi=F, wsb=1 << 30):
        return lib.dflash_accept_sampling_sparse(F, F, dfl.BF16, V, T, qi, F, k, F, F, B, S, F, F,
                                                 F, F, F, F, wsb, None)

    assert call(B=0) == 0
    assert call(k=0) == -2 and call(k=17) == -2
    assert call(S=65) == -2 and call(V=524289) == -2
    assert call(T=0.0) == -1 and call(qi=None) == -1
    assert call(wsb=16) == -3


def test_noalloc_rejects_calls_beyond_its_scratch():
    """The fixed-scratch draft pass refuses a call whose workspace exceeds its
    array, with DFLASH_EWORKSPACE and a message, before any HIP call."""
    lib = dfl.raw_lib()
    limit = dfl.draft_block_noalloc_limit()
    assert limit == 64 << 20
    need = dfl.draft_workspace_bytes(QWEN3_8B_DRAFT, 32, 8192)
    assert need > limit
    fake = ctypes.c_void_p(0x100000)
    c = dfl.make_config(QWEN3_8B_DRAFT)
    w, kv = dfl.CWeights(), dfl.CKVCache()
    st = lib.dflash_draft_block_noalloc(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), fake,
                                        fake, fake, 600, 32, 8192, None, fake, fake, fake, None,
                                        None)
    assert st == -3
    assert b"scratch" in lib.dflash_last_error()
    bad = dfl.make_config(dataclasses.replace(TINY, head_dim=96))
    st = lib.dflash_draft_block_noalloc(ctypes.byref(bad), ctypes.byref(w), ctypes.byref(kv),
                                        fake, fake, fake, 4, 1, 64, None, fake, fake, fake, None,
                                        None)
    assert st == -1


def test_relay_argument_errors():
    """Host-visible relay errors come back before any launch: a field given on
    one side only, negative sizes, a NULL pool."""
    lib = dfl.raw_lib()
    fake = ctypes.c_void_p(0x100000)
    p = dfl.CRequestPool()
    p.anchor, p.seq_len, p.capacity, p.max_pages = 0x100000, 0x100000, 4, 0
    assert lib.dflash_relay_resolve(None, fake, 2, fake, fake, None, None, None) == -1
    # page_table on the batch side but not in the pool
    assert lib.dflash_relay_resolve(ctypes.byref(p), fake, 2, fake, fake, fake, None, None) == -1
    assert b"page_table" in lib.dflash_last_error()
    assert lib.dflash_relay_stash(ctypes.byref(p), fake, -1, fake, fake, None, None, None) == -1
    # n_pages in the pool but not on the batch side
    p.n_pages = 0x100000
    assert lib.dflash_relay_stash(ctypes.byref(p), fake, 2, fake, fake, None, None, None) == -1
    # an empty batch is a no-op
    p.n_pages = None
    assert lib.dflash_relay_stash(ctypes.byref(p), None, 0, fake, fake, None, None, None) == 0


def test_checked_mode_argument_errors():
    """The checked-mode calls refuse NULL pointers and negative sizes before any
    launch; an empty batch or row set only resets the report (not run here:
    that is a launch).  Their report size matches the binding's."""
    lib = dfl.raw_lib()
    fake = ctypes.c_void_p(0x100000)
    c = dfl.make_config(TINY)
    kv = dfl.CKVCache()
    kv.num_pages = 4
    assert lib.dflash_check_draft_inputs(None, ctypes.byref(kv), fake, fake, fake, 4, 1, 64,
                                         fake, None) == -1
    assert lib.dflash_check_draft_inputs(ctypes.byref(c), ctypes.byref(kv), fake, fake, fake, 4,
                                         1, 64, None, None) == -1
    assert lib.dflash_check_draft_inputs(ctypes.byref(c), ctypes.byref(kv), None, fake, fake, 4,
                                         1, 64, fake, None) == -1
    assert lib.dflash_check_draft_inputs(ctypes.byref(c), ctypes.byref(kv), fake, fake, fake, 0,
                                         1, 64, fake, None) == -1
    assert lib.dflash_check_draft_inputs(ctypes.byref(c), ctypes.byref(kv), fake, fake, fake, 4,
                                         -1, 64, fake, None) == -1
    assert lib.dflash_check_context_inputs(ctypes.byref(c), ctypes.byref(kv), fake, fake, None,
                                           -1, 4, fake, None) == -1
    assert lib.dflash_check_context_inputs(ctypes.byref(c), ctypes.byref(kv), None, fake, None,
                                           1, 4, fake, None) == -1
    assert lib.dflash_check_context_inputs(ctypes.byref(c), ctypes.byref(kv), fake, fake, None,
                                           1 << 16, 1 << 16, fake, None) == -1
    assert lib.dflash_check_accept_inputs(fake, fake, fake, 2, 0, 100, fake, None) == -1
    assert lib.dflash_check_accept_inputs(fake, None, fake, 2, 4, 100, fake, None) == -1
    assert lib.dflash_check_accept_inputs(fake, fake, fake, 2, 4, 0, fake, None) == -1
    assert lib.dflash_check_accept_inputs(fake, fake, fake, 2, 4, 100, None, None) == -1
    header = open(os.path.join(ROOT, "include", "dflash.h")).read()
    assert f"#define DFLASH_CHECKS {dfl.CHECKS}" in header
