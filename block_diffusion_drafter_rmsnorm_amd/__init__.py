"""Python binding of libdflash.so, the DFlash draft-and-accept path on MI355X.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory and the stream.  The functions carry
the names of the C entry points (include/dflash.h) and take torch tensors.

Importing fails loudly when the library has not been built
(``python block_diffusion_drafter_rmsnorm_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, List, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DFLASH_LIBRARY selects another build of the same sources (the tests load the
# host-sanitized one through it); by default the in-tree library.
LIB_PATH = os.environ.get("DFLASH_LIBRARY") or os.path.join(_HERE, "libdflash.so")
MAX_LAYERS = 16
CHECKS = 4  # DFLASH_CHECKS: (count, first index) pairs of a checked-mode report

F32, BF16, FP8_E4M3 = 0, 1, 2
_DT_CODE = {"f32": F32, "bf16": BF16, "fp8_e4m3": FP8_E4M3}
_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported configuration",
          -3: "workspace too small", -4: "HIP runtime error"}


class DFlashError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class CConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("feat_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("mask_token_id", ctypes.c_int32),
                ("page_size", ctypes.c_int32),
                ("sliding_window", ctypes.c_int32 * MAX_LAYERS),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("context_window", ctypes.c_int32)]


_LAYER_FIELDS = ["in_norm", "w_qkv", "q_norm", "k_norm", "w_o", "post_norm", "w_gate", "w_up",
                 "w_down"]


class CLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _LAYER_FIELDS]


class CWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("fc", ctypes.c_void_p), ("hidden_norm", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p), ("layer", CLayerWeights * MAX_LAYERS)]


class CSelector(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("w_h", ctypes.c_void_p),
                ("rank", ctypes.c_int32), ("top_k", ctypes.c_int32)]


class CKVCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p * MAX_LAYERS), ("v", ctypes.c_void_p * MAX_LAYERS),
                ("num_pages", ctypes.c_int64)]


class CRequestPool(ctypes.Structure):
    _fields_ = [("anchor", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("n_pages", ctypes.c_void_p),
                ("capacity", ctypes.c_int32), ("max_pages", ctypes.c_int32)]


EXPORTED = ["dflash_context_workspace_bytes", "dflash_draft_workspace_bytes",
            "dflash_project_context", "dflash_draft_block", "dflash_accept",
            "dflash_accept_logits_workspace_bytes", "dflash_accept_logits",
            "dflash_accept_sampling_workspace_bytes", "dflash_accept_sampling",
            "dflash_selector_workspace_bytes", "dflash_draft_block_selector",
            "dflash_accept_sampling_sparse", "dflash_reserve_pages", "dflash_release_pages",
            "dflash_lm_head_workspace_bytes", "dflash_lm_head_argmax",
            "dflash_packed_matrix_bytes", "dflash_pack_matrix",
            "dflash_draft_block_noalloc_limit", "dflash_draft_block_noalloc",
            "dflash_relay_resolve", "dflash_relay_stash",
            "dflash_check_draft_inputs", "dflash_check_context_inputs",
            "dflash_check_accept_inputs",
            "dflash_status_string", "dflash_last_error"]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python block_diffusion_drafter_rmsnorm_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    missing = [n for n in EXPORTED if not hasattr(lib, n)]
    if missing:
        raise ImportError(f"{LIB_PATH} is stale (missing {missing}): rebuild it")
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp, wp, kvp = ctypes.POINTER(CConfig), ctypes.POINTER(CWeights), ctypes.POINTER(CKVCache)
    lib.dflash_context_workspace_bytes.argtypes = [cfgp, I64]
    lib.dflash_context_workspace_bytes.restype = SZ
    lib.dflash_draft_workspace_bytes.argtypes = [cfgp, I32, I32]
    lib.dflash_draft_workspace_bytes.restype = SZ
    lib.dflash_project_context.argtypes = [cfgp, wp, kvp, P, I64, P, P, P, I32, I32, P, SZ, P]
    lib.dflash_project_context.restype = I32
    lib.dflash_draft_block.argtypes = [cfgp, wp, kvp, P, P, P, I32, I32, I32, P, P, P, P, P, P,
                                       SZ, P]
    lib.dflash_draft_block.restype = I32
    lib.dflash_draft_block_noalloc_limit.argtypes = []
    lib.dflash_draft_block_noalloc_limit.restype = SZ
    lib.dflash_draft_block_noalloc.argtypes = [cfgp, wp, kvp, P, P, P, I32, I32, I32, P, P, P, P,
                                               P, P]
    lib.dflash_draft_block_noalloc.restype = I32
    lib.dflash_accept.argtypes = [P, P, P, I32, I32, P, P, P, P, P, P]
    lib.dflash_accept.restype = I32
    lib.dflash_accept_logits_workspace_bytes.argtypes = [I32, I32, I32]
    lib.dflash_accept_logits_workspace_bytes.restype = SZ
    lib.dflash_accept_logits.argtypes = [P, P, I32, I32, P, I32, I32, P, P, P, P, P, P, SZ, P]
    lib.dflash_accept_logits.restype = I32
    lib.dflash_accept_sampling_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.dflash_accept_sampling_workspace_bytes.restype = SZ
    F = ctypes.c_float
    lib.dflash_accept_sampling.argtypes = [P, P, P, I32, I32, F, F, P, P, I32, I32, P, P, P, P, P,
                                           P, SZ, P]
    lib.dflash_accept_sampling.restype = I32
    lib.dflash_accept_sampling_sparse.argtypes = [P, P, I32, I32, F, P, P, I32, P, P, I32, I32, P,
                                                  P, P, P, P, P, SZ, P]
    lib.dflash_accept_sampling_sparse.restype = I32
    lib.dflash_reserve_pages.argtypes = [P, I32, I32, I32, P, I32, P, P, I32, P, P, P]
    lib.dflash_reserve_pages.restype = I32
    lib.dflash_release_pages.argtypes = [P, I32, P, I32, P, P, I32, P, P]
    lib.dflash_release_pages.restype = I32
    poolp = ctypes.POINTER(CRequestPool)
    lib.dflash_relay_resolve.argtypes = [poolp, P, I32, P, P, P, P, P]
    lib.dflash_relay_resolve.restype = I32
    lib.dflash_relay_stash.argtypes = [poolp, P, I32, P, P, P, P, P]
    lib.dflash_relay_stash.restype = I32
    selp = ctypes.POINTER(CSelector)
    lib.dflash_selector_workspace_bytes.argtypes = [cfgp, selp, I32, I32]
    lib.dflash_selector_workspace_bytes.restype = SZ
    lib.dflash_draft_block_selector.argtypes = [cfgp, wp, kvp, selp, P, P, P, I32, I32, I32, P, P,
                                                P, P, P, P, P, F, P, P, SZ, P]
    lib.dflash_draft_block_selector.restype = I32
    lib.dflash_lm_head_workspace_bytes.argtypes = [cfgp, I32]
    lib.dflash_lm_head_workspace_bytes.restype = SZ
    lib.dflash_lm_head_argmax.argtypes = [cfgp, P, P, I32, P, P, P, SZ, P]
    lib.dflash_lm_head_argmax.restype = I32
    lib.dflash_packed_matrix_bytes.argtypes = [I32, I32, I32]
    lib.dflash_packed_matrix_bytes.restype = SZ
    lib.dflash_pack_matrix.argtypes = [P, P, I32, I32, I32, P]
    lib.dflash_pack_matrix.restype = I32
    lib.dflash_check_draft_inputs.argtypes = [cfgp, kvp, P, P, P, I32, I32, I32, P, P]
    lib.dflash_check_draft_inputs.restype = I32
    lib.dflash_check_context_inputs.argtypes = [cfgp, kvp, P, P, P, I32, I32, P, P]
    lib.dflash_check_context_inputs.restype = I32
    lib.dflash_check_accept_inputs.argtypes = [P, P, P, I32, I32, I32, P, P]
    lib.dflash_check_accept_inputs.restype = I32
    lib.dflash_status_string.argtypes = [I32]
    lib.dflash_status_string.restype = ctypes.c_char_p
    lib.dflash_last_error.argtypes = []
    lib.dflash_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


def _check(status: int):
    if status != 0:
        raise DFlashError(status, _lib.dflash_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_config(cfg) -> CConfig:
    """C config from a workloads.configs.DFlashConfig-like object."""
    c = CConfig()
    c.hidden, c.n_layers, c.n_q_heads = cfg.hidden, cfg.n_layers, cfg.n_q_heads
    c.n_kv_heads, c.head_dim, c.inter, c.vocab = cfg.n_kv_heads, cfg.head_dim, cfg.inter, cfg.vocab
    c.feat_dim = cfg.n_target_layers * cfg.target_hidden
    c.block_size, c.mask_token_id, c.page_size = cfg.block_size, cfg.mask_token_id, cfg.page_size
    for l in range(MAX_LAYERS):
        c.sliding_window[l] = int(cfg.sliding_window[l]) if l < len(cfg.sliding_window) else 0
    c.rms_eps, c.rope_theta = float(cfg.rms_eps), float(cfg.rope_theta)
    c.act_dtype, c.kv_dtype = _DT_CODE[cfg.act_dtype], _DT_CODE[cfg.kv_dtype]
    c.context_window = int(getattr(cfg, "context_window", 0))
    return c


PACKED_FIELDS = ("lm_head", "fc")
PACKED_LAYER_FIELDS = ("w_qkv", "w_o", "w_gate", "w_up", "w_down")
_MAT_DT = {torch.bfloat16: BF16, torch.float32: F32}


def packed_matrix_bytes(rows: int, cols: int, dtype: torch.dtype) -> int:
    return int(_lib.dflash_packed_matrix_bytes(int(rows), int(cols), _MAT_DT[dtype]))


def dflash_pack_matrix(w: torch.Tensor, stream=None) -> torch.Tensor:
    """Fragment-packed copy (a new 1-D tensor) of a row-major [rows, cols] matrix."""
    rows, cols = w.shape
    n = packed_matrix_bytes(rows, cols, w.dtype)
    if n == 0:
        raise DFlashError(-2, f"cannot pack a {tuple(w.shape)} {w.dtype} matrix")
    src = w.contiguous()
    out = torch.empty(n // w.element_size(), dtype=w.dtype, device=w.device)
    _check(_lib.dflash_pack_matrix(_ptr(src), _ptr(out), rows, cols, _MAT_DT[w.dtype],
                                   _stream(stream)))
    return out


def make_weights(W: Dict) -> CWeights:
    """C weight table from the dict of device tensors (row-major matrices).

    The projection matrices are packed into new tensors, which the returned
    table keeps alive in its ``packed`` attribute ({name: tensor} and, per
    layer, ``packed["layers"][l]``); the other tensors (embedding, gains) are
    referenced in place and the caller keeps them alive."""
    w = CWeights()
    packed = {"layers": []}
    for n in ("embed", "lm_head", "fc", "hidden_norm", "final_norm"):
        t = W.get(n)
        if t is not None and n in PACKED_FIELDS:
            t = packed[n] = dflash_pack_matrix(t)
        setattr(w, n, None if t is None else t.data_ptr())
    for l, Lw in enumerate(W["layers"]):
        packed["layers"].append({})
        if Lw is None:
            continue
        for n in _LAYER_FIELDS:
            t = Lw.get(n)
            if t is not None and n in PACKED_LAYER_FIELDS:
                t = packed["layers"][l][n] = dflash_pack_matrix(t)
            setattr(w.layer[l], n, None if t is None else t.data_ptr())
    w.packed = packed
    return w


@dataclass
class KVCache:
    """Paged draft cache: per layer K pages [num_pages, nkv, page, D] and V
    pages stored transposed, [num_pages, nkv, D, page]."""
    k: List[torch.Tensor]
    v: List[torch.Tensor]
    num_pages: int

    @staticmethod
    def allocate(cfg, num_pages: int, device="cuda", fill=None) -> "KVCache":
        kshp = (num_pages, cfg.n_kv_heads, cfg.page_size, cfg.head_dim)
        vshp = (num_pages, cfg.n_kv_heads, cfg.head_dim, cfg.page_size)
        dt = _TORCH_DT[cfg.kv_dtype]

        def mk(shp):
            if fill is None:
                return torch.empty(shp, dtype=dt, device=device)
            return torch.full(shp, fill, dtype=dt, device=device)
        return KVCache([mk(kshp) for _ in range(cfg.n_layers)],
                       [mk(vshp) for _ in range(cfg.n_layers)], num_pages)

    def c_struct(self) -> CKVCache:
        c = CKVCache()
        for l, (k, v) in enumerate(zip(self.k, self.v)):
            c.k[l] = k.data_ptr()
            c.v[l] = v.data_ptr()
        c.num_pages = self.num_pages
        return c


def context_workspace_bytes(cfg, rows: int) -> int:
    return int(_lib.dflash_context_workspace_bytes(ctypes.byref(make_config(cfg)), int(rows)))


def draft_workspace_bytes(cfg, batch: int, max_prefix_len: int) -> int:
    return int(_lib.dflash_draft_workspace_bytes(ctypes.byref(make_config(cfg)), int(batch),
                                                 int(max_prefix_len)))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- checked mode
# Device-side checks of the values the calls read from device memory (the
# rules are listed with dflash_check_*_inputs in dflash.h).  Each returns
# {rule: (count, first index)} for the rules that have violations; the
# `checked=True` flag of the calls below runs them first, synchronises, and
# raises ValueError instead of launching when any rule is violated.
CHECK_RULES = {
    "draft": ("anchor id outside [0, vocab)", "prefix_len outside [0, max_prefix_len]",
              "block does not fit the page-table row", "page-table entry outside the pool"),
    "context": ("live row's slot outside the pool", "live row's position < 0",
                "valid_rows outside [0, rows_per_req]"),
    "accept": ("candidate id outside [0, vocab)", "posterior id outside [0, vocab)",
               "prefix_len < 0"),
}


def _report(kind: str, report: torch.Tensor) -> Dict[str, tuple]:
    r = report.cpu().tolist()  # synchronises with the stream the check ran on
    names = CHECK_RULES[kind]
    return {names[k]: (r[2 * k], r[2 * k + 1]) for k in range(len(names)) if r[2 * k] > 0}


def _report_buffer(device) -> torch.Tensor:
    return torch.empty(2 * CHECKS, dtype=torch.int32, device=device)


def check_draft_inputs(cfg, cache: KVCache, anchor: torch.Tensor, prefix_len: torch.Tensor,
                       page_table: torch.Tensor, max_prefix_len: int, stream=None,
                       c_cfg: Optional[CConfig] = None, c_cache: Optional[CKVCache] = None):
    c_cfg = c_cfg if c_cfg is not None else make_config(cfg)
    c_cache = c_cache if c_cache is not None else cache.c_struct()
    report = _report_buffer(anchor.device)
    _check(_lib.dflash_check_draft_inputs(
        ctypes.byref(c_cfg), ctypes.byref(c_cache), _ptr(anchor), _ptr(prefix_len),
        _ptr(page_table), int(page_table.shape[1]), int(anchor.shape[0]), int(max_prefix_len),
        _ptr(report), _stream(stream)))
    return _report("draft", report)


def check_context_inputs(cfg, cache: KVCache, positions: torch.Tensor, slots: torch.Tensor,
                         valid_rows: Optional[torch.Tensor], n_req: int, rows_per_req: int,
                         stream=None, c_cfg: Optional[CConfig] = None,
                         c_cache: Optional[CKVCache] = None):
    c_cfg = c_cfg if c_cfg is not None else make_config(cfg)
    c_cache = c_cache if c_cache is not None else cache.c_struct()
    report = _report_buffer(slots.device)
    _check(_lib.dflash_check_context_inputs(
        ctypes.byref(c_cfg), ctypes.byref(c_cache), _ptr(positions), _ptr(slots),
        _ptr(valid_rows), int(n_req), int(rows_per_req), _ptr(report), _stream(stream)))
    return _report("context", report)


def check_accept_inputs(candidates: torch.Tensor, posterior: torch.Tensor,
                        prefix_len: torch.Tensor, vocab: int, stream=None):
    B, S = candidates.shape
    report = _report_buffer(candidates.device)
    _check(_lib.dflash_check_accept_inputs(_ptr(candidates), _ptr(posterior), _ptr(prefix_len),
                                           int(B), int(S), int(vocab), _ptr(report),
                                           _stream(stream)))
    return _report("accept", report)


def _raise_if(found: Dict[str, tuple], call: str):
    if found:
        raise ValueError(f"{call}: device inputs break the contract: " +
                         "; ".join(f"{k} ({n}x, first at {i})" for k, (n, i) in found.items()))


def dflash_project_context(cfg, weights: CWeights, cache: KVCache, feats: torch.Tensor,
                           positions: torch.Tensor, slots: torch.Tensor,
                           valid_rows: Optional[torch.Tensor], n_req: int, rows_per_req: int,
                           ws: torch.Tensor, stream=None, c_cfg: Optional[CConfig] = None,
                           c_cache: Optional[CKVCache] = None, checked: bool = False):
    c_cfg = c_cfg if c_cfg is not None else make_config(cfg)
    c_cache = c_cache if c_cache is not None else cache.c_struct()
    if checked:
        _raise_if(check_context_inputs(cfg, cache, positions, slots, valid_rows, n_req,
                                       rows_per_req, stream, c_cfg, c_cache),
                  "dflash_project_context")
    _check(_lib.dflash_project_context(
        ctypes.byref(c_cfg), ctypes.byref(weights), ctypes.byref(c_cache), _ptr(feats),
        int(feats.stride(0)), _ptr(positions), _ptr(slots), _ptr(valid_rows), int(n_req),
        int(rows_per_req), _ptr(ws), int(ws.numel()), _stream(stream)))


def dflash_draft_block(cfg, weights: CWeights, cache: KVCache, anchor: torch.Tensor,
                       prefix_len: torch.Tensor, page_table: torch.Tensor, max_prefix_len: int,
                       positions: torch.Tensor, slots: torch.Tensor, candidates: torch.Tensor,
                       ws: torch.Tensor, block_ids: Optional[torch.Tensor] = None,
                       logits: Optional[torch.Tensor] = None, stream=None,
                       c_cfg: Optional[CConfig] = None, c_cache: Optional[CKVCache] = None,
                       checked: bool = False):
    c_cfg = c_cfg if c_cfg is not None else make_config(cfg)
    c_cache = c_cache if c_cache is not None else cache.c_struct()
    if checked:
        _raise_if(check_draft_inputs(cfg, cache, anchor, prefix_len, page_table, max_prefix_len,
                                     stream, c_cfg, c_cache), "dflash_draft_block")
    _check(_lib.dflash_draft_block(
        ctypes.byref(c_cfg), ctypes.byref(weights), ctypes.byref(c_cache), _ptr(anchor),
        _ptr(prefix_len), _ptr(page_table), int(page_table.shape[1]), int(anchor.shape[0]),
        int(max_prefix_len), _ptr(block_ids), _ptr(positions), _ptr(slots), _ptr(candidates),
        _ptr(logits), _ptr(ws), int(ws.numel()), _stream(stream)))


def draft_block_noalloc_limit() -> int:
    return int(_lib.dflash_draft_block_noalloc_limit())


def dflash_draft_block_noalloc(cfg, weights: CWeights, cache: KVCache, anchor: torch.Tensor,
                               prefix_len: torch.Tensor, page_table: torch.Tensor,
                               max_prefix_len: int, positions: torch.Tensor, slots: torch.Tensor,
                               candidates: torch.Tensor, block_ids: Optional[torch.Tensor] = None,
                               logits: Optional[torch.Tensor] = None, stream=None,
                               c_cfg: Optional[CConfig] = None,
                               c_cache: Optional[CKVCache] = None):
    """dflash_draft_block on the library's fixed scratch array (no workspace argument)."""
    c_cfg = c_cfg if c_cfg is not None else make_config(cfg)
    c_cache = c_cache if c_cache is not None else cache.c_struct()
    _check(_lib.dflash_draft_block_noalloc(
        ctypes.byref(c_cfg), ctypes.byref(weights), ctypes.byref(c_cache), _ptr(anchor),
        _ptr(prefix_len), _ptr(page_table), int(page_table.shape[1]), int(anchor.shape[0]),
        int(max_prefix_len), _ptr(block_ids), _ptr(positions), _ptr(slots), _ptr(candidates),
        _ptr(logits), _stream(stream)))


def dflash_accept(candidates: torch.Tensor, posterior: torch.Tensor, prefix_len: torch.Tensor,
                  accept_len: torch.Tensor, commit_len: torch.Tensor, out_tokens: torch.Tensor,
                  next_anchor: torch.Tensor, new_seq_len: torch.Tensor, stream=None,
                  checked_vocab: Optional[int] = None):
    """checked_vocab: run the checked mode with this vocabulary size first."""
    B, S = candidates.shape
    if checked_vocab is not None:
        _raise_if(check_accept_inputs(candidates, posterior, prefix_len, checked_vocab, stream),
                  "dflash_accept")
    _check(_lib.dflash_accept(_ptr(candidates), _ptr(posterior), _ptr(prefix_len), int(B), int(S),
                              _ptr(accept_len), _ptr(commit_len), _ptr(out_tokens),
                              _ptr(next_anchor), _ptr(new_seq_len), _stream(stream)))


def accept_sampling_workspace_bytes(batch: int, block_size: int, vocab: int,
                                    has_draft_logits: bool) -> int:
    return int(_lib.dflash_accept_sampling_workspace_bytes(int(batch), int(block_size),
                                                           int(vocab), int(bool(has_draft_logits))))


_LOGITS_DT = {torch.float32: F32, torch.bfloat16: BF16}


def accept_logits_workspace_bytes(batch: int, block_size: int, vocab: int) -> int:
    return int(_lib.dflash_accept_logits_workspace_bytes(int(batch), int(block_size), int(vocab)))


def dflash_accept_logits(candidates: torch.Tensor, target_logits: torch.Tensor,
                         prefix_len: torch.Tensor, accept_len: torch.Tensor,
                         commit_len: torch.Tensor, out_tokens: torch.Tensor,
                         next_anchor: torch.Tensor, new_seq_len: torch.Tensor, ws: torch.Tensor,
                         stream=None):
    """Greedy accept against the argmax of target_logits [B, S, V] (f32 or bf16);
    ws from workspace(accept_logits_workspace_bytes())."""
    B, S = candidates.shape
    V = int(target_logits.shape[-1])
    dt = _LOGITS_DT.get(target_logits.dtype)
    if dt is None:
        raise DFlashError(-2, f"logits dtype {target_logits.dtype} (supported: f32, bf16)")
    _check(_lib.dflash_accept_logits(
        _ptr(candidates), _ptr(target_logits), dt, V, _ptr(prefix_len), int(B), int(S),
        _ptr(accept_len), _ptr(commit_len), _ptr(out_tokens), _ptr(next_anchor),
        _ptr(new_seq_len), _ptr(ws), int(ws.numel()), _stream(stream)))


def dflash_accept_sampling(candidates: torch.Tensor, target_logits: torch.Tensor,
                           uniforms: torch.Tensor, prefix_len: torch.Tensor,
                           accept_len: torch.Tensor, commit_len: torch.Tensor,
                           out_tokens: torch.Tensor, next_anchor: torch.Tensor,
                           new_seq_len: torch.Tensor, ws: torch.Tensor,
                           target_temperature: float = 1.0,
                           draft_logits: Optional[torch.Tensor] = None,
                           draft_temperature: float = 1.0, stream=None):
    """target_logits [B, S, V]; draft_logits None (argmax drafts) or [B, S-1, V] of the
    same dtype; uniforms [B, S] f32; ws from workspace(accept_sampling_workspace_bytes())."""
    B, S = candidates.shape
    V = int(target_logits.shape[-1])
    if draft_logits is not None and draft_logits.dtype != target_logits.dtype:
        raise DFlashError(-1, "draft_logits and target_logits must share a dtype")
    dt = _LOGITS_DT.get(target_logits.dtype)
    if dt is None:
        raise DFlashError(-2, f"logits dtype {target_logits.dtype} (supported: f32, bf16)")
    _check(_lib.dflash_accept_sampling(
        _ptr(candidates), _ptr(target_logits), _ptr(draft_logits), dt, V,
        float(target_temperature), float(draft_temperature), _ptr(uniforms), _ptr(prefix_len),
        int(B), int(S), _ptr(accept_len), _ptr(commit_len), _ptr(out_tokens), _ptr(next_anchor),
        _ptr(new_seq_len), _ptr(ws), int(ws.numel()), _stream(stream)))


class Selector:
    """DFlash 2 selector weights: a, b [V, rank] (act dtype), w_h [rank, H]
    (packed here, once).  The tensors are kept alive by this object."""

    def __init__(self, a: torch.Tensor, b: torch.Tensor, w_h: torch.Tensor, top_k: int = 8):
        self.a, self.b = a.contiguous(), b.contiguous()
        self.w_h = dflash_pack_matrix(w_h.contiguous())
        self.c = CSelector(self.a.data_ptr(), self.b.data_ptr(), self.w_h.data_ptr(),
                           int(a.shape[1]), int(top_k))


def selector_workspace_bytes(cfg, sel: "Selector", batch: int, max_prefix_len: int) -> int:
    return int(_lib.dflash_selector_workspace_bytes(ctypes.byref(make_config(cfg)),
                                                    ctypes.byref(sel.c), int(batch),
                                                    int(max_prefix_len)))


def dflash_draft_block_selector(cfg, weights: CWeights, cache: "KVCache", sel: "Selector",
                                anchor: torch.Tensor, prefix_len: torch.Tensor,
                                page_table: torch.Tensor, max_prefix_len: int,
                                positions: torch.Tensor, slots: torch.Tensor,
                                candidates: torch.Tensor, cand_ids: torch.Tensor,
                                q_rows: torch.Tensor, ws: torch.Tensor,
                                uniforms: Optional[torch.Tensor] = None, temperature: float = 1.0,
                                block_ids: Optional[torch.Tensor] = None,
                                logits: Optional[torch.Tensor] = None, stream=None):
    c_cfg = make_config(cfg)
    c_cache = cache.c_struct()
    _check(_lib.dflash_draft_block_selector(
        ctypes.byref(c_cfg), ctypes.byref(weights), ctypes.byref(c_cache), ctypes.byref(sel.c),
        _ptr(anchor), _ptr(prefix_len), _ptr(page_table), int(page_table.shape[1]),
        int(anchor.shape[0]), int(max_prefix_len), _ptr(block_ids), _ptr(positions), _ptr(slots),
        _ptr(candidates), _ptr(cand_ids), _ptr(q_rows), _ptr(uniforms), float(temperature),
        _ptr(logits), _ptr(ws), int(ws.numel()), _stream(stream)))


def dflash_accept_sampling_sparse(candidates: torch.Tensor, target_logits: torch.Tensor,
                                  q_ids: torch.Tensor, q_probs: torch.Tensor,
                                  uniforms: torch.Tensor, prefix_len: torch.Tensor,
                                  accept_len: torch.Tensor, commit_len: torch.Tensor,
                                  out_tokens: torch.Tensor, next_anchor: torch.Tensor,
                                  new_seq_len: torch.Tensor, ws: torch.Tensor,
                                  target_temperature: float = 1.0, stream=None):
    """q_ids / q_probs [B, S-1, K]: the selector's cand_ids and q_rows; ws from
    workspace(accept_sampling_workspace_bytes(B, S, V, False))."""
    B, S = candidates.shape
    dt = _LOGITS_DT.get(target_logits.dtype)
    if dt is None:
        raise DFlashError(-2, f"logits dtype {target_logits.dtype} (supported: f32, bf16)")
    _check(_lib.dflash_accept_sampling_sparse(
        _ptr(candidates), _ptr(target_logits), dt, int(target_logits.shape[-1]),
        float(target_temperature), _ptr(q_ids), _ptr(q_probs), int(q_ids.shape[-1]),
        _ptr(uniforms), _ptr(prefix_len), int(B), int(S), _ptr(accept_len), _ptr(commit_len),
        _ptr(out_tokens), _ptr(next_anchor), _ptr(new_seq_len), _ptr(ws), int(ws.numel()),
        _stream(stream)))


def dflash_reserve_pages(seq_len: torch.Tensor, block_size: int, page_size: int,
                         page_table: torch.Tensor, n_pages: torch.Tensor,
                         free_pages: torch.Tensor, free_count: torch.Tensor,
                         status: torch.Tensor, stream=None):
    _check(_lib.dflash_reserve_pages(_ptr(seq_len), int(seq_len.shape[0]), int(block_size),
                                     int(page_size), _ptr(page_table), int(page_table.shape[1]),
                                     _ptr(n_pages), _ptr(free_pages), int(free_pages.numel()),
                                     _ptr(free_count), _ptr(status), _stream(stream)))


def dflash_release_pages(mask: torch.Tensor, page_table: torch.Tensor, n_pages: torch.Tensor,
                         free_pages: torch.Tensor, free_count: torch.Tensor, stream=None):
    _check(_lib.dflash_release_pages(_ptr(mask), int(mask.shape[0]), _ptr(page_table),
                                     int(page_table.shape[1]), _ptr(n_pages), _ptr(free_pages),
                                     int(free_pages.numel()), _ptr(free_count), _stream(stream)))


def lm_head_workspace_bytes(cfg, rows: int) -> int:
    return int(_lib.dflash_lm_head_workspace_bytes(ctypes.byref(make_config(cfg)), int(rows)))


def dflash_lm_head_argmax(cfg, lm_head: torch.Tensor, hidden: torch.Tensor, ids: torch.Tensor,
                          ws: torch.Tensor, logits: Optional[torch.Tensor] = None, stream=None,
                          c_cfg: Optional[CConfig] = None):
    """lm_head: the packed matrix (dflash_pack_matrix or make_weights(W).packed)."""
    c_cfg = c_cfg if c_cfg is not None else make_config(cfg)
    _check(_lib.dflash_lm_head_argmax(ctypes.byref(c_cfg), _ptr(lm_head), _ptr(hidden),
                                      int(hidden.shape[0]), _ptr(logits), _ptr(ids), _ptr(ws),
                                      int(ws.numel()), _stream(stream)))


def raw_lib():
    """The ctypes library handle (for ABI tests)."""
    return _lib


def make_request_pool(anchor: torch.Tensor, seq_len: torch.Tensor,
                      page_table: Optional[torch.Tensor] = None,
                      n_pages: Optional[torch.Tensor] = None) -> CRequestPool:
    """C request-pool table over int32 device tensors [capacity] (page_table
    [capacity, max_pages]); the caller keeps the tensors alive."""
    p = CRequestPool()
    p.anchor, p.seq_len = anchor.data_ptr(), seq_len.data_ptr()
    p.page_table = None if page_table is None else page_table.data_ptr()
    p.n_pages = None if n_pages is None else n_pages.data_ptr()
    p.capacity = int(anchor.shape[0])
    p.max_pages = 0 if page_table is None else int(page_table.shape[1])
    return p


def dflash_relay_resolve(pool: CRequestPool, req_slots: torch.Tensor, anchor: torch.Tensor,
                         prefix_len: torch.Tensor, page_table: Optional[torch.Tensor] = None,
                         n_pages: Optional[torch.Tensor] = None, stream=None):
    _check(_lib.dflash_relay_resolve(ctypes.byref(pool), _ptr(req_slots), int(req_slots.shape[0]),
                                     _ptr(anchor), _ptr(prefix_len), _ptr(page_table),
                                     _ptr(n_pages), _stream(stream)))


def dflash_relay_stash(pool: CRequestPool, req_slots: torch.Tensor, next_anchor: torch.Tensor,
                       new_seq_len: torch.Tensor, page_table: Optional[torch.Tensor] = None,
                       n_pages: Optional[torch.Tensor] = None, stream=None):
    _check(_lib.dflash_relay_stash(ctypes.byref(pool), _ptr(req_slots), int(req_slots.shape[0]),
                                   _ptr(next_anchor), _ptr(new_seq_len), _ptr(page_table),
                                   _ptr(n_pages), _stream(stream)))
