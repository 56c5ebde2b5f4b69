"""Shared plumbing of the GPU parity tests: seeded inputs, calls through the
C ABI binding, and the matching oracle calls on CPU copies of the same
inputs.  Layout conversion only; no method arithmetic."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from oracle.formats import e4m3_decode
from workloads import synth
from tests.helpers import np_weights, paged_to_slots, to_np


def dfl():
    import block_diffusion_drafter_rmsnorm_amd as m
    return m


class Setup:
    """Inputs of one workload on one device, plus their CPU/numpy views."""

    def __init__(self, wl, device="cuda", gen_device=None, seed=None, weights=True,
                 random_cache=True, extra_tokens=None, skip=()):
        self.wl, self.cfg = wl, wl.cfg
        cfg = self.cfg
        self.device = device
        gd = gen_device or device
        s = wl.seed if seed is None else seed
        self.seed = s
        self.B, self.S, self.P = wl.batch, cfg.block_size, cfg.page_size
        self.L = synth.prefix_lengths(wl, "cpu", s).to(torch.int32)
        extra = 2 * cfg.block_size if extra_tokens is None else extra_tokens
        self.pt, self.num_pages = synth.page_table(self.L, cfg, s, extra)
        self.anchor = synth.randint(0, cfg.vocab - 1, (self.B,), s, "anchor", "cpu").to(torch.int32)
        self.W = synth.weights(cfg, s, gd, skip=skip) if weights else None
        if self.W is not None and gd != device:
            self.W = _to(self.W, device)
        self.cache = None
        if random_cache:
            K, V = synth.kv_pool_random(cfg, self.num_pages, s, gd)
            m = dfl()
            self.cache = m.KVCache([k.to(device) for k in K], [v.to(device) for v in V],
                                   self.num_pages)
        self._npW = None
        self._cw = None

    def c_weights(self):
        """The C weight table (projection matrices packed once, on first use)."""
        if self._cw is None:
            self._cw = dfl().make_weights(self.W)
        return self._cw

    # ------------------------------------------------------------ oracle views
    def np_W(self):
        if self._npW is None:
            self._npW = np_weights(_to(self.W, "cpu"))
        return self._npW

    def oracle_cache(self):
        c = oracle.OracleCache.__new__(oracle.OracleCache)
        c.k, c.v = [], []
        for k, v in zip(self.cache.k, self.cache.v):
            c.k.append(self._pool_values(k))
            c.v.append(self._pool_values(v, transposed=True))
        return c

    def _pool_values(self, pool, transposed=False):
        if self.cfg.kv_dtype == "fp8_e4m3":
            a = e4m3_decode(pool.cpu().numpy())
        else:
            a = pool.detach().to("cpu", torch.float64).numpy()
        return paged_to_slots(a, self.P, transposed)

    # ------------------------------------------------------------ GPU calls
    def draft(self, max_prefix=None, logits=True, ws=None):
        m = dfl()
        cfg, B, S = self.cfg, self.B, self.S
        dev = self.device
        mp = int(self.L.max()) if max_prefix is None else max_prefix
        if ws is None:
            ws = m.workspace(m.draft_workspace_bytes(cfg, B, mp), dev)
        out = dict(
            positions=torch.empty((B, S), dtype=torch.int32, device=dev),
            slots=torch.empty((B, S), dtype=torch.int32, device=dev),
            candidates=torch.empty((B, S), dtype=torch.int32, device=dev),
            block_ids=torch.empty((B, S), dtype=torch.int32, device=dev),
            logits=torch.empty((B, S - 1, cfg.vocab), dtype=synth._DT[cfg.act_dtype],
                               device=dev) if logits else None)
        cw = self.c_weights()
        m.dflash_draft_block(cfg, cw, self.cache, self.anchor.to(dev), self.L.to(dev),
                             self.pt.to(dev), mp, out["positions"], out["slots"],
                             out["candidates"], ws, block_ids=out["block_ids"],
                             logits=out["logits"])
        torch.cuda.synchronize()
        return out

    def inject(self, feats, positions, slots, valid=None, n_req=None, rows_per_req=None, ws=None):
        m = dfl()
        dev = self.device
        T = feats.shape[0]
        if n_req is None:
            n_req, rows_per_req = 1, T
        if ws is None:
            ws = m.workspace(m.context_workspace_bytes(self.cfg, T), dev)
        cw = self.c_weights()
        m.dflash_project_context(self.cfg, cw, self.cache, feats.to(dev), positions.to(dev),
                                 slots.to(dev), None if valid is None else valid.to(dev), n_req,
                                 rows_per_req, ws)
        torch.cuda.synchronize()


def _to(W, device):
    out = {k: (None if v is None else v.to(device)) for k, v in W.items() if k != "layers"}
    out["layers"] = [None if Lw is None else {k: v.to(device) for k, v in Lw.items()}
                     for Lw in W["layers"]]
    return out


# ------------------------------------------------------------------ metrics
def logits_row_rel_err(gpu, orc):
    """max |gpu - oracle| / max |oracle| per logits row."""
    g = np.asarray(gpu, np.float64)
    o = np.asarray(orc, np.float64)
    return np.max(np.abs(g - o), axis=-1) / np.max(np.abs(o), axis=-1)


def top2_margin(orc):
    s = np.sort(np.asarray(orc, np.float64), axis=-1)
    return s[..., -1] - s[..., -2]


def argmax_checked_rows(orc, margin):
    """Rows whose oracle top-2 margin exceeds `margin` on the scale the logits
    tolerance is stated on (a fraction of the row's max |oracle logit|): a
    path within a relative error bound e of that scale can reorder any two
    logits closer than 2 e of it, so its argmax must agree wherever the
    margin exceeds 2 e (5e-2 > 2 x 2e-2 for bf16; 1e-3 > 2 x 1e-4 for fp32)."""
    o = np.asarray(orc, np.float64)
    return top2_margin(o) > margin * np.max(np.abs(o), axis=-1)


def e4m3_spacing(x):
    """Distance between adjacent E4M3 values around |x|."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.exp2(e - 3)
