"""No entry point reads a workspace value it did not write in the same call:
every call that takes a workspace gives bitwise the same outputs when the
workspace starts zeroed and when it starts filled with 0xFF bytes (NaN as
fp32 and bf16, -1 as int32).  Draft pass (argmax and selector), injection,
accept from logits and the sampled verify, on small shapes through the C ABI."""
import numpy as np
import pytest
import torch

from workloads import synth
from workloads.configs import get_workload
from tests.gpu_harness import Setup, dfl

pytestmark = pytest.mark.gpu


def _both(run, nbytes):
    """run(ws) -> list of output tensors, with a zeroed and a 0xFF workspace."""
    m = dfl()
    outs = []
    for fill in (0, 0xFF):
        ws = m.workspace(nbytes)
        ws.fill_(fill)
        outs.append([t.clone() for t in run(ws)])
        torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["small_bf16", "small_swa_fp8", "tiny_f32", "small_bf16_wide"])
def test_draft_and_injection_ignore_workspace_contents(name):
    m = dfl()
    wl = get_workload(name)
    cfg = wl.cfg
    st = Setup(wl)
    B, S = st.B, st.S
    mp = int(st.L.max())
    print(f"[poison] {name}: draft pass and injection", flush=True)

    def draft(ws):
        out = st.draft(max_prefix=mp, ws=ws)
        return [out["positions"], out["slots"], out["candidates"], out["logits"]]
    _both(draft, m.draft_workspace_bytes(cfg, B, mp))

    T = 77
    feats = synth.features(T, cfg, 9, "poison_feats", "cpu")
    g = torch.Generator().manual_seed(9)
    pos = torch.randint(0, 5000, (T,), generator=g, dtype=torch.int32)
    slots = torch.randperm(st.num_pages * cfg.page_size, generator=g)[:T].to(torch.int32)
    valid = torch.tensor([3, 16, 0, 11], dtype=torch.int32)  # a prefix-valid 4 x 19 grid

    def inject(ws):
        st.inject(feats[:76], pos[:76], slots[:76], valid, 4, 19, ws=ws)
        return [t.clone() for t in st.cache.k + st.cache.v]
    _both(inject, m.context_workspace_bytes(cfg, 76))

    # 48 rows: the narrow K/V store's fp32 partials live in the workspace
    valid3 = torch.tensor([5, 16, 0], dtype=torch.int32)

    def inject_narrow(ws):
        st.inject(feats[:48], pos[:48], slots[:48], valid3, 3, 16, ws=ws)
        return [t.clone() for t in st.cache.k + st.cache.v]
    _both(inject_narrow, m.context_workspace_bytes(cfg, 48))


def test_selector_and_verify_ignore_workspace_contents():
    m = dfl()
    wl = get_workload("small_bf16")
    cfg = wl.cfg
    st = Setup(wl)
    B, S, V, H = st.B, st.S, cfg.vocab, cfg.hidden
    mp = int(st.L.max())
    r, K = 32, 8
    g = torch.Generator().manual_seed(4)
    A = (torch.randn((V, r), generator=g) * 0.3).to(torch.bfloat16).cuda()
    Bt = (torch.randn((V, r), generator=g) * 0.3).to(torch.bfloat16).cuda()
    Wh = (torch.randn((r, H), generator=g) * 0.02).to(torch.bfloat16).cuda()
    sel = m.Selector(A, Bt, Wh, K)
    uni = torch.rand((B, S - 1), generator=g).cuda()
    cw = st.c_weights()
    dev = "cuda"
    print("[poison] selector pass", flush=True)

    def selector(ws):
        pos = torch.empty((B, S), dtype=torch.int32, device=dev)
        sl, cand = torch.empty_like(pos), torch.empty_like(pos)
        cid = torch.empty((B, S - 1, K), dtype=torch.int32, device=dev)
        q = torch.empty((B, S - 1, K), dtype=torch.float32, device=dev)
        m.dflash_draft_block_selector(cfg, cw, st.cache, sel, st.anchor.to(dev), st.L.to(dev),
                                      st.pt.to(dev), mp, pos, sl, cand, cid, q, ws, uniforms=uni)
        return [pos, sl, cand, cid, q]
    _both(selector, m.selector_workspace_bytes(cfg, sel, B, mp))

    Bv, Sv, Vv = 5, 8, 4099
    cand = torch.randint(0, Vv, (Bv, Sv), generator=g, dtype=torch.int32).cuda()
    tl = (torch.randn((Bv, Sv, Vv), generator=g) * 2).to(torch.bfloat16).cuda()
    dl = (torch.randn((Bv, Sv - 1, Vv), generator=g) * 2).to(torch.bfloat16).cuda()
    un = torch.rand((Bv, Sv), generator=g).cuda()
    L = torch.randint(0, 1000, (Bv,), generator=g, dtype=torch.int32).cuda()
    print("[poison] accept from logits, sampled verify", flush=True)

    def outs():
        return [torch.empty(Bv, dtype=torch.int32, device=dev) for _ in range(4)] + \
            [torch.empty((Bv, Sv), dtype=torch.int32, device=dev)]

    def accept_logits(ws):
        o = outs()
        m.dflash_accept_logits(cand, tl, L, o[0], o[1], o[4], o[2], o[3], ws)
        return o
    _both(accept_logits, m.accept_logits_workspace_bytes(Bv, Sv, Vv))

    def sampling(ws):
        o = outs()
        m.dflash_accept_sampling(cand, tl, un, L, o[0], o[1], o[4], o[2], o[3], ws,
                                 target_temperature=0.8, draft_logits=dl, draft_temperature=1.1)
        return o
    _both(sampling, m.accept_sampling_workspace_bytes(Bv, Sv, Vv, True))
