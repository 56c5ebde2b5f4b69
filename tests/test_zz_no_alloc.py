"""dflash_draft_block_noalloc (the draft pass on the library's fixed scratch
array, for callers that cannot allocate) against dflash_draft_block with a
caller workspace, through the C ABI: two calls in a row on one device, the
second on a smaller input (fewer requests, shorter prefixes), each compared
with the workspace entry point on the same inputs.  Both run the same kernels
in the same launch configuration, so every output (ids, positions, slots,
logits) must be bitwise equal."""
import pytest
import torch

from workloads.configs import get_workload
from tests.gpu_harness import Setup, dfl

pytestmark = pytest.mark.gpu


def _outs(cfg, B, S, logits_dtype):
    dev = "cuda"
    return dict(positions=torch.empty((B, S), dtype=torch.int32, device=dev),
                slots=torch.empty((B, S), dtype=torch.int32, device=dev),
                candidates=torch.empty((B, S), dtype=torch.int32, device=dev),
                block_ids=torch.empty((B, S), dtype=torch.int32, device=dev),
                logits=torch.empty((B, S - 1, cfg.vocab), dtype=logits_dtype, device=dev))


def _both(su, B, L, max_prefix):
    """The two entry points on requests 0..B-1 with prefix lengths L."""
    m = dfl()
    cfg, S = su.cfg, su.S
    ldt = torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16
    anchor = su.anchor[:B].cuda()
    Ld = L[:B].cuda()
    pt = su.pt[:B].contiguous().cuda()
    cw = su.c_weights()
    ref, got = _outs(cfg, B, S, ldt), _outs(cfg, B, S, ldt)
    ws = m.workspace(m.draft_workspace_bytes(cfg, B, max_prefix), "cuda")
    m.dflash_draft_block(cfg, cw, su.cache, anchor, Ld, pt, max_prefix, ref["positions"],
                         ref["slots"], ref["candidates"], ws, block_ids=ref["block_ids"],
                         logits=ref["logits"])
    m.dflash_draft_block_noalloc(cfg, cw, su.cache, anchor, Ld, pt, max_prefix,
                                 got["positions"], got["slots"], got["candidates"],
                                 block_ids=got["block_ids"], logits=got["logits"])
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(ref[k], got[k]), f"{k} differs (batch {B}, max prefix {max_prefix})"


@pytest.mark.parametrize("name", ["small_bf16", "small_swa_fp8", "tiny_f32"])
def test_noalloc_matches_workspace_entry_point(name):
    wl = get_workload(name)
    su = Setup(wl)
    m = dfl()
    B = su.B
    Lmax = int(su.L.max())
    assert m.draft_workspace_bytes(su.cfg, B, Lmax) <= m.draft_block_noalloc_limit()
    print(f"[noalloc] {name}: batch {B}, max prefix {Lmax}", flush=True)
    _both(su, B, su.L, Lmax)
    # second call: fewer requests and shorter prefixes (the scratch keeps the
    # first call's contents)
    B2 = max(1, B - 1)
    L2 = torch.clamp(su.L - 7, min=0).to(torch.int32)
    print(f"[noalloc] {name}: batch {B2}, max prefix {int(L2[:B2].max())}", flush=True)
    _both(su, B2, L2, int(L2[:B2].max()))
