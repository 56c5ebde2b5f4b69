"""GPU parity of the device-side cache reservation (dflash_reserve_pages,
dflash_release_pages) against the oracle: page tables, page counts, the free
stack and the status are integers and must match bit for bit, over several
cycles of reservations, commits and releases."""
import numpy as np
import pytest
import torch

from oracle.reserve import reserve as o_reserve, release as o_release

pytestmark = pytest.mark.gpu


def dfl():
    import block_diffusion_drafter_rmsnorm_amd as m
    return m


def _state(B, maxp, n_pool, seed):
    rng = np.random.default_rng(seed)
    stack = rng.permutation(n_pool).astype(np.int32)
    pt = np.full((B, maxp), -1, np.int32)
    n = np.zeros(B, np.int32)
    return rng, stack, pt, n


def _dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrs]


@pytest.mark.parametrize("B,S,P,maxp,n_pool", [(7, 16, 16, 40, 300), (300, 8, 16, 12, 1100),
                                               (33, 4, 32, 6, 120)])
def test_reserve_release_parity_over_cycles(B, S, P, maxp, n_pool):
    m = dfl()
    rng, stack, pt, n = _state(B, maxp, n_pool, B)
    top = n_pool
    L = rng.integers(0, 60, B).astype(np.int32)
    d_pt, d_n, d_stack = _dev(pt, n, stack)
    d_top = torch.tensor([top], dtype=torch.int32, device="cuda")
    d_st = torch.zeros(1, dtype=torch.int32, device="cuda")
    saw_shortage = False
    for cycle in range(12):
        d_L, = _dev(L)
        m.dflash_reserve_pages(d_L, S, P, d_pt, d_n, d_stack, d_top, d_st)
        pt, n, stack, top, st = o_reserve(L, S, P, pt, n, stack, top)
        torch.cuda.synchronize()
        assert int(d_st.item()) == st, cycle
        assert int(d_top.item()) == top, cycle
        assert np.array_equal(d_n.cpu().numpy(), n), cycle
        assert np.array_equal(d_pt.cpu().numpy(), pt), cycle
        assert np.array_equal(d_stack.cpu().numpy()[:top], stack[:top]), cycle
        saw_shortage |= st != 0
        L = (L + rng.integers(1, S + 1, B)).astype(np.int32)
        done = (rng.random(B) < 0.15).astype(np.int32)
        d_mask, = _dev(done)
        m.dflash_release_pages(d_mask, d_pt, d_n, d_stack, d_top)
        pt, n, stack, top = o_release(done, pt, n, stack, top)
        torch.cuda.synchronize()
        assert int(d_top.item()) == top
        assert np.array_equal(d_n.cpu().numpy(), n)
        assert np.array_equal(d_stack.cpu().numpy()[:top], stack[:top])
        L[done == 1] = rng.integers(0, 30, int(done.sum()))
    if B == 300:
        assert saw_shortage                 # the pool runs out partway through a chunk
