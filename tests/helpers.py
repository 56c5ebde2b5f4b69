"""Test-harness plumbing: tensor conversion and layout changes only."""
import numpy as np
import torch


def to_np(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float32).numpy() if t.is_floating_point() \
            else t.detach().cpu().numpy()
    return np.asarray(t)


def np_weights(W):
    out = {k: to_np(v) for k, v in W.items() if k != "layers"}
    out["layers"] = [None if Lw is None else {k: to_np(v) for k, v in Lw.items()}
                     for Lw in W["layers"]]
    return out


def paged_to_slots(pool, page_size, transposed=False):
    """K pool [pages, nkv, P, D] (or a V pool [pages, nkv, D, P] when
    transposed) -> [pages * P, nkv, D] (slot = page * P + offset)."""
    a = pool if isinstance(pool, np.ndarray) else to_np(pool)
    if transposed:
        a = a.transpose(0, 1, 3, 2)
    pages, nkv, P, D = a.shape
    assert P == page_size
    return a.transpose(0, 2, 1, 3).reshape(pages * P, nkv, D)
