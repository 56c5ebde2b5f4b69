"""The oracle's fp32 timing setting (oracle.precision): the same steps in
fp32, used only to time the oracle as a CPU baseline.  It must compute in
fp32 inside the block, return to fp64 after it (also after an error), and
agree with the fp64 oracle to fp32 rounding: logits within 1e-4 of the row
maximum and the same draft ids wherever the fp64 top-2 gap is clear."""
import numpy as np
import pytest

import oracle
from oracle.precision import real, working_precision
from workloads import synth
from workloads.configs import TINY
from tests.helpers import np_weights


def _run(cfg, W, seed=3):
    L = np.array([37, 5, 60])
    pt, npages = synth.page_table(__import__("torch").tensor(L), cfg, seed, 32)
    pt = pt.numpy()
    cache = oracle.OracleCache(cfg, npages * cfg.page_size)
    P = cfg.page_size
    for r, Lr in enumerate(L):
        pos = np.arange(Lr)
        f = synth.features(int(Lr), cfg, 10 + r).numpy()
        oracle.project_context(cfg, W, cache, f, pos, pt[r, pos // P] * P + pos % P)
    return cache, oracle.draft_block(cfg, W, cache, [4, 9, 11], L, pt)


def test_f32_setting_computes_in_f32_and_matches_f64():
    cfg = TINY
    W = np_weights(synth.weights(cfg, 0, "cpu"))
    c64, d64 = _run(cfg, W)
    assert real() is np.float64 and d64["logits"].dtype == np.float64
    with working_precision("f32"):
        assert real() is np.float32
        c32, d32 = _run(cfg, W)
    assert real() is np.float64
    assert d32["logits"].dtype == np.float32 and c32.k[0].dtype == np.float32
    lg64 = d64["logits"]
    err = np.abs(d32["logits"] - lg64).max(-1) / np.abs(lg64).max(-1)
    assert err.max() < 1e-4, err.max()
    srt = np.sort(lg64, -1)
    clear = (srt[..., -1] - srt[..., -2]) > 1e-3 * np.abs(lg64).max(-1)
    assert clear.sum() >= 6             # of 9 rows
    assert np.array_equal(d32["draft_ids"][clear], d64["draft_ids"][clear])


def test_setting_restored_after_an_error():
    with pytest.raises(RuntimeError):
        with working_precision("f32"):
            raise RuntimeError("inside")
    assert real() is np.float64
    with pytest.raises(ValueError):
        with working_precision("f16"):
            pass
