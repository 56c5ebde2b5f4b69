"""Working precision of the oracle's floating-point arithmetic (TEST
INFRASTRUCTURE ONLY).

Every parity check and pin runs the oracle in fp64, the default.  The one
other setting, fp32, exists so that the benchmark's CPU baseline can time the
oracle at the precision a CPU implementation of the path would compute in;
the steps and their order are the same in both settings, only the dtype the
arrays are held in changes.

    with working_precision("f32"):
        oracle.draft_block(...)
"""
from contextlib import contextmanager

import numpy as np

_DTYPES = {"f64": np.float64, "f32": np.float32}
_current = [np.float64]


def real():
    """The dtype floating-point arrays are computed in."""
    return _current[0]


@contextmanager
def working_precision(name):
    """Compute in `name` ("f64" or "f32") inside the block; fp64 again after."""
    if name not in _DTYPES:
        raise ValueError(f"unknown working precision {name!r}")
    prev = _current[0]
    _current[0] = _DTYPES[name]
    try:
        yield
    finally:
        _current[0] = prev
