"""Row-chunked, thread-parallel calls of oracle functions (test infrastructure).

The oracle's quantizers act row by row and its QDQ product is separable over
output columns, so a full-size check can hand the oracle row chunks and
concatenate what it returns: the same function, the same arithmetic on every
element, only the calls are split. NumPy releases the GIL inside its array
kernels, so the chunks run in parallel threads. BLAS is held to one thread per
call while the pool runs, so that the threads do not oversubscribe the cores.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

WORKERS = max(1, min(12, os.cpu_count() or 1))
_pool = ThreadPoolExecutor(max_workers=WORKERS)


def _blas_limit(n):
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=n, user_api="blas")
    except Exception:  # pragma: no cover - threadpoolctl is optional
        import contextlib
        return contextlib.nullcontext()


def _chunks(n, chunk):
    return [(i, min(n, i + chunk)) for i in range(0, n, chunk)]


def map_rows(fn, *arrays, chunk=2048):
    """fn(*[a[i:j] for a in arrays]) over row chunks, outputs concatenated along axis 0.

    ``fn`` may return one array or a tuple of arrays (each row-aligned)."""
    n = arrays[0].shape[0]
    parts = _chunks(n, chunk)
    with _blas_limit(1):
        outs = list(_pool.map(lambda ij: fn(*[a[ij[0]:ij[1]] for a in arrays]), parts))
    if isinstance(outs[0], tuple):
        return tuple(np.concatenate([o[t] for o in outs], axis=0) for t in range(len(outs[0])))
    return np.concatenate(outs, axis=0)


def map_cols(fn, *w_arrays, chunk=1024):
    """fn(*[w[i:j] for w in w_arrays]) -> [rows, j - i] blocks, joined along axis 1.

    For products y = A W^T: the weight's rows are y's columns."""
    n = w_arrays[0].shape[0]
    parts = _chunks(n, chunk)
    with _blas_limit(1):
        outs = list(_pool.map(lambda ij: fn(*[w[ij[0]:ij[1]] for w in w_arrays]), parts))
    return np.concatenate(outs, axis=1)
