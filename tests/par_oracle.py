"""Row-parallel calls of the CPU oracle for full-size parity checks (test infrastructure).

The oracle stays the plain single-threaded C code: this only splits the output rows of one
product into chunks, calls the oracle on each chunk from a thread pool (ctypes releases the
interpreter lock during a call) and joins the chunks in row order.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

WORKERS = max(1, min(16, os.cpu_count() or 1))


def _split(rows):
    rows = np.asarray(rows, dtype=np.int64)
    return [c for c in np.array_split(rows, WORKERS * 4) if c.size]


def _join(parts, axis):
    return (np.concatenate([p[0] for p in parts], axis=axis),
            np.concatenate([p[1] for p in parts], axis=axis))


def gemv_batched(qweight, scales, X, K, rows):
    """oracle.gemv_batched over `rows`, as (Y [M][rows], mag [M][rows])."""
    with ThreadPoolExecutor(WORKERS) as ex:
        parts = list(ex.map(lambda r: oracle.gemv_batched(qweight, scales, X, K, rows=r),
                            _split(rows)))
    return _join(parts, -1)


def moe_gemv_batched(qweight, scales, ids, X, K, rows):
    """oracle.moe_gemv_batched over `rows`, as (Y [M][topk][rows], mag)."""
    with ThreadPoolExecutor(WORKERS) as ex:
        parts = list(ex.map(lambda r: oracle.moe_gemv_batched(qweight, scales, ids, X, K, rows=r),
                            _split(rows)))
    return _join(parts, -1)


def quantize_pack(w_bf16, K, rows):
    """oracle.quantize_pack of the rows `rows` of w_bf16, as (qweight, scales) in that order."""
    with ThreadPoolExecutor(WORKERS) as ex:
        parts = list(ex.map(lambda r: oracle.quantize_pack(w_bf16[r], K), _split(rows)))
    return _join(parts, 0)
