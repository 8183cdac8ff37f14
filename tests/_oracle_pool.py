"""Run the fp64 oracle head by head in a thread pool, for full-size parity tests.

The oracle is applied unchanged to one head at a time; numpy releases the interpreter lock
inside its matrix products and exponentials, so the heads run side by side, each with one
BLAS thread.  The pool is sized to the cores this process may use, at most 16.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def by_heads(fn, q, k, v, *args, heads=None, **kwargs):
    """Stack ``fn(q[:, h:h+1], k[:, h:h+1], v[:, h:h+1], *args, **kwargs)[:, 0]`` over heads
    along axis 1 (``fn`` returns [rows, 1, d])."""
    heads = list(range(q.shape[1])) if heads is None else [int(h) for h in heads]

    def one(h):
        return fn(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], *args, **kwargs)[:, 0]

    with threadpool_limits(1):
        with ThreadPoolExecutor(workers()) as ex:
            outs = list(ex.map(one, heads))
    return np.stack(outs, axis=1)
