"""Runs CPU-oracle calls over chunks of requests on a pool of host threads.

Requests are independent in every oracle function (each takes the request
ids its uniforms are drawn for), so a batch can be split into chunks and the
chunk results concatenated along the request axis.  ctypes releases the GIL
for the duration of each C call, so the chunks run on separate cores.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os

import numpy as np


def workers() -> int:
    """Host threads to use: every core, at most 16 (one GPU's share of a
    shared host)."""
    return max(1, min(16, os.cpu_count() or 1))


def merge(parts):
    """Concatenates a list of result dataclasses along their first axis."""
    cls = type(parts[0])
    out = {}
    for f in dataclasses.fields(cls):
        vals = [getattr(p, f.name) for p in parts]
        out[f.name] = None if vals[0] is None else np.concatenate(vals, axis=0)
    return cls(**out)


def map_requests(fn, req, chunk: int = 8, nthreads: int | None = None):
    """fn(list of request ids) -> result dataclass; returns the merged result
    for `req` in order."""
    req = list(req)
    chunks = [req[i:i + chunk] for i in range(0, len(req), chunk)]
    n = nthreads or workers()
    if n == 1 or len(chunks) == 1:
        parts = [fn(c) for c in chunks]
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=n) as ex:
            parts = list(ex.map(fn, chunks))
    return merge(parts)
