"""Oracle of the pipeline search's Pareto filter.

Test infrastructure: only the tests, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use anything under oracle/.  The Pareto set of the
search ("Beyond Compression Ratio: High-Throughput KV Compression for
Disaggregated LLM Serving", Sec. 4.2) written as its definition: a point is
kept when no other point is at most as large in every measured quantity and
smaller in one.
"""
from __future__ import annotations


def dominates(q, p, keys):
    return all(q[k] <= p[k] for k in keys) and any(q[k] < p[k] for k in keys)


def pareto_front(points, keys=("stream_bytes", "enc_ms", "dec_ms")):
    """Indices of the non-dominated points, in index order."""
    return [i for i, p in enumerate(points)
            if not any(dominates(q, p, keys) for j, q in enumerate(points) if j != i)]
