"""Pipeline search (FastKVComp Sec. 4.2) host logic: the candidate list and
the Pareto filter against the definition in the oracle.  CPU only."""
import os
import random
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "oracle"))
sys.path.insert(0, ROOT)

import kvc_search_oracle as PO  # noqa: E402
from kv_cache_compression_kvc_amd import search as S  # noqa: E402


def test_pareto_oracle_worked_example():
    pts = [{"stream_bytes": a, "enc_ms": b, "dec_ms": c}
           for a, b, c in [(3, 1, 1), (1, 3, 3), (2, 2, 2), (3, 3, 3), (1, 3, 3), (2, 1, 5)]]
    # (3, 3, 3) is dominated by (2, 2, 2); the two equal points dominate neither
    assert PO.pareto_front(pts) == [0, 1, 2, 4, 5]


def test_pareto_matches_definition():
    rng = random.Random(11)
    for trial in range(300):
        n = rng.randint(1, 40)
        grid = rng.choice([3, 10, 1000])        # coarse grids give ties
        pts = [{"stream_bytes": rng.randrange(grid), "enc_ms": rng.randrange(grid) / 7,
                "dec_ms": rng.randrange(grid) / 3} for _ in range(n)]
        assert sorted(S.pareto_front(pts)) == PO.pareto_front(pts), trial
        for q in pts:
            q["rel_err"] = rng.randrange(grid) / 11
        assert sorted(S.pareto_front(pts, S.SEARCH_KEYS)) == PO.pareto_front(pts, S.SEARCH_KEYS), trial


def test_candidates():
    c = S.candidate_pipelines(3)
    assert c[0] == ()
    assert len(c) == 1 + 11 * 4 + 11 * 11 * 4
    assert all(p[-1].startswith("RZE_") for p in c[1:])
    assert ("TUPL8_1", "BIT_8", "RZE_2") in c and ("TUPL8_1", "RZE_2") in c
    assert len(set(c)) == len(c)
