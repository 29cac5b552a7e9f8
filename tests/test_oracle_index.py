"""Pins for the oracle's index / gather / scatter and for the synthetic selection rule (CPU)."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _brute_index(keep, B, S):
    """Brute force with explicit loops (tiny inputs only)."""
    idx, inv, cu = [], [], [0]
    for t in range(B * S):
        if keep[t]:
            inv.append(len(idx))
            idx.append(t)
        else:
            inv.append(-1)
        if (t + 1) % S == 0:
            cu.append(len(idx))
    return idx, inv, cu


def test_index_golden():
    g = json.load(open(os.path.join(GOLD, "index_tiny.json")))
    ix = oracle.build_index(np.array(g["keep"], np.uint8), g["B"], g["S"])
    assert ix["idx"].tolist() == g["idx"]
    assert ix["inv"].tolist() == g["inv"]
    assert ix["cu_seqlens"].tolist() == g["cu_seqlens"]
    assert ix["count"] == g["count"]
    assert ix["partition"].tolist() == g["partition"]


@pytest.mark.parametrize("B,S,p", [(1, 1, 0.5), (1, 7, 0.0), (1, 7, 1.0), (3, 11, 0.4), (4, 33, 0.7),
                                   (2, 64, 0.05)])
def test_index_brute_force_and_invariants(B, S, p):
    rng = np.random.default_rng(B * 1000 + S)
    keep = (rng.random(B * S) < p).astype(np.uint8)
    if p == 1.0:
        keep[:] = 1
    ix = oracle.build_index(keep, B, S)
    idx, inv, cu = _brute_index(keep, B, S)
    assert ix["idx"].tolist() == idx
    assert ix["inv"].tolist() == inv
    assert ix["cu_seqlens"].tolist() == cu
    n = ix["count"]
    assert n == int(keep.sum())
    assert np.all(np.diff(ix["idx"]) > 0)
    assert np.all(keep[ix["idx"]] == 1)
    assert np.all(ix["inv"][ix["idx"]] == np.arange(n))
    assert np.all((ix["inv"] == -1) == (keep == 0))
    assert np.all(np.diff(ix["cu_seqlens"]) >= 0) and ix["cu_seqlens"][-1] == n
    assert sorted(ix["partition"].tolist()) == list(range(B * S))


def test_nonzero_byte_means_keep():
    keep = np.array([0, 2, 255, 0, 1], np.uint8)
    assert oracle.build_index(keep, 1, 5)["idx"].tolist() == [1, 2, 4]


def test_gather_scatter_round_trip_bitwise():
    rng = np.random.default_rng(3)
    M, C = 50, 24
    src = rng.integers(0, 2 ** 16, size=(M, C), dtype=np.uint16)
    keep = (rng.random(M) < 0.6).astype(np.uint8)
    ix = oracle.build_index(keep, 1, M)
    g = oracle.gather_rows(src, ix["idx"])
    for c, t in enumerate(ix["idx"]):
        assert np.array_equal(g[c], src[t])
    s = oracle.scatter_rows(g, ix["idx"], M)
    assert np.array_equal(s[keep == 1], src[keep == 1])
    assert np.all(s[keep == 0] == 0)


@pytest.mark.parametrize("name,expect", [("linear_fp32", 154), ("tinyllama", 4916), ("qwen25", 4916),
                                         ("phi15", 4916), ("tinyllama_22l", 4916)])
def test_selection_counts(name, expect):
    cfg = synth.get_config(name)
    keep = synth.make_keep(cfg.M, cfg.r_pct, cfg.seed)
    assert int(keep.sum()) == expect


def test_phi_sweep_counts_and_nesting():
    M = synth.get_config("phi15").M
    keeps = [synth.make_keep(M, r, 0) for r in (0, 20, 40, 60)]
    assert [int(k.sum()) for k in keeps] == [8192, 6554, 4916, 3277]
    for hi, lo in zip(keeps[1:], keeps[:-1]):
        assert np.all(hi <= lo)  # a larger filter ratio keeps a subset


def test_selection_keeps_highest_scores():
    M, r = 1000, 40
    keep = synth.make_keep(M, r, 5)
    score = np.exp(synth.rng_for(5, "score").standard_normal(M))
    assert score[keep == 1].min() >= score[keep == 0].max()
