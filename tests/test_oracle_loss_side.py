"""Pins for the oracle's loss-side steps: token selection, the cross-entropy / LM-head backward and
the embedding gradient.  Brute force from the definitions, torch.autograd (CPU, float64) of the
masked loss, central finite differences, and the input generator's own selection rule."""
import numpy as np
import pytest
import torch

import oracle
import synth


# ------------------------------------------------------------------------------------------------
# selection
# ------------------------------------------------------------------------------------------------


def _brute_keep(score, n_keep):
    """Token t is kept iff fewer than n_keep tokens rank above it; u ranks above t when u is a
    number and t is NaN, or both are numbers (or both NaN) and u's score is larger, or equal with
    u earlier."""
    s = [float(v) for v in score]
    M = len(s)

    def above(u, t):
        nu, nt = s[u] != s[u], s[t] != s[t]
        if nu != nt:
            return nt
        if nu or s[u] == s[t]:
            return u < t
        return s[u] > s[t]

    return np.array([1 if sum(above(u, t) for u in range(M) if u != t) < n_keep else 0
                     for t in range(M)], np.uint8)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_select_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    M = 37
    # few distinct values (many ties), signed zeros, infinities and NaNs
    score = rng.choice(np.array([-1.5, -0.0, 0.0, 0.25, 2.0, np.inf, -np.inf, np.nan]), size=M)
    for n_keep in (0, 1, 5, 18, 36, 37):
        got = oracle.select_topk(score, n_keep)
        assert got.sum() == n_keep
        np.testing.assert_array_equal(got, _brute_keep(score, n_keep))


def test_select_topk_nested_and_matches_input_recipe():
    """Masks for growing n_keep are nested, and the rule reproduces the input generator's global
    top-k on its LogNormal scores (independent code)."""
    M, seed = 8192, 0
    score = np.exp(synth.rng_for(seed, "score").standard_normal(M))
    prev = np.zeros(M, np.uint8)
    for r in (60, 40, 20, 0):
        keep = oracle.select_topk(score, M - synth.n_filtered(M, r))
        assert np.all(keep >= prev)
        np.testing.assert_array_equal(keep, synth.make_keep(M, r, seed))
        prev = keep


# ------------------------------------------------------------------------------------------------
# cross-entropy and LM head
# ------------------------------------------------------------------------------------------------


def _masked_ce(z, y, keep, scale):
    lz = torch.nn.functional.cross_entropy(z, y, reduction="none")
    return scale * (lz * keep).sum()


def test_ce_logits_bwd_autograd_fd():
    rng = np.random.default_rng(3)
    M, V = 11, 17
    z = rng.standard_normal((M, V)) * 3
    y = rng.integers(0, V, M)
    keep = (rng.random(M) < 0.6).astype(np.uint8)
    scale = 1.0 / max(int(keep.sum()), 1)
    got = oracle.ce_logits_bwd(z, y, keep, scale)
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    _masked_ce(zt, torch.tensor(y), torch.tensor(keep, dtype=torch.float64), scale).backward()
    np.testing.assert_allclose(got, zt.grad.numpy(), rtol=1e-12, atol=1e-14)
    # central finite differences on a few entries
    h = 1e-6

    def f(zz):
        return float(_masked_ce(torch.tensor(zz), torch.tensor(y),
                                torch.tensor(keep, dtype=torch.float64), scale))

    for i in range(0, M * V, 7):
        zp, zm = z.copy(), z.copy()
        zp.flat[i] += h
        zm.flat[i] -= h
        assert abs((f(zp) - f(zm)) / (2 * h) - got.flat[i]) <= 1e-7
    # softmax - onehot sums to zero over a kept row; filtered rows are exactly zero
    np.testing.assert_allclose(got.sum(axis=1), 0.0, atol=1e-12)
    assert np.all(got[keep == 0] == 0.0)


def test_ce_ignored_labels_match_torch_ignore_index():
    rng = np.random.default_rng(6)
    M, V = 12, 10
    z = rng.standard_normal((M, V))
    y = rng.integers(0, V, M)
    y[[1, 4, 9]] = -100
    keep = np.ones(M, np.uint8)
    keep[2] = 0
    got = oracle.ce_logits_bwd(z, y, keep, 0.5)
    zt = torch.tensor(z, requires_grad=True)
    lz = torch.nn.functional.cross_entropy(zt, torch.tensor(y), reduction="none", ignore_index=-100)
    (0.5 * (lz * torch.tensor(keep, dtype=torch.float64)).sum()).backward()
    np.testing.assert_allclose(got, zt.grad.numpy(), rtol=1e-12, atol=1e-14)
    assert np.all(got[[1, 2, 4, 9]] == 0.0)


def test_lm_head_bwd_autograd():
    rng = np.random.default_rng(4)
    M, H, V = 13, 8, 19
    h = rng.standard_normal((M, H))
    w = rng.standard_normal((V, H)) * 0.3
    y = rng.integers(0, V, M)
    keep = (rng.random(M) < 0.5).astype(np.uint8)
    keep[0] = 1
    scale = 0.37
    out = oracle.lm_head_bwd(h @ w.T, y, h, w, keep, scale)
    ht = torch.tensor(h, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    _masked_ce(ht @ wt.T, torch.tensor(y), torch.tensor(keep, dtype=torch.float64), scale).backward()
    np.testing.assert_allclose(out["dh"], ht.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(out["dw_lm"], wt.grad.numpy(), rtol=1e-11, atol=1e-13)
    assert np.all(out["dh"][keep == 0] == 0.0)


# ------------------------------------------------------------------------------------------------
# embedding
# ------------------------------------------------------------------------------------------------


def test_embedding_bwd_brute_force_and_autograd():
    rng = np.random.default_rng(5)
    M, H, V = 40, 6, 9
    dx = rng.standard_normal((M, H))
    ids = rng.integers(0, V, M)
    ids[:5] = 3  # a frequent token
    ids[7], ids[8] = -1, V + 2  # no embedding row: skipped
    keep = (rng.random(M) < 0.6).astype(np.uint8)
    keep[7] = keep[8] = 1
    got = oracle.embedding_bwd(dx, ids, keep, V)
    ref = np.zeros((V, H))
    for t in range(M):
        if keep[t] and 0 <= ids[t] < V:
            for j in range(H):
                ref[ids[t], j] += dx[t, j]
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    E = torch.tensor(rng.standard_normal((V, H)), requires_grad=True)
    ok = (ids >= 0) & (ids < V)
    x = torch.nn.functional.embedding(torch.tensor(np.where(ok, ids, 0)), E)
    w = torch.tensor(keep * ok, dtype=torch.float64)[:, None]
    (x * torch.tensor(dx) * w).sum().backward()
    np.testing.assert_allclose(got, E.grad.numpy(), rtol=1e-12, atol=1e-12)
    # ids no kept token uses get an exactly zero row
    used = set(ids[(keep != 0) & ok].tolist())
    for v in range(V):
        if v not in used:
            assert np.all(got[v] == 0.0)


# ------------------------------------------------------------------------------------------------
# per-token loss (the score token selection ranks by) and masked vocabulary entries
# ------------------------------------------------------------------------------------------------


def test_ce_loss_matches_torch_and_brute_force():
    import math
    rng = np.random.default_rng(7)
    M, V = 19, 23
    z = rng.standard_normal((M, V)) * 3
    y = rng.integers(0, V, M)
    y[[2, 11]] = -100
    got = oracle.ce_loss(z, y)
    ref = torch.nn.functional.cross_entropy(torch.tensor(z), torch.tensor(y), reduction="none",
                                            ignore_index=-100).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
    for t in range(M):  # the definition, one token at a time
        want = 0.0 if not 0 <= y[t] < V else math.log(sum(math.exp(v) for v in z[t])) - z[t, y[t]]
        assert abs(got[t] - want) <= 1e-12 * max(1.0, abs(want))
    # labels past the vocabulary also mean "no target"
    y2 = y.copy()
    y2[5] = V + 3
    assert oracle.ce_loss(z, y2)[5] == 0.0
    # a constant shift of a row's logits leaves its loss unchanged; the loss is never negative
    np.testing.assert_allclose(oracle.ce_loss(z + 17.0, y), got, rtol=0, atol=1e-11)
    assert np.all(got >= 0.0)


def test_masked_logits_minus_inf():
    """Whole runs of -inf logits (masked vocabulary entries) drop out of the softmax: the loss and
    its gradient equal those of the row without them (and torch's, which handles -inf the same)."""
    rng = np.random.default_rng(8)
    M, V = 6, 40
    z = rng.standard_normal((M, V)) * 2
    z[0, :16] = -np.inf       # two 8-wide blocks at the start of the row
    z[1, 8:32] = -np.inf      # three blocks in the middle
    z[2, 32:] = -np.inf       # the tail
    y = np.array([20, 3, 5, 7, 9, 11])
    keep = np.ones(M, np.uint8)
    g = oracle.ce_logits_bwd(z, y, keep, 1.0)
    zt = torch.tensor(z, requires_grad=True)
    torch.nn.functional.cross_entropy(zt, torch.tensor(y), reduction="sum").backward()
    np.testing.assert_allclose(g, zt.grad.numpy(), rtol=1e-12, atol=1e-14)
    assert np.all(g[np.isinf(z)] == 0.0)
    loss = oracle.ce_loss(z, y)
    for t in range(3):
        fin = np.isfinite(z[t])
        keep_cols = np.flatnonzero(fin)
        want = oracle.ce_loss(z[t:t + 1, fin], [int(np.searchsorted(keep_cols, y[t]))])[0]
        assert abs(loss[t] - want) <= 1e-12


def test_oracle_float32_precision_close_to_float64():
    """The float32 run of the oracle (the benchmark's CPU baseline) agrees with the float64 one
    on a small layer within 1e-4 of each gradient's largest entry."""
    cfg = synth.get_config("small_llama")
    inp = synth.make_layer_inputs(cfg)
    args = (cfg, synth.floats(inp["weights"]), synth.floats(inp["saved"]),
            synth.bf16_bits_to_f32(inp["dy"]), inp["keep"])
    ref = oracle.layer_bwd(*args)
    with oracle.precision(np.float32):
        got = oracle.layer_bwd(*args)
    for k, r in ref.items():
        assert got[k].dtype == np.float32, k
        err = np.abs(got[k].astype(np.float64) - r).max() / np.abs(r).max()
        assert err <= 1e-4, (k, err)
    assert oracle.layer_bwd(*args)["dx"].dtype == np.float64  # the switch is scoped
