"""Pins for the oracle's filtered attention backward and whole-layer / stack backward (CPU).

Independent routes used: a hand-derived closed form (golden), torch.autograd of explicit surrogate
forwards (tests/torch_ref.py), central finite differences of a NumPy surrogate, and the special cases
r = 0 and suffix masks, where the method coincides with the ordinary gradient."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import torch_ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")

TINY_LLAMA = synth.LayerShape("tiny_llama", "llama", B=2, S=6, H=8, nq=4, nkv=2, d=4, I=12, rot=4,
                              rope_base=1.0e4, eps=1e-5)
TINY_PHI = synth.LayerShape("tiny_phi", "phi", B=2, S=6, H=8, nq=2, nkv=2, d=4, I=12, rot=2,
                            rope_base=1.0e4, eps=1e-5)
# kept query 2 attends filtered key 1, etc.: a non-suffix mask
KEEP = np.array([1, 0, 1, 1, 0, 1, 0, 1, 1, 0, 1, 1], np.uint8)
SUFFIX = np.array([1, 1, 1, 1, 0, 0, 1, 1, 1, 0, 0, 0], np.uint8)


def test_attention_golden_two_tokens():
    g = json.load(open(os.path.join(GOLD, "attn_two_token.json")))
    a = {k: np.array(g[k], np.float64)[:, None] for k in ("q", "k", "v", "o", "dout")}
    lse = np.array(g["lse"])[:, None]
    for mode in ("filtered", "full_d"):
        dq, dk, dv = oracle.attention_bwd(a["q"], a["k"], a["v"], a["o"], lse, a["dout"], g["keep"],
                                          1, 2, 1, 1, 1, mode=mode)
        np.testing.assert_allclose(dq[:, 0], g[mode]["dq"], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(dk[:, 0], g[mode]["dk"], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(dv[:, 0], g[mode]["dv"], rtol=1e-14, atol=1e-15)
    _, _, dv = oracle.attention_bwd(a["q"], a["k"], a["v"], a["o"], lse, a["dout"], g["keep"],
                                    1, 2, 1, 1, 1, mode="loss_only")
    np.testing.assert_allclose(dv[:, 0], g["loss_only_dv"], rtol=1e-14)


def _attn_case(seed=0, B=2, S=6, nq=4, nkv=2, d=4):
    rng = np.random.default_rng(seed)
    M = B * S
    q = rng.standard_normal((M, nq * d))
    k = rng.standard_normal((M, nkv * d))
    v = rng.standard_normal((M, nkv * d))
    do = rng.standard_normal((M, nq * d))
    return q, k, v, do


def _torch_attn_grads(q, k, v, do, keep, B, S, nq, nkv, d, variant, loss_keep):
    qt, kt, vt = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    o, lse = torch_ref.attention_fwd(qt, kt, vt, keep, B, S, nq, nkv, d, variant)
    kf = torch.tensor(loss_keep, dtype=torch.float64)[:, None]
    (o * torch.tensor(do) * kf).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(), o.detach().numpy(), lse.numpy()


@pytest.mark.parametrize("mode,variant", [("filtered", "drop_keys"), ("full_d", "sg_keys")])
def test_attention_equals_autograd_of_surrogate(mode, variant):
    B, S, nq, nkv, d = 2, 6, 4, 2, 4
    q, k, v, do = _attn_case()
    # the true forward output (plain) and lse are what the backward is handed
    _, _, _, o_true, lse = _torch_attn_grads(q, k, v, do, KEEP, B, S, nq, nkv, d, "plain", KEEP)
    gq, gk, gv, _, _ = _torch_attn_grads(q, k, v, do, KEEP, B, S, nq, nkv, d, variant, KEEP)
    dq, dk, dv = oracle.attention_bwd(q, k, v, o_true, lse, do, KEEP, B, S, nq, nkv, d, mode=mode)
    for a, b in ((dq, gq), (dk, gk), (dv, gv)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)
    for a in (dq, dk, dv):
        assert np.all(a[KEEP == 0] == 0.0)


def test_attention_filtered_fd_of_numpy_surrogate():
    """Central differences of g(q,k,v) = sum_{i kept} dO_i . sum_{j kept, j<=i} e_ij v_j /
    (sum_{j kept, j<=i} e_ij + c_i), c_i = filtered keys' exp-scores frozen at the base point."""
    B, S, nq, nkv, d = 1, 6, 2, 1, 3
    rng = np.random.default_rng(7)
    q, k, v, do = _attn_case(7, B, S, nq, nkv, d)
    keep = np.array([1, 0, 1, 0, 1, 1], np.uint8)
    tau = 1 / math.sqrt(d)
    kb = keep.astype(bool)

    def scores(qq, kk):
        out = []
        for h in range(nq):
            s = tau * qq.reshape(S, nq, d)[:, h] @ kk.reshape(S, 1, d)[:, 0].T
            out.append(np.where(np.tril(np.ones((S, S), bool)), np.exp(s), 0.0))
        return out

    c0 = [(e * ~kb[None, :]).sum(1) for e in scores(q, k)]

    def g(qq, kk, vv):
        tot = 0.0
        for h, e in enumerate(scores(qq, kk)):
            ek = e * kb[None, :]
            ot = (ek @ vv) / (ek.sum(1) + c0[h])[:, None]
            tot += float((ot * do.reshape(S, nq, d)[:, h] * kb[:, None]).sum())
        return tot

    lse = np.stack([np.log(e.sum(1)) for e in scores(q, k)], 1)
    dq, dk, dv = oracle.attention_bwd(q, k, v, np.zeros_like(q), lse, do, keep, B, S, nq, nkv, d)
    hh = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for i in range(arr.size):
            ap, am = arr.copy(), arr.copy()
            ap.flat[i] += hh
            am.flat[i] -= hh
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = ap, am
            fd = (g(*args_p) - g(*args_m)) / (2 * hh)
            assert abs(fd - grad.flat[i]) <= 1e-6 * max(1.0, abs(fd)), (which, i, fd, grad.flat[i])
    del rng


@pytest.mark.parametrize("mode", ["filtered", "full_d"])
def test_attention_r0_and_suffix_equal_true_gradient(mode):
    B, S, nq, nkv, d = 2, 6, 4, 2, 4
    q, k, v, do = _attn_case(3)
    for keep in (np.ones(12, np.uint8), SUFFIX):
        gq, gk, gv, o, lse = _torch_attn_grads(q, k, v, do, keep, B, S, nq, nkv, d, "plain", keep)
        dq, dk, dv = oracle.attention_bwd(q, k, v, o, lse, do, keep, B, S, nq, nkv, d, mode=mode)
        for a, b in ((dq, gq), (dk, gk), (dv, gv)):
            np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_figure3_contrast_loss_only_densifies_dv():
    """Filtering the loss alone leaves non-zero V gradients on filtered keys that kept queries
    attend (Figure 3); filtering P removes them (Figure 5)."""
    B, S, nq, nkv, d = 2, 6, 4, 2, 4
    q, k, v, do = _attn_case(5)
    gq, gk, gv, o, lse = _torch_attn_grads(q, k, v, do, KEEP, B, S, nq, nkv, d, "plain", KEEP)
    dq, dk, dv = oracle.attention_bwd(q, k, v, o, lse, do, KEEP, B, S, nq, nkv, d, mode="loss_only")
    np.testing.assert_allclose(dv, gv, rtol=1e-10, atol=1e-12)  # loss-only = true masked gradient
    np.testing.assert_allclose(dk, gk, rtol=1e-10, atol=1e-12)
    filt_attended = [1, 4, 9]  # filtered tokens with a later kept token in the same sequence
    assert np.all(np.abs(dv[filt_attended]).max(axis=1) > 1e-3)
    _, _, dvf = oracle.attention_bwd(q, k, v, o, lse, do, KEEP, B, S, nq, nkv, d, mode="filtered")
    assert np.all(dvf[KEEP == 0] == 0.0)


# ------------------------------------------------------------------------------------------------
# whole layers
# ------------------------------------------------------------------------------------------------


def _tiny_layer_inputs(cfg, seed):
    rng = np.random.default_rng(seed)
    H, I = cfg.H, cfg.I
    w = {"w_qkv": 0.3 * rng.standard_normal((cfg.n_qkv, H)),
         "w_o": 0.3 * rng.standard_normal((H, cfg.nq * cfg.d))}
    if cfg.kind == "llama":
        w.update(w_gateup=0.3 * rng.standard_normal((2 * I, H)), w_down=0.3 * rng.standard_normal((H, I)),
                 gamma1=1 + 0.1 * rng.standard_normal(H), gamma2=1 + 0.1 * rng.standard_normal(H))
    else:
        w.update(w_fc1=0.3 * rng.standard_normal((I, H)), w_fc2=0.3 * rng.standard_normal((H, I)),
                 gamma=1 + 0.1 * rng.standard_normal(H), beta=0.1 * rng.standard_normal(H))
    x = rng.standard_normal((cfg.M, H))
    dy = rng.standard_normal((cfg.M, H))
    return w, x, dy


def _check_layer(cfg, mode, variant, keep, seed=0):
    w, x, dy = _tiny_layer_inputs(cfg, seed)
    ref, saved = torch_ref.layer_grads(cfg, w, x, dy, keep, variant)
    out = oracle.layer_bwd(cfg, w, saved, dy, keep, mode)
    for name, val in out.items():
        np.testing.assert_allclose(val, ref[name], rtol=1e-9, atol=1e-11, err_msg=name)
    assert np.all(out["dx"][np.asarray(keep) == 0] == 0.0)


@pytest.mark.parametrize("cfg", [TINY_LLAMA, TINY_PHI], ids=["llama", "phi"])
@pytest.mark.parametrize("mode,variant", [("filtered", "drop_keys"), ("full_d", "sg_keys")])
def test_layer_equals_autograd_of_surrogate(cfg, mode, variant):
    _check_layer(cfg, mode, variant, KEEP)


@pytest.mark.parametrize("cfg", [TINY_LLAMA, TINY_PHI], ids=["llama", "phi"])
@pytest.mark.parametrize("mode", ["filtered", "full_d"])
def test_layer_r0_and_suffix_equal_plain_autograd(cfg, mode):
    _check_layer(cfg, mode, "plain", np.ones(cfg.M, np.uint8))
    _check_layer(cfg, mode, "plain", SUFFIX, seed=1)


@pytest.mark.parametrize("mode,variant", [("filtered", "drop_keys"), ("full_d", "sg_keys")])
def test_stack_of_three_layers(mode, variant):
    cfg = TINY_LLAMA
    ws, x, dy = [], None, None
    for s in range(3):
        w, x0, dy0 = _tiny_layer_inputs(cfg, 10 + s)
        ws.append(w)
        if s == 0:
            x, dy = x0, dy0
    dx_ref, g_ref, saved = torch_ref.stack_grads(cfg, ws, x, dy, KEEP, variant)
    layers = [{"weights": w, "saved": sv} for w, sv in zip(ws, saved)]
    outs = oracle.model_bwd(cfg, layers, dy, KEEP, mode)
    np.testing.assert_allclose(outs[0]["dx"], dx_ref, rtol=1e-9, atol=1e-11)
    for o, g in zip(outs, g_ref):
        for name, val in g.items():
            np.testing.assert_allclose(o[name], val, rtol=1e-9, atol=1e-11, err_msg=name)
    for o in outs:
        assert np.all(o["dx"][KEEP == 0] == 0.0)
