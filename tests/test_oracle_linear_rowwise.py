"""Pins for the oracle's linear and row-wise backward pieces: central finite differences of forwards
written here, torch.autograd, and a library GELU."""
import numpy as np
import pytest
import torch

import oracle
import synth


def _fd(f, x, idxs, h=1e-6):
    out = []
    for i in idxs:
        xp, xm = x.copy(), x.copy()
        xp.flat[i] += h
        xm.flat[i] -= h
        out.append((f(xp) - f(xm)) / (2 * h))
    return np.array(out)


def test_linear_fd_and_zero_rows():
    rng = np.random.default_rng(0)
    M, K, N = 9, 5, 4
    x, w, dy = rng.standard_normal((M, K)), rng.standard_normal((N, K)), rng.standard_normal((M, N))
    keep = np.array([1, 0, 1, 1, 0, 1, 0, 1, 1], np.uint8)
    out = oracle.linear_bwd(x, dy, w, keep, bias=True)

    def loss_x(xx):
        return float(((xx @ w.T) * dy * keep[:, None]).sum())

    def loss_w(ww):
        return float(((x @ ww.T) * dy * keep[:, None]).sum())

    ii = list(range(0, M * K, 3))
    np.testing.assert_allclose(_fd(loss_x, x, ii), out["dx"].flat[ii], rtol=1e-7, atol=1e-8)
    jj = list(range(N * K))
    np.testing.assert_allclose(_fd(loss_w, w, jj), out["dw"].flat[jj], rtol=1e-7, atol=1e-8)
    assert np.all(out["dx"][keep == 0] == 0.0)
    np.testing.assert_allclose(out["db"], (dy * keep[:, None]).sum(0))


def test_linear_torch_autograd_and_r0():
    inp = synth.make_linear_inputs(synth.get_config("linear_fp32"))
    for keep in (inp["keep"], np.ones_like(inp["keep"])):
        x = torch.tensor(inp["x"], dtype=torch.float64, requires_grad=True)
        w = torch.tensor(inp["w"], dtype=torch.float64, requires_grad=True)
        k = torch.tensor(keep, dtype=torch.float64)[:, None]
        ((x @ w.T) * torch.tensor(inp["dy"], dtype=torch.float64) * k).sum().backward()
        out = oracle.linear_bwd(inp["x"], inp["dy"], inp["w"], keep)
        np.testing.assert_allclose(out["dx"], x.grad.numpy(), rtol=1e-12, atol=1e-10)
        np.testing.assert_allclose(out["dw"], w.grad.numpy(), rtol=1e-12, atol=1e-10)


def test_linear_dw_is_sum_over_kept_rows_only():
    rng = np.random.default_rng(1)
    x, w, dy = rng.standard_normal((7, 3)), rng.standard_normal((2, 3)), rng.standard_normal((7, 2))
    keep = np.array([0, 1, 0, 0, 1, 1, 0], np.uint8)
    dw = np.zeros((2, 3))
    for t in np.flatnonzero(keep):
        dw += np.outer(dy[t], x[t])
    np.testing.assert_allclose(oracle.linear_bwd(x, dy, w, keep)["dw"], dw, rtol=1e-13)


def test_rmsnorm_fd():
    rng = np.random.default_rng(2)
    M, H, eps = 3, 6, 1e-5
    x, gamma, dy = rng.standard_normal((M, H)), 1 + 0.1 * rng.standard_normal(H), rng.standard_normal((M, H))

    def fwd(xx, gg):
        return xx / np.sqrt((xx * xx).mean(1, keepdims=True) + eps) * gg

    rstd = 1 / np.sqrt((x * x).mean(1) + eps)
    dx, dg = oracle.rmsnorm_bwd(dy, x, rstd, gamma)
    np.testing.assert_allclose(_fd(lambda xx: (fwd(xx, gamma) * dy).sum(), x, range(M * H)), dx.ravel(),
                               rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(_fd(lambda gg: (fwd(x, gg) * dy).sum(), gamma, range(H)), dg,
                               rtol=1e-6, atol=1e-8)


def test_layernorm_fd():
    rng = np.random.default_rng(3)
    M, H, eps = 3, 7, 1e-5
    x, dy = rng.standard_normal((M, H)) + 0.3, rng.standard_normal((M, H))
    gamma, beta = 1 + 0.1 * rng.standard_normal(H), 0.1 * rng.standard_normal(H)

    def fwd(xx, gg, bb):
        mu = xx.mean(1, keepdims=True)
        return (xx - mu) / np.sqrt(((xx - mu) ** 2).mean(1, keepdims=True) + eps) * gg + bb

    mean = x.mean(1)
    rstd = 1 / np.sqrt(((x - mean[:, None]) ** 2).mean(1) + eps)
    dx, dg, db = oracle.layernorm_bwd(dy, x, mean, rstd, gamma)
    np.testing.assert_allclose(_fd(lambda xx: (fwd(xx, gamma, beta) * dy).sum(), x, range(M * H)),
                               dx.ravel(), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(_fd(lambda gg: (fwd(x, gg, beta) * dy).sum(), gamma, range(H)), dg,
                               rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(_fd(lambda bb: (fwd(x, gamma, bb) * dy).sum(), beta, range(H)), db,
                               rtol=1e-6, atol=1e-8)


def test_swiglu_fd():
    rng = np.random.default_rng(4)
    g, u, da = rng.standard_normal(20) * 3, rng.standard_normal(20), rng.standard_normal(20)

    def fwd(gg, uu):
        return gg / (1 + np.exp(-gg)) * uu

    dg, du = oracle.swiglu_bwd(da, g, u)
    np.testing.assert_allclose(_fd(lambda gg: (fwd(gg, u) * da).sum(), g, range(20)), dg, rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(_fd(lambda uu: (fwd(g, uu) * da).sum(), u, range(20)), du, rtol=1e-6, atol=1e-9)


def test_gelu_tanh_matches_torch_and_fd():
    f = np.linspace(-6, 6, 97)
    ref = torch.nn.functional.gelu(torch.tensor(f), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(f), ref, rtol=1e-13, atol=1e-15)
    da = np.cos(f)
    h = 1e-6
    fd = (oracle.gelu_tanh(f + h) - oracle.gelu_tanh(f - h)) / (2 * h) * da  # elementwise map
    np.testing.assert_allclose(fd, oracle.gelu_tanh_bwd(da, f), rtol=1e-6, atol=1e-9)
    ft = torch.tensor(f, requires_grad=True)
    (torch.nn.functional.gelu(ft, approximate="tanh") * torch.tensor(da)).sum().backward()
    np.testing.assert_allclose(oracle.gelu_tanh_bwd(da, f), ft.grad.numpy(), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("d,rot,base", [(8, 8, 1e4), (8, 4, 1e4), (16, 16, 1e6)])
def test_rope_bwd_is_transpose_of_forward(d, rot, base):
    from tests.torch_ref import rope_fwd
    rng = np.random.default_rng(5)
    M, nh = 13, 3
    pos = np.arange(M) * 7 % 11
    x, dy = rng.standard_normal((M, nh * d)), rng.standard_normal((M, nh * d))
    y = rope_fwd(torch.tensor(x), torch.tensor(pos), nh, d, rot, base).numpy()
    dx = oracle.rope_bwd(dy, pos, nh, d, rot, base)
    # <R x, dy> == <x, R^T dy> and R is orthogonal (norm preserving, R^T R = I)
    np.testing.assert_allclose((y * dy).sum(), (x * dx).sum(), rtol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(dx, axis=1), np.linalg.norm(dy, axis=1), rtol=1e-12)
    back = oracle.rope_bwd(y, pos, nh, d, rot, base)
    np.testing.assert_allclose(back, x, rtol=1e-12, atol=1e-12)
    if rot < d:
        np.testing.assert_array_equal(dx.reshape(M, nh, d)[:, :, rot:], dy.reshape(M, nh, d)[:, :, rot:])
    # position 0 is the identity
    z = oracle.rope_bwd(dy[:1], np.zeros(1), nh, d, rot, base)
    np.testing.assert_allclose(z, dy[:1], rtol=0, atol=0)
