"""Independent references for pinning the oracle: forward passes written in PyTorch (CPU, float64)
and differentiated by torch.autograd.  Nothing here calls the oracle's backward formulas.

The filtered backward is the exact gradient of an explicit surrogate forward:
  * "plain"  : ordinary causal softmax attention;
  * "sg_keys": every contribution of a filtered token to another token's attention output is held
               constant (detached) - the numerator and the normaliser terms of filtered keys.
               Its gradient at the true forward is the method with D_i = dO_i . O_i.
  * "drop_keys": filtered keys are removed from the numerator, their normaliser term is held
               constant.  Its gradient is the method with D~_i = sum_j P~_ij dP_ij; its forward
               value differs from the true output, so callers save the surrogate's own activations.
The loss is sum over kept tokens of dY_t . y_t (the filtered tokens' loss is dropped).
"""
import math

import torch

DT = torch.float64


def rope_fwd(x, pos, nheads, d, rot, base):
    """Rotary embedding written as a complex rotation of the pairs (m, m + rot/2)."""
    if rot == 0:
        return x
    half = rot // 2
    M = x.shape[0]
    x3 = x.reshape(M, nheads, d)
    theta = base ** (-2.0 * torch.arange(half, dtype=DT) / rot)
    ang = pos.to(DT)[:, None] * theta[None, :]
    rot_c = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    z = torch.complex(x3[:, :, :half], x3[:, :, half:rot]) * rot_c
    out = torch.cat([z.real, z.imag, x3[:, :, rot:]], dim=2)
    return out.reshape(M, nheads * d)


def attention_fwd(q, k, v, keep, B, S, nq, nkv, d, variant="plain"):
    """Returns (o [M, nq*d], lse [M, nq]); lse is over all causal keys and is detached."""
    M = B * S
    tau = 1.0 / math.sqrt(d)
    G = nq // nkv
    q3, k3, v3 = q.reshape(M, nq, d), k.reshape(M, nkv, d), v.reshape(M, nkv, d)
    keep = torch.as_tensor(keep).reshape(-1).bool()
    causal = torch.tril(torch.ones(S, S, dtype=torch.bool))
    outs, lses = [], []
    for b in range(B):
        rs = slice(b * S, (b + 1) * S)
        kb = keep[rs].to(DT)
        oh, lh = [], []
        for h in range(nq):
            g = h // G
            s = tau * (q3[rs, h, :] @ k3[rs, g, :].T)
            s = s.masked_fill(~causal, float("-inf"))
            m = s.max(dim=1, keepdim=True).values.detach()
            e = torch.exp(s - m)
            lh.append((m + torch.log(e.sum(dim=1, keepdim=True))).detach()[:, 0])
            vv = v3[rs, g, :]
            if variant == "plain":
                o = (e @ vv) / e.sum(dim=1, keepdim=True)
            elif variant == "sg_keys":
                ek, ef = e * kb[None, :], e * (1.0 - kb[None, :])
                num = ek @ vv + (ef @ vv).detach()
                den = ek.sum(dim=1, keepdim=True) + ef.sum(dim=1, keepdim=True).detach()
                o = num / den
            elif variant == "drop_keys":
                ek, ef = e * kb[None, :], e * (1.0 - kb[None, :])
                o = (ek @ vv) / (ek.sum(dim=1, keepdim=True) + ef.sum(dim=1, keepdim=True).detach())
            else:
                raise ValueError(variant)
            oh.append(o)
        outs.append(torch.stack(oh, dim=1))
        lses.append(torch.stack(lh, dim=1))
    return torch.cat(outs, 0).reshape(M, nq * d), torch.cat(lses, 0)


def _t(a, grad=False):
    t = torch.tensor(a, dtype=DT)
    return t.requires_grad_(grad)


def llama_forward(cfg, w, x, keep, variant="plain"):
    """w: dict of float64 tensors; x [M, H].  Returns (y, saved)."""
    M, H, I, d, nq, nkv = cfg.M, cfg.H, cfg.I, cfg.d, cfg.nq, cfg.nkv
    pos = torch.arange(M) % cfg.S
    rstd1 = torch.rsqrt((x * x).mean(dim=1, keepdim=True) + cfg.eps)
    xn1 = x * rstd1 * w["gamma1"]
    qkv = xn1 @ w["w_qkv"].T
    q = rope_fwd(qkv[:, : nq * d], pos, nq, d, cfg.rot, cfg.rope_base)
    k = rope_fwd(qkv[:, nq * d:(nq + nkv) * d], pos, nkv, d, cfg.rot, cfg.rope_base)
    v = qkv[:, (nq + nkv) * d:]
    o, lse = attention_fwd(q, k, v, keep, cfg.B, cfg.S, nq, nkv, d, variant)
    h = x + o @ w["w_o"].T
    rstd2 = torch.rsqrt((h * h).mean(dim=1, keepdim=True) + cfg.eps)
    xn2 = h * rstd2 * w["gamma2"]
    gu = xn2 @ w["w_gateup"].T
    gate, up = gu[:, :I], gu[:, I:]
    y = h + (torch.nn.functional.silu(gate) * up) @ w["w_down"].T
    saved = {"x": x, "rstd1": rstd1[:, 0], "q": q, "k": k, "v": v, "o": o, "lse": lse, "h": h,
             "rstd2": rstd2[:, 0], "gate": gate, "up": up}
    return y, {kk: vv.detach().numpy().copy() for kk, vv in saved.items()}


def phi_forward(cfg, w, x, keep, variant="plain"):
    M, I, d, nq, nkv = cfg.M, cfg.I, cfg.d, cfg.nq, cfg.nkv
    pos = torch.arange(M) % cfg.S
    mean = x.mean(dim=1, keepdim=True)
    rstd = torch.rsqrt(((x - mean) ** 2).mean(dim=1, keepdim=True) + cfg.eps)
    xn = (x - mean) * rstd * w["gamma"] + w["beta"]
    qkv = xn @ w["w_qkv"].T
    q = rope_fwd(qkv[:, : nq * d], pos, nq, d, cfg.rot, cfg.rope_base)
    k = rope_fwd(qkv[:, nq * d:(nq + nkv) * d], pos, nkv, d, cfg.rot, cfg.rope_base)
    v = qkv[:, (nq + nkv) * d:]
    o, lse = attention_fwd(q, k, v, keep, cfg.B, cfg.S, nq, nkv, d, variant)
    f = xn @ w["w_fc1"].T
    y = x + o @ w["w_o"].T + torch.nn.functional.gelu(f, approximate="tanh") @ w["w_fc2"].T
    saved = {"x": x, "mean": mean[:, 0], "rstd": rstd[:, 0], "q": q, "k": k, "v": v, "o": o,
             "lse": lse, "f": f}
    return y, {kk: vv.detach().numpy().copy() for kk, vv in saved.items()}


def layer_grads(cfg, w_np, x_np, dy_np, keep, variant="plain"):
    """torch.autograd gradients of sum_{t kept} dY_t . y_t.  Returns (grads, saved)."""
    w = {k: _t(v, True) for k, v in w_np.items()}
    x = _t(x_np, True)
    fwd = llama_forward if cfg.kind == "llama" else phi_forward
    y, saved = fwd(cfg, w, x, keep, variant)
    kf = torch.as_tensor(keep).reshape(-1, 1).to(DT)
    loss = (y * _t(dy_np) * kf).sum()
    loss.backward()
    g = {"dx": x.grad.numpy()}
    for k, v in w.items():
        name = "d" + k if k.startswith(("gamma", "beta")) else "d" + k
        g[name] = v.grad.numpy()
    return g, saved


def stack_grads(cfg, ws_np, x_np, dy_np, keep, variant="plain"):
    """Gradients of a stack of layers (bottom first) through torch.autograd."""
    ws = [{k: _t(v, True) for k, v in w.items()} for w in ws_np]
    x = _t(x_np, True)
    fwd = llama_forward if cfg.kind == "llama" else phi_forward
    h = x
    saved_all = []
    for w in ws:
        h, saved = fwd(cfg, w, h, keep, variant)
        saved_all.append(saved)
    kf = torch.as_tensor(keep).reshape(-1, 1).to(DT)
    (h * _t(dy_np) * kf).sum().backward()
    grads = [{"d" + k: v.grad.numpy() for k, v in w.items()} for w in ws]
    return x.grad.numpy(), grads, saved_all
