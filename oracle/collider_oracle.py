"""Plain CPU oracle for Collider-style filtered transformer-layer backward.

TEST INFRASTRUCTURE.  Imported only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg; the HIP product path never imports, links or runs it, and it imports nothing from there.

Source: "Enhancing Token Filtering Efficiency in Large Language Model Training with Collider"
(arXiv 2502.00340), abstract and TL;DR, captions of Figures 2, 3 and 5.  What it computes:
  * backward token filtering drops the training loss of filtered tokens (Figure 2(b)), so the
    upstream gradient rows of filtered tokens are zero;
  * the activations of filtered tokens are filtered in the backward of *every* layer (abstract),
    including the attention softmax activation P, whose filtered-token entries would otherwise make
    G_V = P^T G_O dense (Figure 3); the Q/K backward activations are filtered as well (Figure 5);
  * the resulting sparse GEMMs equal dense GEMMs over the kept tokens only (abstract).

This oracle computes all of it the plain way: float64, the full token layout (M = B*S rows), the
keep mask applied explicitly (zeroed upstream-gradient rows, zeroed columns of P), dense NumPy matmuls
and per-(sequence, head) attention loops.  No compaction, blocking or fusion.  Inputs may be any
float dtype; they are upcast to float64.  Readings of points the pages leave open:
  * P is filtered on its key columns (a filtered query row of G_O is already zero, so zeroing rows
    alone cannot make G_V sparse);
  * the softmax-backward row term is, by default, taken from the filtered activation:
    D~_i = sum_j P~_ij dP_ij ("filtered").  The alternative D_i = dO_i . O_i ("full_d") is kept
    behind the `mode` switch;
  * P keeps the forward's normalisation (log-sum-exp over all causal keys): backward filtering does
    not change the forward (Figure 2(b));
  * weights use the [out, in] layout, y = x @ w.T;
  * rotary embedding is rotate-half over the first `rot` dims of each head, position = s (t mod S).

Pins (tests/test_oracle_*.py): hand-derived golden cases, central finite differences, torch.autograd
of explicit surrogate forwards whose exact gradient the method is, the r = 0 and suffix-mask special
cases, and exact-zero rows.  No function here is "parity unpinned".
"""
import numpy as np

__all__ = [
    "build_index", "gather_rows", "scatter_rows", "linear_bwd",
    "silu", "sigmoid", "gelu_tanh", "gelu_tanh_bwd", "swiglu_bwd",
    "rmsnorm_bwd", "layernorm_bwd", "rope_bwd", "attention_bwd",
    "llama_layer_bwd", "phi_layer_bwd", "layer_bwd", "model_bwd", "MODES",
    "select_topk", "ce_loss", "ce_logits_bwd", "lm_head_bwd", "embedding_bwd", "precision",
]

MODES = ("filtered", "full_d", "loss_only")


# Floating-point type of the oracle's arithmetic.  float64 everywhere the oracle is pinned and
# compared; `precision(np.float32)` switches it for a timed float32 run (the CPU baseline of the
# benchmark), whose results tests check against the float64 ones.
_DTYPE = np.float64


class precision:
    """Context manager: run the oracle's float arithmetic in `dtype` (float64 or float32)."""

    def __init__(self, dtype):
        if np.dtype(dtype) not in (np.dtype(np.float64), np.dtype(np.float32)):
            raise ValueError(dtype)
        self.dtype, self.prev = np.dtype(dtype).type, None

    def __enter__(self):
        global _DTYPE
        self.prev, _DTYPE = _DTYPE, self.dtype
        return self

    def __exit__(self, *exc):
        global _DTYPE
        _DTYPE = self.prev
        return False


def _f64(a):
    return np.asarray(a, dtype=_DTYPE)


def _keep_bool(keep):
    return np.asarray(keep).reshape(-1) != 0


# ---------------------------------------------------------------------------------------------
# mask -> index, gather, scatter  (integer / bit-copy work)
# ---------------------------------------------------------------------------------------------


def build_index(keep, B, S):
    """Stable compaction of a per-token keep mask (Figure 2(b): filtering is per token).

    idx[c]       = flat position of the c-th kept token, ascending (c < count)
    inv[t]       = c if token t is kept, else -1
    cu_seqlens[b]= number of kept tokens before sequence b (length B + 1, last entry = count)
    partition    = kept positions ascending followed by filtered positions ascending
    """
    keep = _keep_bool(keep)
    M = B * S
    if keep.size != M:
        raise ValueError("keep has %d entries, expected B*S = %d" % (keep.size, M))
    idx = np.flatnonzero(keep).astype(np.int32)
    count = int(idx.size)
    inv = np.full(M, -1, dtype=np.int32)
    inv[idx] = np.arange(count, dtype=np.int32)
    cu = np.array([np.count_nonzero(keep[: b * S]) for b in range(B + 1)], dtype=np.int32)
    partition = np.concatenate([idx, np.flatnonzero(~keep).astype(np.int32)])
    return {"idx": idx, "inv": inv, "cu_seqlens": cu, "count": count, "partition": partition}


def gather_rows(src, idx):
    """Dimension-reduced copy: row c of the result is row idx[c] of src (abstract)."""
    return np.asarray(src)[np.asarray(idx, dtype=np.int64)]


def scatter_rows(src_compact, idx, M):
    """Inverse of gather: full layout with the rows of filtered tokens exactly zero."""
    src_compact = np.asarray(src_compact)
    out = np.zeros((M,) + src_compact.shape[1:], dtype=src_compact.dtype)
    out[np.asarray(idx, dtype=np.int64)] = src_compact
    return out


# ---------------------------------------------------------------------------------------------
# linear layer (abstract: sparse GEMM -> dimension-reduced dense GEMM; Figure 2(b))
# ---------------------------------------------------------------------------------------------


def linear_bwd(x, dy, w, keep, bias=False):
    """y = x @ w.T with the loss of filtered tokens dropped: dY~ = diag(keep) dY,
    dX = dY~ @ w, dW = dY~^T @ x (stored [out, in]), db = column sums of dY~."""
    k = _keep_bool(keep).astype(_DTYPE)[:, None]
    dyk = _f64(dy) * k
    out = {"dx": dyk @ _f64(w), "dw": dyk.T @ _f64(x)}
    if bias:
        out["db"] = dyk.sum(axis=0)
    return out


# ---------------------------------------------------------------------------------------------
# row-wise vector-Jacobian products (the per-layer activation backward of the abstract)
# ---------------------------------------------------------------------------------------------


def sigmoid(z):
    z = _f64(z)
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    z = _f64(z)
    return z * sigmoid(z)


_GELU_C = np.sqrt(2.0 / np.pi)
_GELU_A = 0.044715


def gelu_tanh(f):
    """GELU with the tanh approximation of Hendrycks and Gimpel."""
    f = _f64(f)
    return 0.5 * f * (1.0 + np.tanh(_GELU_C * (f + _GELU_A * f ** 3)))


def gelu_tanh_bwd(da, f):
    f = _f64(f)
    t = np.tanh(_GELU_C * (f + _GELU_A * f ** 3))
    deriv = 0.5 * (1.0 + t) + 0.5 * f * (1.0 - t * t) * _GELU_C * (1.0 + 3.0 * _GELU_A * f * f)
    return _f64(da) * deriv


def swiglu_bwd(da, gate, up):
    """a = silu(gate) * up.  Returns (dgate, dup)."""
    g, u, da = _f64(gate), _f64(up), _f64(da)
    s = sigmoid(g)
    dgate = da * u * s * (1.0 + g * (1.0 - s))
    dup = da * g * s
    return dgate, dup


def rmsnorm_bwd(dy, x, rstd, gamma):
    """y = x * rstd * gamma with rstd = 1/sqrt(mean(x^2) + eps) saved by the forward.
    Returns (dx, dgamma)."""
    dy, x, rstd, gamma = _f64(dy), _f64(x), _f64(rstd)[:, None], _f64(gamma)[None, :]
    xhat = x * rstd
    g = dy * gamma
    dx = rstd * (g - xhat * (g * xhat).mean(axis=1, keepdims=True))
    return dx, (dy * xhat).sum(axis=0)


def layernorm_bwd(dy, x, mean, rstd, gamma):
    """y = (x - mean) * rstd * gamma + beta.  Returns (dx, dgamma, dbeta)."""
    dy, x = _f64(dy), _f64(x)
    mean, rstd, gamma = _f64(mean)[:, None], _f64(rstd)[:, None], _f64(gamma)[None, :]
    xhat = (x - mean) * rstd
    g = dy * gamma
    dx = rstd * (g - g.mean(axis=1, keepdims=True) - xhat * (g * xhat).mean(axis=1, keepdims=True))
    return dx, (dy * xhat).sum(axis=0), dy.sum(axis=0)


def rope_bwd(dy, pos, nheads, d, rot, base):
    """Transpose of the rotate-half rotary embedding on the first `rot` dims of each head:
    for m < rot/2, angle = pos * base^(-2m/rot),
      dx_m          = dy_m cos + dy_{m+rot/2} sin
      dx_{m+rot/2}  = dy_{m+rot/2} cos - dy_m sin;  dims >= rot pass through."""
    dy = _f64(dy)
    if rot == 0:
        return dy.copy()
    half = rot // 2
    theta = float(base) ** (-2.0 * np.arange(half, dtype=np.float64) / rot)
    ang = _f64(pos)[:, None] * theta[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    d3 = dy.reshape(dy.shape[0], nheads, d)
    out = d3.copy()
    a, b = d3[:, :, :half], d3[:, :, half:rot]
    out[:, :, :half] = a * c + b * s
    out[:, :, half:rot] = b * c - a * s
    return out.reshape(dy.shape)


# ---------------------------------------------------------------------------------------------
# attention backward with the softmax activation filtered (Figures 3 and 5)
# ---------------------------------------------------------------------------------------------


def attention_bwd(q, k, v, o, lse, dout, keep, B, S, nq, nkv, d, mode="filtered", scale=None):
    """Causal (grouped-query) attention backward per sequence, full token layout.

    q [M, nq*d], k and v [M, nkv*d], o [M, nq*d] and lse [M, nq] are the forward's (post-rotary q, k;
    lse = natural-log log-sum-exp of scale * q.k over all causal keys).  Head h reads KV head
    h // (nq // nkv).  mode:
      "filtered"  - P~ = P with filtered-token columns zeroed; D~_i = sum_j P~_ij dP_ij;
      "full_d"    - P~ as above; D_i = dO'_i . O_i;
      "loss_only" - P not filtered (loss filtering alone, the Figure 3 baseline).
    In every mode dO' = diag(keep) dO.  Returns (dq, dk, dv) in the input layouts.
    """
    if mode not in MODES:
        raise ValueError(mode)
    M = B * S
    tau = 1.0 / np.sqrt(d) if scale is None else float(scale)
    G = nq // nkv
    keepb = _keep_bool(keep)
    q3, k3, v3 = _f64(q).reshape(M, nq, d), _f64(k).reshape(M, nkv, d), _f64(v).reshape(M, nkv, d)
    o3, do3, lse2 = _f64(o).reshape(M, nq, d), _f64(dout).reshape(M, nq, d), _f64(lse).reshape(M, nq)
    dq = np.zeros((M, nq, d), _DTYPE)
    dk = np.zeros((M, nkv, d), _DTYPE)
    dv = np.zeros((M, nkv, d), _DTYPE)
    causal = np.tril(np.ones((S, S), dtype=bool))
    for b in range(B):
        rows = slice(b * S, (b + 1) * S)
        kb = keepb[rows].astype(_DTYPE)
        for h in range(nq):
            g = h // G
            qq, kk, vv = q3[rows, h, :], k3[rows, g, :], v3[rows, g, :]
            P = np.where(causal, np.exp(tau * (qq @ kk.T) - lse2[rows, h][:, None]), 0.0)
            dO = do3[rows, h, :] * kb[:, None]
            Pt = P if mode == "loss_only" else P * kb[None, :]
            dP = dO @ vv.T
            if mode == "full_d":
                D = (dO * o3[rows, h, :]).sum(axis=1)
            else:
                D = (Pt * dP).sum(axis=1)
            dS = Pt * (dP - D[:, None])
            dq[rows, h, :] = tau * (dS @ kk)
            dk[rows, g, :] += tau * (dS.T @ qq)
            dv[rows, g, :] += Pt.T @ dO
    return dq.reshape(M, nq * d), dk.reshape(M, nkv * d), dv.reshape(M, nkv * d)


# ---------------------------------------------------------------------------------------------
# whole layers and the layer chain (abstract: filter activations across all layers)
# ---------------------------------------------------------------------------------------------


def _split_cfg(cfg):
    return cfg.B, cfg.S, cfg.H, cfg.nq, cfg.nkv, cfg.d, cfg.I


def llama_layer_bwd(cfg, w, saved, dy, keep, mode="filtered"):
    """Pre-norm RMSNorm / GQA attention / SwiGLU layer.

    w: w_qkv [(nq+2nkv)d, H], w_o [H, nq d], w_gateup [2I, H] (gate rows first), w_down [H, I],
       gamma1, gamma2 [H].
    saved: x, rstd1, q, k (post-rotary), v, o, lse, h (= x + attention output), rstd2, gate, up.
    Returns dx and the weight / gain gradients (all float64, full token layout)."""
    B, S, H, nq, nkv, d, I = _split_cfg(cfg)
    M = B * S
    kf = _keep_bool(keep).astype(_DTYPE)[:, None]
    pos = np.arange(M) % S
    dYp = _f64(dy) * kf
    gate, up = _f64(saved["gate"]), _f64(saved["up"])
    a = silu(gate) * up
    dA = dYp @ _f64(w["w_down"])
    dw_down = dYp.T @ a
    dgate, dup = swiglu_bwd(dA, gate, up)
    dGU = np.concatenate([dgate, dup], axis=1)
    h, rstd2, gamma2 = _f64(saved["h"]), _f64(saved["rstd2"]), _f64(w["gamma2"])
    xn2 = h * rstd2[:, None] * gamma2[None, :]
    dXn2 = dGU @ _f64(w["w_gateup"])
    dw_gateup = dGU.T @ xn2
    dh_n, dgamma2 = rmsnorm_bwd(dXn2, h, rstd2, gamma2)
    dh = dYp + dh_n
    o = _f64(saved["o"])
    dO = dh @ _f64(w["w_o"])
    dw_o = dh.T @ o
    dq, dk, dv = attention_bwd(saved["q"], saved["k"], saved["v"], o, saved["lse"], dO, keep,
                               B, S, nq, nkv, d, mode=mode)
    dq = rope_bwd(dq, pos, nq, d, cfg.rot, cfg.rope_base)
    dk = rope_bwd(dk, pos, nkv, d, cfg.rot, cfg.rope_base)
    dQKV = np.concatenate([dq, dk, dv], axis=1)
    x, rstd1, gamma1 = _f64(saved["x"]), _f64(saved["rstd1"]), _f64(w["gamma1"])
    xn1 = x * rstd1[:, None] * gamma1[None, :]
    dXn1 = dQKV @ _f64(w["w_qkv"])
    dw_qkv = dQKV.T @ xn1
    dx_n, dgamma1 = rmsnorm_bwd(dXn1, x, rstd1, gamma1)
    return {"dx": dh + dx_n, "dw_qkv": dw_qkv, "dw_o": dw_o, "dw_gateup": dw_gateup,
            "dw_down": dw_down, "dgamma1": dgamma1, "dgamma2": dgamma2}


def phi_layer_bwd(cfg, w, saved, dy, keep, mode="filtered"):
    """Parallel block: xn = LayerNorm(x); y = x + Attn(xn) @ w_o.T + gelu_tanh(xn @ w_fc1.T) @ w_fc2.T.

    w: w_qkv [3 nq d, H], w_o [H, nq d], w_fc1 [I, H], w_fc2 [H, I], gamma, beta [H].
    saved: x, mean, rstd, q, k (post-rotary), v, o, lse, f (fc1 pre-activation)."""
    B, S, H, nq, nkv, d, I = _split_cfg(cfg)
    M = B * S
    kf = _keep_bool(keep).astype(_DTYPE)[:, None]
    pos = np.arange(M) % S
    dYp = _f64(dy) * kf
    f = _f64(saved["f"])
    dA = dYp @ _f64(w["w_fc2"])
    dw_fc2 = dYp.T @ gelu_tanh(f)
    dF = gelu_tanh_bwd(dA, f)
    o = _f64(saved["o"])
    dO = dYp @ _f64(w["w_o"])
    dw_o = dYp.T @ o
    dq, dk, dv = attention_bwd(saved["q"], saved["k"], saved["v"], o, saved["lse"], dO, keep,
                               B, S, nq, nkv, d, mode=mode)
    dq = rope_bwd(dq, pos, nq, d, cfg.rot, cfg.rope_base)
    dk = rope_bwd(dk, pos, nkv, d, cfg.rot, cfg.rope_base)
    dQKV = np.concatenate([dq, dk, dv], axis=1)
    x, mean, rstd = _f64(saved["x"]), _f64(saved["mean"]), _f64(saved["rstd"])
    gamma, beta = _f64(w["gamma"]), _f64(w["beta"])
    xn = (x - mean[:, None]) * rstd[:, None] * gamma[None, :] + beta[None, :]
    dXn = dQKV @ _f64(w["w_qkv"]) + dF @ _f64(w["w_fc1"])
    dw_qkv = dQKV.T @ xn
    dw_fc1 = dF.T @ xn
    dx_n, dgamma, dbeta = layernorm_bwd(dXn, x, mean, rstd, gamma)
    return {"dx": dYp + dx_n, "dw_qkv": dw_qkv, "dw_o": dw_o, "dw_fc1": dw_fc1, "dw_fc2": dw_fc2,
            "dgamma": dgamma, "dbeta": dbeta}


def layer_bwd(cfg, w, saved, dy, keep, mode="filtered"):
    if cfg.kind == "llama":
        return llama_layer_bwd(cfg, w, saved, dy, keep, mode)
    if cfg.kind == "phi":
        return phi_layer_bwd(cfg, w, saved, dy, keep, mode)
    raise ValueError(cfg.kind)


def model_bwd(cfg, layers, dy, keep, mode="filtered"):
    """Backward through a stack of layers, top to bottom; the same keep mask in every layer and the
    dx of layer l+1 is the upstream gradient of layer l.  Returns the per-layer outputs, bottom first."""
    g = dy
    outs = []
    for layer in reversed(layers):
        out = layer_bwd(cfg, layer["weights"], layer["saved"], g, keep, mode)
        outs.append(out)
        g = out["dx"]
    return outs[::-1]


# ---------------------------------------------------------------------------------------------
# loss side of the backward (Figure 2(b): the per-token training loss decides which tokens are
# filtered; the loss of a filtered token is dropped, so it sends no gradient into the LM head,
# the layers below it or the token embedding)
# ---------------------------------------------------------------------------------------------


def select_topk(score, n_keep):
    """Token selection on per-token scores: keep the n_keep tokens with the largest score.

    Order: by descending score, equal scores by ascending position; -0.0 equals +0.0; NaN ranks
    below every number (NaN scores are filtered first).  Returns a uint8 mask (1 = kept)."""
    s = np.asarray(score, dtype=np.float64).reshape(-1)
    M = s.size
    n_keep = max(0, min(int(n_keep), M))
    nan = np.isnan(s)
    # lexsort: the last key is the primary one
    order = np.lexsort((np.arange(M), -np.where(nan, 0.0, s), nan))
    keep = np.zeros(M, dtype=np.uint8)
    keep[order[:n_keep]] = 1
    return keep


def ce_loss(logits, labels):
    """Per-token cross-entropy loss of every token (Figure 2(b): the training loss whose per-token
    values decide which tokens backward filtering drops): loss_t = logsumexp(z_t) - z_t[y_t], natural
    log.  A label outside [0, V) marks a token without a target: loss 0.  -inf logits (masked
    vocabulary entries) contribute exp(-inf) = 0 to the sum."""
    z = _f64(logits)
    y = np.asarray(labels, dtype=np.int64).reshape(-1)
    V = z.shape[1]
    valid = (y >= 0) & (y < V)
    zmax = z.max(axis=1)
    lse = zmax + np.log(np.exp(z - zmax[:, None]).sum(axis=1))
    zy = z[np.arange(z.shape[0]), np.where(valid, y, 0)]
    return np.where(valid, lse - zy, 0.0)


def ce_logits_bwd(logits, labels, keep, scale):
    """Gradient of L = scale * sum over kept t of CE(logits_t, labels_t) with respect to the
    logits, CE(z, y) = logsumexp(z) - z_y:  dL/dz_t = scale * (softmax(z_t) - onehot(y_t)) for a
    kept token, 0 for a filtered one (its loss is dropped).  A label outside [0, V) (torch's ignore
    index -100, say) marks a token without a target: no loss, zero gradient."""
    z = _f64(logits)
    y = np.asarray(labels, dtype=np.int64).reshape(-1)
    V = z.shape[1]
    valid = (y >= 0) & (y < V)
    k = _keep_bool(keep) & valid
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    p = e / e.sum(axis=1, keepdims=True)
    rows = np.flatnonzero(valid)
    p[rows, y[rows]] -= 1.0
    return float(scale) * p * k[:, None]


def lm_head_bwd(logits, labels, h, w_lm, keep, scale):
    """Backward of the LM head logits = h @ w_lm.T (w_lm [V, H], torch layout) under the per-token
    loss of ce_logits_bwd: dh = dlogits @ w_lm, dw_lm = dlogits^T @ h.  Rows of filtered tokens of
    dlogits are zero, so dh's filtered rows are exactly zero and dw_lm sums over kept tokens only."""
    g = ce_logits_bwd(logits, labels, keep, scale)
    return {"dlogits": g, "dh": g @ _f64(w_lm), "dw_lm": g.T @ _f64(h)}


def embedding_bwd(dx, token_ids, keep, V):
    """Gradient of the token embedding table E [V, H] under x_t = E[id_t]: row v of dE is the sum of
    dx_t over the kept tokens t with id_t = v (a filtered token's dx is zero).  Ids outside [0, V)
    have no embedding row and are skipped."""
    ids = np.asarray(token_ids, dtype=np.int64).reshape(-1)
    use = _keep_bool(keep) & (ids >= 0) & (ids < int(V))
    g = _f64(dx)[use]
    dE = np.zeros((int(V), _f64(dx).shape[1]), _DTYPE)
    np.add.at(dE, ids[use], g)
    return dE
