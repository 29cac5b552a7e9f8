"""Seeded input generation: random draws, the keep mask, and the forward pass.

Every tensor is drawn from its own PCG64 stream, keyed by (seed, tensor name), so a tensor does not
change when another one is added.  Floating-point tensors the backward reads are stored rounded to
bfloat16 (round to nearest even) as uint16 bit patterns; per-row statistics (rstd, mean, lse) and
norm gains are float32.  Both the oracle and the device path receive exactly these arrays.

Token selection (the keep mask) is the harness's part of token filtering: each token gets a
LogNormal(0, 1) score (a stand-in for the per-token loss a filter ranks by) and the
floor(M * r_pct / 100) lowest-scoring tokens of the flattened batch are filtered; among equal scores
the lower flat position is kept.  The paper leaves its selector open (it cites one, Figure 4 caption).
"""
import sys
import zlib

import numpy as np

from .configs import LayerShape, LinearShape

# ---------------------------------------------------------------------------------------------
# bfloat16 helpers (storage format only)
# ---------------------------------------------------------------------------------------------


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even, returning the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _round_bf16(a) -> np.ndarray:
    """float32 array -> float32 array holding the nearest bfloat16 values."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


# ---------------------------------------------------------------------------------------------
# random streams and the keep mask
# ---------------------------------------------------------------------------------------------


def rng_for(seed: int, name: str) -> np.random.Generator:
    key = zlib.crc32(name.encode("utf-8"))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(key,))))


def n_filtered(M: int, r_pct: int) -> int:
    """Number of filtered tokens for an integer percentage (no floating-point ambiguity)."""
    return (M * int(r_pct)) // 100


def make_keep(M: int, r_pct: int, seed: int, pattern: str = "topk") -> np.ndarray:
    """uint8 keep mask of length M (1 = kept).

    pattern "topk":   global top-(M - n_filt) by LogNormal score, ties keep the lower position.
    pattern "suffix": within each row of a [B, S] view the filtered tokens are the last ones
                      (used only by tests; needs the caller to pass M = S for one sequence).
    """
    n_filt = n_filtered(M, r_pct)
    if pattern == "topk":
        score = np.exp(rng_for(seed, "score").standard_normal(M))
        order = np.lexsort((np.arange(M), -score))  # by descending score, then ascending position
        keep = np.zeros(M, dtype=np.uint8)
        keep[order[: M - n_filt]] = 1
        return keep
    if pattern == "suffix":
        keep = np.ones(M, dtype=np.uint8)
        if n_filt:
            keep[M - n_filt:] = 0
        return keep
    raise ValueError(pattern)


def suffix_keep(B: int, S: int, r_pct: int) -> np.ndarray:
    """Every sequence keeps a prefix and filters its last floor(S*r/100) tokens."""
    return np.concatenate([make_keep(S, r_pct, 0, "suffix") for _ in range(B)])


# ---------------------------------------------------------------------------------------------
# linear layer inputs
# ---------------------------------------------------------------------------------------------


def make_linear_inputs(cfg: LinearShape, seed=None, r_pct=None) -> dict:
    seed = cfg.seed if seed is None else seed
    r_pct = cfg.r_pct if r_pct is None else r_pct
    M = cfg.M
    return {
        "x": rng_for(seed, "x").standard_normal((M, cfg.K)).astype(np.float32),
        "w": rng_for(seed, "w").standard_normal((cfg.N, cfg.K)).astype(np.float32),
        "dy": rng_for(seed, "dy").standard_normal((M, cfg.N)).astype(np.float32),
        "keep": make_keep(M, r_pct, seed),
    }


# ---------------------------------------------------------------------------------------------
# model forward (float32) producing the saved activations
# ---------------------------------------------------------------------------------------------


def _rope_fwd(x, pos, nheads, d, rot, base):
    """Rotate-half rotary embedding on the first `rot` dims of each head (forward)."""
    if rot == 0:
        return x
    half = rot // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / rot)
    ang = pos.astype(np.float64)[:, None] * theta[None, :]
    c = np.cos(ang).astype(np.float32)[:, None, :]
    s = np.sin(ang).astype(np.float32)[:, None, :]
    x3 = x.reshape(x.shape[0], nheads, d).copy()
    a = x3[:, :, :half].copy()
    b = x3[:, :, half:rot].copy()
    x3[:, :, :half] = a * c - b * s
    x3[:, :, half:rot] = b * c + a * s
    return x3.reshape(x.shape)


def _attention_fwd(q, k, v, B, S, nq, nkv, d, chunk=1024):
    """Causal softmax attention per sequence; returns o [M, nq*d] and lse [M, nq] (natural log,
    softmax scale 1/sqrt(d) included)."""
    M = B * S
    tau = 1.0 / np.sqrt(d)
    G = nq // nkv
    o = np.zeros((M, nq * d), np.float32)
    lse = np.zeros((M, nq), np.float32)
    q3 = q.reshape(M, nq, d)
    k3 = k.reshape(M, nkv, d)
    v3 = v.reshape(M, nkv, d)
    o3 = o.reshape(M, nq, d)
    for b in range(B):
        r0 = b * S
        for h in range(nq):
            if S >= 16384 and h % 8 == 0:  # long sequences take minutes on the host: say where we are
                print(f"[synth] attention forward: sequence {b + 1}/{B}, head {h + 1}/{nq} (S={S})",
                      file=sys.stderr, flush=True)
            g = h // G
            kk = k3[r0:r0 + S, g, :]
            vv = v3[r0:r0 + S, g, :]
            for i0 in range(0, S, chunk):
                i1 = min(S, i0 + chunk)
                s = (q3[r0 + i0:r0 + i1, h, :] @ kk[:i1].T) * np.float32(tau)
                rows = np.arange(i0, i1)[:, None]
                cols = np.arange(i1)[None, :]
                s = np.where(cols <= rows, s, -np.inf)
                mx = s.max(axis=1, keepdims=True)
                e = np.exp(s - mx)
                z = e.sum(axis=1, keepdims=True)
                lse[r0 + i0:r0 + i1, h] = (mx + np.log(z))[:, 0]
                o3[r0 + i0:r0 + i1, h, :] = (e / z) @ vv[:i1]
    return o, lse


def _gelu_tanh(f):
    c = np.float32(np.sqrt(2.0 / np.pi))
    return 0.5 * f * (1.0 + np.tanh(c * (f + np.float32(0.044715) * f * f * f)))


def make_layer_weights(cfg: LayerShape, seed: int, layer: int = 0) -> dict:
    p = f"L{layer}."
    H, I = cfg.H, cfg.I

    def wdraw(name, shape):
        return f32_to_bf16_bits(0.02 * rng_for(seed, p + name).standard_normal(shape).astype(np.float32))

    def gdraw(name, shape, base):
        return (base + 0.02 * rng_for(seed, p + name).standard_normal(shape)).astype(np.float32)

    w = {
        "w_qkv": wdraw("w_qkv", (cfg.n_qkv, H)),
        "w_o": wdraw("w_o", (H, cfg.nq * cfg.d)),
    }
    if cfg.kind == "llama":
        w["w_gateup"] = wdraw("w_gateup", (2 * I, H))
        w["w_down"] = wdraw("w_down", (H, I))
        w["gamma1"] = gdraw("gamma1", (H,), 1.0)
        w["gamma2"] = gdraw("gamma2", (H,), 1.0)
    elif cfg.kind == "phi":
        w["w_fc1"] = wdraw("w_fc1", (I, H))
        w["w_fc2"] = wdraw("w_fc2", (H, I))
        w["gamma"] = gdraw("gamma", (H,), 1.0)
        w["beta"] = gdraw("beta", (H,), 0.0)
    else:
        raise ValueError(cfg.kind)
    return w


def layer_forward(cfg: LayerShape, w: dict, x_bits: np.ndarray) -> tuple:
    """Forward pass of one layer in float32 from bf16 input bits.

    Returns (saved, y_bits): `saved` is the set of activations the backward reads (bf16 bits or
    float32), y_bits the layer output rounded to bf16.
    """
    M, H, I, d = cfg.M, cfg.H, cfg.I, cfg.d
    nq, nkv = cfg.nq, cfg.nkv
    pos = np.arange(M) % cfg.S
    x = bf16_bits_to_f32(x_bits)
    wf = {k: (bf16_bits_to_f32(v) if v.dtype == np.uint16 else v) for k, v in w.items()}
    saved = {"x": x_bits}
    if cfg.kind == "llama":
        rstd1 = (1.0 / np.sqrt((x.astype(np.float64) ** 2).mean(axis=1) + cfg.eps)).astype(np.float32)
        xn1 = x * rstd1[:, None] * wf["gamma1"][None, :]
    else:
        x64 = x.astype(np.float64)
        mean = x64.mean(axis=1)
        rstd = 1.0 / np.sqrt(((x64 - mean[:, None]) ** 2).mean(axis=1) + cfg.eps)
        mean, rstd = mean.astype(np.float32), rstd.astype(np.float32)
        xn1 = (x - mean[:, None]) * rstd[:, None] * wf["gamma"][None, :] + wf["beta"][None, :]
        saved["mean"], saved["rstd"] = mean, rstd
    qkv = xn1 @ wf["w_qkv"].T
    q = _rope_fwd(qkv[:, : nq * d], pos, nq, d, cfg.rot, cfg.rope_base)
    k = _rope_fwd(qkv[:, nq * d:(nq + nkv) * d], pos, nkv, d, cfg.rot, cfg.rope_base)
    v = qkv[:, (nq + nkv) * d:]
    q, k, v = _round_bf16(q), _round_bf16(k), _round_bf16(v)
    o, lse = _attention_fwd(q, k, v, cfg.B, cfg.S, nq, nkv, d)
    o = _round_bf16(o)
    saved.update(q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v),
                 o=f32_to_bf16_bits(o), lse=lse)
    attn = o @ wf["w_o"].T
    if cfg.kind == "llama":
        saved["rstd1"] = rstd1
        h = _round_bf16(x + attn)
        rstd2 = (1.0 / np.sqrt((h.astype(np.float64) ** 2).mean(axis=1) + cfg.eps)).astype(np.float32)
        xn2 = h * rstd2[:, None] * wf["gamma2"][None, :]
        gu = xn2 @ wf["w_gateup"].T
        gate, up = _round_bf16(gu[:, :I]), _round_bf16(gu[:, I:])
        a = gate / (1.0 + np.exp(-gate)) * up
        y = h + a @ wf["w_down"].T
        saved.update(h=f32_to_bf16_bits(h), rstd2=rstd2, gate=f32_to_bf16_bits(gate),
                     up=f32_to_bf16_bits(up))
    else:
        f = _round_bf16(xn1 @ wf["w_fc1"].T)
        y = x + attn + _gelu_tanh(f) @ wf["w_fc2"].T
        saved["f"] = f32_to_bf16_bits(f)
    return saved, f32_to_bf16_bits(y)


def make_layer_inputs(cfg: LayerShape, seed=None, r_pct=None, keep=None) -> dict:
    """One layer: weights, saved activations from a forward pass, upstream gradient dY ~ N(0,1)
    (filtered rows deliberately non-zero) and the keep mask."""
    seed = cfg.seed if seed is None else seed
    r_pct = cfg.r_pct if r_pct is None else r_pct
    w = make_layer_weights(cfg, seed)
    x_bits = f32_to_bf16_bits(rng_for(seed, "x").standard_normal((cfg.M, cfg.H)).astype(np.float32))
    saved, _ = layer_forward(cfg, w, x_bits)
    dy = f32_to_bf16_bits(rng_for(seed, "dy").standard_normal((cfg.M, cfg.H)).astype(np.float32))
    if keep is None:
        keep = make_keep(cfg.M, r_pct, seed)
    return {"cfg": cfg, "weights": w, "saved": saved, "dy": dy, "keep": keep}


def make_model_inputs(cfg: LayerShape, seed=None, r_pct=None, n_layers=None) -> dict:
    """A stack of layers: one consistent forward from x0 ~ N(0,1), per-layer weights and saved
    activations, dY of the top layer ~ N(0,1), one keep mask shared by every layer."""
    seed = cfg.seed if seed is None else seed
    r_pct = cfg.r_pct if r_pct is None else r_pct
    L = cfg.n_layers if n_layers is None else n_layers
    x_bits = f32_to_bf16_bits(rng_for(seed, "x").standard_normal((cfg.M, cfg.H)).astype(np.float32))
    layers = []
    for li in range(L):
        w = make_layer_weights(cfg, seed, li)
        saved, x_bits = layer_forward(cfg, w, x_bits)
        layers.append({"weights": w, "saved": saved})
    dy = f32_to_bf16_bits(rng_for(seed, "dy").standard_normal((cfg.M, cfg.H)).astype(np.float32))
    return {"cfg": cfg, "layers": layers, "dy": dy, "keep": make_keep(cfg.M, r_pct, seed)}


def floats(d: dict) -> dict:
    """Copy of a dict with bf16 bit arrays (uint16) widened to float32; other entries unchanged."""
    return {k: (bf16_bits_to_f32(v) if isinstance(v, np.ndarray) and v.dtype == np.uint16 else v)
            for k, v in d.items()}
