"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bars: bit-exact for index / gather / scatter; max|d|/max|ref| <= 2e-2 for bf16 outputs and <= 1e-4
for the fp32 linear layer; rows of filtered tokens exactly zero in full-layout outputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
import token_filtered_backward_amd as tfb
from tests.helpers import BF16_TOL, F32_TOL, bf16_dev, f32_dev, rel_err, to64, upcast

pytestmark = pytest.mark.gpu


def _keep(M, pattern, seed=0, r=40):
    rng = np.random.default_rng(seed)
    if pattern == "all":
        return np.ones(M, np.uint8)
    if pattern == "none":
        return np.zeros(M, np.uint8)
    if pattern == "rand":
        return (rng.random(M) < 0.6).astype(np.uint8) * rng.integers(1, 256, M).astype(np.uint8)
    return synth.make_keep(M, r, seed)


def _dev_keep(keep):
    return torch.from_numpy(np.ascontiguousarray(keep, np.uint8)).cuda()


# ------------------------------------------------------------------------------------------------
# index, gather, scatter: bit-exact
# ------------------------------------------------------------------------------------------------


@pytest.mark.parametrize("B,S,pattern", [(1, 1, "all"), (1, 1, "none"), (1, 7, "none"), (3, 11, "rand"),
                                         (4, 2048, "topk"), (2, 4096, "topk"), (1, 8192, "topk"),
                                         (5, 3001, "rand"), (1, 70000, "rand"), (2, 5, "all"),
                                         (1, 16384, "topk"), (1, 16385, "rand"), (3, 400001, "rand"),
                                         (1024, 1024, "topk"), (1, 1 << 22, "rand")])
def test_build_index_bit_exact(B, S, pattern):
    keep = _keep(B * S, pattern, seed=B + S)
    ix = tfb.build_index(_dev_keep(keep), B, S)
    torch.cuda.synchronize()
    ref = oracle.build_index(keep, B, S)
    assert ix.M_kept == ref["count"]
    assert np.array_equal(ix.idx.cpu().numpy(), ref["partition"])
    assert np.array_equal(ix.inv.cpu().numpy(), ref["inv"])
    assert np.array_equal(ix.cu_seqlens.cpu().numpy(), ref["cu_seqlens"])
    assert int(ix.count.cpu()[0]) == ref["count"]


@pytest.mark.parametrize("B,S,pattern", [(4, 2048, "topk"), (5, 3001, "rand"), (1, 70000, "rand"),
                                         (1, 7, "none"), (2, 5, "all"), (3, 400001, "rand")])
@pytest.mark.parametrize("delta", [0, -5, 3])
def test_build_index_with_announced_count(B, S, pattern, delta):
    """The index build that takes the kept count from the caller: with the true count it equals the
    ordinary build bit for bit; with a wrong one it flags the mismatch and keeps inv / cu_seqlens
    inside the announced count (idx stays the full partition, count the true count)."""
    keep = _keep(B * S, pattern, seed=B * S + 1)
    ref = oracle.build_index(keep, B, S)
    n = ref["count"]
    expect = min(max(n + delta, 0), B * S)
    ix = tfb.build_index(_dev_keep(keep), B, S, expect=expect)
    assert ix.M_kept == expect
    idx, inv = ix.idx.cpu().numpy(), ix.inv.cpu().numpy()
    cu, count, mm = ix.cu_seqlens.cpu().numpy(), int(ix.count.cpu()[0]), int(ix.mismatch.cpu()[0])
    assert count == n and np.array_equal(idx, ref["partition"])
    assert mm == int(expect != n)
    exp_inv = np.where(ref["inv"] < expect, ref["inv"], -1)
    assert np.array_equal(inv, exp_inv)
    assert np.array_equal(cu, np.minimum(ref["cu_seqlens"], expect))
    if expect == n:
        ix.check()
    else:
        with pytest.raises(tfb.ColliderError):
            ix.check()


@pytest.mark.parametrize("cols,dtype", [(2048, torch.bfloat16), (256, torch.bfloat16), (32, torch.float32),
                                        (12, torch.bfloat16), (5, torch.float32), (4096, torch.float32)])
def test_gather_scatter_bit_exact(cols, dtype):
    B, S = 3, 517
    M = B * S
    keep = _keep(M, "topk", seed=cols)
    ix = tfb.build_index(_dev_keep(keep), B, S)
    rng = np.random.default_rng(cols)
    if dtype == torch.bfloat16:
        bits = rng.integers(0, 2 ** 16, size=(M, cols), dtype=np.uint16)
        src = bf16_dev(bits)
        src_np = bits
    else:
        src_np = rng.standard_normal((M, cols)).astype(np.float32)
        src = f32_dev(src_np)
    mk = ix.M_kept
    dst = torch.empty((mk, cols), dtype=dtype, device="cuda")
    tfb.collider_gather_rows(src, dst, ix.idx, mk)
    ref_idx = oracle.build_index(keep, B, S)["idx"]
    got = dst.cpu().view(torch.int16).numpy().view(np.uint16) if dtype == torch.bfloat16 else dst.cpu().numpy()
    assert np.array_equal(got, oracle.gather_rows(src_np, ref_idx))
    # scatter back with zero fill over a poisoned destination
    full = torch.full((M, cols), float("nan"), dtype=dtype, device="cuda")
    tfb.collider_scatter_rows(dst, full, ix.inv, M, zero_fill_filtered=True)
    back = full.cpu().view(torch.int16).numpy().view(np.uint16) if dtype == torch.bfloat16 else full.cpu().numpy()
    assert np.array_equal(back, oracle.scatter_rows(got, ref_idx, M))
    # without zero fill the filtered rows are untouched
    full2 = torch.full((M, cols), 7.0, dtype=dtype, device="cuda")
    tfb.collider_scatter_rows(dst, full2, ix.inv, M, zero_fill_filtered=False)
    f2 = full2.float().cpu().numpy()
    assert np.all(f2[keep == 0] == 7.0)


# ------------------------------------------------------------------------------------------------
# linear layer
# ------------------------------------------------------------------------------------------------


def test_linear_fp32_single_layer():
    cfg = synth.get_config("linear_fp32")
    inp = synth.make_linear_inputs(cfg)
    keep = inp["keep"]
    ix = tfb.build_index(_dev_keep(keep), cfg.B, cfg.S)
    assert ix.M_kept == 154
    x, dy, w = f32_dev(inp["x"]), f32_dev(inp["dy"]), f32_dev(inp["w"])
    mk = ix.M_kept
    x_c = torch.empty((mk, cfg.K), device="cuda")
    dy_c = torch.empty((mk, cfg.N), device="cuda")
    tfb.collider_gather_rows(x, x_c, ix.idx, mk)
    tfb.collider_gather_rows(dy, dy_c, ix.idx, mk)
    dx_c = torch.empty((mk, cfg.K), device="cuda")
    dw = torch.empty((cfg.N, cfg.K), device="cuda")
    db = torch.empty(cfg.N, device="cuda")
    tfb.collider_linear_bwd_reduced(x_c, dy_c, w, dx_c, dw, db)
    dx = torch.empty((cfg.M, cfg.K), device="cuda")
    tfb.collider_scatter_rows(dx_c, dx, ix.inv, cfg.M)
    ref = oracle.linear_bwd(inp["x"], inp["dy"], inp["w"], keep, bias=True)
    assert rel_err(to64(dx), ref["dx"]) <= F32_TOL
    assert rel_err(to64(dw), ref["dw"]) <= F32_TOL
    assert rel_err(to64(db), ref["db"]) <= F32_TOL
    assert np.all(to64(dx)[keep == 0] == 0.0)


@pytest.mark.parametrize("Mk,K,N", [(1, 8, 8), (77, 64, 136), (300, 256, 512), (1000, 520, 264),
                                    (4916, 2048, 2048), (4916, 2048, 5632), (4916, 5632, 2048),
                                    (4916, 1536, 8960), (0, 64, 64)])
def test_linear_bf16(Mk, K, N):
    rng = np.random.default_rng(Mk + K + N)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((Mk, K)).astype(np.float32))
    dyb = synth.f32_to_bf16_bits(rng.standard_normal((Mk, N)).astype(np.float32))
    wb = synth.f32_to_bf16_bits(0.02 * rng.standard_normal((N, K)).astype(np.float32))
    x, dy, w = bf16_dev(xb), bf16_dev(dyb), bf16_dev(wb)
    dx = torch.empty((Mk, K), dtype=torch.bfloat16, device="cuda")
    dw = torch.full((N, K), float("nan"), device="cuda")
    db = torch.full((N,), float("nan"), device="cuda")
    tfb.collider_linear_bwd_reduced(x, dy, w, dx, dw, db)
    ref = oracle.linear_bwd(synth.bf16_bits_to_f32(xb), synth.bf16_bits_to_f32(dyb),
                            synth.bf16_bits_to_f32(wb), np.ones(Mk, np.uint8), bias=True)
    if Mk == 0:
        assert np.all(to64(dw) == 0.0) and np.all(to64(db) == 0.0)
        return
    assert rel_err(to64(dx), ref["dx"]) <= 1e-2
    assert rel_err(to64(dw), ref["dw"]) <= 1e-3
    assert rel_err(to64(db), ref["db"]) <= 1e-3
    # accumulate adds onto the previous contents
    tfb.collider_linear_bwd_reduced(x, dy, w, None, dw, None, accumulate=True)
    assert rel_err(to64(dw), 2 * ref["dw"]) <= 1e-3


@pytest.fixture
def gemm_policy():
    """Sets a GEMM work-decomposition policy for one test and restores the cost model after it."""
    def set_(policy):
        tfb.collider_gemm_set_policy(policy)
    yield set_
    tfb.collider_gemm_set_policy(tfb.GEMM_POLICY_AUTO)


@pytest.mark.parametrize("policy", [tfb.GEMM_POLICY_SPLITK, tfb.GEMM_POLICY_STREAMK, tfb.GEMM_POLICY_TILES])
@pytest.mark.parametrize("Mk,K,N", [(77, 64, 136), (300, 256, 512), (1000, 520, 264), (2500, 768, 1280),
                                    (4916, 2048, 5632), (4916, 5632, 2048)])
def test_linear_bf16_policies(gemm_policy, policy, Mk, K, N):
    """Every work decomposition (whole tiles, K-splits, stream-K with its fix-up pass) meets the
    bar, and repeating a call reproduces it bitwise."""
    gemm_policy(policy)
    rng = np.random.default_rng(Mk * 7 + K + N)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((Mk, K)).astype(np.float32))
    dyb = synth.f32_to_bf16_bits(rng.standard_normal((Mk, N)).astype(np.float32))
    wb = synth.f32_to_bf16_bits(0.02 * rng.standard_normal((N, K)).astype(np.float32))
    x, dy, w = bf16_dev(xb), bf16_dev(dyb), bf16_dev(wb)
    dx = torch.full((Mk, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    dw = torch.full((N, K), float("nan"), device="cuda")
    tfb.collider_linear_bwd_reduced(x, dy, w, dx, dw)
    ref = oracle.linear_bwd(synth.bf16_bits_to_f32(xb), synth.bf16_bits_to_f32(dyb),
                            synth.bf16_bits_to_f32(wb), np.ones(Mk, np.uint8))
    assert rel_err(to64(dx), ref["dx"]) <= 1e-2
    assert rel_err(to64(dw), ref["dw"]) <= 1e-3
    dx2, dw2 = torch.empty_like(dx), torch.empty_like(dw)
    tfb.collider_linear_bwd_reduced(x, dy, w, dx2, dw2)
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16)) and torch.equal(dw, dw2)
    tfb.collider_linear_bwd_reduced(x, dy, w, None, dw, accumulate=True)
    assert rel_err(to64(dw), 2 * ref["dw"]) <= 1e-3


# ------------------------------------------------------------------------------------------------
# attention
# ------------------------------------------------------------------------------------------------


def _attn_case(name, r, dmode, seed=0):
    cfg = synth.get_config(name)
    inp = synth.make_layer_inputs(cfg, seed=seed, r_pct=r)
    keep = inp["keep"]
    sv = upcast(inp["saved"])
    rng = np.random.default_rng(seed + 1)
    dob = synth.f32_to_bf16_bits(rng.standard_normal((cfg.M, cfg.nq * cfg.d)).astype(np.float32))
    mode = "filtered" if dmode == 0 else "full_d"
    dq, dk, dv = oracle.attention_bwd(sv["q"], sv["k"], sv["v"], sv["o"], sv["lse"],
                                      synth.bf16_bits_to_f32(dob), keep, cfg.B, cfg.S, cfg.nq, cfg.nkv,
                                      cfg.d, mode=mode)
    pos = np.arange(cfg.M) % cfg.S
    dq = oracle.rope_bwd(dq, pos, cfg.nq, cfg.d, cfg.rot, cfg.rope_base)
    dk = oracle.rope_bwd(dk, pos, cfg.nkv, cfg.d, cfg.rot, cfg.rope_base)
    return cfg, inp, dob, (dq, dk, dv)


@pytest.mark.parametrize("name", ["small_llama", "small_llama_d128", "small_phi"])
@pytest.mark.parametrize("dmode", [0, 1])
@pytest.mark.parametrize("r", [0, 40, 90])
def test_attention_parity(name, dmode, r):
    check_attention(name, r, dmode)


def check_attention(name, r, dmode):
    """collider_attn_bwd_filtered on compacted q, k, v, o, lse, dO against the oracle's attention
    backward (then its RoPE backward) on the full token layout, at the kept rows."""
    cfg, inp, dob, ref = _attn_case(name, r, dmode)
    keep = inp["keep"]
    ix = tfb.build_index(_dev_keep(keep), cfg.B, cfg.S)
    mk = ix.M_kept
    nqd, nkvd = cfg.nq * cfg.d, cfg.nkv * cfg.d
    full = {k: bf16_dev(inp["saved"][k]) for k in ("q", "k", "v", "o")}
    full["lse"] = f32_dev(inp["saved"]["lse"])
    full["do"] = bf16_dev(dob)
    comp = {}
    for k, t in full.items():
        comp[k] = torch.empty((mk, t.shape[1]), dtype=t.dtype, device="cuda")
        tfb.collider_gather_rows(t, comp[k], ix.idx, mk)
    out = {k: torch.empty((mk, n), dtype=torch.bfloat16, device="cuda") for k, n in
           (("dq", nqd), ("dk", nkvd), ("dv", nkvd))}
    acfg = tfb.AttnCfg(cfg.nq, cfg.nkv, cfg.d, cfg.rot, cfg.rope_base, 0.0, dmode)
    io = tfb.AttnIO(comp["q"].data_ptr(), nqd, comp["k"].data_ptr(), nkvd, comp["v"].data_ptr(), nkvd,
                    comp["o"].data_ptr(), nqd, comp["lse"].data_ptr(), cfg.nq, comp["do"].data_ptr(), nqd,
                    out["dq"].data_ptr(), nqd, out["dk"].data_ptr(), nkvd, out["dv"].data_ptr(), nkvd)
    cix = ix.c()
    ws = torch.empty(max(1, tfb.collider_attn_workspace_bytes(acfg, cix)), dtype=torch.uint8, device="cuda")
    tfb.collider_attn_bwd_filtered(acfg, cix, io, ws)
    idx = ix.idx[:mk].cpu().numpy()
    for name_, r_ in zip(("dq", "dk", "dv"), ref):
        e = rel_err(to64(out[name_]), r_[idx])
        assert e <= BF16_TOL, (name_, e)


# ------------------------------------------------------------------------------------------------
# whole layer
# ------------------------------------------------------------------------------------------------


def _upload_layer(inp):
    cfg = inp["cfg"]
    W = {}
    for k, v in inp["weights"].items():
        W[k] = bf16_dev(v) if v.dtype == np.uint16 else f32_dev(v)
    S = {}
    for k, v in inp["saved"].items():
        S[k] = bf16_dev(v) if v.dtype == np.uint16 else f32_dev(v)
    if cfg.kind == "llama":
        weights = dict(w_qkv=W["w_qkv"], w_o=W["w_o"], w_gateup=W["w_gateup"], w_down=W["w_down"],
                       gamma1=W["gamma1"], gamma2=W["gamma2"])
        saved = dict(x=S["x"], q=S["q"], k=S["k"], v=S["v"], o=S["o"], lse=S["lse"], rstd1=S["rstd1"],
                     h=S["h"], rstd2=S["rstd2"], gate=S["gate"], up=S["up"])
    else:
        weights = dict(w_qkv=W["w_qkv"], w_o=W["w_o"], w_fc1=W["w_fc1"], w_fc2=W["w_fc2"],
                       ln_gamma=W["gamma"], ln_beta=W["beta"])
        saved = dict(x=S["x"], q=S["q"], k=S["k"], v=S["v"], o=S["o"], lse=S["lse"], rstd1=S["rstd"],
                     mean=S["mean"], f=S["f"])
    return weights, saved, bf16_dev(inp["dy"])


GRAD_NAMES = {"llama": {"dx": "dx", "dw_qkv": "dw_qkv", "dw_o": "dw_o", "dw_gateup": "dw_gateup",
                        "dw_down": "dw_down", "dgamma1": "dgamma1", "dgamma2": "dgamma2"},
              "phi": {"dx": "dx", "dw_qkv": "dw_qkv", "dw_o": "dw_o", "dw_fc1": "dw_fc1", "dw_fc2": "dw_fc2",
                      "dln_gamma": "dgamma", "dln_beta": "dbeta"}}


def run_layer_and_compare(inp, dmode, tol=BF16_TOL):
    cfg = inp["cfg"]
    keep = inp["keep"]
    weights, saved, dy = _upload_layer(inp)
    ix = tfb.build_index(_dev_keep(keep), cfg.B, cfg.S)
    lcfg = tfb.layer_cfg(cfg, dmode=dmode)
    grads = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda")
    for g in grads.values():
        g.fill_(float("nan"))
    tfb.layer_bwd(lcfg, weights, saved, dy, ix, grads)
    torch.cuda.synchronize()
    ref = oracle.layer_bwd(cfg, upcast(inp["weights"]), upcast(inp["saved"]),
                           synth.bf16_bits_to_f32(inp["dy"]), keep,
                           "filtered" if dmode == 0 else "full_d")
    errs = {}
    for gname, oname in GRAD_NAMES[cfg.kind].items():
        errs[gname] = rel_err(to64(grads[gname]), ref[oname])
    assert np.all(to64(grads["dx"])[keep == 0] == 0.0)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, errs
    return errs


@pytest.mark.parametrize("name", ["small_llama", "small_llama_d128", "small_phi"])
@pytest.mark.parametrize("dmode", [0, 1])
@pytest.mark.parametrize("r", [0, 40, 75])
def test_layer_parity_small(name, dmode, r):
    inp = synth.make_layer_inputs(synth.get_config(name), r_pct=r)
    run_layer_and_compare(inp, dmode)


@pytest.mark.parametrize("name", ["small_llama", "small_llama_d128", "small_phi"])
@pytest.mark.parametrize("r", [0, 40])
def test_layer_weight_layouts(name, r):
    """Weights stored [in, out] give the same gradients as [out, in] - dx and the norm gains bit for
    bit, every weight gradient as the exact transpose - and match the oracle."""
    cfg = synth.get_config(name)
    inp = synth.make_layer_inputs(cfg, r_pct=r)
    weights, saved, dy = _upload_layer(inp)
    ix = tfb.build_index(_dev_keep(inp["keep"]), cfg.B, cfg.S)
    out = {}
    for layout, w in ((tfb.WEIGHTS_OUT_IN, weights), (tfb.WEIGHTS_IN_OUT, tfb.to_in_out(weights))):
        lcfg = tfb.layer_cfg(cfg, weight_layout=layout)
        grads = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda")
        for g in grads.values():
            g.fill_(float("nan"))
        tfb.layer_bwd(lcfg, w, saved, dy, ix, grads)
        torch.cuda.synchronize()
        out[layout] = grads
    g0, g1 = out[tfb.WEIGHTS_OUT_IN], out[tfb.WEIGHTS_IN_OUT]
    for k in g0:
        a = g1[k].t() if k.startswith("dw_") else g1[k]
        b = g0[k]
        assert a.shape == b.shape, k
        same = torch.equal(a.contiguous().view(torch.int16), b.view(torch.int16)) if b.dtype == torch.bfloat16 \
            else torch.equal(a.contiguous(), b)
        assert same, k
    ref = oracle.layer_bwd(cfg, upcast(inp["weights"]), upcast(inp["saved"]),
                           synth.bf16_bits_to_f32(inp["dy"]), inp["keep"], "filtered")
    for gname, oname in GRAD_NAMES[cfg.kind].items():
        got = to64(g1[gname])
        got = got.T if gname.startswith("dw_") else got
        assert rel_err(got, ref[oname]) <= BF16_TOL, gname


@pytest.mark.parametrize("policy", [tfb.GEMM_POLICY_SPLITK, tfb.GEMM_POLICY_STREAMK, tfb.GEMM_POLICY_TILES])
@pytest.mark.parametrize("name", ["small_llama", "small_phi"])
def test_layer_parity_gemm_policies(gemm_policy, policy, name):
    """The fused SwiGLU / GELU / fp32 epilogues give the same gradients through every GEMM work
    decomposition, including the stream-K fix-up pass."""
    gemm_policy(policy)
    inp = synth.make_layer_inputs(synth.get_config(name), r_pct=40)
    run_layer_and_compare(inp, 0)


@pytest.mark.parametrize("name,layout", [("small_llama", 0), ("small_phi", 0), ("small_llama", 1),
                                         ("small_phi", 1)])
def test_layer_all_filtered(name, layout):
    cfg = synth.get_config(name)
    inp = synth.make_layer_inputs(cfg, keep=np.zeros(cfg.M, np.uint8))
    weights, saved, dy = _upload_layer(inp)
    if layout == tfb.WEIGHTS_IN_OUT:
        weights = tfb.to_in_out(weights)
    ix = tfb.build_index(_dev_keep(inp["keep"]), cfg.B, cfg.S)
    assert ix.M_kept == 0
    lcfg = tfb.layer_cfg(cfg, weight_layout=layout)
    grads = tfb.make_grads(lcfg, cfg.M, 0, "cuda")
    for g in grads.values():
        g.fill_(float("nan"))
    tfb.layer_bwd(lcfg, weights, saved, dy, ix, grads)
    for k, g in grads.items():
        assert torch.all(g == 0).item(), k


@pytest.mark.parametrize("layout", [0, 1])
def test_layer_compact_chain_matches_full_layout(layout):
    """dx_compact of the upper layer feeding dy_compact of the lower one equals the full-layout path."""
    cfg = synth.get_config("small_llama")
    inp = synth.make_layer_inputs(cfg)
    weights, saved, dy = _upload_layer(inp)
    if layout == tfb.WEIGHTS_IN_OUT:
        weights = tfb.to_in_out(weights)
    ix = tfb.build_index(_dev_keep(inp["keep"]), cfg.B, cfg.S)
    lcfg = tfb.layer_cfg(cfg, weight_layout=layout)
    g_full = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda")
    tfb.layer_bwd(lcfg, weights, saved, dy, ix, g_full)
    g_c = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda", dx_compact=True)
    tfb.layer_bwd(lcfg, weights, saved, dy, ix, g_c, dx_compact=True)
    idx = ix.idx[: ix.M_kept].long()
    assert torch.equal(g_c["dx"], g_full["dx"][idx])
    # feed the compact dx down as a compact dy: equals feeding the full-layout dx
    g1 = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda")
    tfb.layer_bwd(lcfg, weights, saved, g_full["dx"], ix, g1)
    g2 = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda")
    tfb.layer_bwd(lcfg, weights, saved, g_c["dx"], ix, g2, dy_compact=True)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


@pytest.mark.parametrize("name", ["small_llama", "small_phi"])
def test_layer_every_token_kept_is_the_dense_path(name):
    """An index that keeps every token gives exactly the unfiltered baseline's gradients, in the
    full layout, compact (dx_compact) and from a compact dy alike."""
    cfg = synth.get_config(name)
    inp = synth.make_layer_inputs(cfg, r_pct=0)
    weights, saved, dy = _upload_layer(inp)
    keep = np.ones(cfg.M, dtype=np.uint8)
    ix = tfb.build_index(_dev_keep(keep), cfg.B, cfg.S)
    assert ix.M_kept == cfg.M
    g_dense = tfb.make_grads(tfb.layer_cfg(cfg, unfiltered=True), cfg.M, cfg.M, "cuda")
    tfb.layer_bwd(tfb.layer_cfg(cfg, unfiltered=True), weights, saved, dy, tfb.dense_index(cfg.B, cfg.S),
                  g_dense)
    lcfg = tfb.layer_cfg(cfg)
    g_full = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda")
    tfb.layer_bwd(lcfg, weights, saved, dy, ix, g_full)
    g_c = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda", dx_compact=True)
    tfb.layer_bwd(lcfg, weights, saved, dy, ix, g_c, dx_compact=True, dy_compact=True)
    for k in g_dense:
        assert torch.equal(g_full[k], g_dense[k]), k
        assert torch.equal(g_c[k], g_dense[k]), k


@pytest.mark.parametrize("name,layout", [("small_llama", 0), ("small_llama", 1), ("small_phi", 0),
                                         ("small_phi", 1)])
def test_layer_accumulate_adds_onto_weight_and_gain_gradients(name, layout):
    """accumulate != 0 adds every weight, gain and bias gradient onto what its buffer holds (one
    fp32 addition: bit for bit the old value plus the gradient of a call without accumulate) and
    writes dx as that call does."""
    cfg = synth.get_config(name)
    inp = synth.make_layer_inputs(cfg, seed=2)
    weights, saved, dy = _upload_layer(inp)
    if layout == tfb.WEIGHTS_IN_OUT:
        weights = tfb.to_in_out(weights)
    ix = tfb.build_index(_dev_keep(inp["keep"]), cfg.B, cfg.S)
    lcfg = tfb.layer_cfg(cfg, weight_layout=layout)
    fresh = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda")
    tfb.layer_bwd(lcfg, weights, saved, dy, ix, fresh)
    acfg = tfb.layer_cfg(cfg, accumulate=True, weight_layout=layout)
    acc = tfb.make_grads(acfg, cfg.M, ix.M_kept, "cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    prior = {}
    for k, g in acc.items():
        if g.dtype == torch.float32:
            g.copy_(torch.randn(g.shape, generator=gen, device="cuda"))
        else:
            g.fill_(float("nan"))
        prior[k] = g.clone()
    tfb.layer_bwd(acfg, weights, saved, dy, ix, acc)
    torch.cuda.synchronize()
    for k in fresh:
        if k == "dx":
            assert torch.equal(acc[k].view(torch.int16), fresh[k].view(torch.int16)), k
        else:
            assert torch.equal(acc[k], prior[k] + fresh[k]), k


@pytest.mark.parametrize("name", ["small_llama", "small_phi"])
def test_stack_of_layers(name):
    """Three layers from one consistent forward, chained top to bottom with compact gradients
    between layers (the same mask in every layer), against the oracle's stack backward."""
    cfg = synth.get_config(name)
    model = synth.make_model_inputs(cfg, seed=3, r_pct=40, n_layers=3)
    keep = model["keep"]
    ix = tfb.build_index(_dev_keep(keep), cfg.B, cfg.S)
    lcfg = tfb.layer_cfg(cfg)
    lb = tfb.LayerBackward(lcfg, cfg.B, cfg.S, "cuda")
    g = bf16_dev(model["dy"])
    outs = []
    for li in reversed(range(3)):
        inp = dict(cfg=cfg, weights=model["layers"][li]["weights"], saved=model["layers"][li]["saved"],
                   dy=model["dy"])
        weights, saved, _ = _upload_layer(inp)
        grads = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda", dx_compact=li > 0)
        lb(weights, saved, g, ix, grads, dy_compact=li < 2, dx_compact=li > 0)
        outs.append(grads)
        g = grads["dx"]
    torch.cuda.synchronize()
    ref = oracle.model_bwd(cfg, [{"weights": upcast(l["weights"]), "saved": upcast(l["saved"])}
                                 for l in model["layers"]], synth.bf16_bits_to_f32(model["dy"]), keep)
    idx = ix.idx[:ix.M_kept].cpu().numpy()
    for li, grads in zip(reversed(range(3)), outs):
        for gname, oname in GRAD_NAMES[cfg.kind].items():
            r = ref[li][oname]
            if gname == "dx" and li > 0:
                r = r[idx]  # compact rows
            e = rel_err(to64(grads[gname]), r)
            assert e <= BF16_TOL, (li, gname, e)
    assert np.all(to64(outs[-1]["dx"])[keep == 0] == 0.0)


@pytest.mark.parametrize("base,changes", [
    ("small_llama", dict(H=4608, B=1, S=160)),             # hidden > 4096: the two-sweep norm backward
    ("small_phi", dict(H=4160, B=1, S=160)),               # ... with a ragged last 8-vector per lane
    ("small_llama", dict(nq=6, nkv=2, rot=24)),            # head count not a multiple of 4, rotary
    ("small_llama_d128", dict(nq=3, nkv=1, rot=40)),       # widths not multiples of 16 (rot/2 and
    ("small_phi", dict(nq=6, nkv=6, rot=20)),              # rot fall inside groups of 8 columns)
])
@pytest.mark.parametrize("dmode", [0, 1])
def test_layer_parity_wider_shapes(base, changes, dmode):
    """Layer shapes outside the benchmark models' envelope: hidden sizes past 4096 and head counts /
    rotary widths that do not divide into the kernels' vector widths, against the oracle."""
    cfg = synth.get_config(base).with_(name=base + "_wide", **changes)
    inp = synth.make_layer_inputs(cfg, r_pct=40)
    run_layer_and_compare(inp, dmode)


@pytest.mark.parametrize("name", ["small_llama", "small_phi"])
def test_layer_graph_replay_matches_eager(name):
    """The layer recorded into a HIP graph and replayed gives the eager result bit for bit, on every
    replay, with eager work and synchronisation between replays and with a new mask of the same
    kept count rebuilt in place, the count taken from the device or announced by the host."""
    cfg = synth.get_config(name)
    inp = synth.make_layer_inputs(cfg, r_pct=40)
    weights, saved, dy = _upload_layer(inp)
    lcfg = tfb.layer_cfg(cfg)
    keep1 = inp["keep"]
    keep2 = synth.make_keep(cfg.M, 40, 77)  # another mask, same kept count
    assert keep1.sum() == keep2.sum()

    def eager(keep):
        ix = tfb.build_index(_dev_keep(keep), cfg.B, cfg.S)
        g = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda")
        tfb.LayerBackward(lcfg, cfg.B, cfg.S, "cuda")(weights, saved, dy, ix, g)
        torch.cuda.synchronize()
        return {k: v.clone() for k, v in g.items()}

    ref1, ref2 = eager(keep1), eager(keep2)
    lb = tfb.LayerBackward(lcfg, cfg.B, cfg.S, "cuda")
    ix = tfb.build_index(_dev_keep(keep1), cfg.B, cfg.S)
    grads = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda")
    junk = torch.zeros(1 << 20, device="cuda")
    for rep, (keep, ref) in enumerate([(keep1, ref1), (keep1, ref1), (keep2, ref2), (keep1, ref1)]):
        # odd replays take the kept count from the host (no wait for the index build)
        ix = tfb.build_index(_dev_keep(keep), cfg.B, cfg.S, out=ix,
                             expect=int(keep.sum()) if rep % 2 else None)
        for gt in grads.values():
            gt.fill_(float("nan"))
        lb(weights, saved, dy, ix, grads, graph=True)
        junk.add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
        for k in ref:
            a, b = grads[k], ref[k]
            same = torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 \
                else torch.equal(a, b)
            assert same, (rep, k)
        ix.check()


@pytest.mark.parametrize("name", ["small_llama", "small_phi"])
def test_index_and_layer_in_one_graph(name):
    """A whole step - the index build from the mask, with the kept count announced by the host, and
    the layer - recorded into one HIP graph: every replay gives the eager result bit for bit, with a
    new mask of the same kept count written into the captured mask buffer between replays, and eager
    work and synchronisation in between."""
    cfg = synth.get_config(name)
    inp = synth.make_layer_inputs(cfg, r_pct=40)
    weights, saved, dy = _upload_layer(inp)
    lcfg = tfb.layer_cfg(cfg)
    keep1 = inp["keep"]
    keep2 = synth.make_keep(cfg.M, 40, 77)  # another mask, same kept count
    n = int(keep1.sum())
    assert n == int(keep2.sum())

    def eager(keep):
        ix = tfb.build_index(_dev_keep(keep), cfg.B, cfg.S)
        g = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda")
        tfb.LayerBackward(lcfg, cfg.B, cfg.S, "cuda")(weights, saved, dy, ix, g)
        torch.cuda.synchronize()
        return {k: v.clone() for k, v in g.items()}

    ref1, ref2 = eager(keep1), eager(keep2)
    keep_dev = _dev_keep(keep1)
    ix = tfb.build_index(keep_dev, cfg.B, cfg.S)
    lb = tfb.LayerBackward(lcfg, cfg.B, cfg.S, "cuda")
    grads = tfb.make_grads(lcfg, cfg.M, n, "cuda")

    def step():
        tfb.build_index(keep_dev, cfg.B, cfg.S, out=ix, expect=n)
        lb(weights, saved, dy, ix, grads)

    step()  # eager first: workspace and mismatch flag exist before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    junk = torch.zeros(1 << 20, device="cuda")
    for rep, (keep, ref) in enumerate([(keep1, ref1), (keep2, ref2), (keep2, ref2), (keep1, ref1)]):
        keep_dev.copy_(_dev_keep(keep))
        for gt in grads.values():
            gt.fill_(float("nan"))
        graph.replay()
        junk.add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
        for k in ref:
            a, b = grads[k], ref[k]
            same = torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 \
                else torch.equal(a, b)
            assert same, (rep, k)
        ix.check()


def test_layer_repeat_is_deterministic():
    cfg = synth.get_config("small_llama")
    inp = synth.make_layer_inputs(cfg)
    weights, saved, dy = _upload_layer(inp)
    ix = tfb.build_index(_dev_keep(inp["keep"]), cfg.B, cfg.S)
    lcfg = tfb.layer_cfg(cfg)
    a = tfb.layer_bwd(lcfg, weights, saved, dy, ix)
    b = tfb.layer_bwd(lcfg, weights, saved, dy, ix)
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("name,layout", [("small_llama", 0), ("small_llama_d128", 0), ("small_phi", 0),
                                         ("small_llama", 1), ("small_phi", 1)])
def test_unfiltered_baseline(name, layout):
    """The dense baseline equals the filtered path with every token kept (same kernels, same
    numerics, dmode FULL) and the oracle's ordinary backward, in either weight layout."""
    cfg = synth.get_config(name)
    inp = synth.make_layer_inputs(cfg, keep=np.ones(cfg.M, np.uint8))
    weights, saved, dy = _upload_layer(inp)
    if layout == tfb.WEIGHTS_IN_OUT:
        weights = tfb.to_in_out(weights)
    g_unf = tfb.layer_bwd(tfb.layer_cfg(cfg, unfiltered=True, weight_layout=layout), weights, saved, dy,
                          tfb.dense_index(cfg.B, cfg.S))
    ix = tfb.build_index(_dev_keep(inp["keep"]), cfg.B, cfg.S)
    g_all = tfb.layer_bwd(tfb.layer_cfg(cfg, dmode=tfb.ATTN_D_FULL, weight_layout=layout), weights, saved,
                          dy, ix)
    for k in g_unf:
        assert torch.equal(g_unf[k], g_all[k]), k
    # with every token kept the filtered row term is the full one (the layer takes the cheaper form)
    g_def = tfb.layer_bwd(tfb.layer_cfg(cfg, weight_layout=layout), weights, saved, dy, ix)
    for k in g_unf:
        assert torch.equal(g_unf[k], g_def[k]), k
    ref = oracle.layer_bwd(cfg, upcast(inp["weights"]), upcast(inp["saved"]),
                           synth.bf16_bits_to_f32(inp["dy"]), inp["keep"], "full_d")
    for gname, oname in GRAD_NAMES[cfg.kind].items():
        got = to64(g_unf[gname])
        if layout == tfb.WEIGHTS_IN_OUT and gname.startswith("dw_"):
            got = got.T
        assert rel_err(got, ref[oname]) <= BF16_TOL, gname


def _degenerate_keep(B, S, kind):
    keep = np.zeros((B, S), np.uint8)
    if kind == "one_token":            # a single kept token, in the middle of the batch
        keep[B // 2, S // 2] = 1
    elif kind == "middle_sequence_empty":  # sequences kept whole except an empty one between them
        keep[:] = 1
        keep[B // 2] = 0
    elif kind == "first_tokens":       # only each sequence's first token (the shortest causal rows)
        keep[:, 0] = 1
    elif kind == "last_tokens":        # only each sequence's last token (the longest causal rows)
        keep[:, -1] = 1
    elif kind == "alternate":          # every other token
        keep[:, ::2] = 1
    return keep.reshape(-1)


@pytest.mark.parametrize("name", ["small_llama", "small_llama_d128", "small_phi"])
@pytest.mark.parametrize("B,S", [(1, 1), (3, 5), (2, 129)])
@pytest.mark.parametrize("kind", ["one_token", "middle_sequence_empty", "first_tokens", "last_tokens",
                                  "alternate"])
def test_layer_degenerate_shapes(name, B, S, kind):
    """Very short sequences (S = 1, 5; 129 crosses one 128-row attention block), a single kept token,
    an empty sequence between kept ones, only first or only last tokens kept, every other token."""
    cfg = synth.get_config(name).with_(B=B, S=S)
    keep = _degenerate_keep(B, S, kind)
    if keep.sum() == 0:
        keep[0] = 1
    inp = synth.make_layer_inputs(cfg, keep=keep)
    run_layer_and_compare(inp, 0)
