"""GPU parity at the full layer sizes the benchmark runs (TinyLlama-, Qwen2.5- and Phi-1.5-shaped
layers; the Phi layer over a filter-ratio sweep), through the same entry point and launch
configuration: the layer backward on two streams, GEMM plans for concurrent work.  Every gradient is
compared whole against the float64 oracle (a few seconds of host time per layer).

Bars: max|d|/max|ref| <= 2e-2 for every gradient, rows of filtered tokens in dx exactly zero."""
import functools

import numpy as np
import pytest
import torch

import oracle
import synth
import token_filtered_backward_amd as tfb
from tests.helpers import BF16_TOL, to64, upcast
from tests.test_gpu_parity import GRAD_NAMES, _dev_keep, _upload_layer, check_attention

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def _inputs(name, r, n_layers=None):
    cfg = synth.get_config(name)
    if n_layers is not None:
        cfg = cfg.with_(n_layers=n_layers)
    return synth.make_layer_inputs(cfg, seed=0, r_pct=r)


def _run(inp, dmode, unfiltered=False, weight_layout=0):
    cfg = inp["cfg"]
    weights, saved, dy = _upload_layer(inp)
    if weight_layout == tfb.WEIGHTS_IN_OUT:
        weights = tfb.to_in_out(weights)
    if unfiltered:
        ix = tfb.dense_index(cfg.B, cfg.S)
    else:
        ix = tfb.build_index(_dev_keep(inp["keep"]), cfg.B, cfg.S)
    lcfg = tfb.layer_cfg(cfg, dmode=dmode, unfiltered=unfiltered, weight_layout=weight_layout)
    grads = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda")
    for g in grads.values():
        g.fill_(float("nan"))
    tfb.LayerBackward(lcfg, cfg.B, cfg.S, "cuda")(weights, saved, dy, ix, grads)
    torch.cuda.synchronize()
    # weight gradients in the [out, in] layout the oracle returns
    return {k: (to64(v).T if weight_layout and k.startswith("dw_") else to64(v)) for k, v in grads.items()}


def _compare(cfg, got, ref, keep):
    errs = {g: float(np.max(np.abs(got[g] - ref[o])) / max(np.max(np.abs(ref[o])), 1e-30))
            for g, o in GRAD_NAMES[cfg.kind].items()}
    print(cfg.name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert np.all(got["dx"][keep == 0] == 0.0)
    bad = {k: v for k, v in errs.items() if not v <= BF16_TOL}
    assert not bad, errs


@pytest.mark.parametrize("name,r,dmode,layout", [("tinyllama", 40, 0, 0), ("tinyllama", 40, 1, 0),
                                                 ("tinyllama", 40, 0, 1), ("qwen25", 40, 0, 0),
                                                 ("qwen25", 40, 0, 1), ("phi15", 0, 0, 0),
                                                 ("phi15", 20, 0, 0), ("phi15", 40, 0, 0),
                                                 ("phi15", 60, 0, 0), ("phi15", 40, 0, 1)])
def test_layer_fullsize(name, r, dmode, layout):
    cfg = synth.get_config(name)
    inp = synth.make_layer_inputs(cfg, seed=0, r_pct=r)
    got = _run(inp, dmode, weight_layout=layout)
    ref = oracle.layer_bwd(cfg, upcast(inp["weights"]), upcast(inp["saved"]),
                           synth.bf16_bits_to_f32(inp["dy"]), inp["keep"],
                           "filtered" if dmode == 0 else "full_d")
    _compare(cfg, got, ref, inp["keep"])


def test_unfiltered_baseline_fullsize():
    """The dense baseline the speedup is measured against computes the ordinary gradient."""
    cfg = synth.get_config("tinyllama")
    inp = synth.make_layer_inputs(cfg, seed=0, r_pct=0)
    got = _run(inp, 1, unfiltered=True)
    ref = oracle.layer_bwd(cfg, upcast(inp["weights"]), upcast(inp["saved"]),
                           synth.bf16_bits_to_f32(inp["dy"]), np.ones(cfg.M, np.uint8), "full_d")
    _compare(cfg, got, ref, np.ones(cfg.M, np.uint8))


@pytest.mark.timeout(900)
def test_layer_long_context_fullsize():
    """One layer of the long-context stack (B 1 x S 8192, 40% filtered) against the oracle."""
    inp = _inputs("tinyllama_22l", 40, 1)
    cfg = inp["cfg"]
    got = _run(inp, 0)
    ref = oracle.layer_bwd(cfg, upcast(inp["weights"]), upcast(inp["saved"]),
                           synth.bf16_bits_to_f32(inp["dy"]), inp["keep"], "filtered")
    _compare(cfg, got, ref, inp["keep"])


@pytest.mark.timeout(900)
def test_attention_long_context():
    """Filtered attention backward over one sequence of 16384 tokens (4 query heads on 1 KV head,
    head_dim 64, 40% filtered: 9831 kept rows, about 4.8e7 kept causal pairs per head) against the
    float64 oracle: the long-context end of the sequence-length sweep."""
    print("attention long context: B 1 x S 16384, oracle on the host (about a minute)", flush=True)
    check_attention("longctx_attn", 40, 0)


def test_stack_compact_chain_fullsize():
    """22 layers at B 1 x S 8192 chained with compact gradients equal, bit for bit, the same stack
    run with full-layout scatter / gather between layers; filtered rows of the bottom dx are zero.
    (One synthetic layer's saved set and weights serve every layer.)"""
    cfg = synth.get_config("tinyllama_22l")
    inp = _inputs("tinyllama_22l", 40, 1)
    weights, saved, dy = _upload_layer(inp)
    keep = _dev_keep(inp["keep"])
    ix = tfb.build_index(keep, cfg.B, cfg.S)
    lcfg = tfb.layer_cfg(cfg)
    lb = tfb.LayerBackward(lcfg, cfg.B, cfg.S, "cuda")
    L = cfg.n_layers
    gc = [tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda", dx_compact=True) for _ in range(2)]
    out_c = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda")
    lb(weights, saved, dy, ix, gc[0], dx_compact=True)
    for layer in range(1, L - 1):
        lb(weights, saved, gc[(layer - 1) % 2]["dx"], ix, gc[layer % 2], dy_compact=True, dx_compact=True)
    lb(weights, saved, gc[(L - 2) % 2]["dx"], ix, out_c, dy_compact=True)
    gf = [tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda") for _ in range(2)]
    lb(weights, saved, dy, ix, gf[0])
    for layer in range(1, L):
        lb(weights, saved, gf[(layer - 1) % 2]["dx"], ix, gf[layer % 2])
    torch.cuda.synchronize()
    last = gf[(L - 1) % 2]
    for k in out_c:
        a, b = out_c[k], last[k]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), k
    dx = to64(out_c["dx"])
    assert np.all(np.isfinite(dx)) and np.all(dx[inp["keep"] == 0] == 0.0)
    assert np.abs(dx[inp["keep"] != 0]).max() > 0


@pytest.mark.timeout(900)
def test_loss_side_fullsize():
    """The loss-side steps at the benchmark's shape (B 4 x S 2048, hidden 2048, vocab 32000, 40%
    filtered by the device's own top-k on the LogNormal scores): LM-head cross-entropy backward
    and embedding gradient against the float64 oracle."""
    from tests.helpers import bf16_dev, rel_err
    B, S, H, V = 4, 2048, 2048, 32000
    M = B * S
    rng = np.random.default_rng(11)
    score = np.exp(synth.rng_for(0, "score").standard_normal(M)).astype(np.float32)
    keep_d = tfb.select_keep(torch.from_numpy(score).cuda(), M - synth.n_filtered(M, 40))
    keep = keep_d.cpu().numpy()
    assert np.array_equal(keep, oracle.select_topk(score, M - synth.n_filtered(M, 40)))
    ix = tfb.build_index(keep_d, B, S)
    mk = ix.M_kept
    logits = synth.f32_to_bf16_bits((rng.standard_normal((M, V)) * 2.0).astype(np.float32))
    h = synth.f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((V, H)) * 0.02).astype(np.float32))
    labels = rng.integers(0, V, M).astype(np.int32)
    dh = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((V, H), dtype=torch.float32, device="cuda")
    print("loss side full size: LM head", flush=True)
    tfb.collider_lm_head_bwd(bf16_dev(logits), torch.from_numpy(labels).cuda(), bf16_dev(h), bf16_dev(w),
                             ix.c(), 1.0 / mk, dh, dw)
    torch.cuda.synchronize()
    f = synth.bf16_bits_to_f32
    ref = oracle.lm_head_bwd(f(logits), labels, f(h), f(w), keep, 1.0 / mk)
    got_dh = to64(dh)
    errs = {"dh": rel_err(got_dh, ref["dh"]), "dw_lm": rel_err(to64(dw), ref["dw_lm"])}
    print(errs, flush=True)
    assert np.all(got_dh[keep == 0] == 0.0)
    assert all(e <= BF16_TOL for e in errs.values()), errs
    del ref, logits
    print("loss side full size: embedding", flush=True)
    ids = rng.integers(0, V, M).astype(np.int32)
    dxc = synth.f32_to_bf16_bits(rng.standard_normal((mk, H)).astype(np.float32))
    dE = torch.empty((V, H), dtype=torch.float32, device="cuda")
    tfb.collider_embedding_bwd(bf16_dev(dxc), torch.from_numpy(ids).cuda(), ix.c(), dE, dx_compact=True)
    torch.cuda.synchronize()
    dx_full = np.zeros((M, H))
    dx_full[keep != 0] = f(dxc)
    e = rel_err(to64(dE), oracle.embedding_bwd(dx_full, ids, keep, V))
    print("embedding", e, flush=True)
    assert e <= 1e-5
