"""The long-context stack (TinyLlama-shaped layers at B 1 x S 8192, 40% filtered) end to end
against the oracle: one consistent host forward through the stack gives every layer its own
weights and saved activations; the GPU runs the layers top to bottom with compact gradients between
them (one index, built once; the bottom layer writes dx in the full token layout), exactly as the
filtered backward of a model runs; the oracle runs the same stack in the full token layout with the
mask applied explicitly.  Every layer's weight and gain gradients, every intermediate dx (kept rows)
and the bottom dx are compared element by element; the per-layer errors are printed so that their
growth with depth is visible.

The oracle runs in float32 here (its float32 results are checked against float64 in
tests/test_oracle_loss_side.py; the float32 rounding error, about 1e-6 relative, is far below
the 2e-2 bar) so that three layers of S = 8192 attention fit the test's time."""
import os
import time

import numpy as np
import pytest
import torch

import oracle
import synth
import token_filtered_backward_amd as tfb
from tests.helpers import BF16_TOL, rel_err, to64
from tests.test_gpu_parity import GRAD_NAMES, _dev_keep, _upload_layer

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[chain]", *a, flush=True)


def run_chain(n_layers, seed=0, r_pct=40):
    """Returns ({grad name: [error per layer, bottom first]}, {dx: [error per layer]})."""
    cfg = synth.get_config("tinyllama_22l").with_(n_layers=n_layers)
    t0 = time.time()
    _say(f"host forward of {n_layers} layers at B {cfg.B} x S {cfg.S} ...")
    inp = synth.make_model_inputs(cfg, seed=seed, r_pct=r_pct, n_layers=n_layers)
    _say(f"forward done in {time.time() - t0:.0f}s")
    keep = inp["keep"]
    ix = tfb.build_index(_dev_keep(keep), cfg.B, cfg.S)
    lcfg = tfb.layer_cfg(cfg)
    lb = tfb.LayerBackward(lcfg, cfg.B, cfg.S, "cuda")
    L = n_layers
    got = [None] * L
    dy = None
    for li in reversed(range(L)):  # top layer first
        one = {"cfg": cfg, "weights": inp["layers"][li]["weights"], "saved": inp["layers"][li]["saved"],
               "dy": inp["dy"]}
        weights, saved, dy_top = _upload_layer(one)
        top, bottom = li == L - 1, li == 0
        g = tfb.make_grads(lcfg, cfg.M, ix.M_kept, "cuda", dx_compact=not bottom)
        for t in g.values():
            t.fill_(float("nan"))
        lb(weights, saved, dy_top if top else dy, ix, g, dy_compact=not top, dx_compact=not bottom)
        torch.cuda.synchronize()
        got[li] = {k: to64(v) for k, v in g.items()}
        dy = g["dx"]
    _say(f"GPU chain done; oracle (float32) ...")
    layers = [{"weights": synth.floats(l["weights"]), "saved": synth.floats(l["saved"])}
              for l in inp["layers"]]
    kept = np.flatnonzero(keep)
    grad_err, dx_err = {k: [] for k in GRAD_NAMES["llama"] if k != "dx"}, []
    g_ref = synth.bf16_bits_to_f32(inp["dy"])
    with oracle.precision(np.float32):
        for li in reversed(range(L)):
            t1 = time.time()
            ref = oracle.layer_bwd(cfg, layers[li]["weights"], layers[li]["saved"], g_ref, keep)
            errs = {k: rel_err(got[li][k], ref[o]) for k, o in GRAD_NAMES["llama"].items() if k != "dx"}
            dx_ref = ref["dx"]
            dx_got = got[li]["dx"]
            if li > 0:  # compact rows: the kept tokens in ascending order
                e = rel_err(dx_got, dx_ref[kept])
                assert np.all(dx_ref[keep == 0] == 0.0)
            else:
                e = rel_err(dx_got, dx_ref)
                assert np.all(dx_got[keep == 0] == 0.0)
            for k, v in errs.items():
                grad_err[k].insert(0, v)
            dx_err.insert(0, e)
            _say(f"layer {li} (depth {L - li} from the top): dx {e:.2e} "
                 + " ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f"  [{time.time() - t1:.0f}s]")
            g_ref = dx_ref
    return grad_err, dx_err


@pytest.mark.timeout(3000)
def test_long_context_stack_against_oracle():
    # three layers by default (about a minute of host time); COLLIDER_CHAIN_LAYERS=22 runs the whole
    # 22-layer stack (about eight minutes, mostly the host forward and the oracle)
    grad_err, dx_err = run_chain(int(os.environ.get("COLLIDER_CHAIN_LAYERS", "3")))
    bad = {(k, li): e for k, v in grad_err.items() for li, e in enumerate(v) if not e <= BF16_TOL}
    bad.update({("dx", li): e for li, e in enumerate(dx_err) if not e <= BF16_TOL})
    assert not bad, bad
