"""GPU parity of the loss-side steps through the C ABI: token selection (bit-exact), the LM-head
cross-entropy backward over kept tokens (bf16 bar) and the embedding gradient (float32 sums of
bf16 rows in a fixed order), against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import token_filtered_backward_amd as tfb
from tests.helpers import BF16_TOL, bf16_dev, rel_err, to64
from tests.test_gpu_parity import _dev_keep

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------------------------------------
# selection
# ------------------------------------------------------------------------------------------------


def _scores(M, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "lognormal":
        return np.exp(rng.standard_normal(M)).astype(np.float32)
    if kind == "ties":  # few distinct values, signed zeros, infinities, NaN
        vals = np.array([-1.5, -0.0, 0.0, 0.25, 2.0, np.inf, -np.inf, np.nan], np.float32)
        return rng.choice(vals, size=M)
    if kind == "const":
        return np.full(M, 0.75, np.float32)
    if kind == "normal":
        return rng.standard_normal(M).astype(np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("M,kind", [(1, "lognormal"), (7, "ties"), (1000, "ties"), (8192, "lognormal"),
                                    (8192, "const"), (70001, "normal"), (70001, "ties")])
def test_select_keep_bit_exact(M, kind):
    score = _scores(M, kind, M)
    dev = torch.from_numpy(score).cuda()
    for n_keep in sorted({0, 1, M // 3, M // 2, M - 1, M}):
        got = tfb.select_keep(dev, n_keep).cpu().numpy()
        ref = oracle.select_topk(score, n_keep)
        assert np.array_equal(got, ref), (M, kind, n_keep, int(np.sum(got != ref)))


@pytest.mark.parametrize("M,kind", [(8193, "ties"), (300007, "lognormal"), (300007, "ties"),
                                    (300007, "const"), ((1 << 20) + 3, "normal"), (9000011, "ties")])
def test_select_keep_multi_workgroup_bit_exact(M, kind):
    """The selection spread over many workgroups (token counts above 8192; past 2048 x 4096 tokens
    each workgroup walks several 4096-token steps) keeps the same tokens as the oracle, ties in
    token order across chunk boundaries included, and as the one-workgroup kernel."""
    score = _scores(M, kind, M)
    dev = torch.from_numpy(score).cuda()
    need = tfb.collider_select_workspace_bytes(M)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for n_keep in sorted({0, 1, M // 3, M - M // 5, M - 1, M} if M < 400000 else {1, M // 3, M - M // 5, M - 1}):
        keep = torch.empty(M, dtype=torch.uint8, device="cuda")
        tfb.collider_select_keep_ws(dev, n_keep, keep, ws)
        got = keep.cpu().numpy()
        ref = oracle.select_topk(score, n_keep)
        assert np.array_equal(got, ref), (M, kind, n_keep, int(np.sum(got != ref)))
    if M < 400000:
        one = torch.empty(M, dtype=torch.uint8, device="cuda")
        tfb.collider_select_keep(dev, M // 3, one)
        keep = torch.empty(M, dtype=torch.uint8, device="cuda")
        tfb.collider_select_keep_ws(dev, M // 3, keep, ws)
        assert torch.equal(one, keep)


def test_select_keep_matches_the_layer_inputs_mask():
    """On the generator's LogNormal scores (as float32) the device selection gives the 40% mask the
    layer benchmarks use."""
    M = 8192
    score = np.exp(synth.rng_for(0, "score").standard_normal(M))
    s32 = score.astype(np.float32)
    got = tfb.select_keep(torch.from_numpy(s32).cuda(), M - synth.n_filtered(M, 40)).cpu().numpy()
    assert np.array_equal(got, oracle.select_topk(s32, M - synth.n_filtered(M, 40)))
    # float32 rounding of these scores creates no tie, so the mask is the generator's
    assert np.array_equal(got, synth.make_keep(M, 40, 0))


# ------------------------------------------------------------------------------------------------
# LM head cross-entropy backward
# ------------------------------------------------------------------------------------------------


def _lm_case(B, S, H, V, r, seed, pattern="topk"):
    rng = np.random.default_rng(seed)
    M = B * S
    logits = synth.f32_to_bf16_bits((rng.standard_normal((M, V)) * 2.0).astype(np.float32))
    h = synth.f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((V, H)) * 0.02).astype(np.float32))
    labels = rng.integers(0, V, M).astype(np.int32)
    labels[rng.random(M) < 0.05] = -100  # tokens without a target
    keep = synth.make_keep(M, r, seed) if pattern == "topk" else np.zeros(M, np.uint8)
    return logits, labels, h, w, keep


@pytest.mark.parametrize("B,S,H,V,r", [(2, 200, 256, 1000, 40), (1, 64, 64, 40000, 40),
                                       (1, 48, 64, 72000, 25), (2, 130, 128, 8, 0)])
@pytest.mark.parametrize("dh_compact", [False, True])
def test_lm_head_bwd_parity(B, S, H, V, r, dh_compact):
    logits, labels, h, w, keep = _lm_case(B, S, H, V, r, seed=V + S)
    M = B * S
    ix = tfb.build_index(_dev_keep(keep), B, S)
    mk = ix.M_kept
    scale = 1.0 / max(mk, 1)
    dh = torch.full((mk if dh_compact else M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    dw = torch.full((V, H), float("nan"), dtype=torch.float32, device="cuda")
    tfb.collider_lm_head_bwd(bf16_dev(logits), torch.from_numpy(labels).cuda(), bf16_dev(h), bf16_dev(w),
                             ix.c(), scale, dh, dw, dh_compact=dh_compact)
    torch.cuda.synchronize()
    f = synth.bf16_bits_to_f32
    ref = oracle.lm_head_bwd(f(logits), labels, f(h), f(w), keep, scale)
    got_dh = to64(dh)
    ref_dh = ref["dh"][keep != 0] if dh_compact else ref["dh"]
    assert rel_err(got_dh, ref_dh) <= BF16_TOL
    assert rel_err(to64(dw), ref["dw_lm"]) <= BF16_TOL
    if not dh_compact:
        assert np.all(got_dh[keep == 0] == 0.0)


def test_lm_head_bwd_all_filtered_and_accumulate():
    B, S, H, V = 1, 96, 64, 512
    logits, labels, h, w, _ = _lm_case(B, S, H, V, 40, seed=7)
    keep = np.zeros(B * S, np.uint8)
    ix = tfb.build_index(_dev_keep(keep), B, S)
    dh = torch.full((B * S, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    dw = torch.full((V, H), 3.0, dtype=torch.float32, device="cuda")
    args = (bf16_dev(logits), torch.from_numpy(labels).cuda(), bf16_dev(h), bf16_dev(w), ix.c(), 1.0)
    tfb.collider_lm_head_bwd(*args, dh, dw, accumulate=True)
    torch.cuda.synchronize()
    assert torch.all(dh.float() == 0.0) and torch.all(dw == 3.0)
    tfb.collider_lm_head_bwd(*args, dh, dw)
    torch.cuda.synchronize()
    assert torch.all(dw == 0.0)
    # nothing kept, compact dh: an empty output is accepted
    dw0 = torch.full((V, H), 2.0, dtype=torch.float32, device="cuda")
    tfb.collider_lm_head_bwd(*args, torch.empty((0, H), dtype=torch.bfloat16, device="cuda"), dw0,
                             dh_compact=True)
    torch.cuda.synchronize()
    assert torch.all(dw0 == 0.0)
    # accumulate on a real mask adds the overwrite result
    keep = synth.make_keep(B * S, 40, 7)
    ix = tfb.build_index(_dev_keep(keep), B, S)
    args = (bf16_dev(logits), torch.from_numpy(labels).cuda(), bf16_dev(h), bf16_dev(w), ix.c(), 0.25)
    dw1 = torch.empty((V, H), dtype=torch.float32, device="cuda")
    tfb.collider_lm_head_bwd(*args, dh, dw1)
    dw2 = torch.full((V, H), 1.5, dtype=torch.float32, device="cuda")
    tfb.collider_lm_head_bwd(*args, dh, dw2, accumulate=True)
    torch.cuda.synchronize()
    assert torch.allclose(dw2, dw1 + 1.5, rtol=0, atol=1e-6)


# ------------------------------------------------------------------------------------------------
# embedding gradient
# ------------------------------------------------------------------------------------------------


@pytest.mark.parametrize("B,S,H,V,r", [(2, 200, 256, 1000, 40), (1, 3000, 64, 50, 20), (4, 2048, 128, 32000, 40),
                                       (2, 1500, 64, 50000, 40), (2, 600, 896, 3000, 40),
                                       (1, 77, 64, 16, 100)])
@pytest.mark.parametrize("dx_compact", [False, True])
def test_embedding_bwd_parity(B, S, H, V, r, dx_compact):
    rng = np.random.default_rng(S + V)
    M = B * S
    keep = synth.make_keep(M, r, 1)
    ids = rng.integers(0, V, M).astype(np.int32)
    ids[: M // 10] = V // 2                     # a frequent token
    ids[rng.random(M) < 0.01] = -1             # ids outside [0, V) are skipped
    ix = tfb.build_index(_dev_keep(keep), B, S)
    mk = ix.M_kept
    dxf = synth.f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    dx_dev = bf16_dev(dxf[keep != 0] if dx_compact else dxf)
    if mk == 0 and dx_compact:
        dx_dev = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    dE = torch.full((V, H), float("nan"), dtype=torch.float32, device="cuda")
    tfb.collider_embedding_bwd(dx_dev, torch.from_numpy(ids).cuda(), ix.c(), dE, dx_compact=dx_compact)
    torch.cuda.synchronize()
    ref = oracle.embedding_bwd(synth.bf16_bits_to_f32(dxf), ids, keep, V)
    got = to64(dE)
    assert np.all(np.isfinite(got))
    assert rel_err(got, ref) <= 1e-5
    used = np.zeros(V, bool)
    ok = (ids >= 0) & (ids < V) & (keep != 0)
    used[ids[ok]] = True
    assert np.all(got[~used] == 0.0)
    # deterministic: a second call gives the same bits; accumulate adds
    dE2 = torch.empty_like(dE)
    tfb.collider_embedding_bwd(dx_dev, torch.from_numpy(ids).cuda(), ix.c(), dE2, dx_compact=dx_compact)
    dE3 = torch.ones_like(dE)
    tfb.collider_embedding_bwd(dx_dev, torch.from_numpy(ids).cuda(), ix.c(), dE3, dx_compact=dx_compact,
                               accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dE, dE2)
    assert torch.allclose(dE3, dE + 1.0, rtol=0, atol=1e-5)


# ------------------------------------------------------------------------------------------------
# per-token loss -> selection -> index, on the device
# ------------------------------------------------------------------------------------------------


def _logits_case(M, V, seed, minus_inf=False):
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal((M, V)) * 2.0).astype(np.float32)
    labels = rng.integers(0, V, M).astype(np.int32)
    labels[rng.random(M) < 0.05] = -100
    if M > 3:
        labels[3] = V + 3  # past the vocabulary: no target either
    if minus_inf:
        # whole 8-wide blocks of -inf (masked vocabulary entries), at the start of a row, in the
        # middle, at the end, and runs long enough to cover a thread's whole share of a row; every
        # row keeps at least one finite 8-wide block (a row of -inf only has no defined loss)
        def blocks(n):
            return max(0, min(n, V - 8)) // 8 * 8
        z[0, :blocks(64)] = -np.inf
        if M > 1:
            z[1, 8:8 + blocks(min(8 * 300, V - 16))] = -np.inf
        if M > 2:
            z[2, V - blocks(16):] = -np.inf
        z[4::5, :blocks(V // 2)] = -np.inf
        # labels on finite entries
        for t in range(min(M, 5)):
            fin = np.flatnonzero(np.isfinite(z[t]))
            if labels[t] >= 0 and labels[t] < V and fin.size:
                labels[t] = fin[len(fin) // 2]
        rows = np.arange(4, M, 5)
        labels[rows] = np.where(labels[rows] >= 0, V - 1, labels[rows])
    return synth.f32_to_bf16_bits(z), labels


@pytest.mark.parametrize("M,V", [(400, 1000), (64, 40000), (37, 72000), (130, 8), (1, 32000)])
@pytest.mark.parametrize("minus_inf", [False, True])
def test_ce_loss_parity(M, V, minus_inf):
    bits, labels = _logits_case(M, V, seed=M + V, minus_inf=minus_inf)
    got = tfb.ce_loss(bf16_dev(bits), torch.from_numpy(labels).cuda()).cpu().numpy().astype(np.float64)
    ref = oracle.ce_loss(synth.bf16_bits_to_f32(bits), labels)
    assert np.all(np.isfinite(got))
    assert rel_err(got, ref) <= 1e-5, rel_err(got, ref)
    assert np.all(got[(labels < 0) | (labels >= V)] == 0.0)


def test_loss_select_index_chain():
    """logits -> per-token loss -> keep the 60% largest -> index, all on the device (the loss side
    of Figure 2(b) up to the layers): the mask is the oracle's selection of the device's own loss
    values bit for bit, and the index the oracle's index of that mask."""
    B, S, V = 4, 512, 4096
    M = B * S
    bits, labels = _logits_case(M, V, seed=5)
    loss = tfb.ce_loss(bf16_dev(bits), torch.from_numpy(labels).cuda())
    n_keep = M - synth.n_filtered(M, 40)
    keep = tfb.select_keep(loss, n_keep)
    ix = tfb.build_index(keep, B, S)
    loss_np = loss.cpu().numpy()
    assert rel_err(loss_np, oracle.ce_loss(synth.bf16_bits_to_f32(bits), labels)) <= 1e-5
    keep_ref = oracle.select_topk(loss_np, n_keep)
    assert np.array_equal(keep.cpu().numpy(), keep_ref)
    ref = oracle.build_index(keep_ref, B, S)
    assert ix.M_kept == ref["count"] == n_keep
    assert np.array_equal(ix.idx.cpu().numpy()[:n_keep], ref["idx"])
    assert np.array_equal(ix.inv.cpu().numpy(), ref["inv"])
    # tokens without a target have loss 0 and are ranked below every token with a positive loss
    assert np.all(keep_ref[(labels < 0) | (labels >= V)] == 0)


@pytest.mark.parametrize("V", [1000, 40000, 72000])
def test_lm_head_bwd_minus_inf_blocks(V):
    """LM-head backward on logit rows holding whole 8-wide blocks of -inf: finite gradients equal to
    the oracle's (the -inf entries get exactly zero gradient)."""
    B, S, H = 1, 64, 128
    M = B * S
    bits, labels = _logits_case(M, V, seed=V, minus_inf=True)
    rng = np.random.default_rng(V + 1)
    h = synth.f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((V, H)) * 0.02).astype(np.float32))
    keep = np.ones(M, np.uint8)
    keep[1::3] = 0
    ix = tfb.build_index(_dev_keep(keep), B, S)
    dh = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((V, H), dtype=torch.float32, device="cuda")
    tfb.collider_lm_head_bwd(bf16_dev(bits), torch.from_numpy(labels).cuda(), bf16_dev(h), bf16_dev(w),
                             ix.c(), 1.0 / ix.M_kept, dh, dw)
    torch.cuda.synchronize()
    f = synth.bf16_bits_to_f32
    ref = oracle.lm_head_bwd(f(bits), labels, f(h), f(w), keep, 1.0 / ix.M_kept)
    got_dh, got_dw = to64(dh), to64(dw)
    assert np.all(np.isfinite(got_dh)) and np.all(np.isfinite(got_dw))
    assert rel_err(got_dh, ref["dh"]) <= BF16_TOL and rel_err(got_dw, ref["dw_lm"]) <= BF16_TOL
