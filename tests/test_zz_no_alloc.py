"""The allocation-free embedding gradient (collider_embedding_bwd_noalloc, for callers that cannot
allocate device memory) against the workspace entry point collider_embedding_bwd: the same result
bit for bit on two calls in a row - the second with a smaller input, so that stale scratch from the
first would show - and the oracle's result within the float32 bar; sizes past the scratch limits are
rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

import oracle
import token_filtered_backward_amd as tfb
from tests.helpers import bf16_dev, rel_err, to64
from tests.test_gpu_parity import _dev_keep

pytestmark = pytest.mark.gpu

import synth  # noqa: E402


def _case(B, S, H, V, r, seed, compact):
    rng = np.random.default_rng(seed)
    M = B * S
    keep = synth.make_keep(M, r, seed)
    ids = rng.integers(0, V, M).astype(np.int32)
    ids[: M // 10] = 7  # a frequent id
    ids[rng.random(M) < 0.02] = -1  # no embedding row
    ix = tfb.build_index(_dev_keep(keep), B, S)
    rows = ix.M_kept if compact else M
    dx_bits = synth.f32_to_bf16_bits(rng.standard_normal((max(rows, 1), H)).astype(np.float32))
    return keep, ids, ix, dx_bits[:rows]


def _run_pair(B, S, H, V, r, seed, compact, accumulate=False):
    keep, ids, ix, dx_bits = _case(B, S, H, V, r, seed, compact)
    dx = bf16_dev(dx_bits) if dx_bits.shape[0] else None
    ids_d = torch.from_numpy(ids).cuda()
    init = torch.randn((V, H), device="cuda") if accumulate else None
    a = init.clone() if accumulate else torch.full((V, H), float("nan"), device="cuda")
    b = init.clone() if accumulate else torch.full((V, H), float("nan"), device="cuda")
    tfb.collider_embedding_bwd(dx, ids_d, ix.c(), a, dx_compact=compact, accumulate=accumulate)
    tfb.collider_embedding_bwd_noalloc(dx, ids_d, ix.c(), b, dx_compact=compact, accumulate=accumulate)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # the oracle, on the full-layout dx the call saw
    M = B * S
    f = synth.bf16_bits_to_f32(dx_bits).astype(np.float64)
    dx_full = np.zeros((M, H))
    if compact:
        dx_full[keep != 0] = f
    else:
        dx_full = f
    ref = oracle.embedding_bwd(dx_full, ids, keep, V)
    if accumulate:
        ref = ref + to64(init)
    assert rel_err(to64(b), ref) <= 1e-5
    return b


def test_noalloc_matches_workspace_entry_two_calls_shrinking():
    big = _run_pair(4, 2048, 256, 32000, 40, seed=1, compact=True)
    small = _run_pair(1, 300, 128, 5000, 60, seed=2, compact=False)
    assert big.shape != small.shape


def test_noalloc_large_vocab_and_accumulate():
    _run_pair(2, 1000, 64, 100000, 40, seed=3, compact=True)  # cursors in global memory
    _run_pair(2, 700, 64, 3000, 25, seed=4, compact=False, accumulate=True)
    _run_pair(1, 64, 64, 500, 100, seed=5, compact=True)  # nothing kept


def test_noalloc_rejects_sizes_past_the_scratch():
    B, S, H = 1, 64, 64
    keep = np.ones(B * S, np.uint8)
    ix = tfb.build_index(_dev_keep(keep), B, S)
    ids = torch.zeros(B * S, dtype=torch.int32, device="cuda")
    dx = torch.zeros((B * S, H), dtype=torch.bfloat16, device="cuda")
    V = (1 << 18) + 1
    dE = torch.zeros((V, H), device="cuda")
    with pytest.raises(tfb.ColliderError, match="status 5"):
        tfb.collider_embedding_bwd_noalloc(dx, ids, ix.c(), dE, dx_compact=True)
    M = (1 << 20) + 8
    big = tfb.build_index(torch.ones(M, dtype=torch.uint8, device="cuda"), 1, M)
    ids2 = torch.zeros(M, dtype=torch.int32, device="cuda")
    dx2 = torch.zeros((M, 8), dtype=torch.bfloat16, device="cuda")
    dE2 = torch.zeros((16, 8), device="cuda")
    with pytest.raises(tfb.ColliderError, match="status 5"):
        tfb.collider_embedding_bwd_noalloc(dx2, ids2, big.c(), dE2, dx_compact=True)
