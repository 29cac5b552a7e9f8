"""The C ABI library loads, exports every function include/collider.h declares, and rejects bad
arguments on the host before touching the GPU (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import synth
import token_filtered_backward_amd as tfb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "collider.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tfb.LIB_PATH), reason="libcollider.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(collider_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("collider_build_index", "collider_index_count_host", "collider_gather_rows",
              "collider_scatter_rows", "collider_linear_bwd_reduced", "collider_attn_bwd_filtered",
              "collider_layer_bwd"):
        assert n in names


def test_library_resolves_every_symbol_at_load():
    """Loading with immediate binding fails on any symbol the library uses but does not define."""
    ctypes.CDLL(tfb.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(tfb.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_status_strings():
    L = tfb.lib()
    for s in range(7):
        assert L.collider_status_string(s)
    assert L.collider_status_string(5).decode() == "workspace missing or too small"


def test_host_validation_errors():
    L = tfb.lib()
    p = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    assert L.collider_build_index(None, 1, 1, p, p, p, p, None) == 1
    assert L.collider_build_index(p, 0, 1, p, p, p, p, None) == 2
    assert L.collider_build_index_expect(p, 2, 4, -1, p, p, p, p, p, None) == 2   # count < 0
    assert L.collider_build_index_expect(p, 2, 4, 9, p, p, p, p, p, None) == 2    # count > B*S
    assert L.collider_build_index_expect(p, 2, 4, 3, p, p, p, p, None, None) == 1  # no flag
    assert L.collider_gather_rows(p, 8, p, 8, p, 1, 8, 7, None) == 4          # bad dtype
    assert L.collider_gather_rows(p, 4, p, 8, p, 1, 8, 1, None) == 2          # ld < row
    assert L.collider_gather_rows(None, 8, p, 8, p, 1, 8, 1, None) == 1
    assert L.collider_scatter_rows(p, 8, None, 8, p, 4, 8, 1, 1, None) == 1
    # linear: K not a multiple of 8 for bf16, missing workspace
    assert L.collider_linear_bwd_reduced(1, 4, 12, 8, p, 12, p, 8, p, p, p, None, 0, None, 0, None) == 3
    a16 = ctypes.c_void_p(0x10000)
    assert L.collider_linear_bwd_reduced(1, 4096, 2048, 2048, a16, 2048, a16, 2048, a16, a16, a16, None, 0,
                                         None, 0, None) == 5                  # workspace missing
    cfg = tfb.AttnCfg(8, 2, 96, 0, 0.0, 0.0, 0)
    ix = tfb.CollIndex(p, p, p, p, 1, 8, 8)
    io = tfb.AttnIO()
    assert L.collider_attn_bwd_filtered(ctypes.byref(cfg), ctypes.byref(ix), ctypes.byref(io), None, 0, None) == 4
    cfg = tfb.AttnCfg(6, 4, 64, 0, 0.0, 0.0, 0)                                # nq % nkv != 0
    assert L.collider_attn_bwd_filtered(ctypes.byref(cfg), ctypes.byref(ix), ctypes.byref(io), None, 0, None) == 2
    cfg = tfb.AttnCfg(8, 2, 64, 25, 1e4, 0.0, 0)                               # odd rotary width
    assert L.collider_attn_bwd_filtered(ctypes.byref(cfg), ctypes.byref(ix), ctypes.byref(io), None, 0, None) == 4
    cfg = tfb.AttnCfg(8, 2, 64, 64, 1e4, 0.0, 0)
    ix_bad = tfb.CollIndex(p, p, p, p, 1, 8, 9)                                # M_kept > M
    assert L.collider_attn_bwd_filtered(ctypes.byref(cfg), ctypes.byref(ix_bad), ctypes.byref(io), None, 0, None) == 2
    io.q = io.k = io.v = io.lse = io.dout = io.dq = io.dk = io.dv = 0x10008    # misaligned
    io.ld_q = io.ld_do = io.ld_dq = 512
    io.ld_k = io.ld_v = io.ld_dk = io.ld_dv = 128
    io.ld_lse = 8
    assert L.collider_attn_bwd_filtered(ctypes.byref(cfg), ctypes.byref(ix), ctypes.byref(io), None, 0, None) == 3
    io.q = io.k = io.v = io.lse = io.dout = io.dq = io.dk = io.dv = 0x10000
    assert L.collider_attn_bwd_filtered(ctypes.byref(cfg), ctypes.byref(ix), ctypes.byref(io), None, 0, None) == 5


def test_layer_validation_and_workspace_sizes():
    L = tfb.lib()
    for name in ("tinyllama", "qwen25", "phi15", "small_llama", "small_phi"):
        shape = synth.get_config(name)
        cfg = tfb.layer_cfg(shape)
        mk = shape.M - synth.n_filtered(shape.M, 40)
        need = L.collider_layer_workspace_bytes(ctypes.byref(cfg), shape.B, shape.S, mk)
        assert need > 0
        # more kept tokens never needs less workspace; M_kept > M is rejected
        assert L.collider_layer_workspace_bytes(ctypes.byref(cfg), shape.B, shape.S, shape.M) >= need
        assert L.collider_layer_workspace_bytes(ctypes.byref(cfg), shape.B, shape.S, shape.M + 1) == 0
    shape = synth.get_config("tinyllama")
    bad = tfb.layer_cfg(shape.with_(H=5004))                  # hidden not a multiple of 8
    assert L.collider_layer_workspace_bytes(ctypes.byref(bad), 1, 8, 8) == 0
    cfg = tfb.layer_cfg(shape)
    ix = tfb.CollIndex(0x1000, 0x1000, 0x1000, 0x1000, 4, 2048, 4916)
    w, sv, g = tfb.LayerWeights(), tfb.LayerSaved(), tfb.LayerGrads()
    assert L.collider_layer_bwd(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(sv), ctypes.c_void_p(0x1000),
                                0, ctypes.byref(ix), ctypes.byref(g), 0, None, 0, None) == 1
    cfg.kind = 7
    assert L.collider_layer_bwd(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(sv), ctypes.c_void_p(0x1000),
                                0, ctypes.byref(ix), ctypes.byref(g), 0, None, 0, None) == 4
    # weight layouts: [in, out] for both layer kinds; unknown layouts rejected
    io = tfb.layer_cfg(shape, weight_layout=tfb.WEIGHTS_IN_OUT)
    assert L.collider_layer_workspace_bytes(ctypes.byref(io), 4, 2048, 4916) > 0
    phi_io = tfb.layer_cfg(synth.get_config("phi15"), weight_layout=tfb.WEIGHTS_IN_OUT)
    assert L.collider_layer_workspace_bytes(ctypes.byref(phi_io), 4, 2048, 4916) > 0
    io.weight_layout = 2
    assert L.collider_layer_workspace_bytes(ctypes.byref(io), 4, 2048, 4916) == 0


def test_linear_workspace_size_is_host_only():
    assert tfb.collider_linear_workspace_bytes(tfb.BF16, 4916, 2048, 2048) > 0
    assert tfb.collider_linear_workspace_bytes(tfb.F32, 154, 256, 256) > 0


def test_gemm_policy_values():
    L = tfb.lib()
    assert L.collider_gemm_set_policy(7) == 2 and L.collider_gemm_set_policy(-1) == 2
    for p in (1, 2, 3, 0):
        assert L.collider_gemm_set_policy(p) == 0


def test_gemm_plans_fill_the_cus_on_ragged_token_counts():
    """Host-side planner: whole-tile plans for the layer's concurrent GEMMs pick a tile height that
    fills 256 CUs for the ragged kept-token count, and the dense counts keep 256-row tiles."""
    plan = tfb.collider_gemm_describe_plan
    assert plan(4916, 2048, 11264, 0, concurrent=True)["bm"] == 160   # 248 tiles
    assert plan(4916, 5632, 2048, 0, concurrent=True)["bm"] == 224    # 484 tiles, 2 waves
    assert plan(5500, 2048, 2048, 0, concurrent=True)["bm"] == 192    # 232 tiles
    assert plan(8192, 2048, 11264, 0, concurrent=True)["bm"] == 256   # 256 tiles
    for shape in ((4916, 2048, 11264, 0), (11264, 2048, 4916, 1), (2048, 2048, 4916, 1), (77, 136, 64, 0)):
        p = plan(*shape, concurrent=True)
        assert p["splits"] == 1 and p["sk_tiles"] == 0
        bm, bn = p["bm"], p["bn"]
        assert p["dp_tiles"] == -(-shape[0] // bm) * -(-shape[1] // bn)
    # token-major operands only take 128 / 256-row tiles
    for M in (2048, 2560, 5632, 11264):
        assert plan(M, 2048, 4916, 1)["bm"] in (128, 256)
    L = tfb.lib()
    out = (ctypes.c_int32 * 7)()
    assert L.collider_gemm_describe_plan(0, 8, 8, 0, 0, out) == 2
    assert L.collider_gemm_describe_plan(8, 12, 8, 0, 0, out) == 2
    assert L.collider_gemm_describe_plan(8, 8, 8, 2, 0, out) == 2


def test_loss_side_validation():
    L = tfb.lib()
    p = ctypes.c_void_p(0x10000)
    assert L.collider_select_keep(None, 8, 4, p, None) == 1
    assert L.collider_select_keep(p, 0, 4, p, None) == 2
    # the many-workgroup selection: no workspace up to 8192 tokens, one histogram per chunk above
    assert L.collider_select_workspace_bytes(8192) == 0
    assert L.collider_select_workspace_bytes(8193) == (4 + 4 * 257) * 4
    assert L.collider_select_workspace_bytes(1 << 30) == (4 + 2048 * 257) * 4
    assert L.collider_select_keep_ws(p, 9000, 4, ctypes.c_void_p(0x10004), ctypes.c_void_p(0x10004), 1 << 20, None) == 3
    assert L.collider_select_keep_ws(None, 9000, 4, p, p, 1 << 20, None) == 1
    assert L.collider_select_keep_ws(p, 0, 4, p, p, 1 << 20, None) == 2
    assert L.collider_select_keep_ws(p, 9000, 4, p, None, 0, None) == 5
    assert L.collider_select_keep_ws(p, 9000, 4, p, p, 16, None) == 5
    ix = tfb.CollIndex(p, p, p, p, 2, 64, 77)
    # V not a multiple of 8, then a missing workspace
    assert L.collider_lm_head_bwd(p, 1004, p, p, 256, p, ctypes.byref(ix), 256, 1004, 1.0, p, 0, p, 0,
                                  None, 0, None) == 3
    assert L.collider_lm_head_bwd(p, 1000, p, p, 256, p, ctypes.byref(ix), 256, 1000, 1.0, p, 0, p, 0,
                                  None, 0, None) == 5
    assert L.collider_lm_head_bwd(p, 1000, None, p, 256, p, ctypes.byref(ix), 256, 1000, 1.0, p, 0, p, 0,
                                  None, 0, None) == 1
    assert L.collider_lm_head_workspace_bytes(77, 256, 1000) >= 77 * 1000 * 2 + 2 * 77 * 256 * 2
    assert L.collider_embedding_bwd(p, 256, 1, None, ctypes.byref(ix), 256, 1000, p, 0, None, 0, None) == 1
    assert L.collider_embedding_bwd(p, 256, 1, p, ctypes.byref(ix), 252, 1000, p, 0, None, 0, None) == 3
    assert L.collider_embedding_bwd(p, 256, 1, p, ctypes.byref(ix), 256, 1000, p, 0, None, 0, None) == 5
    assert L.collider_embedding_workspace_bytes(77, 1000) >= (3 * 1000 + 1 + 77) * 4
