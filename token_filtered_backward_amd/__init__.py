"""Python binding of libcollider (filtered transformer-layer backward on MI355X).

Argument marshalling only: every step runs in the HIP kernels of libcollider.so.  Torch tensors
supply device memory and the current HIP stream.  Functions named collider_* mirror the C entry
points of include/collider.h one to one; build_index / layer_bwd are conveniences on top of them.
There is no CPU fallback: if the library is missing or a call fails, an exception is raised.

Method: "Enhancing Token Filtering Efficiency in Large Language Model Training with Collider"
(arXiv 2502.00340), abstract and Figures 2, 3, 5.
"""
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcollider.so")

F32, BF16 = 0, 1
ATTN_D_FILTERED, ATTN_D_FULL = 0, 1
LAYER_LLAMA, LAYER_PHI = 0, 1
WEIGHTS_OUT_IN, WEIGHTS_IN_OUT = 0, 1

_c_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class CollIndex(ctypes.Structure):
    _fields_ = [("idx", _c_p), ("inv", _c_p), ("cu_seqlens", _c_p), ("count", _c_p),
                ("B", _i32), ("S", _i32), ("M_kept", _i32)]


class AttnCfg(ctypes.Structure):
    _fields_ = [("n_q_heads", _i32), ("n_kv_heads", _i32), ("head_dim", _i32), ("rot_dims", _i32),
                ("rope_base", ctypes.c_float), ("softmax_scale", ctypes.c_float), ("dmode", _i32)]


class AttnIO(ctypes.Structure):
    _fields_ = [("q", _c_p), ("ld_q", _i64), ("k", _c_p), ("ld_k", _i64), ("v", _c_p), ("ld_v", _i64),
                ("o", _c_p), ("ld_o", _i64), ("lse", _c_p), ("ld_lse", _i64), ("dout", _c_p),
                ("ld_do", _i64), ("dq", _c_p), ("ld_dq", _i64), ("dk", _c_p), ("ld_dk", _i64),
                ("dv", _c_p), ("ld_dv", _i64)]


class LayerCfg(ctypes.Structure):
    _fields_ = [("kind", _i32), ("hidden", _i32), ("n_q_heads", _i32), ("n_kv_heads", _i32),
                ("head_dim", _i32), ("rot_dims", _i32), ("inter", _i32),
                ("rope_base", ctypes.c_float), ("dmode", _i32), ("accumulate", _i32),
                ("unfiltered", _i32), ("weight_layout", _i32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, _c_p) for n in ("w_qkv", "w_o", "w_gateup", "w_down", "w_fc1", "w_fc2",
                                    "gamma1", "gamma2", "ln_gamma", "ln_beta")]


class LayerSaved(ctypes.Structure):
    _fields_ = [(n, _c_p) for n in ("x", "q", "k", "v", "o", "lse", "rstd1", "mean", "h", "rstd2",
                                    "gate", "up", "f")]


class LayerGrads(ctypes.Structure):
    _fields_ = [(n, _c_p) for n in ("dx", "dw_qkv", "dw_o", "dw_gateup", "dw_down", "dw_fc1",
                                    "dw_fc2", "dgamma1", "dgamma2", "dln_gamma", "dln_beta")]


_lib = None


def lib():
    """Load libcollider.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m token_filtered_backward_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    st = _i32
    sz = ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "collider_status_string": (ctypes.c_char_p, [_i32]),
        "collider_build_index": (st, [_c_p, _i32, _i32, _c_p, _c_p, _c_p, _c_p, _c_p]),
        "collider_build_index_expect": (st, [_c_p, _i32, _i32, _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]),
        "collider_index_count_host": (st, [_c_p, P(_i32), _c_p]),
        "collider_gather_rows": (st, [_c_p, _i64, _c_p, _i64, _c_p, _i32, _i32, _i32, _c_p]),
        "collider_scatter_rows": (st, [_c_p, _i64, _c_p, _i64, _c_p, _i32, _i32, _i32, _i32, _c_p]),
        "collider_linear_workspace_bytes": (sz, [_i32, _i32, _i32, _i32]),
        "collider_linear_bwd_reduced": (st, [_i32, _i32, _i32, _i32, _c_p, _i64, _c_p, _i64, _c_p,
                                             _c_p, _c_p, _c_p, _i32, _c_p, sz, _c_p]),
        "collider_attn_workspace_bytes": (sz, [P(AttnCfg), P(CollIndex)]),
        "collider_attn_bwd_filtered": (st, [P(AttnCfg), P(CollIndex), P(AttnIO), _c_p, sz, _c_p]),
        "collider_layer_workspace_bytes": (sz, [P(LayerCfg), _i32, _i32, _i32]),
        "collider_layer_bwd": (st, [P(LayerCfg), P(LayerWeights), P(LayerSaved), _c_p, _i32,
                                    P(CollIndex), P(LayerGrads), _i32, _c_p, sz, _c_p]),
        "collider_profile_enable": (st, [_i32]),
        "collider_gemm_set_policy": (st, [_i32]),
        "collider_gemm_describe_plan": (st, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_i32)]),
        "collider_profile_collect": (_i32, [ctypes.c_char_p, _i32, P(ctypes.c_double), P(_i32), _i32]),
        "collider_select_keep": (st, [_c_p, _i32, _i32, _c_p, _c_p]),
        "collider_select_workspace_bytes": (sz, [_i32]),
        "collider_select_keep_ws": (st, [_c_p, _i32, _i32, _c_p, _c_p, sz, _c_p]),
        "collider_ce_loss": (st, [_c_p, _i64, _c_p, _i32, _i32, _c_p, _c_p]),
        "collider_side_streams_live": (_i32, []),
        "collider_release_resources": (st, []),
        "collider_lm_head_workspace_bytes": (sz, [_i32, _i32, _i32]),
        "collider_lm_head_bwd": (st, [_c_p, _i64, _c_p, _c_p, _i64, _c_p, P(CollIndex), _i32, _i32,
                                      ctypes.c_float, _c_p, _i32, _c_p, _i32, _c_p, sz, _c_p]),
        "collider_embedding_workspace_bytes": (sz, [_i32, _i32]),
        "collider_embedding_bwd_noalloc": (st, [_c_p, _i64, _i32, _c_p, P(CollIndex), _i32, _i32, _c_p,
                                                _i32, _c_p]),
        "collider_embedding_bwd": (st, [_c_p, _i64, _i32, _c_p, P(CollIndex), _i32, _i32, _c_p, _i32,
                                        _c_p, sz, _c_p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


class ColliderError(RuntimeError):
    pass


def _check(status: int, what: str):
    if status != 0:
        msg = lib().collider_status_string(status).decode()
        raise ColliderError(f"{what}: status {status} ({msg})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ld(t):
    """Row stride in elements of a 2-D tensor with unit column stride (shape-derived when the
    stride is not meaningful: empty or single-row tensors)."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.shape[0] <= 1 or t.numel() == 0:
        return t.shape[1]
    if t.stride(1) != 1:
        raise ValueError("columns must be contiguous")
    return t.stride(0)


def _dt(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------------------------------------
# one-to-one wrappers of the C entry points
# ------------------------------------------------------------------------------------------------


def collider_build_index(keep, B, S, idx, inv, cu_seqlens, count, stream=None):
    _check(lib().collider_build_index(_ptr(keep), B, S, _ptr(idx), _ptr(inv), _ptr(cu_seqlens),
                                      _ptr(count), _stream(stream)), "collider_build_index")


def collider_build_index_expect(keep, B, S, expected_count, idx, inv, cu_seqlens, count, mismatch,
                                stream=None):
    _check(lib().collider_build_index_expect(_ptr(keep), B, S, int(expected_count), _ptr(idx), _ptr(inv),
                                             _ptr(cu_seqlens), _ptr(count), _ptr(mismatch),
                                             _stream(stream)), "collider_build_index_expect")


def collider_index_count_host(count, stream=None) -> int:
    out = _i32(0)
    _check(lib().collider_index_count_host(_ptr(count), ctypes.byref(out), _stream(stream)),
           "collider_index_count_host")
    return int(out.value)


def collider_gather_rows(src, dst, idx, n_rows, stream=None):
    """dst[c, :] = src[idx[c], :] for c < n_rows (2-D tensors with unit column stride)."""
    _check(lib().collider_gather_rows(_ptr(src), _ld(src), _ptr(dst), _ld(dst), _ptr(idx),
                                      n_rows, src.shape[1], _dt(src), _stream(stream)),
           "collider_gather_rows")


def collider_scatter_rows(src, dst, inv, M, zero_fill_filtered=True, stream=None):
    _check(lib().collider_scatter_rows(_ptr(src), _ld(src), _ptr(dst), _ld(dst), _ptr(inv),
                                       M, dst.shape[1], int(zero_fill_filtered), _dt(dst),
                                       _stream(stream)), "collider_scatter_rows")


def collider_linear_workspace_bytes(dt, M_kept, K, N) -> int:
    return int(lib().collider_linear_workspace_bytes(dt, M_kept, K, N))


def collider_linear_bwd_reduced(x, dy, w, dx, dw, db=None, accumulate=False, ws=None, stream=None):
    """dx = dy @ w, dw = dy^T @ x, db = colsum(dy) over the M_kept = x.shape[0] compacted rows."""
    Mk, K = x.shape
    N = w.shape[0]
    dt = _dt(w)
    if ws is None:
        nbytes = collider_linear_workspace_bytes(dt, Mk, K, N)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w.device)
    _check(lib().collider_linear_bwd_reduced(dt, Mk, K, N, _ptr(x), _ld(x), _ptr(dy), _ld(dy),
                                             _ptr(w), _ptr(dx), _ptr(dw), _ptr(db), int(accumulate),
                                             _ptr(ws), ws.numel(), _stream(stream)),
           "collider_linear_bwd_reduced")


def collider_attn_workspace_bytes(cfg: AttnCfg, ix: CollIndex) -> int:
    return int(lib().collider_attn_workspace_bytes(ctypes.byref(cfg), ctypes.byref(ix)))


def collider_attn_bwd_filtered(cfg: AttnCfg, ix: CollIndex, io: AttnIO, ws, stream=None):
    _check(lib().collider_attn_bwd_filtered(ctypes.byref(cfg), ctypes.byref(ix), ctypes.byref(io),
                                            _ptr(ws), ws.numel(), _stream(stream)),
           "collider_attn_bwd_filtered")


def collider_select_keep(score, n_keep, keep, stream=None):
    """keep[t] = 1 for the n_keep largest scores (float32 [M]; ties: lower t first), else 0."""
    _check(lib().collider_select_keep(_ptr(score), score.numel(), int(n_keep), _ptr(keep),
                                      _stream(stream)), "collider_select_keep")


def collider_select_workspace_bytes(M) -> int:
    return int(lib().collider_select_workspace_bytes(int(M)))


def collider_select_keep_ws(score, n_keep, keep, ws, stream=None):
    """collider_select_keep over many workgroups (same mask); ws: uint8 device tensor of at least
    collider_select_workspace_bytes(M) bytes (may be None when that is 0)."""
    _check(lib().collider_select_keep_ws(_ptr(score), score.numel(), int(n_keep), _ptr(keep),
                                         _ptr(ws) if ws is not None else None,
                                         ws.numel() if ws is not None else 0, _stream(stream)),
           "collider_select_keep_ws")


def collider_ce_loss(logits, labels, loss, stream=None):
    """loss[t] = logsumexp(logits[t]) - logits[t, labels[t]] (0 for a label outside [0, V)) for
    every token: logits bf16 [M, V], labels int32 [M], loss float32 [M]."""
    M, V = logits.shape
    if logits.dtype != torch.bfloat16 or labels.dtype != torch.int32 or loss.dtype != torch.float32:
        raise TypeError("logits must be bfloat16, labels int32 and loss float32")
    if labels.numel() != M or loss.numel() != M:
        raise ValueError("labels and loss need one entry per logits row")
    _check(lib().collider_ce_loss(_ptr(logits), _ld(logits), _ptr(labels), M, V, _ptr(loss),
                                  _stream(stream)), "collider_ce_loss")


def ce_loss(logits: torch.Tensor, labels: torch.Tensor, stream=None) -> torch.Tensor:
    loss = torch.empty(logits.shape[0], dtype=torch.float32, device=logits.device)
    collider_ce_loss(logits, labels, loss, stream)
    return loss


def collider_side_streams_live() -> int:
    """Side-stream sets the library holds (leased or idle, every device)."""
    return int(lib().collider_side_streams_live())


def collider_release_resources():
    """Destroy the library's idle side streams and pooled timing events."""
    _check(lib().collider_release_resources(), "collider_release_resources")


def select_keep(score: torch.Tensor, n_keep: int, stream=None) -> torch.Tensor:
    if score.dtype != torch.float32 or not score.is_contiguous():
        raise TypeError("score must be a contiguous float32 tensor")
    keep = torch.empty(score.numel(), dtype=torch.uint8, device=score.device)
    need = collider_select_workspace_bytes(score.numel())
    if need:  # large token counts: the selection spread over the GPU
        ws = torch.empty(need, dtype=torch.uint8, device=score.device)
        collider_select_keep_ws(score, n_keep, keep, ws, stream)
    else:
        collider_select_keep(score, n_keep, keep, stream)
    return keep


def collider_lm_head_workspace_bytes(M_kept, H, V) -> int:
    return int(lib().collider_lm_head_workspace_bytes(M_kept, H, V))


def collider_lm_head_bwd(logits, labels, h, w_lm, ix: CollIndex, loss_scale, dh, dw_lm,
                         dh_compact=False, accumulate=False, ws=None, stream=None):
    """Cross-entropy backward through the LM head over kept tokens: logits bf16 [M, V] (full
    layout), labels int32 [M], h bf16 [M, H], w_lm bf16 [V, H] -> dh bf16 ([M_kept, H] when
    dh_compact, else [M, H] with zero filtered rows) and dw_lm float32 [V, H]."""
    V, H = w_lm.shape
    for name, t, dt in (("logits", logits, torch.bfloat16), ("h", h, torch.bfloat16), ("w_lm", w_lm, torch.bfloat16),
                        ("labels", labels, torch.int32), ("dh", dh, torch.bfloat16), ("dw_lm", dw_lm, torch.float32)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
    if ws is None:
        ws = torch.empty(max(1, collider_lm_head_workspace_bytes(ix.M_kept, H, V)), dtype=torch.uint8,
                         device=h.device)
    _check(lib().collider_lm_head_bwd(_ptr(logits), _ld(logits), _ptr(labels), _ptr(h), _ld(h),
                                      _ptr(w_lm), ctypes.byref(ix), H, V, float(loss_scale), _ptr(dh),
                                      int(bool(dh_compact)), _ptr(dw_lm), int(bool(accumulate)),
                                      _ptr(ws), ws.numel(), _stream(stream)), "collider_lm_head_bwd")


def collider_embedding_workspace_bytes(M_kept, V) -> int:
    return int(lib().collider_embedding_workspace_bytes(M_kept, V))


def collider_embedding_bwd(dx, ids, ix: CollIndex, dE, dx_compact=False, accumulate=False, ws=None,
                           stream=None):
    """dE[v] (+)= sum of dx rows of the kept tokens with ids == v (token order); dx bf16 [M_kept, H]
    (dx_compact) or [M, H], ids int32 [M], dE float32 [V, H]."""
    V, H = dE.shape
    if dE.dtype != torch.float32 or ids.dtype != torch.int32 or (dx is not None and dx.dtype != torch.bfloat16):
        raise TypeError("dx must be bfloat16, ids int32 and dE float32")
    if ws is None:
        ws = torch.empty(max(1, collider_embedding_workspace_bytes(ix.M_kept, V)), dtype=torch.uint8,
                         device=dE.device)
    _check(lib().collider_embedding_bwd(_ptr(dx), _ld(dx) if dx is not None else H,
                                        int(bool(dx_compact)), _ptr(ids), ctypes.byref(ix), H, V,
                                        _ptr(dE), int(bool(accumulate)), _ptr(ws), ws.numel(),
                                        _stream(stream)), "collider_embedding_bwd")


def collider_embedding_bwd_noalloc(dx, ids, ix: CollIndex, dE, dx_compact=False, accumulate=False,
                                   stream=None):
    """collider_embedding_bwd without a workspace (the library's fixed device scratch; V <= 262144,
    M_kept <= 1048576; calls that overlap on one GPU race)."""
    V, H = dE.shape
    if dE.dtype != torch.float32 or ids.dtype != torch.int32 or (dx is not None and dx.dtype != torch.bfloat16):
        raise TypeError("dx must be bfloat16, ids int32 and dE float32")
    _check(lib().collider_embedding_bwd_noalloc(_ptr(dx), _ld(dx) if dx is not None else H,
                                                int(bool(dx_compact)), _ptr(ids), ctypes.byref(ix), H, V,
                                                _ptr(dE), int(bool(accumulate)), _stream(stream)),
           "collider_embedding_bwd_noalloc")


def collider_layer_workspace_bytes(cfg: LayerCfg, B, S, M_kept) -> int:
    return int(lib().collider_layer_workspace_bytes(ctypes.byref(cfg), B, S, M_kept))


def collider_layer_bwd(cfg: LayerCfg, w: LayerWeights, saved: LayerSaved, dy, dy_compact,
                       ix: CollIndex, grads: LayerGrads, dx_compact, ws, stream=None):
    _check(lib().collider_layer_bwd(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(saved), _ptr(dy),
                                    int(dy_compact), ctypes.byref(ix), ctypes.byref(grads),
                                    int(dx_compact), _ptr(ws), ws.numel(), _stream(stream)),
           "collider_layer_bwd")


GEMM_POLICY_AUTO, GEMM_POLICY_SPLITK, GEMM_POLICY_STREAMK, GEMM_POLICY_TILES = 0, 1, 2, 3


def collider_gemm_set_policy(policy: int):
    """GEMM work decomposition for the calling thread (0 cost model, 1 tiles + K-splits,
    2 stream-K, 3 whole tiles only).  Query workspace sizes after changing it."""
    _check(lib().collider_gemm_set_policy(int(policy)), "collider_gemm_set_policy")


def collider_gemm_describe_plan(M, N, K, layout, concurrent=False):
    """{bm, bn, splits, dp_tiles, sk_tiles, grid, lds} of the bf16 GEMM plan (host only)."""
    out = (_i32 * 7)()
    _check(lib().collider_gemm_describe_plan(int(M), int(N), int(K), int(layout), int(concurrent), out),
           "collider_gemm_describe_plan")
    return dict(zip(("bm", "bn", "splits", "dp_tiles", "sk_tiles", "grid", "lds"), list(out)))


def collider_profile_enable(on: bool):
    _check(lib().collider_profile_enable(int(on)), "collider_profile_enable")


def collider_profile_collect(max_kernels=64):
    """{kernel name: (total ms, launches)} recorded since the last collect."""
    cap = 64 * max_kernels
    names = ctypes.create_string_buffer(cap)
    ms = (ctypes.c_double * max_kernels)()
    cnt = (_i32 * max_kernels)()
    n = lib().collider_profile_collect(names, cap, ms, cnt, max_kernels)
    if n < 0:
        raise ColliderError("collider_profile_collect failed")
    out, parts = {}, names.raw.split(b"\0")
    for i in range(n):
        out[parts[i].decode()] = (float(ms[i]), int(cnt[i]))
    return out


# ------------------------------------------------------------------------------------------------
# conveniences
# ------------------------------------------------------------------------------------------------


@dataclass
class Index:
    idx: torch.Tensor
    inv: torch.Tensor
    cu_seqlens: torch.Tensor
    count: torch.Tensor
    B: int
    S: int
    M_kept: int
    mismatch: torch.Tensor = None  # set by build_index(..., expect=n): device flag, 1 = count != n

    def c(self) -> CollIndex:
        return CollIndex(self.idx.data_ptr(), self.inv.data_ptr(), self.cu_seqlens.data_ptr(),
                         self.count.data_ptr(), self.B, self.S, self.M_kept)

    def check(self):
        """For an index built with an announced count: raise if the mask kept another number of
        tokens (waits for the index build)."""
        if self.mismatch is not None and int(self.mismatch.item()) != 0:
            raise ColliderError(f"keep mask holds {int(self.count.item())} kept tokens, "
                                f"{self.M_kept} were announced")


def build_index(keep: torch.Tensor, B: int, S: int, stream=None, out: "Index" = None,
                expect: int = None) -> Index:
    """Compact a [B*S] uint8 keep mask on the device.  Without `expect` this waits once for the
    kept count.  With `expect` (the number of tokens the mask is known to keep, e.g. a top-k) it
    does not wait: the device checks the count, and Index.check() reports a mismatch.  With `out`
    the index is rebuilt in that index's buffers (same addresses every step)."""
    dev = keep.device
    M = B * S
    if out is not None and out.B == B and out.S == S and out.idx.numel() == M:
        idx, inv, cu, count, mm = out.idx, out.inv, out.cu_seqlens, out.count, out.mismatch
    else:
        idx = torch.empty(M, dtype=torch.int32, device=dev)
        inv = torch.empty(M, dtype=torch.int32, device=dev)
        cu = torch.empty(B + 1, dtype=torch.int32, device=dev)
        count = torch.empty(1, dtype=torch.int32, device=dev)
        mm = None
    if expect is None:
        collider_build_index(keep, B, S, idx, inv, cu, count, stream)
        mk = collider_index_count_host(count, stream)
        mm = None
    else:
        if mm is None:
            mm = torch.zeros(1, dtype=torch.int32, device=dev)
        collider_build_index_expect(keep, B, S, expect, idx, inv, cu, count, mm, stream)
        mk = int(expect)
    if out is not None and out.idx is idx:
        out.M_kept, out.mismatch = mk, mm
        return out
    return Index(idx, inv, cu, count, B, S, mk, mm)


def layer_cfg(shape, dmode=ATTN_D_FILTERED, accumulate=False, unfiltered=False,
              weight_layout=WEIGHTS_OUT_IN) -> LayerCfg:
    """LayerCfg from any object with kind/H/nq/nkv/d/rot/I/rope_base attributes.
    unfiltered=True selects the ordinary dense backward over all tokens (the baseline);
    weight_layout=WEIGHTS_IN_OUT takes every projection weight (and returns its gradient) as
    W [in, out] instead of w [out, in]."""
    return LayerCfg(LAYER_LLAMA if shape.kind == "llama" else LAYER_PHI, shape.H, shape.nq, shape.nkv,
                    shape.d, shape.rot, shape.I, float(shape.rope_base), dmode, int(accumulate),
                    int(unfiltered), int(weight_layout))


def to_in_out(weights: dict) -> dict:
    """The projection weights of a [out, in] weight dict as contiguous [in, out] matrices (the
    norm parameters unchanged), for weight_layout=WEIGHTS_IN_OUT."""
    proj = ("w_qkv", "w_o", "w_gateup", "w_down", "w_fc1", "w_fc2")
    return {k: (v.t().contiguous() if k in proj and v is not None else v) for k, v in weights.items()}


def dense_index(B: int, S: int) -> Index:
    """Index placeholder for the unfiltered baseline (only B and S are read)."""
    z = torch.empty(0, dtype=torch.int32)
    return Index(z, z, z, z, B, S, B * S)


def _struct(cls, tensors: dict):
    return cls(**{k: (v.data_ptr() if v is not None else None) for k, v in tensors.items()})


def make_grads(cfg: LayerCfg, M: int, M_kept: int, device, dx_compact=False) -> dict:
    H, I, d = cfg.hidden, cfg.inter, cfg.head_dim
    nqkv = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * d
    f32 = dict(dtype=torch.float32, device=device)
    io = cfg.weight_layout == WEIGHTS_IN_OUT

    def w(rows, cols):  # a weight gradient in the weights' layout
        return torch.empty((cols, rows) if io else (rows, cols), **f32)

    g = {"dx": torch.empty((M_kept if dx_compact else M, H), dtype=torch.bfloat16, device=device),
         "dw_qkv": w(nqkv, H), "dw_o": w(H, cfg.n_q_heads * d)}
    if cfg.kind == LAYER_LLAMA:
        g.update(dw_gateup=w(2 * I, H), dw_down=w(H, I),
                 dgamma1=torch.empty(H, **f32), dgamma2=torch.empty(H, **f32))
    else:
        g.update(dw_fc1=w(I, H), dw_fc2=w(H, I),
                 dln_gamma=torch.empty(H, **f32), dln_beta=torch.empty(H, **f32))
    return g


class LayerBackward:
    """Reusable filtered layer backward: holds the workspace; call with an Index per step."""

    def __init__(self, cfg: LayerCfg, B: int, S: int, device="cuda"):
        self.cfg, self.B, self.S, self.device = cfg, B, S, device
        self.ws = None

    def workspace(self, M_kept: int):
        need = collider_layer_workspace_bytes(self.cfg, self.B, self.S, M_kept)
        if need == 0:
            raise ColliderError("invalid layer configuration")
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self.ws

    def _args(self, weights, saved, dy, index, grads, dy_compact, dx_compact):
        """ctypes arguments of one call, reused while every pointer stays the same (building the
        structures costs more host time than the library's launches)."""
        key = (tuple(t.data_ptr() for t in weights.values()), tuple(saved.keys()),
               tuple(t.data_ptr() for t in saved.values()), tuple(grads.keys()),
               tuple(t.data_ptr() for t in grads.values()), dy.data_ptr(), index.idx.data_ptr(),
               index.M_kept, bool(dy_compact), bool(dx_compact), tuple(weights.keys()))
        if getattr(self, "_key", None) != key:
            ws = self.workspace(index.M_kept)
            self._key = key
            self._cargs = (ctypes.byref(self.cfg), ctypes.byref(_struct(LayerWeights, weights)),
                           ctypes.byref(_struct(LayerSaved, saved)), ctypes.c_void_p(dy.data_ptr()),
                           int(dy_compact), ctypes.byref(index.c()),
                           ctypes.byref(_struct(LayerGrads, grads)), int(dx_compact),
                           ctypes.c_void_p(ws.data_ptr()), ws.numel())
        return self._cargs

    def __call__(self, weights: dict, saved: dict, dy, index: Index, grads: dict, dy_compact=False,
                 dx_compact=False, stream=None, graph=False):
        """graph=True records the call into a HIP graph on first use and replays it while every
        pointer and the kept count stay the same (one launch instead of the layer's ~30; with
        top-k selection the kept count is the same every step).  The index buffers must then be
        reused across steps (build_index(..., out=index)).  The graph is captured and replayed on
        the current stream: graph=True does not take an explicit `stream` (make the stream current
        with torch.cuda.stream(...) instead)."""
        if graph and stream is not None and stream != torch.cuda.current_stream():
            raise ValueError("graph=True replays on the current stream; pass no other stream "
                             "(wrap the call in torch.cuda.stream(s) instead)")
        args = self._args(weights, saved, dy, index, grads, dy_compact, dx_compact)
        if not graph:
            _check(lib().collider_layer_bwd(*args, _stream(stream)), "collider_layer_bwd")
            return grads
        key = (self._key, torch.cuda.current_stream().cuda_stream)
        if getattr(self, "_graph_key", None) != key:
            # one eager call first: the library's one-time set-up (side stream, kernel attributes)
            # must not happen inside the capture
            _check(lib().collider_layer_bwd(*args, _stream()), "collider_layer_bwd")
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                _check(lib().collider_layer_bwd(*args, _stream()), "collider_layer_bwd")
            self._graph, self._graph_key = g, key
        self._graph.replay()  # on the current stream, after the work already queued there
        return grads


def layer_bwd(cfg: LayerCfg, weights: dict, saved: dict, dy, index: Index, grads=None, **kw):
    """One filtered layer backward: returns the dict of gradients (allocated if not given)."""
    if grads is None:
        grads = make_grads(cfg, index.B * index.S, index.M_kept, dy.device, kw.get("dx_compact", False))
    return LayerBackward(cfg, index.B, index.S, dy.device)(weights, saved, dy, index, grads, **kw)
