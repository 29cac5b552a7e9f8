#!/usr/bin/env python3
"""Filtered transformer-layer backward on one MI355X.

One step = the whole filtered path for one batch: keep mask -> index (built on the device every
step; top-k fixes the kept count, so the host may announce it instead of waiting for it - both
are timed), gathers, every reduced GEMM, the filtered attention backward, norm / activation backward and
the scatter of dx, for one TinyLlama-shaped layer (B 4 x S 2048, hidden 2048, 32/4 heads x 64,
SwiGLU 5632) with 40% of the tokens filtered by top-k on a LogNormal score.  Inputs are synthetic
(seeded generator, random-init weights) and resident in HBM before timing starts.

Prints one JSON line: value = ms per filtered layer backward (back-to-back steps), the speedup over
the unfiltered dense backward of the same layer (same kernels on all tokens, no index / gather /
scatter, D = dO . O), the reduced-GEMM roofline (bf16 MFMA) from per-kernel HIP events, and the
CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config tinyllama] [--r 40]
                    [--seq S [--tokens T]]      (long-context sweep: S per sequence, B = T / S)
                    [--loss-side [--vocab V]]   (the loss-side steps instead of the layer)
                    [--sparse-sweep]            (Figure 4: torch.sparse vs dense vs reduced GEMMs)
                    [--index-sweep]             (mask -> index build time from 8192 to 4M tokens)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "filtered layer-bwd ms, MFMA util & speedup vs unfiltered at 40% filter"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(cfg, M_kept, seq_counts):
    """Algorithmic work of one filtered layer backward (never the dense work avoided)."""
    H, I, d, nq, nkv = cfg.H, cfg.I, cfg.d, cfg.nq, cfg.nkv
    nqkv = (nq + 2 * nkv) * d
    if cfg.kind == "llama":
        proj = H * nqkv + H * nq * d + 2 * I * H + H * I
    else:
        proj = H * nqkv + H * nq * d + I * H + H * I
    gemm_flops = 4.0 * M_kept * proj                      # dX and dW: 2 * M' * K * N each
    pairs = sum(n * (n + 1) // 2 for n in seq_counts)     # causal kept (query, key) pairs per head
    attn_flops = 10.0 * d * nq * pairs                    # S, dP, dV, dK, dQ
    # the filtered softmax-backward row term (reading A): accumulated in the dQ kernel's one sweep,
    # whose only extra matrix work is sum_j P_ij K_j
    attn_dt_flops = 2.0 * d * nq * pairs
    # the one gather left: dY's kept rows (read + write); attention and the recompute kernels read
    # the other saved tensors through the index
    gather_bytes = 2.0 * M_kept * 2 * H
    # reduced-GEMM bytes: bf16 operands read once, outputs written once (bf16 dX, fp32 dW), plus
    # the activation-backward epilogue's reads of the saved pre-activations
    Mk, nqd = M_kept, nq * d
    if cfg.kind == "llama":
        gemm_bytes = [2 * (Mk * H + H * I) + 8 * Mk * I,                  # dA (SwiGLU epilogue)
                      2 * Mk * H + 2 * Mk * I + 4 * H * I,                 # dW down
                      2 * (2 * Mk * I + 2 * I * H + Mk * H),               # dX gate/up
                      4 * Mk * I + 2 * Mk * H + 8 * I * H,                 # dW gate/up
                      2 * (Mk * H + H * nqd + Mk * nqd),                   # dO
                      2 * Mk * H + 2 * Mk * nqd + 4 * H * nqd,             # dW o
                      2 * (Mk * nqkv + nqkv * H + Mk * H),                 # dX qkv
                      2 * Mk * nqkv + 2 * Mk * H + 4 * nqkv * H]           # dW qkv
    else:
        gemm_bytes = [2 * (Mk * H + H * I) + 4 * Mk * I,                  # dF (GELU epilogue)
                      2 * Mk * H + 2 * Mk * I + 4 * H * I,                 # dW fc2
                      2 * (Mk * H + H * nqd + Mk * nqd),                   # dO
                      2 * Mk * H + 2 * Mk * nqd + 4 * H * nqd,             # dW o
                      2 * (Mk * (nqkv + I) + (nqkv + I) * H + Mk * H),     # dX (qkv and fc1)
                      2 * Mk * nqkv + 2 * Mk * H + 4 * nqkv * H,           # dW qkv
                      2 * Mk * I + 2 * Mk * H + 4 * I * H]                 # dW fc1
    # the scatter writes +0.0 to the filtered rows of dx; the last norm backward writes the kept rows
    scatter_bytes = 2.0 * (cfg.M - M_kept) * H
    return {"gemm_flops": gemm_flops, "attn_flops": attn_flops, "attn_dt_flops": attn_dt_flops,
            "pairs": pairs, "gather_bytes": gather_bytes, "scatter_bytes": scatter_bytes,
            "gemm_bytes": float(sum(gemm_bytes)),
            "gemm_launches": len(gemm_bytes)}


TRAFFIC_FILE = "profiles/gemm_bf16_tinyllama_b4s2048_r40_traffic.md"


def measured_traffic(cfg, r_pct):
    """HBM bytes per reduced-GEMM launch from the committed counter runs (rocprofv3 FETCH_SIZE and
    WRITE_SIZE, calibrated on a plain copy), or None when they were taken on another workload or on
    a GEMM source other than the one built here."""
    import hashlib
    import re
    if (cfg.name, cfg.B, cfg.S, r_pct) != ("tinyllama", 4, 2048, 40):
        return None
    path = os.path.join(ROOT, TRAFFIC_FILE)
    src = os.path.join(ROOT, "token_filtered_backward_amd", "csrc", "gemm.hip")
    try:
        text = open(path).read()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    h = re.search(r"gemm_source_sha256: ([0-9a-f]+)", text)
    if not m or not h or h.group(1) != sha:
        return None
    return float(m.group(1))


def host_cpu():
    """(cores this process may run on, CPU model name) of the host: the affinity mask's size, or
    the OMP_NUM_THREADS share when the host sets a smaller one."""
    cores = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and 0 < int(share) < cores:
        cores = int(share)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def cpu_baseline(cfg, inp, min_seconds=8.0):
    """The oracle as it stands, in float32 (its float64 arithmetic switched to float32), on whole
    sequences of the same workload, scaled to one layer.  BLAS runs one thread per core this
    process may use."""
    import numpy as np

    import oracle
    import synth
    import contextlib
    cores, model = host_cpu()
    try:
        from threadpoolctl import threadpool_limits
        blas = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        blas = contextlib.nullcontext()
    S = cfg.S
    one = cfg.with_(B=1)
    w = synth.floats(inp["weights"])
    done, t_total = 0, 0.0
    with blas, oracle.precision(np.float32):
        for b in range(cfg.B):
            rows = slice(b * S, (b + 1) * S)
            sv = {k: v[rows] for k, v in synth.floats(inp["saved"]).items()}
            dy = synth.bf16_bits_to_f32(inp["dy"][rows])
            keep = inp["keep"][rows]
            t0 = time.perf_counter()
            oracle.layer_bwd(one, w, sv, dy, keep, "filtered")
            t_total += time.perf_counter() - t0
            done += 1
            if t_total >= min_seconds:
                break
    ms = t_total * 1e3 * cfg.B / done
    return {"value": round(ms, 1), "unit": "ms", "cores": int(cores), "kind": "oracle",
            "cpu_model": model, "precision": "float32",
            "sample": f"{done} of {cfg.B} sequences (S={S}) of the same layer, float32 NumPy oracle with "
                      f"{cores} BLAS threads, scaled x{cfg.B / done:g} (the layer's work is linear in the "
                      "sequence count)"}


def calibration_copy(mb):
    """One elementwise kernel over `mb` MiB (reads mb MiB, writes mb MiB): a plain copy of known size
    that calibrates HBM byte counters in a profiler run."""
    if mb <= 0:
        return
    import torch
    n = mb << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    log(f"[bench] calibration copy of {mb} MiB done")


def lm_head_traffic(cfg, r_pct, vocab):
    """HBM bytes per LM-head GEMM launch from the committed counter runs, or None for another
    workload or another GEMM / entry-point source than the one built here."""
    import hashlib
    import re
    if (cfg.name, cfg.B, cfg.S, r_pct, vocab) != ("tinyllama", 4, 2048, 40, 32000):
        return None
    path = os.path.join(ROOT, "profiles", "gemm_bf16_lm_head_b4s2048_v32000_r40_traffic.md")
    csrc = os.path.join(ROOT, "token_filtered_backward_amd", "csrc")
    try:
        text = open(path).read()
        shas = {n: hashlib.sha256(open(os.path.join(csrc, n), "rb").read()).hexdigest()
                for n in ("gemm.hip", "api.hip")}
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    ok = all(re.search(rf"{re.escape(n)}_sha256: {h}", text) for n, h in shas.items())
    return float(m.group(1)) if m and ok else None


def loss_side_bench(args, cfg, emit=True):
    """The loss-side steps of one batch: logits -> per-token cross-entropy loss of every token ->
    keep mask (device top-k on the loss) -> index -> LM-head cross-entropy backward over the kept
    tokens (dh stays compact for the top layer) -> embedding gradient from the bottom layer's
    compact dx.  Unfiltered: the per-token loss (a training step computes it either way) and the
    same LM-head and embedding backward over every token (no selection or index)."""
    import numpy as np
    import torch

    import synth
    import token_filtered_backward_amd as tfb

    dev = "cuda"
    calibration_copy(getattr(args, "copy_calibration_mb", 0))
    B, S, M, H, V = cfg.B, cfg.S, cfg.M, cfg.H, args.vocab
    n_keep = M - synth.n_filtered(M, args.r)
    log(f"[bench] loss side: M={M} H={H} V={V} r={args.r}% (kept {n_keep})")
    rng = np.random.default_rng(args.seed)
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    logits = (torch.randn((M, V), generator=g, device=dev) * 2.0).to(torch.bfloat16)
    h = torch.randn((M, H), generator=g, device=dev).to(torch.bfloat16)
    w_lm = (torch.randn((V, H), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    labels = torch.from_numpy(rng.integers(0, V, M).astype(np.int32)).to(dev)
    # token ids of text follow Zipf's law: id v (by frequency rank) with probability ~ 1 / (v+1)^1.1,
    # so that a few ids carry many tokens (the most frequent one about a tenth of the batch)
    zipf_p = 1.0 / np.arange(1, V + 1, dtype=np.float64) ** 1.1
    ids = torch.from_numpy(rng.choice(V, size=M, p=zipf_p / zipf_p.sum()).astype(np.int32)).to(dev)
    dx = torch.randn((n_keep, H), generator=g, device=dev).to(torch.bfloat16)
    dx_full = torch.randn((M, H), generator=g, device=dev).to(torch.bfloat16)
    keep = torch.empty(M, dtype=torch.uint8, device=dev)
    loss = torch.empty(M, dtype=torch.float32, device=dev)
    ixp = tfb.build_index(torch.ones(M, dtype=torch.uint8, device=dev), B, S)
    dh = torch.empty((n_keep, H), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((V, H), dtype=torch.float32, device=dev)
    dE = torch.empty((V, H), dtype=torch.float32, device=dev)
    ws_lm = torch.empty(tfb.collider_lm_head_workspace_bytes(M, H, V), dtype=torch.uint8, device=dev)
    ws_e = torch.empty(tfb.collider_embedding_workspace_bytes(M, V), dtype=torch.uint8, device=dev)
    # every token kept (a real index: the LM-head path reads rows through it, so the unfiltered
    # step also copies h once, about 1% of its time)
    uix = tfb.build_index(torch.ones(M, dtype=torch.uint8, device=dev), B, S)
    dh_u = torch.empty((M, H), dtype=torch.bfloat16, device=dev)

    def step():
        tfb.collider_ce_loss(logits, labels, loss)
        tfb.collider_select_keep(loss, n_keep, keep)
        ix = tfb.build_index(keep, B, S, out=ixp, expect=n_keep)
        c = ix.c()
        tfb.collider_lm_head_bwd(logits, labels, h, w_lm, c, 1.0 / n_keep, dh, dw, dh_compact=True, ws=ws_lm)
        tfb.collider_embedding_bwd(dx, ids, c, dE, dx_compact=True, ws=ws_e)

    def step_unf():
        tfb.collider_ce_loss(logits, labels, loss)
        c = uix.c()
        tfb.collider_lm_head_bwd(logits, labels, h, w_lm, c, 1.0 / M, dh_u, dw, dh_compact=True, ws=ws_lm)
        tfb.collider_embedding_bwd(dx_full, ids, c, dE, dx_compact=True, ws=ws_e)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / args.steps

    ms_f = timed(step)
    ixp.check()
    ms_u = timed(step_unf)
    log(f"[bench] loss side filtered {ms_f:.3f} ms, unfiltered {ms_u:.3f} ms")

    def kernels(fn):
        n = max(3, min(args.steps, 10))
        torch.cuda.synchronize()
        tfb.collider_profile_collect()
        tfb.collider_profile_enable(True)
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        prof = tfb.collider_profile_collect()
        tfb.collider_profile_enable(False)
        return {k: v[0] / n for k, v in prof.items()}

    kf, ku = kernels(step), kernels(step_unf)
    gemm_ms = kf.get("lm_head_dh", 0.0) + kf.get("lm_head_dw", 0.0)
    gemm_flops = 2 * 2.0 * n_keep * H * V
    ce_bytes = 2.0 * n_keep * V * 2
    emb_ms = sum(v for k, v in kf.items() if k.startswith("embed_"))
    emb_bytes = 4.0 * V * H + 2.0 * n_keep * H
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None
    out = {
        "metric": "loss-side bwd ms (per-token loss, token selection, LM-head cross-entropy bwd, "
                  f"embedding grad) at {args.r}% filter",
        "value": round(ms_f, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_f, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"loss side of a {cfg.name}-shaped model, B{B}xS{S}, hidden {H}, vocab {V}, "
                               f"{args.r}% filtered", "M": M, "M_kept": n_keep, "hidden": H, "vocab": V},
        "ms_unfiltered": round(ms_u, 4), "speedup_vs_unfiltered": round(ms_u / ms_f, 3),
        "kernel_ms_per_step": {k: round(v, 4) for k, v in sorted(kf.items(), key=lambda kv: -kv[1])},
        "kernel_ms_per_step_unfiltered": {k: round(v, 4) for k, v in sorted(ku.items(), key=lambda kv: -kv[1])},
        "ce_grad_gbs": round(ce_bytes / (kf["ce_grad"] * 1e-3) / 1e9, 1) if kf.get("ce_grad") else None,
        "embedding_gbs": round(emb_bytes / (emb_ms * 1e-3) / 1e9, 1) if emb_ms else None,
        "select_ms": round(kf.get("select_topk", 0.0), 4),
        "ce_loss_ms": round(kf.get("ce_loss", 0.0), 4),
        "ce_loss_gbs": round(2.0 * M * V / (kf["ce_loss"] * 1e-3) / 1e9, 1) if kf.get("ce_loss") else None,
        "roofline": {"kernel": "gemm_bf16 (the LM head's dh and dW reduced GEMMs)", "bound": "mfma",
                     "achieved": None if gemm_tflops is None else round(gemm_tflops, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": None if gemm_tflops is None else round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": lm_head_traffic(cfg, args.r, V), "flops_per_launch": gemm_flops / 2,
                     "algorithmic_bytes_per_launch": (2.0 * n_keep * V + 2.0 * V * H + 2.0 * n_keep * H
                                                      + 2.0 * n_keep * V + 2.0 * n_keep * H + 4.0 * V * H) / 2,
                     "avg_launch_ms": round(gemm_ms / 2, 5)},
    }
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            cores = len(os.sched_getaffinity(0))
        rows = 512  # kept rows of the sample (the LM-head work is linear in the kept-row count)
        lg = logits[:rows].float().cpu().numpy()
        t0 = time.perf_counter()
        oracle.lm_head_bwd(lg, labels[:rows].cpu().numpy(), h[:rows].float().cpu().numpy(),
                           w_lm.float().cpu().numpy(), np.ones(rows, np.uint8), 1.0 / rows)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(dt * 1e3 * n_keep / rows, 1), "unit": "ms", "cores": int(cores),
                               "kind": "oracle",
                               "sample": f"LM-head backward of {rows} kept rows (float64 NumPy), scaled x"
                                         f"{n_keep / rows:g} to the {n_keep} kept rows; selection and "
                                         "embedding gradient not included"}
    if emit:
        print(json.dumps(out), flush=True)
    return out


def sparse_sweep_bench(args, cfg):
    """Figure 4 on this GPU: the linear backward of the gate/up projection of the layer (the
    row-sparse gradient dG [M, 2I] of a filtered batch, its input X [M, H], weight w [2I, H]) over a
    filter-ratio sweep, computed three ways:
      dense   torch.matmul (hipBLASLt) on all M rows, filtered rows of dG zeroed - what filtering
              only the loss costs;
      sparse  torch.sparse.mm with dG in CSR (rows of filtered tokens empty), float32 - PyTorch's
              sparse GEMM, the comparison of the Figure 4 caption;
      reduced this library: gather of the kept rows of dG and X, then collider_linear_bwd_reduced
              (dense GEMMs over the M' kept rows); beside it torch.matmul on the same compacted
              rows (the vendor GEMM on the reduced shapes).
    Each is dX = dG w plus dW = dG^T X.  Context only (no target)."""
    import numpy as np
    import torch

    import synth
    import token_filtered_backward_amd as tfb

    dev = "cuda"
    M, H, N = cfg.M, cfg.H, 2 * cfg.I
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    dG = torch.randn((M, N), generator=g, device=dev).to(torch.bfloat16)
    X = torch.randn((M, H), generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn((N, H), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    reps = max(3, min(args.steps, 10))

    def t_ms(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    # The sparse leg runs in float32 only: the ROCm sparse library's SpMM documents no type
    # combination with bf16 inputs and a bf16 result (bf16 inputs need a float32 result), which is
    # what torch.sparse.mm on two bf16 operands would ask for.
    def sparse_ms(a, b):
        """ms of torch.sparse.mm(a as float32 CSR, b as float32)."""
        a_sp = a.float().to_sparse_csr()
        b_ = b.float()
        return t_ms(lambda: torch.sparse.mm(a_sp, b_))

    rows = []
    for r in (0, 10, 20, 30, 40, 50, 60, 70, 80, 90, 95, 99):
        keep_np = synth.make_keep(M, r, args.seed)
        keep = torch.from_numpy(keep_np).to(dev)
        dGm = dG * keep[:, None].to(torch.bfloat16)
        dGmT = dGm.t().contiguous()
        ix = tfb.build_index(keep, cfg.B, cfg.S)
        mk = ix.M_kept
        row = {"r_pct": r, "M_kept": mk}
        row["dense_bf16_ms"] = t_ms(lambda: (torch.matmul(dGm, w), torch.matmul(dGmT, X)))
        dGf, dGfT, Xf, wf = dGm.float(), dGmT.float(), X.float(), w.float()
        row["dense_f32_ms"] = t_ms(lambda: (torch.matmul(dGf, wf), torch.matmul(dGfT, Xf)))
        row["sparse_f32_ms"] = sparse_ms(dGm, w) + sparse_ms(dGmT, X)
        dGk = torch.empty((max(mk, 1), N), dtype=torch.bfloat16, device=dev)
        Xk = torch.empty((max(mk, 1), H), dtype=torch.bfloat16, device=dev)
        dx = torch.empty((max(mk, 1), H), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((N, H), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, tfb.collider_linear_workspace_bytes(tfb.BF16, mk, H, N)), dtype=torch.uint8,
                         device=dev)

        def reduced(gather=True):
            if gather and mk:
                tfb.collider_gather_rows(dG, dGk, ix.idx, mk)
                tfb.collider_gather_rows(X, Xk, ix.idx, mk)
            tfb.collider_linear_bwd_reduced(Xk[:mk], dGk[:mk], w, dx[:mk], dw, ws=ws)

        row["reduced_ms"] = t_ms(reduced)
        row["reduced_gemms_only_ms"] = t_ms(lambda: reduced(False))
        # the vendor GEMM (torch.matmul, hipBLASLt) on the same compacted rows: dX = dG' w and
        # dW = dG'^T X' with dG'^T made contiguous beforehand (untimed)
        if mk:
            dGkT = dGk[:mk].t().contiguous()
            row["reduced_rows_hipblaslt_ms"] = t_ms(lambda: (torch.matmul(dGk[:mk], w), torch.matmul(dGkT, Xk[:mk])))
            del dGkT
        else:
            row["reduced_rows_hipblaslt_ms"] = 0.0
        rows.append(row)
        log(f"[bench] sparse sweep r={r}%: " + ", ".join(
            f"{k} {v:.3f}" if isinstance(v, float) else f"{k} {v}" for k, v in row.items() if k != "r_pct"))
        del dGm, dGmT, dGf, dGfT, Xf, wf

    def crossover(key, dense_key):
        for row in rows:
            if row[key] < row[dense_key]:
                return row["r_pct"]
        return None

    out = {"metric": "Figure 4 sweep: linear backward (dX + dW) of the gate/up projection, ms, dense vs "
                     "torch.sparse vs dimension-reduced dense", "unit": "ms", "n_gpus": 1,
           "higher_is_better": False, "data": "synthetic", "dtype": "bf16",
           "config": {"workload": f"{cfg.name}-shaped gate/up projection backward, dG [{M}, {N}], X [{M}, {H}], "
                                  f"w [{N}, {H}]", "M": M, "N": N, "K": H},
           "rows": rows,
           "sparse_f32_beats_dense_from_r_pct": {"dense_f32": crossover("sparse_f32_ms", "dense_f32_ms"),
                                                 "dense_bf16": crossover("sparse_f32_ms", "dense_bf16_ms")},
           "reduced_beats_dense_bf16_from_r_pct": crossover("reduced_ms", "dense_bf16_ms"),
           "torch": torch.__version__}
    print(json.dumps(out), flush=True)
    return out


def index_sweep_bench(args):
    """Mask -> index over growing token counts (one sequence per 8192 tokens, 40% filtered by the
    generator's top-k): microseconds per build, from HIP events around a replayed HIP graph of 50
    builds (device time; checked against the eager build bit for bit), and around 50 eager
    back-to-back calls (which include the host's launch cost)."""
    import numpy as np
    import torch

    import synth
    import token_filtered_backward_amd as tfb

    rows = []
    for M in (8192, 65536, 262144, 1 << 20, 1 << 22):
        S = 8192
        B = M // S
        keep = torch.from_numpy(synth.make_keep(M, 40, args.seed)).cuda()
        ix = tfb.build_index(keep, B, S)
        n_keep = ix.M_kept
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(5):
            tfb.build_index(keep, B, S, out=ix, expect=n_keep)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(50):
            tfb.build_index(keep, B, S, out=ix, expect=n_keep)
        e1.record()
        e1.synchronize()
        us_eager = e0.elapsed_time(e1) * 1e3 / 50
        ref = [t.clone() for t in (ix.idx, ix.inv, ix.cu_seqlens, ix.count)]
        for t in (ix.idx, ix.inv, ix.cu_seqlens):
            t.fill_(-5)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(50):
                tfb.build_index(keep, B, S, out=ix, expect=n_keep)
        g.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(ref, (ix.idx, ix.inv, ix.cu_seqlens, ix.count))):
            raise RuntimeError(f"index build in a graph differs from the eager build (M={M})")
        reps = 5
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (50 * reps)
        rows.append({"M": M, "B": B, "S": S, "us_per_build": round(us, 2),
                     "GB_per_s": round(9.0 * M / (us * 1e-6) / 1e9, 1),
                     "us_per_build_eager": round(us_eager, 2)})
        log(f"[bench] index build M={M}: {us:.2f} us (graph), {us_eager:.2f} us (eager calls)")
    out = {"metric": "mask -> index build, us per call (graph of back-to-back builds, kept count announced)",
           "unit": "us",
           "n_gpus": 1, "higher_is_better": False, "data": "synthetic", "rows": rows,
           "config": {"workload": "keep mask of M tokens, sequences of 8192, 40% filtered"}}
    print(json.dumps(out), flush=True)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="tinyllama")
    ap.add_argument("--r", type=int, default=40, help="filtered percentage")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--seq", type=int, default=0,
                    help="sequence length S (long-context sweep); the batch becomes tokens / S")
    ap.add_argument("--tokens", type=int, default=0,
                    help="tokens per batch B*S with --seq (default: the config's own B*S)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfiltered", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch every kernel eagerly each step")
    ap.add_argument("--weight-layout", choices=("in_out", "out_in"), default=None,
                    help="projection weights stored [in, out] (y = x W, the pages' notation) or "
                         "[out, in] (torch nn.Linear); default: in_out for LLAMA-kind layers, "
                         "out_in for PHI-kind ones")
    ap.add_argument("--dmode", choices=("filtered", "full"), default="filtered",
                    help="softmax-backward row term of the filtered attention: sum over kept keys of "
                         "P~ dP (filtered, the default) or dO . O (full)")
    ap.add_argument("--loss-side", action="store_true",
                    help="time the loss-side steps (token selection, LM-head cross-entropy backward, "
                         "embedding gradient) at the config's token count and hidden size")
    ap.add_argument("--vocab", type=int, default=32000, help="vocabulary size for --loss-side")
    ap.add_argument("--index-sweep", action="store_true",
                    help="time the mask -> index build from 8192 to 4M tokens")
    ap.add_argument("--sparse-sweep", action="store_true",
                    help="Figure 4 on this GPU: torch.sparse vs dense GEMM vs the reduced GEMMs over a "
                         "filter-ratio sweep (gate/up projection of the config's layer)")
    ap.add_argument("--no-loss-side", action="store_true",
                    help="skip the loss-side summary the default layer run appends")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a plain copy of "
                         "known size, to calibrate HBM byte counters in a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}); the filtered layer backward "
              "is data-parallel and needs no second GPU to measure", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import token_filtered_backward_amd as tfb

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    cfg = synth.get_config(args.config)
    if args.loss_side:
        loss_side_bench(args, cfg)
        return
    if args.sparse_sweep:
        sparse_sweep_bench(args, cfg)
        return
    if args.index_sweep:
        index_sweep_bench(args)
        return
    if args.seq:
        tokens = args.tokens or cfg.M
        if tokens % args.seq:
            print(f"--tokens {tokens} is not a multiple of --seq {args.seq}", file=sys.stderr)
            sys.exit(2)
        cfg = cfg.with_(B=tokens // args.seq, S=args.seq)
    log(f"[bench] generating inputs for {cfg.name} (B={cfg.B} S={cfg.S} r={args.r}%) ...")
    t0 = time.perf_counter()
    inp = synth.make_layer_inputs(cfg, seed=args.seed, r_pct=args.r)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f}s")

    def up(v):
        if v.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(dev)

    W = {k: up(v) for k, v in inp["weights"].items()}
    Sv = {k: up(v) for k, v in inp["saved"].items()}
    if cfg.kind == "llama":
        weights = {k: W[k] for k in ("w_qkv", "w_o", "w_gateup", "w_down", "gamma1", "gamma2")}
        saved = {k: Sv[k] for k in ("x", "q", "k", "v", "o", "lse", "rstd1", "h", "rstd2", "gate", "up")}
    else:
        weights = dict(w_qkv=W["w_qkv"], w_o=W["w_o"], w_fc1=W["w_fc1"], w_fc2=W["w_fc2"],
                       ln_gamma=W["gamma"], ln_beta=W["beta"])
        saved = dict(x=Sv["x"], q=Sv["q"], k=Sv["k"], v=Sv["v"], o=Sv["o"], lse=Sv["lse"],
                     rstd1=Sv["rstd"], mean=Sv["mean"], f=Sv["f"])
    dy = up(inp["dy"])
    keep = torch.from_numpy(inp["keep"]).to(dev)
    B, S, M = cfg.B, cfg.S, cfg.M
    # weight storage layout (set up once, before timing; the weight gradients come out in it)
    wl = args.weight_layout or ("in_out" if cfg.kind == "llama" else "out_in")
    layout = tfb.WEIGHTS_IN_OUT if wl == "in_out" else tfb.WEIGHTS_OUT_IN
    if layout == tfb.WEIGHTS_IN_OUT:
        weights = tfb.to_in_out(weights)

    dmode = tfb.ATTN_D_FULL if args.dmode == "full" else tfb.ATTN_D_FILTERED
    lcfg = tfb.layer_cfg(cfg, dmode=dmode, weight_layout=layout)
    lb = tfb.LayerBackward(lcfg, B, S, dev)
    ix0 = tfb.build_index(keep, B, S)
    grads = tfb.make_grads(lcfg, M, ix0.M_kept, dev)
    lb.workspace(ix0.M_kept)

    L = cfg.n_layers
    if L > 1:
        # a stack of L layers of the same shape (the saved set and weights of one layer serve every
        # layer: the work does not depend on the values).  Gradients stay compact between layers;
        # the bottom layer scatters dx to the full token layout.
        gc = [tfb.make_grads(lcfg, M, ix0.M_kept, dev, dx_compact=True) for _ in range(2)]

    ixp = tfb.build_index(keep, B, S)  # index buffers reused every step
    # the filter keeps a fixed number of tokens (top-k over the batch), so the host knows the kept
    # count: the index is still built on the device every step, but the host does not wait for it
    n_kept = M - M * args.r // 100
    assert n_kept == ix0.M_kept, (n_kept, ix0.M_kept)

    def step_filtered(graph=False, wait_count=False):
        ix = tfb.build_index(keep, B, S, out=ixp, expect=None if wait_count else n_kept)
        if L == 1:
            lb(weights, saved, dy, ix, grads, graph=graph)
            return
        lb(weights, saved, dy, ix, gc[0], dx_compact=True)
        for layer in range(1, L - 1):
            lb(weights, saved, gc[(layer - 1) % 2]["dx"], ix, gc[layer % 2], dy_compact=True,
               dx_compact=True)
        lb(weights, saved, gc[(L - 2) % 2]["dx"], ix, grads, dy_compact=True)

    ucfg = tfb.layer_cfg(cfg, unfiltered=True, weight_layout=layout)
    ub = tfb.LayerBackward(ucfg, B, S, dev)
    uix = tfb.dense_index(B, S)
    ugrads = [tfb.make_grads(ucfg, M, M, dev) for _ in range(2 if L > 1 else 1)]

    def step_unfiltered(graph=False):
        if L == 1:
            ub(weights, saved, dy, uix, ugrads[0], graph=graph)
            return
        ub(weights, saved, dy, uix, ugrads[0])
        for layer in range(1, L):
            ub(weights, saved, ugrads[(layer - 1) % 2]["dx"], uix, ugrads[layer % 2])

    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)  # > 256 MB MALL
    calibration_copy(args.copy_calibration_mb)

    def timed(fn, K, W_):
        for _ in range(W_):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(K):
            fn()
        torch.cuda.synchronize()
        warm = (time.perf_counter() - t) * 1e3 / K
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cold = []
        for _ in range(K):
            flush.fill_(1)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            cold.append(e0.elapsed_time(e1))
        return warm, float(np.median(cold))

    # Each path is timed with eager launches and as a replayed HIP graph of the layer (one launch;
    # the index is rebuilt in place every step, and top-k keeps the kept count fixed); the filtered
    # path both with the kept count announced by the host and with the host waiting for the
    # device's count every step.  Each path is reported in its fastest mode (all modes are listed),
    # so the speedup never rests on a slower baseline.
    graph = L == 1 and not args.no_graph

    # Each mode is reported by its cold median (caches flushed before every step); the warm
    # back-to-back mean is kept beside it.
    def best_of(variants, label):
        res = {}
        for name, fn in variants.items():
            res[name] = timed(fn, args.steps, args.warmup)
            log(f"[bench] {label}, {name}: cold median {res[name][1]:.3f} ms/step (warm {res[name][0]:.3f})")
        mode = min(res, key=lambda m: res[m][1])
        return res[mode][0], res[mode][1], mode, {m: {"cold": round(v[1], 4), "warm": round(v[0], 4)}
                                                 for m, v in res.items()}

    log(f"[bench] timing: warmup {args.warmup}, steps {args.steps}")
    vf = {"eager": lambda: step_filtered(), "eager, host waits for count": lambda: step_filtered(False, True)}
    if graph:
        vf["graph"] = lambda: step_filtered(True)
        vf["graph, host waits for count"] = lambda: step_filtered(True, True)
        # the whole step (index build with the announced count, then the layer) as one HIP graph,
        # captured after an eager step; one replay must reproduce the eager step bit for bit
        step_filtered()
        torch.cuda.synchronize()
        ref = {k: v.clone() for k, v in grads.items()}
        g_step = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step):
            step_filtered()
        for v in grads.values():
            v.fill_(float("nan"))
        g_step.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            a, b = (grads[k].view(torch.int16), v.view(torch.int16)) if v.dtype == torch.bfloat16 else (grads[k], v)
            assert torch.equal(a, b), f"whole-step graph replay differs from the eager step in {k}"
        vf["graph of the whole step"] = g_step.replay
    ms_f, ms_f_cold, mode_f, modes_f = best_of(vf, "filtered")
    ixp.check()
    ms_u = ms_u_cold = mode_u = modes_u = None
    if not args.no_unfiltered:
        vu = {"eager": lambda: step_unfiltered()}
        if graph:
            vu["graph"] = lambda: step_unfiltered(True)
        ms_u, ms_u_cold, mode_u, modes_u = best_of(vu, "unfiltered")

    # per-kernel durations from HIP events recorded by the library on its launch stream
    n_prof = max(3, min(args.steps, 10))
    torch.cuda.synchronize()
    tfb.collider_profile_collect()
    tfb.collider_profile_enable(True)
    for _ in range(n_prof):
        step_filtered()
    torch.cuda.synchronize()
    prof = tfb.collider_profile_collect()
    tfb.collider_profile_enable(False)
    kernels = {k: round(v[0] / n_prof, 4) for k, v in sorted(prof.items(), key=lambda kv: -kv[1][0])}
    kernels_unf = None
    if not args.no_unfiltered:
        tfb.collider_profile_enable(True)
        for _ in range(n_prof):
            step_unfiltered()
        torch.cuda.synchronize()
        prof_u = tfb.collider_profile_collect()
        tfb.collider_profile_enable(False)
        kernels_unf = {k: round(v[0] / n_prof, 4)
                       for k, v in sorted(prof_u.items(), key=lambda kv: -kv[1][0])}
    gemm_names = [k for k in prof if k.startswith("gemm_") and k not in ("gemm_splitk_reduce", "gemm_sk_fixup")]
    gemm_ms = sum(prof[k][0] for k in gemm_names) / n_prof
    gemm_launches = sum(prof[k][1] for k in gemm_names) / n_prof

    # context for the gather / scatter rates: a plain device-to-device copy (torch) of the same
    # byte count on the same GPU, each copy after a 512 MB write that flushes L2 and the MALL, so
    # that it reads from HBM as the layer's gathers do (median of 10)
    def copy_rate_cold(nbytes):
        n = max(int(nbytes) // 2 // 16 * 16, 16)  # read + write: half the bytes each way
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b_ = torch.empty_like(a)
        b_.copy_(a)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(10):
            flush.fill_(1)
            c0.record()
            b_.copy_(a)
            c1.record()
            c1.synchronize()
            ts.append(c0.elapsed_time(c1))
        return 2.0 * n / (float(np.median(ts)) * 1e-3) / 1e9

    ix = tfb.build_index(keep, B, S)
    cu = ix.cu_seqlens.cpu().numpy()
    seq_counts = [int(cu[b + 1] - cu[b]) for b in range(B)]
    work = algorithmic_work(cfg, ix.M_kept, seq_counts)
    if L > 1:  # every layer's GEMMs and attention; dY gathered by the top layer only, dx
        # scattered by the bottom one
        work = dict(work, gemm_flops=L * work["gemm_flops"], attn_flops=L * work["attn_flops"],
                    attn_dt_flops=L * work["attn_dt_flops"],
                    gemm_bytes=L * work["gemm_bytes"], gemm_launches=L * work["gemm_launches"])
    gemm_tflops = work["gemm_flops"] / (gemm_ms * 1e-3) / 1e12
    attn_ms = sum(prof[k][0] for k in prof if k.startswith("attn_")) / n_prof
    # the P K product runs only under reading A with some token filtered (with every token kept the
    # layer takes D = dO . O, which then equals D~)
    dt_flops = work["attn_dt_flops"] if (args.dmode == "filtered" and ix.M_kept < cfg.M) else 0.0
    attn_tflops = (work["attn_flops"] + dt_flops) / (attn_ms * 1e-3) / 1e12 if attn_ms else None
    gather_ms = prof.get("gather_rows", (0.0, 1))[0] / n_prof
    gather_gbs = work["gather_bytes"] / (gather_ms * 1e-3) / 1e9 if gather_ms else None
    scatter_ms = prof.get("scatter_rows", (0.0, 1))[0] / n_prof
    scatter_gbs = work["scatter_bytes"] / (scatter_ms * 1e-3) / 1e9 if scatter_ms else None

    out = {
        "metric": METRIC,
        "value": round(ms_f_cold, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_f_cold, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"{cfg.name}-shaped layer backward, B{B}xS{S}, {args.r}% filtered" if L == 1
                                else f"{L} x {cfg.name}-shaped layers backward (compact chain), B{B}xS{S}, "
                                     f"{args.r}% filtered"),
                   "layers": L,
                   "B": B, "S": S, "hidden": cfg.H, "heads": f"{cfg.nq}/{cfg.nkv}x{cfg.d}",
                   "inter": cfg.I, "M": M, "M_kept": ix.M_kept, "parallelism": "single GPU",
                   "attn_row_term": args.dmode,
                   "weight_layout": "in_out" if layout == tfb.WEIGHTS_IN_OUT else "out_in"},
        "launch_mode": {"filtered": mode_f, "unfiltered": mode_u},
        "ms_by_launch_mode": {"filtered": modes_f, "unfiltered": modes_u},
        "timing": "value: median over the timed steps of one step each, after a 512 MB write that "
                  "flushes L2 and the MALL; *_warm: mean of the same steps run back to back",
        "ms_filtered_warm": round(ms_f, 4),
        "ms_unfiltered": None if ms_u_cold is None else round(ms_u_cold, 4),
        "ms_unfiltered_warm": None if ms_u is None else round(ms_u, 4),
        "speedup_vs_unfiltered": None if ms_u is None else round(ms_u_cold / ms_f_cold, 3),
        "speedup_vs_unfiltered_warm": None if ms_u is None else round(ms_u / ms_f, 3),
        "mfma_util_gemm": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
        "gemm_tflops": round(gemm_tflops, 1),
        "attn_tflops": None if attn_tflops is None else round(attn_tflops, 1),
        "gather_gbs": None if gather_gbs is None else round(gather_gbs, 1),
        "scatter_gbs": None if scatter_gbs is None else round(scatter_gbs, 1),
        "hbm_frac_gather": None if gather_gbs is None else round(gather_gbs / PEAK_HBM_GBS, 4),
        "hbm_frac_scatter": None if scatter_gbs is None else round(scatter_gbs / PEAK_HBM_GBS, 4),
        "copy_gbs_cold_same_bytes_as_gather": round(copy_rate_cold(work["gather_bytes"]), 1),
        "kernel_ms_per_step": kernels,
        "kernel_ms_per_step_unfiltered": kernels_unf,
        "roofline": {
            "kernel": f"gemm_bf16 (all {int(gemm_launches)} reduced-GEMM launches of one layer)",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(cfg, args.r),
            "traffic_source": (f"{TRAFFIC_FILE}: rocprofv3 FETCH_SIZE + WRITE_SIZE of this gemm.hip "
                               "(SHA-256 recorded there and checked here), calibrated on a plain copy; "
                               "not measured in this run") if measured_traffic(cfg, args.r) else None,
            "algorithmic_bytes_per_launch": work["gemm_bytes"] / work["gemm_launches"],
            "flops_per_launch": work["gemm_flops"] / max(gemm_launches, 1),
            "avg_launch_ms": round(gemm_ms / max(gemm_launches, 1), 5),
        },
    }
    if L == 1 and cfg.name == "tinyllama" and not args.seq and not args.no_loss_side:
        # the loss-side steps of the same batch (selection, LM-head cross-entropy backward,
        # embedding gradient), timed on their own; not part of `value`
        try:
            la = argparse.Namespace(seed=args.seed, r=args.r, vocab=args.vocab, steps=10, warmup=3,
                                    no_cpu_baseline=True)
            ls = loss_side_bench(la, cfg, emit=False)
            out["loss_side"] = {k: ls[k] for k in ("value", "unit", "ms_unfiltered", "speedup_vs_unfiltered",
                                                    "ce_grad_gbs", "embedding_gbs", "select_ms",
                                                    "ce_loss_ms", "ce_loss_gbs")}
            out["loss_side"]["workload"] = ls["config"]["workload"]
            out["loss_side"]["gemm_tflops"] = ls["roofline"]["achieved"]
        except Exception as e:  # reported, never fatal to the layer measurement
            out["loss_side"] = {"error": f"{type(e).__name__}: {e}"}
    if not args.no_cpu_baseline and (L > 1 or S > 4096):
        log("[bench] no CPU oracle timing for a layer stack or a sequence longer than 4096 (one "
            "float64 sequence of the layer at this size alone takes minutes)")
    elif not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(cfg, inp)
        log(f"[bench] cpu oracle: {out['cpu_baseline']['value']} ms per layer")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
