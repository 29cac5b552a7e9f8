// Whole-layer filtered backward (Collider paper, abstract: the activations of filtered tokens are
// filtered across all layers; every linear backward becomes a dense GEMM over the kept tokens).
//
// The work of one layer, no host synchronisation (the weight-gradient side of it runs on a side
// stream, see layer_run):
//   gather   dY' (the saved tensors stay in the full layout; their consumers read them through
//            the index)
//   LLAMA                                         PHI (parallel block)
//   a'  = silu(gate')*up'   (recompute)           g' = gelu_tanh(f')       (recompute)
//   dA  = dY' w_down   -> SwiGLU bwd epilogue     dF = dY' w_fc2 -> GELU bwd epilogue
//   dw_down = dY'^T a'                            dw_fc2 = dY'^T g'
//   dXn2 = [dgate|dup] w_gateup                   dO = dY' w_o;  dw_o = dY'^T O'
//   dw_gateup = [dgate|dup]^T xn2'                attention bwd -> [dq|dk|dv]
//   dh = dY' + RMSNorm2 bwd(dXn2)                 dXn = [dq|dk|dv|dF] [w_qkv; w_fc1]
//   dO = dh w_o;  dw_o = dh^T O'                  dw_qkv, dw_fc1 = (...)^T xn'
//   attention bwd -> [dq|dk|dv]                   dx = dY' + LayerNorm bwd(dXn)
//   dXn1 = [dq|dk|dv] w_qkv; dw_qkv = (...)^T xn1'
//   dx = dh + RMSNorm1 bwd(dXn1)
//   the last norm backward writes dx's kept rows (compact, or in place in the full layout, whose
//   filtered rows get +0.0).
// Normalised inputs (xn1', xn2'), activations (a', g') and the attention output O' are recomputed
// or copied from saved tensors read through the index, and written transposed (tokens contiguous)
// for the weight-gradient GEMMs; the SwiGLU / GELU backward is fused into the epilogue of the GEMM
// producing dA.
#include <algorithm>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "internal.h"

namespace collider {

namespace {

// Side streams (default priority) with their fork / join events, leased per call from a pool per
// device: a call takes an idle set (or creates one when every set is leased, so the pool never
// outgrows the number of calls in flight at once on that device) and returns it when its launches
// are enqueued.  A set whose stream still belongs to an open graph capture (it joined the capture
// through the fork event) is not leased again until that capture has ended.  The pool holds no
// per-thread state; collider_release_resources destroys the idle sets.  Everything runs on the
// caller's stream with COLLIDER_SINGLE_STREAM=1 set, and while per-kernel timing is on (so that
// each kernel's events bracket it alone).
struct Side {
  hipStream_t s = nullptr;
  hipEvent_t ev[8] = {};
  int dev = -1;
};

constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
std::vector<Side*> g_side_idle[kMaxDevices];
int g_side_live = 0;

void side_destroy(Side* sd) {
  for (hipEvent_t e : sd->ev)
    if (e) (void)hipEventDestroy(e);
  if (sd->s) (void)hipStreamDestroy(sd->s);
  delete sd;
}

bool side_capturing(const Side* sd) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(sd->s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
}

collider_status side_acquire(Side** out) {
  static const bool single = getenv("COLLIDER_SINGLE_STREAM") != nullptr;
  *out = nullptr;
  if (single || profiling_on()) return COLLIDER_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return COLLIDER_ERR_HIP;
  {
    std::lock_guard<std::mutex> lk(g_side_mu);
    std::vector<Side*>& idle = g_side_idle[dev];
    for (size_t i = idle.size(); i-- > 0;) {
      if (side_capturing(idle[i])) continue;
      *out = idle[i];
      idle.erase(idle.begin() + (std::ptrdiff_t)i);
      return COLLIDER_OK;
    }
  }
  Side* sd = new Side;
  sd->dev = dev;
  bool ok = hipStreamCreateWithFlags(&sd->s, hipStreamNonBlocking) == hipSuccess;
  // The events only order the two streams (hipStreamWaitEvent); the host never queries or waits on
  // them, so they go without the system-scope fence that host inspection needs.  Eager layer calls
  // on MI355X: TinyLlama 1.109 -> 1.094 ms, Phi-1.5 1.169 -> 1.163 ms (the fence sat between the
  // producing kernel and the next one on the recording stream).
  for (hipEvent_t& e : sd->ev)
    ok = ok && hipEventCreateWithFlags(&e, hipEventDisableTiming | hipEventDisableSystemFence) ==
                   hipSuccess;
  if (!ok) {
    side_destroy(sd);
    return COLLIDER_ERR_HIP;
  }
  std::lock_guard<std::mutex> lk(g_side_mu);
  ++g_side_live;
  *out = sd;
  return COLLIDER_OK;
}

// Returns a leased set to its device's pool on scope exit (the events may be recorded again at
// once: every wait on them is already enqueued, and a wait takes the event's state at enqueue).
struct SideLease {
  Side* sd = nullptr;
  ~SideLease() {
    if (!sd) return;
    std::lock_guard<std::mutex> lk(g_side_mu);
    g_side_idle[sd->dev].push_back(sd);
  }
};

}  // namespace

int side_sets_live() {
  std::lock_guard<std::mutex> lk(g_side_mu);
  return g_side_live;
}

int side_release_idle() {
  std::vector<Side*> doomed;
  {
    std::lock_guard<std::mutex> lk(g_side_mu);
    for (std::vector<Side*>& idle : g_side_idle) {
      for (Side* sd : idle)
        if (!side_capturing(sd)) doomed.push_back(sd);
      std::vector<Side*> keep;
      for (Side* sd : idle)
        if (std::find(doomed.begin(), doomed.end(), sd) == doomed.end()) keep.push_back(sd);
      idle.swap(keep);
    }
    g_side_live -= (int)doomed.size();
  }
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (Side* sd : doomed) {
    (void)hipSetDevice(sd->dev);
    side_destroy(sd);
  }
  (void)hipSetDevice(cur);
  return (int)doomed.size();
}

namespace {

struct LayerBufs {

  uint16_t* dy_c;
  // token-contiguous (transposed, [C, ldT]) operands of the weight-gradient GEMMs: the
  // activation, the normalised input, the attention output
  uint16_t *actT, *xnT, *oT;
  uint16_t *dmid, *dqkv, *dxn, *dh, *do_c, *dx_c;
  float *part_g, *part_b;
  uint16_t* dxn1;
  uint16_t* w_stack;  // PHI, [in, out] weights: [W_qkv | W_fc1], [H, nqkv + I]
  void* gemm_ws;   // split-K partials of the GEMMs on the caller's stream
  void* gemm_ws2;  // ... and of the weight-gradient GEMMs on the side stream
  void* attn_ws;
  size_t gemm_ws_bytes, gemm_ws2_bytes, attn_ws_bytes;
};

}  // namespace

collider_status layer_run(const collider_layer_cfg& c, const collider_layer_weights* w,
                          const collider_layer_saved* sv, const void* dy, int dy_compact,
                          const collider_index& ix, collider_layer_grads* gr, int dx_compact,
                          void* ws, size_t ws_bytes, hipStream_t s, size_t* need) {
  const bool llama = c.kind == COLLIDER_LAYER_LLAMA;
  // dense: the unfiltered baseline, or an index that keeps every token (its partition is then the
  // identity, so the full layout is the compacted one and no gather or index lookup is needed)
  const bool unf = c.unfiltered != 0 || ix.M_kept == ix.B * ix.S;
  const int B = ix.B, S = ix.S, M = B * S, Mk = unf ? M : ix.M_kept;
  const int H = c.hidden, I = c.inter, d = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const int nqd = nq * d, nkvd = nkv * d, nqkv = nqd + 2 * nkvd;
  const int mid = llama ? 2 * I : nqkv + I;  // width of [dgate|dup] or [dq|dk|dv|dF]
  const int parts = norm_grad_parts(Mk, H);
  const bool dry = need != nullptr;

  Carver cv(dry ? nullptr : ws);
  LayerBufs b{};
  // the upstream gradient's kept rows are gathered (the first GEMM's operand); the saved tensors
  // attention reads (q, k, v, o, lse) stay in the full layout and are read through the index
  if (unf)
    b.dy_c = (uint16_t*)dy;
  else
    b.dy_c = dy_compact ? (uint16_t*)dy : cv.take<uint16_t>((size_t)Mk * H);
  // tokens of the transposed operands, padded with zero columns to whole 64-token k-tiles
  const int ldT = (Mk + 63) / 64 * 64;
  b.actT = cv.take<uint16_t>((size_t)I * ldT);
  b.xnT = cv.take<uint16_t>((size_t)H * ldT);
  b.oT = cv.take<uint16_t>((size_t)nqd * ldT);
  b.dmid = cv.take<uint16_t>((size_t)Mk * mid);
  // [dq|dk|dv]: its own buffer for LLAMA (attention must not overwrite [dgate|dup] while the
  // side stream's dw_gateup GEMM may still read it); for PHI the first columns of dmid
  b.dqkv = llama ? cv.take<uint16_t>((size_t)Mk * nqkv) : b.dmid;
  const int ldq = llama ? nqkv : mid;
  b.dxn = cv.take<uint16_t>((size_t)Mk * H);
  // the second norm backward's input gets its own buffer: the side stream may still be reading
  // the first one's (for the gain gradient) when the QKV activation-gradient GEMM writes it
  b.dxn1 = llama ? cv.take<uint16_t>((size_t)Mk * H) : b.dxn;
  b.dh = llama ? cv.take<uint16_t>((size_t)Mk * H) : nullptr;
  b.do_c = cv.take<uint16_t>((size_t)Mk * nqd);
  // the last norm backward writes dx itself: compact rows, the full layout when unfiltered, or the
  // kept rows of the full layout (their filtered rows zeroed on the side stream)
  b.dx_c = (uint16_t*)(gr ? gr->dx : nullptr);
  const int dx_full = (!dx_compact && !unf) ? 1 : 0;
  b.part_g = cv.take<float>((size_t)parts * H);
  b.part_b = cv.take<float>((size_t)parts * H);
  // PHI with [in, out] weights: W_qkv and W_fc1 stacked into one [H, nqkv + I] matrix
  b.w_stack = (!llama && c.weight_layout == COLLIDER_WEIGHTS_IN_OUT)
                  ? cv.take<uint16_t>((size_t)H * (nqkv + I)) : nullptr;

  // GEMM problems (pointers are only meaningful when not dry)
  const int32_t* idx = unf ? nullptr : ix.idx;  // row map of the saved tensors (null: identity)
  GemmProblem g_dA{}, g_dw2{}, g_dXmid{}, g_dwmid{}, g_dO{}, g_dwo{}, g_dXin{}, g_dwqkv{}, g_dwfc1{};
  // Weight layouts.  [out, in] (w, y = x w^T): the activation gradient dX = dY w reads w with
  // n = in contiguous (B(k, n) = w[k][n]), the weight gradient is dw = dY^T X [out, in].
  // [in, out] (W = w^T): dX = dY W^T reads each row of W contiguous along the reduction
  // (B(k, n) = W[n][k]), the weight gradient is dW = X^T dY [in, out] - the same GEMM with the
  // operands swapped.  `wout` is the weight's output width (its leading dimension when [out, in]
  // is w's row length `win`).
  const bool w_io = c.weight_layout == COLLIDER_WEIGHTS_IN_OUT;
  auto dx_gemm = [&](GemmProblem& p, int n, int k, const void* A, int64_t lda, const void* Bm,
                     int64_t ldb, int epi, void* C, int64_t ldc) {
    // n: in features, k: out features; ldb: the row length of w [out, in] (= n)
    p.M = Mk; p.N = n; p.K = k;
    p.A = A; p.lda = lda; p.a_kmajor = true;
    p.B0 = Bm; p.ldb = w_io ? k : ldb; p.b_kmajor = w_io;
    p.epi = epi; p.C = C; p.ldc = ldc;
  };
  auto dw_gemm = [&](GemmProblem& p, int m, int n, const void* G, int64_t ldg, const void* XT,
                     float* C) {
    // dw [m = out, n = in] = dY^T [m, M'] X [M', n], with the gradient dY token-major (row stride
    // ldg) and X given transposed, XT [n, ldT] (token-contiguous, zero past the kept tokens).
    // [in, out] weights: dW [in, out] = X^T dY, A = XT read along the reduction; [out, in]:
    // dw = dY^T X, B = XT read along the reduction.
    p.K = Mk;
    if (w_io) {
      p.M = n; p.N = m;
      p.A = XT; p.lda = ldT; p.a_kmajor = true; p.a_kpad = true;
      p.B0 = G; p.ldb = ldg; p.b_kmajor = false;
    } else {
      p.M = m; p.N = n;
      p.A = G; p.lda = ldg; p.a_kmajor = false;
      p.B0 = XT; p.ldb = ldT; p.b_kmajor = true; p.b_kpad = true;
    }
    p.epi = EPI_F32; p.C = C; p.ldc = p.N; p.accumulate = c.accumulate;
  };
  if (llama) {
    dx_gemm(g_dA, I, H, b.dy_c, H, w ? w->w_down : nullptr, I, EPI_SWIGLU, b.dmid, mid);
    g_dA.g = sv ? (const uint16_t*)sv->gate : nullptr;
    g_dA.up = sv ? (const uint16_t*)sv->up : nullptr;
    g_dA.ld_g = I;
    g_dA.rowmap = idx;
    g_dA.out2 = b.dmid ? b.dmid + I : nullptr;
    g_dA.ld_out2 = mid;
    dw_gemm(g_dw2, H, I, b.dy_c, H, b.actT, gr ? gr->dw_down : nullptr);
    dx_gemm(g_dXmid, H, 2 * I, b.dmid, mid, w ? w->w_gateup : nullptr, H, EPI_BF16, b.dxn, H);
    dw_gemm(g_dwmid, 2 * I, H, b.dmid, mid, b.xnT, gr ? gr->dw_gateup : nullptr);
    dx_gemm(g_dO, nqd, H, b.dh, H, w ? w->w_o : nullptr, nqd, EPI_BF16, b.do_c, nqd);
    dw_gemm(g_dwo, H, nqd, b.dh, H, b.oT, gr ? gr->dw_o : nullptr);
    dx_gemm(g_dXin, H, nqkv, b.dqkv, ldq, w ? w->w_qkv : nullptr, H, EPI_BF16, b.dxn1, H);
    dw_gemm(g_dwqkv, nqkv, H, b.dqkv, ldq, b.xnT, gr ? gr->dw_qkv : nullptr);
  } else {
    uint16_t* dF = b.dmid ? b.dmid + nqkv : nullptr;
    dx_gemm(g_dA, I, H, b.dy_c, H, w ? w->w_fc2 : nullptr, I, EPI_GELU, dF, mid);
    g_dA.g = sv ? (const uint16_t*)sv->f : nullptr;
    g_dA.ld_g = I;
    g_dA.rowmap = idx;
    dw_gemm(g_dw2, H, I, b.dy_c, H, b.actT, gr ? gr->dw_fc2 : nullptr);
    dx_gemm(g_dO, nqd, H, b.dy_c, H, w ? w->w_o : nullptr, nqd, EPI_BF16, b.do_c, nqd);
    dw_gemm(g_dwo, H, nqd, b.dy_c, H, b.oT, gr ? gr->dw_o : nullptr);
    dx_gemm(g_dXin, H, nqkv + I, b.dmid, mid, w ? w->w_qkv : nullptr, H, EPI_BF16, b.dxn, H);
    if (w_io) {
      // [in, out]: W_qkv [H, nqkv] and W_fc1 [H, I] have different row lengths, so they are
      // stacked into one [H, nqkv + I] matrix (copied on the side stream, well before this GEMM),
      // whose rows hold the whole reduction
      g_dXin.B0 = b.w_stack;
    } else {
      g_dXin.B1 = w ? w->w_fc1 : nullptr;
      g_dXin.kseg = nqkv;
    }
    dw_gemm(g_dwqkv, nqkv, H, b.dmid, mid, b.xnT, gr ? gr->dw_qkv : nullptr);
    dw_gemm(g_dwfc1, I, H, dF, mid, b.xnT, gr ? gr->dw_fc1 : nullptr);
  }
  g_dA.name = llama ? "gemm_dA_swiglu" : "gemm_dA_gelu";
  g_dw2.name = llama ? "gemm_dw_down" : "gemm_dw_fc2";
  g_dXmid.name = "gemm_dX_gateup";
  g_dwmid.name = "gemm_dw_gateup";
  g_dO.name = "gemm_dO";
  g_dwo.name = "gemm_dw_o";
  g_dXin.name = llama ? "gemm_dX_qkv" : "gemm_dX_qkv_fc1";
  g_dwqkv.name = "gemm_dw_qkv";
  g_dwfc1.name = "gemm_dw_fc1";
  // the two streams run side by side: every layer GEMM takes the plan for concurrent work (the
  // same plan in single-stream mode, so per-kernel timings measure the kernels the layer runs)
  GemmProblem* gl[] = {&g_dA, &g_dw2, &g_dXmid, &g_dwmid, &g_dO, &g_dwo, &g_dXin, &g_dwqkv, &g_dwfc1};
  for (GemmProblem* p : gl) p->concurrent = true;
  size_t gemm_need = 0, gemm_need2 = 0;
  for (const GemmProblem* p : gl) {
    if (p->M <= 0) continue;
    size_t& need_s = p->epi == EPI_F32 ? gemm_need2 : gemm_need;  // dW GEMMs: side stream
    need_s = std::max(need_s, gemm_bf16_workspace_bytes(*p));
  }
  b.gemm_ws = cv.take<char>(gemm_need);
  b.gemm_ws_bytes = gemm_need;
  b.gemm_ws2 = cv.take<char>(gemm_need2);
  b.gemm_ws2_bytes = gemm_need2;

  collider_attn_cfg ac{};
  ac.n_q_heads = nq;
  ac.n_kv_heads = nkv;
  ac.head_dim = d;
  ac.rot_dims = c.rot_dims;
  ac.rope_base = c.rope_base;
  ac.softmax_scale = 0.f;
  // with every token kept the two row terms are the same quantity: D~_i = sum_j P_ij dO_i . v_j =
  // dO_i . O_i, the forward's output over all (here all kept) keys; the second costs no key sweep
  ac.dmode = (unf || Mk == M) ? COLLIDER_ATTN_D_FULL : c.dmode;
  collider_index aix = ix;
  if (unf) {  // every token kept: the attention kernels take cs = b*S and position = row mod S
    aix.idx = nullptr;
    aix.inv = nullptr;
    aix.cu_seqlens = nullptr;
    aix.count = nullptr;
    aix.M_kept = M;
  }
  b.attn_ws_bytes = attn_workspace_bytes(ac, B, S, Mk);
  b.attn_ws = cv.take<char>(b.attn_ws_bytes);

  if (dry) {
    *need = cv.bytes();
    return COLLIDER_OK;
  }
  if (ws_bytes < cv.bytes()) return COLLIDER_ERR_WORKSPACE;

  collider_status st;
#define CHECK(x)                       \
  do {                                 \
    st = (x);                          \
    if (st != COLLIDER_OK) return st;  \
  } while (0)

  // Weight-gradient GEMMs, the operands only they read (normalised / activated / copied saved
  // tensors, written transposed) and the gain gradient of the inner norm run on a side stream,
  // forked from and joined back to the caller's stream with events: that work fills what the dX
  // chain leaves idle, and the critical path dA -> dX -> norm bwd -> dO -> attention -> dX -> norm
  // bwd stays on `s`.  The gain (and bias) gradient of the last norm follows its backward on `s`,
  // which would otherwise sit idle while the side stream finishes its last weight-gradient GEMMs:
  // queued behind those GEMMs it made the tail of the step (0.4-0.9% of the layer on MI355X).
  SideLease lease;
  CHECK(side_acquire(&lease.sd));
  Side* side = lease.sd;
  hipStream_t s1 = side ? side->s : s;
  auto handoff = [&](int e, hipStream_t from, hipStream_t to) -> collider_status {
    if (!side) return COLLIDER_OK;
    if (hipEventRecord(side->ev[e], from) != hipSuccess) return COLLIDER_ERR_HIP;
    return hipStreamWaitEvent(to, side->ev[e], 0) == hipSuccess ? COLLIDER_OK : COLLIDER_ERR_HIP;
  };
  // Fork.  With eager launches the side stream starts before the gather: its first kernels (zero
  // fill, rotary table, transposed recomputes) read only the index and the saved tensors, so they
  // run beside it, and the first side-stream kernel that reads dY' waits for it (event 0).  Under
  // stream capture the fork stays after the gather: replays of the graph built from the early fork
  // ran 8-10% slower (the graph's branches ran with less concurrency), while eager launches gain
  // about 3% from it (TinyLlama- and Qwen2.5-shaped layers, 40%, one MI355X).
  bool early_fork = false;
  if (side) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) == hipSuccess)
      early_fork = cap == hipStreamCaptureStatusNone;
    else
      (void)hipGetLastError();  // no answer (the legacy stream during a capture): the late fork
  }
  if (early_fork) CHECK(handoff(5, s, s1));
  if (Mk > 0 && !unf && !dy_compact) {  // 1. the upstream gradient's kept rows (dA GEMM operand)
    GatherDesc gd{dy, b.dy_c, H * 2 / 16, H * 2 / 16, H * 2 / 16, 0};
    CHECK(launch_gather_rows(&gd, 1, idx, Mk, s));
  }
  if (!early_fork) CHECK(handoff(5, s, s1));  // fork: dY' ready
  // With the early fork the first activation-gradient GEMM(s), which need only dY', are enqueued
  // right after the gather, ahead of the side stream's launches: the host's launches are then off
  // the critical path when it has just waited for the device's kept count (TinyLlama layer in that
  // mode 1.231 -> 1.172 ms, Phi-1.5 1.252 -> 1.228 on MI355X; unchanged with the count announced).
  // The side stream's first reader of dY' waits for event 0.
  if (early_fork) {
    if (hipEventRecord(side->ev[0], s) != hipSuccess) return COLLIDER_ERR_HIP;  // dY' ready
    CHECK(gemm_bf16(g_dA, b.gemm_ws, b.gemm_ws_bytes, s));
    if (!llama) {
      if (hipEventRecord(side->ev[2], s) != hipSuccess) return COLLIDER_ERR_HIP;  // dF ready
      CHECK(gemm_bf16(g_dO, b.gemm_ws, b.gemm_ws_bytes, s));
    }
  }
  if (dx_full)  // the filtered rows of dx: +0.0 (the kept rows come from the last norm backward)
    CHECK(launch_scatter_bytes(nullptr, 0, gr->dx, (int64_t)H * 2, ix.inv, M, H * 2, 2, s1));
  // the rotary table attention reads (S and the rotary configuration only), off the critical path;
  // attention waits on the event recorded after it
  CHECK(attn_rope_prepare(ac, aix, b.attn_ws, b.attn_ws_bytes, s1));
  if (b.w_stack) {  // the stacked [W_qkv | W_fc1] of a PHI layer with [in, out] weights
    CHECK(launch_copy_rows((const uint16_t*)w->w_qkv, nqkv, b.w_stack, nqkv + I, H, nqkv, s1));
    CHECK(launch_copy_rows((const uint16_t*)w->w_fc1, I, b.w_stack + nqkv, nqkv + I, H, I, s1));
  }
  // attention, and everything after it on `s`, waits on the event recorded here
  if (side && hipEventRecord(side->ev[6], s1) != hipSuccess) return COLLIDER_ERR_HIP;
  collider_attn_io io{};  // saved tensors in the full layout, rows idx[c] (all rows when unfiltered)
  io.q = sv ? sv->q : nullptr; io.ld_q = nqd;
  io.k = sv ? sv->k : nullptr; io.ld_k = nkvd;
  io.v = sv ? sv->v : nullptr; io.ld_v = nkvd;
  io.o = sv ? sv->o : nullptr; io.ld_o = nqd;
  io.lse = sv ? sv->lse : nullptr; io.ld_lse = nq;
  io.dout = b.do_c; io.ld_do = nqd;
  io.dq = b.dqkv; io.ld_dq = ldq;
  io.dk = b.dqkv + nqd; io.ld_dk = ldq;
  io.dv = b.dqkv + nqd + nkvd; io.ld_dv = ldq;
  if (llama) {
    CHECK(launch_cols_recompute(COL_SWIGLU, (const uint16_t*)sv->gate, I, (const uint16_t*)sv->up,
                                nullptr, nullptr, nullptr, nullptr, idx, Mk, I, b.actT, ldT, s1));
    CHECK(launch_cols_recompute(COL_NORM, (const uint16_t*)sv->h, H, nullptr, nullptr, sv->rstd2,
                                w->gamma2, nullptr, idx, Mk, H, b.xnT, ldT, s1));
    // dY' ready (event 0, recorded after the gather)
    if (early_fork && hipStreamWaitEvent(s1, side->ev[0], 0) != hipSuccess) return COLLIDER_ERR_HIP;
    CHECK(gemm_bf16(g_dw2, b.gemm_ws2, b.gemm_ws2_bytes, s1));
    if (!early_fork) CHECK(gemm_bf16(g_dA, b.gemm_ws, b.gemm_ws_bytes, s));
    CHECK(handoff(1, s, s1));  // [dgate|dup] ready
    CHECK(gemm_bf16(g_dwmid, b.gemm_ws2, b.gemm_ws2_bytes, s1));
    CHECK(gemm_bf16(g_dXmid, b.gemm_ws, b.gemm_ws_bytes, s));
    CHECK(launch_norm_bwd(b.dxn, b.dy_c, (const uint16_t*)sv->h, nullptr, sv->rstd2, w->gamma2, idx,
                          Mk, H, b.dh, 0, s));
    CHECK(launch_cols_recompute(COL_COPY, (const uint16_t*)sv->o, nqd, nullptr, nullptr, nullptr,
                                nullptr, nullptr, idx, Mk, nqd, b.oT, ldT, s1));
    CHECK(handoff(2, s, s1));  // dh ready (and dXn2, for the gain gradient)
    CHECK(gemm_bf16(g_dwo, b.gemm_ws2, b.gemm_ws2_bytes, s1));
    CHECK(launch_norm_grad_parts(b.dxn, (const uint16_t*)sv->h, nullptr, sv->rstd2, idx, Mk, H,
                                 b.part_g, nullptr, parts, s1));
    CHECK(launch_colsum_parts(b.part_g, Mk > 0 ? parts : 0, H, gr->dgamma2, c.accumulate, s1));
    CHECK(gemm_bf16(g_dO, b.gemm_ws, b.gemm_ws_bytes, s));
    if (side && hipStreamWaitEvent(s, side->ev[6], 0) != hipSuccess) return COLLIDER_ERR_HIP;
    CHECK(attn_bwd(ac, aix, io, b.attn_ws, b.attn_ws_bytes, s, true, idx));
    CHECK(handoff(3, s, s1));  // [dq|dk|dv] ready
    CHECK(launch_cols_recompute(COL_NORM, (const uint16_t*)sv->x, H, nullptr, nullptr, sv->rstd1,
                                w->gamma1, nullptr, idx, Mk, H, b.xnT, ldT, s1));
    CHECK(gemm_bf16(g_dwqkv, b.gemm_ws2, b.gemm_ws2_bytes, s1));
    CHECK(gemm_bf16(g_dXin, b.gemm_ws, b.gemm_ws_bytes, s));
    CHECK(launch_norm_bwd(b.dxn1, b.dh, (const uint16_t*)sv->x, nullptr, sv->rstd1, w->gamma1, idx, Mk,
                          H, b.dx_c, dx_full, s, dx_full ? ix.count : nullptr));
    // partial rows in part_b, which RMSNorm leaves unused: part_g may still be read by the side
    // stream's column sums of the second norm's gain gradient
    CHECK(launch_norm_grad_parts(b.dxn1, (const uint16_t*)sv->x, nullptr, sv->rstd1, idx, Mk, H,
                                 b.part_b, nullptr, parts, s));
    CHECK(launch_colsum_parts(b.part_b, Mk > 0 ? parts : 0, H, gr->dgamma1, c.accumulate, s));
  } else {
    CHECK(launch_cols_recompute(COL_GELU, (const uint16_t*)sv->f, I, nullptr, nullptr, nullptr,
                                nullptr, nullptr, idx, Mk, I, b.actT, ldT, s1));
    CHECK(launch_cols_recompute(COL_NORM, (const uint16_t*)sv->x, H, nullptr, sv->mean, sv->rstd1,
                                w->ln_gamma, w->ln_beta, idx, Mk, H, b.xnT, ldT, s1));
    CHECK(launch_cols_recompute(COL_COPY, (const uint16_t*)sv->o, nqd, nullptr, nullptr, nullptr,
                                nullptr, nullptr, idx, Mk, nqd, b.oT, ldT, s1));
    // dY' ready (event 0, recorded after the gather)
    if (early_fork && hipStreamWaitEvent(s1, side->ev[0], 0) != hipSuccess) return COLLIDER_ERR_HIP;
    CHECK(gemm_bf16(g_dw2, b.gemm_ws2, b.gemm_ws2_bytes, s1));
    CHECK(gemm_bf16(g_dwo, b.gemm_ws2, b.gemm_ws2_bytes, s1));
    if (!early_fork) {
      CHECK(gemm_bf16(g_dA, b.gemm_ws, b.gemm_ws_bytes, s));
      if (side && hipEventRecord(side->ev[2], s) != hipSuccess) return COLLIDER_ERR_HIP;  // dF ready
      CHECK(gemm_bf16(g_dO, b.gemm_ws, b.gemm_ws_bytes, s));
    }
    // dW_fc1 needs only dF (the dA GEMM's output) and xn': it runs while attention holds the
    // caller's stream and the side stream would otherwise wait, instead of behind dW_qkv at the
    // end of the step (Phi-1.5 layer on MI355X: 1.282 -> 1.263 ms with eager launches, 1.313 ->
    // 1.271 replayed as a graph)
    if (side && hipStreamWaitEvent(s1, side->ev[2], 0) != hipSuccess) return COLLIDER_ERR_HIP;
    CHECK(gemm_bf16(g_dwfc1, b.gemm_ws2, b.gemm_ws2_bytes, s1));
    if (side && hipStreamWaitEvent(s, side->ev[6], 0) != hipSuccess) return COLLIDER_ERR_HIP;
    CHECK(attn_bwd(ac, aix, io, b.attn_ws, b.attn_ws_bytes, s, true, idx));
    CHECK(handoff(1, s, s1));  // [dq|dk|dv|dF] ready
    CHECK(gemm_bf16(g_dwqkv, b.gemm_ws2, b.gemm_ws2_bytes, s1));
    CHECK(gemm_bf16(g_dXin, b.gemm_ws, b.gemm_ws_bytes, s));
    CHECK(launch_norm_bwd(b.dxn, b.dy_c, (const uint16_t*)sv->x, sv->mean, sv->rstd1, w->ln_gamma,
                          idx, Mk, H, b.dx_c, dx_full, s, dx_full ? ix.count : nullptr));
    CHECK(launch_norm_grad_parts(b.dxn, (const uint16_t*)sv->x, sv->mean, sv->rstd1, idx, Mk, H,
                                 b.part_g, b.part_b, parts, s));
    CHECK(launch_colsum_parts(b.part_g, Mk > 0 ? parts : 0, H, gr->dln_gamma, c.accumulate, s));
    CHECK(launch_colsum_parts(b.part_b, Mk > 0 ? parts : 0, H, gr->dln_beta, c.accumulate, s));
  }
  CHECK(handoff(4, s1, s));  // join: every weight gradient is complete on the caller's stream
#undef CHECK
  return COLLIDER_OK;
}

}  // namespace collider
