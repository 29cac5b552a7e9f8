// extern "C" entry points of libcollider: argument validation on the host, then launches.
// Nothing here allocates device memory; nothing throws across the interface.
#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace collider {

collider_status layer_run(const collider_layer_cfg& c, const collider_layer_weights* w,
                          const collider_layer_saved* sv, const void* dy, int dy_compact,
                          const collider_index& ix, collider_layer_grads* gr, int dx_compact,
                          void* ws, size_t ws_bytes, hipStream_t s, size_t* need);

// ------------------------------------------------------------------------------------------
// per-kernel event timing (measurement only; off by default)
// ------------------------------------------------------------------------------------------
namespace {
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
// per host thread: one thread's timing switch does not change how another thread's launches run
thread_local bool t_prof_on = false;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t pool_get() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

bool profiling_on() { return t_prof_on; }

ProfScope::ProfScope(const char* n, hipStream_t s) : name(n), stream(s), slot(-1) {
  if (!t_prof_on) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipEvent_t a = pool_get(), b = pool_get();
  if (!a || !b) return;
  (void)hipEventRecord(a, s);
  g_prof_recs.push_back(ProfRec{n, a, b});
  slot = (int)g_prof_recs.size() - 1;
}

ProfScope::~ProfScope() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  (void)hipEventRecord(g_prof_recs[slot].b, stream);
}

}  // namespace collider

using namespace collider;

// ------------------------------------------------------------------------------------------
// validation helpers
// ------------------------------------------------------------------------------------------
static bool bad_ptr16(const void* p) { return p == nullptr || !aligned16(p); }

static collider_status check_index(const collider_index* ix) {
  if (!ix || !ix->idx || !ix->inv || !ix->cu_seqlens || !ix->count) return COLLIDER_ERR_NULL;
  if (ix->B < 1 || ix->S < 1 || (int64_t)ix->B * ix->S > (1 << 30)) return COLLIDER_ERR_SHAPE;
  if (ix->M_kept < 0 || ix->M_kept > ix->B * ix->S) return COLLIDER_ERR_SHAPE;
  return COLLIDER_OK;
}

static collider_status check_attn_cfg(const collider_attn_cfg* c) {
  if (!c) return COLLIDER_ERR_NULL;
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads) return COLLIDER_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return COLLIDER_ERR_UNSUPPORTED;
  if (c->rot_dims < 0 || c->rot_dims > c->head_dim || c->rot_dims % 2) return COLLIDER_ERR_UNSUPPORTED;
  if (c->rot_dims > 0 && !(c->rope_base > 1.f)) return COLLIDER_ERR_SHAPE;
  if (c->softmax_scale < 0.f) return COLLIDER_ERR_SHAPE;
  if (c->dmode != COLLIDER_ATTN_D_FILTERED && c->dmode != COLLIDER_ATTN_D_FULL) return COLLIDER_ERR_SHAPE;
  return COLLIDER_OK;
}

extern "C" {

const char* collider_status_string(collider_status s) {
  switch (s) {
    case COLLIDER_OK: return "ok";
    case COLLIDER_ERR_NULL: return "null pointer argument";
    case COLLIDER_ERR_SHAPE: return "invalid or inconsistent size";
    case COLLIDER_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case COLLIDER_ERR_UNSUPPORTED: return "unsupported configuration";
    case COLLIDER_ERR_WORKSPACE: return "workspace missing or too small";
    case COLLIDER_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

collider_status collider_build_index(const uint8_t* keep, int32_t B, int32_t S, int32_t* idx,
                                     int32_t* inv, int32_t* cu_seqlens, int32_t* count,
                                     hipStream_t stream) {
  if (!keep || !idx || !inv || !cu_seqlens || !count) return COLLIDER_ERR_NULL;
  if (B < 1 || S < 1 || (int64_t)B * S > (1 << 30)) return COLLIDER_ERR_SHAPE;
  return launch_build_index(keep, B, S, idx, inv, cu_seqlens, count, -1, nullptr, stream);
}

collider_status collider_build_index_expect(const uint8_t* keep, int32_t B, int32_t S,
                                            int32_t expected_count, int32_t* idx, int32_t* inv,
                                            int32_t* cu_seqlens, int32_t* count, int32_t* mismatch,
                                            hipStream_t stream) {
  if (!keep || !idx || !inv || !cu_seqlens || !count || !mismatch) return COLLIDER_ERR_NULL;
  if (B < 1 || S < 1 || (int64_t)B * S > (1 << 30)) return COLLIDER_ERR_SHAPE;
  if (expected_count < 0 || (int64_t)expected_count > (int64_t)B * S) return COLLIDER_ERR_SHAPE;
  return launch_build_index(keep, B, S, idx, inv, cu_seqlens, count, expected_count, mismatch,
                            stream);
}

collider_status collider_index_count_host(const int32_t* count_dev, int32_t* count_host,
                                          hipStream_t stream) {
  if (!count_dev || !count_host) return COLLIDER_ERR_NULL;
  if (hipMemcpyAsync(count_host, count_dev, sizeof(int32_t), hipMemcpyDeviceToHost, stream) !=
      hipSuccess)
    return COLLIDER_ERR_HIP;
  return hipStreamSynchronize(stream) == hipSuccess ? COLLIDER_OK : COLLIDER_ERR_HIP;
}

static int dt_size(collider_dtype dt) { return dt == COLLIDER_F32 ? 4 : (dt == COLLIDER_BF16 ? 2 : 0); }

collider_status collider_gather_rows(const void* src, int64_t ld_src, void* dst, int64_t ld_dst,
                                     const int32_t* idx, int32_t n_rows, int32_t row_elems,
                                     collider_dtype dt, hipStream_t stream) {
  const int es = dt_size(dt);
  if (!es) return COLLIDER_ERR_UNSUPPORTED;
  if (n_rows < 0 || row_elems < 0 || ld_src < row_elems || ld_dst < row_elems) return COLLIDER_ERR_SHAPE;
  if (n_rows == 0 || row_elems == 0) return COLLIDER_OK;
  if (!src || !dst || !idx) return COLLIDER_ERR_NULL;
  if (((uintptr_t)src | (uintptr_t)dst) & (es - 1)) return COLLIDER_ERR_ALIGN;
  return launch_gather_bytes(src, ld_src * es, dst, ld_dst * es, idx, n_rows, row_elems * es, stream);
}

collider_status collider_scatter_rows(const void* src, int64_t ld_src, void* dst, int64_t ld_dst,
                                      const int32_t* inv, int32_t M, int32_t row_elems,
                                      int32_t zero_fill_filtered, collider_dtype dt,
                                      hipStream_t stream) {
  const int es = dt_size(dt);
  if (!es) return COLLIDER_ERR_UNSUPPORTED;
  if (M < 0 || row_elems < 0 || ld_src < row_elems || ld_dst < row_elems) return COLLIDER_ERR_SHAPE;
  if (M == 0 || row_elems == 0) return COLLIDER_OK;
  if (!src || !dst || !inv) return COLLIDER_ERR_NULL;
  if (((uintptr_t)src | (uintptr_t)dst) & (es - 1)) return COLLIDER_ERR_ALIGN;
  // any non-zero flag zero-fills the filtered rows (the kernels' mode 2, zeros only, is internal)
  return launch_scatter_bytes(src, ld_src * es, dst, ld_dst * es, inv, M, row_elems * es,
                              zero_fill_filtered ? 1 : 0, stream);
}

static void linear_problems(collider_dtype dt, int32_t Mk, int32_t K, int32_t N, const void* x,
                            int64_t ld_x, const void* dy, int64_t ld_dy, const void* w, void* dx,
                            float* dw, int32_t accumulate, GemmProblem* pdx, GemmProblem* pdw) {
  *pdx = GemmProblem{};
  pdx->M = Mk; pdx->N = K; pdx->K = N;
  pdx->A = dy; pdx->lda = ld_dy; pdx->a_kmajor = true;
  pdx->B0 = w; pdx->ldb = K; pdx->b_kmajor = false;
  pdx->epi = dt == COLLIDER_F32 ? EPI_F32 : EPI_BF16;
  pdx->C = dx; pdx->ldc = K;
  *pdw = GemmProblem{};
  pdw->M = N; pdw->N = K; pdw->K = Mk;
  pdw->A = dy; pdw->lda = ld_dy; pdw->a_kmajor = false;
  pdw->B0 = x; pdw->ldb = ld_x; pdw->b_kmajor = false;
  pdw->epi = EPI_F32; pdw->C = dw; pdw->ldc = K; pdw->accumulate = accumulate;
  pdx->name = "linear_dx";
  pdw->name = "linear_dw";
}

// bf16: x' is copied transposed ([K, ldT], tokens contiguous, zero columns up to a multiple of 64)
// into the workspace, so that the weight-gradient GEMM reads it with 16-byte LDS reads along the
// reduction, as the layer's weight-gradient GEMMs read their transposed operands
static int linear_ldT(int32_t M_kept) { return (M_kept + 63) / 64 * 64; }

static void linear_use_xT(GemmProblem* pdw, const void* xT, int32_t M_kept) {
  pdw->B0 = xT;
  pdw->ldb = linear_ldT(M_kept);
  pdw->b_kmajor = true;
  pdw->b_kpad = true;
}

size_t collider_linear_workspace_bytes(collider_dtype dt, int32_t M_kept, int32_t K, int32_t N) {
  if (M_kept < 0 || K < 1 || N < 1) return 0;
  GemmProblem a, b;
  linear_problems(dt, M_kept, K, N, nullptr, K, nullptr, N, nullptr, nullptr, nullptr, 0, &a, &b);
  Carver cv(nullptr);
  cv.take<float>((size_t)colsum_parts_count(M_kept) * N);  // bias column-sum partials
  if (dt == COLLIDER_BF16) {
    if (M_kept > 0) {
      cv.take<uint16_t>((size_t)K * linear_ldT(M_kept));  // x' transposed
      linear_use_xT(&b, nullptr, M_kept);
    }
    cv.take<char>(std::max(gemm_bf16_workspace_bytes(a), gemm_bf16_workspace_bytes(b)));
  }
  return cv.bytes();
}

collider_status collider_linear_bwd_reduced(collider_dtype dt, int32_t M_kept, int32_t K, int32_t N,
                                            const void* x, int64_t ld_x, const void* dy,
                                            int64_t ld_dy, const void* w, void* dx, float* dw,
                                            float* db, int32_t accumulate, void* ws,
                                            size_t ws_bytes, hipStream_t stream) {
  if (dt != COLLIDER_F32 && dt != COLLIDER_BF16) return COLLIDER_ERR_UNSUPPORTED;
  if (M_kept < 0 || K < 1 || N < 1 || ld_x < K || ld_dy < N) return COLLIDER_ERR_SHAPE;
  if (!w || !dw || (M_kept > 0 && (!x || !dy))) return COLLIDER_ERR_NULL;
  if (dt == COLLIDER_BF16) {
    if (K % 8 || N % 8 || ld_x % 8 || ld_dy % 8) return COLLIDER_ERR_ALIGN;
    if (!aligned16(w) || (M_kept > 0 && (!aligned16(x) || !aligned16(dy))) || (dx && !aligned16(dx)))
      return COLLIDER_ERR_ALIGN;
  }
  const size_t need = collider_linear_workspace_bytes(dt, M_kept, K, N);
  if (need > 0 && (!ws || ws_bytes < need)) return COLLIDER_ERR_WORKSPACE;
  GemmProblem pdx, pdw;
  linear_problems(dt, M_kept, K, N, x, ld_x, dy, ld_dy, w, dx, dw, accumulate, &pdx, &pdw);
  Carver cv(ws);
  float* parts = cv.take<float>((size_t)colsum_parts_count(M_kept) * N);
  uint16_t* xT = (dt == COLLIDER_BF16 && M_kept > 0) ? cv.take<uint16_t>((size_t)K * linear_ldT(M_kept))
                                                     : nullptr;
  char* gws = cv.take<char>(0);
  const size_t gws_bytes = ws_bytes > (size_t)(gws - (char*)ws) ? ws_bytes - (gws - (char*)ws) : 0;
  collider_status st = COLLIDER_OK;
  if (dt == COLLIDER_F32) {
    if (dx) st = gemm_f32(pdx, stream);
    if (st == COLLIDER_OK) st = gemm_f32(pdw, stream);
  } else {
    if (xT) {
      st = launch_cols_recompute(COL_COPY, (const uint16_t*)x, ld_x, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, nullptr, M_kept, K, xT, linear_ldT(M_kept), stream);
      linear_use_xT(&pdw, xT, M_kept);
    }
    if (st == COLLIDER_OK && dx) st = gemm_bf16(pdx, gws, gws_bytes, stream);
    if (st == COLLIDER_OK) st = gemm_bf16(pdw, gws, gws_bytes, stream);
  }
  if (st == COLLIDER_OK && db) {
    if (M_kept > 0)
      st = launch_colsum(dy, ld_dy, M_kept, N, dt == COLLIDER_BF16, db, accumulate, parts, stream);
    else if (!accumulate)
      st = launch_fill_f32(db, N, 0.f, stream);
  }
  return st;
}

size_t collider_attn_workspace_bytes(const collider_attn_cfg* cfg, const collider_index* ix) {
  if (check_attn_cfg(cfg) != COLLIDER_OK || !ix || ix->B < 1 || ix->S < 1 || ix->M_kept < 0) return 0;
  return attn_workspace_bytes(*cfg, ix->B, ix->S, ix->M_kept);
}

collider_status collider_attn_bwd_filtered(const collider_attn_cfg* cfg, const collider_index* ix,
                                           const collider_attn_io* io, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
  collider_status st = check_attn_cfg(cfg);
  if (st != COLLIDER_OK) return st;
  if ((st = check_index(ix)) != COLLIDER_OK) return st;
  if (!io) return COLLIDER_ERR_NULL;
  if (ix->M_kept == 0) return COLLIDER_OK;
  const int d = cfg->head_dim, nqd = cfg->n_q_heads * d, nkvd = cfg->n_kv_heads * d;
  if (!io->q || !io->k || !io->v || !io->lse || !io->dout || !io->dq || !io->dk || !io->dv)
    return COLLIDER_ERR_NULL;
  if (cfg->dmode == COLLIDER_ATTN_D_FULL && !io->o) return COLLIDER_ERR_NULL;
  if (io->ld_q < nqd || io->ld_k < nkvd || io->ld_v < nkvd || io->ld_do < nqd || io->ld_dq < nqd ||
      io->ld_dk < nkvd || io->ld_dv < nkvd || io->ld_lse < cfg->n_q_heads ||
      (io->o && io->ld_o < nqd))
    return COLLIDER_ERR_SHAPE;
  const void* p16[] = {io->q, io->k, io->v, io->dout, io->dq, io->dk, io->dv};
  for (const void* p : p16)
    if (bad_ptr16(p)) return COLLIDER_ERR_ALIGN;
  if ((io->ld_q | io->ld_k | io->ld_v | io->ld_do | io->ld_dq | io->ld_dk | io->ld_dv) % 8)
    return COLLIDER_ERR_ALIGN;
  if (io->o && (bad_ptr16(io->o) || io->ld_o % 8)) return COLLIDER_ERR_ALIGN;
  const size_t need = attn_workspace_bytes(*cfg, ix->B, ix->S, ix->M_kept);
  if (!ws || ws_bytes < need) return COLLIDER_ERR_WORKSPACE;
  return attn_bwd(*cfg, *ix, *io, ws, ws_bytes, stream);
}

static collider_status check_layer(const collider_layer_cfg* c) {
  if (!c) return COLLIDER_ERR_NULL;
  if (c->kind != COLLIDER_LAYER_LLAMA && c->kind != COLLIDER_LAYER_PHI) return COLLIDER_ERR_UNSUPPORTED;
  if (c->hidden < 8 || c->inter < 8 || c->hidden % 8 || c->inter % 8) return COLLIDER_ERR_SHAPE;
  collider_attn_cfg ac{c->n_q_heads, c->n_kv_heads, c->head_dim, c->rot_dims, c->rope_base, 0.f, c->dmode};
  collider_status st = check_attn_cfg(&ac);
  if (st != COLLIDER_OK) return st;
  if (c->kind == COLLIDER_LAYER_PHI && ((c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim) % 64)
    return COLLIDER_ERR_UNSUPPORTED;
  if (c->weight_layout != COLLIDER_WEIGHTS_OUT_IN && c->weight_layout != COLLIDER_WEIGHTS_IN_OUT)
    return COLLIDER_ERR_UNSUPPORTED;
  return COLLIDER_OK;
}

size_t collider_layer_workspace_bytes(const collider_layer_cfg* cfg, int32_t B, int32_t S,
                                      int32_t M_kept) {
  if (check_layer(cfg) != COLLIDER_OK || B < 1 || S < 1 || M_kept < 0 || M_kept > B * S) return 0;
  collider_index ix{};
  ix.B = B;
  ix.S = S;
  ix.M_kept = M_kept;
  size_t need = 0;
  layer_run(*cfg, nullptr, nullptr, nullptr, 0, ix, nullptr, 0, nullptr, 0, nullptr, &need);
  // dy_compact / dx_compact only remove buffers, so this bound covers every variant
  return need;
}

collider_status collider_layer_bwd(const collider_layer_cfg* cfg, const collider_layer_weights* w,
                                   const collider_layer_saved* sv, const void* dy,
                                   int32_t dy_compact, const collider_index* ix,
                                   collider_layer_grads* g, int32_t dx_compact, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  collider_status st = check_layer(cfg);
  if (st != COLLIDER_OK) return st;
  if (cfg->unfiltered) {  // only B and S of the index are read
    if (!ix) return COLLIDER_ERR_NULL;
    if (ix->B < 1 || ix->S < 1 || (int64_t)ix->B * ix->S > (1 << 30)) return COLLIDER_ERR_SHAPE;
    if (dy_compact || dx_compact) return COLLIDER_ERR_UNSUPPORTED;
  } else if ((st = check_index(ix)) != COLLIDER_OK) {
    return st;
  }
  if (!w || !sv || !g || !dy) return COLLIDER_ERR_NULL;
  const bool llama = cfg->kind == COLLIDER_LAYER_LLAMA;
  const void* wp[] = {w->w_qkv, w->w_o, llama ? w->w_gateup : w->w_fc1, llama ? w->w_down : w->w_fc2};
  const void* sp16[] = {sv->x, sv->q, sv->k, sv->v, sv->o, llama ? sv->h : sv->f,
                        llama ? sv->gate : sv->f, llama ? sv->up : sv->f, dy, g->dx};
  for (const void* p : wp)
    if (!p) return COLLIDER_ERR_NULL;
  for (const void* p : sp16)
    if (!p) return COLLIDER_ERR_NULL;
  if (!sv->lse || !sv->rstd1 || (!llama && !sv->mean) || (llama && !sv->rstd2)) return COLLIDER_ERR_NULL;
  if (llama && (!w->gamma1 || !w->gamma2 || !g->dgamma1 || !g->dgamma2 || !g->dw_gateup || !g->dw_down))
    return COLLIDER_ERR_NULL;
  if (!llama && (!w->ln_gamma || !w->ln_beta || !g->dln_gamma || !g->dln_beta || !g->dw_fc1 || !g->dw_fc2))
    return COLLIDER_ERR_NULL;
  if (!g->dw_qkv || !g->dw_o) return COLLIDER_ERR_NULL;
  for (const void* p : wp)
    if (!aligned16(p)) return COLLIDER_ERR_ALIGN;
  for (const void* p : sp16)
    if (!aligned16(p)) return COLLIDER_ERR_ALIGN;
  const float* f16[] = {sv->lse, llama ? w->gamma1 : w->ln_gamma, llama ? w->gamma2 : w->ln_beta};
  for (const float* p : f16)
    if (!aligned16(p)) return COLLIDER_ERR_ALIGN;
  size_t need = 0;
  layer_run(*cfg, nullptr, nullptr, nullptr, dy_compact, *ix, nullptr, dx_compact, nullptr, 0,
            nullptr, &need);
  if (!ws || ws_bytes < need) return COLLIDER_ERR_WORKSPACE;
  return layer_run(*cfg, w, sv, dy, dy_compact, *ix, g, dx_compact, ws, ws_bytes, stream, nullptr);
}

collider_status collider_gemm_set_policy(int32_t policy) {
  if (policy < 0 || policy > 3) return COLLIDER_ERR_SHAPE;
  gemm_set_policy(policy);
  return COLLIDER_OK;
}

collider_status collider_gemm_describe_plan(int32_t M, int32_t N, int32_t K, int32_t layout,
                                           int32_t concurrent, int32_t* out) {
  if (!out) return COLLIDER_ERR_NULL;
  if (M <= 0 || N <= 0 || K < 0 || N % 8 || (layout != 0 && layout != 1)) return COLLIDER_ERR_SHAPE;
  GemmProblem g{};
  g.M = M;
  g.N = N;
  g.K = K;
  g.concurrent = concurrent != 0;
  if (layout == 0) {  // dX = dY w: A [M, K] K-contiguous, B [K, N] N-contiguous, bf16 out
    g.a_kmajor = true;
    g.lda = K;
    g.ldb = N;
    g.epi = EPI_BF16;
  } else {  // dW = dY^T X: both operands token-major [K, M] and [K, N], fp32 out
    g.lda = M;
    g.ldb = N;
    g.epi = EPI_F32;
  }
  int v[7];
  gemm_describe_plan(g, v);
  for (int i = 0; i < 7; ++i) out[i] = v[i];
  return COLLIDER_OK;
}

collider_status collider_profile_enable(int32_t on) {
  t_prof_on = on != 0;
  return COLLIDER_OK;
}

int32_t collider_side_streams_live(void) { return side_sets_live(); }

collider_status collider_release_resources(void) {
  (void)side_release_idle();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_recs.empty()) return COLLIDER_OK;  // events still awaiting collection stay
  for (hipEvent_t e : g_prof_pool) (void)hipEventDestroy(e);
  g_prof_pool.clear();
  return COLLIDER_OK;
}

int32_t collider_profile_collect(char* names, int32_t name_cap, double* total_ms, int32_t* launches,
                                 int32_t max_kernels) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  std::vector<std::string> order;
  std::map<std::string, std::pair<double, int>> agg;
  for (const ProfRec& r : g_prof_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return -1;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return -1;
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      order.push_back(r.name);
      agg[r.name] = {ms, 1};
    } else {
      it->second.first += ms;
      it->second.second += 1;
    }
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  int n = 0, off = 0;
  for (const std::string& nm : order) {
    if (n >= max_kernels) break;
    if (names) {
      if (off + (int)nm.size() + 1 > name_cap) break;
      std::memcpy(names + off, nm.c_str(), nm.size() + 1);
      off += (int)nm.size() + 1;
    }
    if (total_ms) total_ms[n] = agg[nm].first;
    if (launches) launches[n] = agg[nm].second;
    ++n;
  }
  return n;
}

// ------------------------------------------------------------------------------------------
// loss side: token selection, LM-head cross-entropy backward, embedding gradient
// ------------------------------------------------------------------------------------------
collider_status collider_ce_loss(const void* logits, int64_t ld_logits, const int32_t* labels,
                                 int32_t M, int32_t V, float* loss, hipStream_t stream) {
  if (!logits || !labels || !loss) return COLLIDER_ERR_NULL;
  if (M < 1 || M > (1 << 30) || V < 1 || ld_logits < V) return COLLIDER_ERR_SHAPE;
  if (V % 8 || ld_logits % 8 || !aligned16(logits)) return COLLIDER_ERR_ALIGN;
  return launch_ce_loss((const uint16_t*)logits, ld_logits, labels, M, V, loss, stream);
}

collider_status collider_select_keep(const float* score, int32_t M, int32_t n_keep, uint8_t* keep,
                                     hipStream_t stream) {
  if (!score || !keep) return COLLIDER_ERR_NULL;
  if (M < 1 || M > (1 << 30)) return COLLIDER_ERR_SHAPE;
  return launch_select_topk(score, M, n_keep, keep, stream);
}

size_t collider_select_workspace_bytes(int32_t M) {
  return M < 1 || M > (1 << 30) ? 0 : select_workspace_bytes(M);
}

collider_status collider_select_keep_ws(const float* score, int32_t M, int32_t n_keep, uint8_t* keep,
                                        void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!score || !keep) return COLLIDER_ERR_NULL;
  if (M < 1 || M > (1 << 30)) return COLLIDER_ERR_SHAPE;
  const size_t need = select_workspace_bytes(M);
  if (need > 0 && (!ws || ws_bytes < need)) return COLLIDER_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return COLLIDER_ERR_ALIGN;
  return launch_select_topk_multi(score, M, n_keep, keep, (uint32_t*)ws, stream);
}

}  // extern "C"

namespace {
struct LmHeadWs {
  uint16_t *hT, *dl, *dh_c;
  int ldT;
  char* gws;
  size_t gws_bytes, bytes;
};

// The LM head's two reduced GEMMs: dh' = dlogits' w_lm (A K-contiguous, B = w_lm [V, H]) and
// dW_lm = dlogits'^T h'.  h' reaches the second transposed, [H, ldT] with its tokens contiguous
// (ldT = M' rounded up to 64, zero columns past M'), so that its reduction runs along memory.
void lm_head_problems(int32_t Mk, int32_t H, int32_t V, const uint16_t* hT, int ldT,
                      const uint16_t* dl, const void* w_lm, void* dh_c, float* dw_lm,
                      int32_t accumulate, GemmProblem* pdh, GemmProblem* pdw) {
  linear_problems(COLLIDER_BF16, Mk, H, V, nullptr, H, dl, V, w_lm, dh_c, dw_lm, accumulate, pdh, pdw);
  pdw->B0 = hT; pdw->ldb = ldT; pdw->b_kmajor = true; pdw->b_kpad = true;
  pdh->name = "lm_head_dh";
  pdw->name = "lm_head_dw";
  // whole-tile plans: for dh' the cost model (calibrated on the layer's reduction lengths) picks
  // stream-K 256 x 256 tiles, but with the vocabulary-long reduction whole 160-row tiles measured
  // 0.55 ms against 0.76 ms (B 4 x S 2048, hidden 2048, vocab 32000, 40% filtered)
  pdh->concurrent = pdw->concurrent = true;
}

LmHeadWs carve_lm_head(int32_t Mk, int32_t H, int32_t V, void* base) {
  Carver cv(base);
  LmHeadWs w;
  w.ldT = (Mk + 63) / 64 * 64;
  w.hT = cv.take<uint16_t>((size_t)H * w.ldT);
  w.dl = cv.take<uint16_t>((size_t)Mk * V);
  w.dh_c = cv.take<uint16_t>((size_t)Mk * H);
  GemmProblem a, b;
  lm_head_problems(Mk, H, V, nullptr, w.ldT, nullptr, nullptr, nullptr, nullptr, 0, &a, &b);
  w.gws_bytes = std::max(gemm_bf16_workspace_bytes(a), gemm_bf16_workspace_bytes(b));
  w.gws = cv.take<char>(w.gws_bytes);
  w.bytes = cv.bytes();
  return w;
}
}  // namespace

extern "C" {

size_t collider_lm_head_workspace_bytes(int32_t M_kept, int32_t H, int32_t V) {
  if (M_kept < 0 || H < 1 || V < 1) return 0;
  return carve_lm_head(M_kept, H, V, nullptr).bytes;
}

collider_status collider_lm_head_bwd(const void* logits, int64_t ld_logits, const int32_t* labels,
                                     const void* h, int64_t ld_h, const void* w_lm,
                                     const collider_index* ix, int32_t H, int32_t V,
                                     float loss_scale, void* dh, int32_t dh_compact, float* dw_lm,
                                     int32_t accumulate, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  collider_status st = check_index(ix);
  if (st != COLLIDER_OK) return st;
  const int32_t Mk = ix->M_kept, M = ix->B * ix->S;
  // a compact dh has no rows when nothing is kept: NULL is accepted there
  const bool dh_none = dh_compact && Mk == 0;
  if (!logits || !labels || !h || !w_lm || !dw_lm || (!dh && !dh_none)) return COLLIDER_ERR_NULL;
  if (H < 1 || V < 1 || ld_logits < V || ld_h < H) return COLLIDER_ERR_SHAPE;
  if (H % 8 || V % 8 || ld_logits % 8 || ld_h % 8) return COLLIDER_ERR_ALIGN;
  if (!aligned16(logits) || !aligned16(h) || !aligned16(w_lm) || (dh && !aligned16(dh)) ||
      !aligned16(dw_lm))
    return COLLIDER_ERR_ALIGN;
  LmHeadWs w = carve_lm_head(Mk, H, V, ws);
  if (!ws || ws_bytes < w.bytes) return COLLIDER_ERR_WORKSPACE;
  uint16_t* dh_c = dh_compact ? (uint16_t*)dh : w.dh_c;
  if (Mk > 0) {
    // h's kept rows, transposed (the weight gradient's operand), read through the index
    st = launch_cols_recompute(COL_COPY, (const uint16_t*)h, ld_h, nullptr, nullptr, nullptr, nullptr,
                               nullptr, ix->idx, Mk, H, w.hT, w.ldT, stream);
    if (st != COLLIDER_OK) return st;
    st = launch_ce_grad((const uint16_t*)logits, ld_logits, labels, ix->idx, Mk, V, loss_scale, w.dl,
                        V, stream);
    if (st != COLLIDER_OK) return st;
  }
  GemmProblem pdh, pdw;
  lm_head_problems(Mk, H, V, w.hT, w.ldT, w.dl, w_lm, dh_c, dw_lm, accumulate, &pdh, &pdw);
  if (Mk > 0 && (st = gemm_bf16(pdh, w.gws, w.gws_bytes, stream)) != COLLIDER_OK) return st;
  if ((st = gemm_bf16(pdw, w.gws, w.gws_bytes, stream)) != COLLIDER_OK) return st;
  if (!dh_compact)  // full layout: kept rows from dh', filtered rows +0.0
    st = launch_scatter_bytes(dh_c, (int64_t)H * 2, dh, (int64_t)H * 2, ix->inv, M, H * 2, 1, stream);
  return st;
}

}  // extern "C"

namespace {
struct EmbWs {
  int32_t *cnt, *off, *cursor, *sorted, *hist;
  size_t bytes;
};
EmbWs carve_emb(int32_t Mk, int32_t V, void* base) {
  Carver cv(base);
  EmbWs w;
  w.cnt = cv.take<int32_t>((size_t)V);
  w.off = cv.take<int32_t>((size_t)V + 1);
  w.cursor = cv.take<int32_t>((size_t)V);
  w.sorted = cv.take<int32_t>((size_t)(Mk > 0 ? Mk : 1));
  const int chunks = embedding_hist_chunks(Mk, V);  // parallel placement when its histograms fit
  w.hist = chunks ? cv.take<int32_t>((size_t)chunks * V) : nullptr;
  w.bytes = cv.bytes();
  return w;
}
}  // namespace

extern "C" {

size_t collider_embedding_workspace_bytes(int32_t M_kept, int32_t V) {
  if (M_kept < 0 || V < 1) return 0;
  return carve_emb(M_kept, V, nullptr).bytes;
}

collider_status collider_embedding_bwd(const void* dx, int64_t ld_dx, int32_t dx_compact,
                                       const int32_t* ids, const collider_index* ix, int32_t H,
                                       int32_t V, float* dE, int32_t accumulate, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
  collider_status st = check_index(ix);
  if (st != COLLIDER_OK) return st;
  if (!ids || !dE || (ix->M_kept > 0 && !dx)) return COLLIDER_ERR_NULL;
  if (H < 1 || V < 1 || V > (1 << 30) || ld_dx < H) return COLLIDER_ERR_SHAPE;
  if (H % 8 || ld_dx % 8 || (dx && !aligned16(dx)) || !aligned16(dE)) return COLLIDER_ERR_ALIGN;
  EmbWs w = carve_emb(ix->M_kept, V, ws);
  if (!ws || ws_bytes < w.bytes) return COLLIDER_ERR_WORKSPACE;
  return launch_embedding_bwd((const uint16_t*)dx, ld_dx, dx_compact, ids, ix->idx, ix->M_kept, V, H,
                              dE, accumulate, w.cnt, w.off, w.cursor, w.sorted, stream, w.hist);
}

collider_status collider_embedding_bwd_noalloc(const void* dx, int64_t ld_dx, int32_t dx_compact,
                                               const int32_t* ids, const collider_index* ix,
                                               int32_t H, int32_t V, float* dE, int32_t accumulate,
                                               hipStream_t stream) {
  collider_status st = check_index(ix);
  if (st != COLLIDER_OK) return st;
  if (!ids || !dE || (ix->M_kept > 0 && !dx)) return COLLIDER_ERR_NULL;
  if (H < 1 || V < 1 || ld_dx < H) return COLLIDER_ERR_SHAPE;
  if (H % 8 || ld_dx % 8 || (dx && !aligned16(dx)) || !aligned16(dE)) return COLLIDER_ERR_ALIGN;
  if (V > kEmbScratchMaxV || ix->M_kept > kEmbScratchMaxRows) return COLLIDER_ERR_WORKSPACE;
  int32_t *cnt, *off, *cursor, *sorted;
  if ((st = embedding_scratch(&cnt, &off, &cursor, &sorted)) != COLLIDER_OK) return st;
  return launch_embedding_bwd((const uint16_t*)dx, ld_dx, dx_compact, ids, ix->idx, ix->M_kept, V, H,
                              dE, accumulate, cnt, off, cursor, sorted, stream);
}

}  // extern "C"
