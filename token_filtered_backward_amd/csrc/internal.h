// Internal declarations of libcollider (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/collider.h"

namespace collider {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------------
// bf16 helpers (uint16 storage)
// ------------------------------------------------------------------------------------------
// Activation helpers on the hardware transcendental units: v_exp_f32 (2^x) and v_rcp_f32 (1/x,
// about 1 ulp).  Their error is far below the bf16 resolution of every value they feed.
__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}
// tanh(x) = 1 - 2 / (e^(2x) + 1): exact limits +-1 for large |x| (e^(2x) -> inf or 0)
__device__ __forceinline__ float fast_tanh(float x) {
  return 1.f - 2.f * __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(x * 2.8853900817779268f) + 1.f);
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 h = (__bf16)f;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}
__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ------------------------------------------------------------------------------------------
// launch bookkeeping: error check + optional per-kernel event timing
// ------------------------------------------------------------------------------------------
// true while per-kernel event timing is enabled (collider_profile_enable) on the calling thread
bool profiling_on();
// layer.hip: side-stream sets alive (leased or idle), and destruction of the idle ones
int side_sets_live();
int side_release_idle();

struct ProfScope {
  const char* name;
  hipStream_t stream;
  int slot;
  ProfScope(const char* n, hipStream_t s);
  ~ProfScope();
};

#define COLLIDER_LAUNCH(name, stream, ...)                  \
  do {                                                      \
    ::collider::ProfScope _ps(name, stream);                \
    __VA_ARGS__;                                            \
  } while (0)

inline collider_status last_hip_status() {
  return hipGetLastError() == hipSuccess ? COLLIDER_OK : COLLIDER_ERR_HIP;
}

inline bool aligned16(const void* p) { return (((uintptr_t)p) & 15u) == 0; }

// ------------------------------------------------------------------------------------------
// workspace carving (256-byte aligned sub-buffers)
// ------------------------------------------------------------------------------------------
struct Carver {
  char* base;
  size_t off;
  explicit Carver(void* b) : base((char*)b), off(0) {}
  template <class T>
  T* take(size_t n) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? (T*)(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
  size_t bytes() const { return (off + 255) & ~(size_t)255; }
};

// ------------------------------------------------------------------------------------------
// kernel launchers (each returns the launch status)
// ------------------------------------------------------------------------------------------

// mask -> index (index.hip)
// expect >= 0: the count the caller announced (inv / cu never reach past it; *mismatch, when
// given, is set to 1 if the mask keeps another number of tokens, else 0); expect < 0: none
collider_status launch_build_index(const uint8_t* keep, int B, int S, int32_t* idx, int32_t* inv,
                                   int32_t* cu, int32_t* count, int expect, int32_t* mismatch,
                                   hipStream_t s);

// loss.hip
collider_status launch_select_topk(const float* score, int M, int n_keep, uint8_t* keep,
                                   hipStream_t s);
// the same selection over many workgroups, for large token counts (M above 8192); ws holds
// select_workspace_bytes(M) bytes (0 when the single-workgroup kernel serves M)
size_t select_workspace_bytes(int M);
collider_status launch_select_topk_multi(const float* score, int M, int n_keep, uint8_t* keep,
                                         uint32_t* ws, hipStream_t s);
collider_status launch_ce_loss(const uint16_t* logits, int64_t ld, const int32_t* labels, int M, int V,
                               float* loss, hipStream_t s);
collider_status launch_ce_grad(const uint16_t* logits, int64_t ld, const int32_t* labels,
                               const int32_t* rowmap, int rows, int V, float scale, uint16_t* dl,
                               int64_t ldd, hipStream_t s);
// The allocation-free embedding gradient's scratch (a file-scope device array in loss.hip):
// device addresses, on the current device, of cnt / cursor [kEmbScratchMaxV], off
// [kEmbScratchMaxV + 1] and sorted [kEmbScratchMaxRows]
constexpr int kEmbScratchMaxV = 1 << 18;
constexpr int kEmbScratchMaxRows = 1 << 20;
collider_status embedding_scratch(int32_t** cnt, int32_t** off, int32_t** cursor, int32_t** sorted);
// cnt, cursor: [V]; off: [V + 1]; sorted: [rows]; hist (may be null): [embedding_hist_chunks(rows,
// V) * V], the per-chunk histograms of the parallel placement (used when that count is non-zero)
constexpr int64_t kEmbHistMax = 1 << 22;
int embedding_hist_chunks(int rows, int V);
collider_status launch_embedding_bwd(const uint16_t* dx, int64_t ld, int dx_compact,
                                     const int32_t* ids, const int32_t* idx, int rows, int V, int H,
                                     float* dE, int accumulate, int32_t* cnt, int32_t* off,
                                     int32_t* cursor, int32_t* sorted, hipStream_t s,
                                     int32_t* hist = nullptr);

// rows.hip
struct GatherDesc {
  const void* src;
  void* dst;
  int64_t ld_src, ld_dst;  // in 16-byte units
  int32_t row_vec16;       // 16-byte vectors per row
  int32_t tail_bytes;      // bytes after the last whole vector (0, 4, 8, 12 allowed)
};
collider_status launch_gather_rows(const GatherDesc* d, int n_desc, const int32_t* idx, int n_rows,
                                   hipStream_t s);
collider_status launch_gather_bytes(const void* src, int64_t ld_src_b, void* dst, int64_t ld_dst_b,
                                    const int32_t* idx, int n_rows, int row_bytes, hipStream_t s);
// dst[t] = src[inv[t]] for kept t; filtered t: zeros (zero_fill 1) or untouched (0); zero_fill 2:
// only the filtered rows, as zeros (src unused)
collider_status launch_scatter_bytes(const void* src, int64_t ld_src_b, void* dst, int64_t ld_dst_b,
                                     const int32_t* inv, int M, int row_bytes, int zero_fill,
                                     hipStream_t s);

// dst[r, 0:cols] = src[r, 0:cols] for r < rows, bf16 with leading dimensions ld_src / ld_dst
collider_status launch_copy_rows(const uint16_t* src, int64_t ld_src, uint16_t* dst, int64_t ld_dst,
                                 int rows, int cols, hipStream_t s);
// out[col * ldT + c] = bf16(op(row rowmap[c] of x (and x2), col)) for c < rows, 0 up to ldT (a
// multiple of 8 >= rows): the transposed (token-contiguous) operand of a weight-gradient GEMM.
// op: COL_COPY x; COL_NORM (x - mean) rstd gamma + beta (mean, beta may be null: RMSNorm);
// COL_SWIGLU silu(x) x2; COL_GELU gelu_tanh(x).  x, x2 row stride ld_x elements.
enum ColOp { COL_COPY = 0, COL_NORM = 1, COL_SWIGLU = 2, COL_GELU = 3 };
collider_status launch_cols_recompute(int op, const uint16_t* x, int64_t ld_x, const uint16_t* x2,
                                      const float* mean, const float* rstd, const float* gamma,
                                      const float* beta, const int32_t* rowmap, int rows, int C,
                                      uint16_t* out, int64_t ldT, hipStream_t s);
// dx = dres + norm_bwd(dxn; x[rowmap], stats): row c of dx, or row rowmap[c] when dx_full != 0
// (the full token layout); row_limit (device int, may be null): rows c >= *row_limit are skipped
collider_status launch_norm_bwd(const uint16_t* dxn, const uint16_t* dres, const uint16_t* x,
                                const float* mean, const float* rstd, const float* gamma,
                                const int32_t* rowmap, int rows, int H, uint16_t* dx, int dx_full,
                                hipStream_t s, const int32_t* row_limit = nullptr);
// partial column sums for dgamma = sum dxn * xhat (and dbeta = sum dxn when part_dbeta != null):
// n_part rows of H floats each, summed by launch_colsum_parts
collider_status launch_norm_grad_parts(const uint16_t* dxn, const uint16_t* x, const float* mean,
                                       const float* rstd, const int32_t* rowmap, int rows, int H,
                                       float* part_dgamma, float* part_dbeta, int n_part,
                                       hipStream_t s);
int norm_grad_parts(int rows, int H);
// partial-sum rows launch_colsum uses for `rows` rows
int colsum_parts_count(int rows);
collider_status launch_colsum_parts(const float* parts, int n_part, int H, float* out,
                                    int accumulate, hipStream_t s);
// column sums of a bf16 / f32 matrix (bias gradient)
collider_status launch_colsum(const void* x, int64_t ld, int rows, int cols, bool bf16, float* out,
                              int accumulate, float* ws, hipStream_t s);
collider_status launch_fill_f32(float* p, size_t n, float v, hipStream_t s);
// rotary tables cos/sin [S, rot/2] float32
collider_status launch_rope_table(float* cs, int S, int rot, float base, hipStream_t s);

// gemm.hip
enum EpiKind { EPI_BF16 = 0, EPI_F32 = 1, EPI_SWIGLU = 2, EPI_GELU = 3 };
struct GemmProblem {
  // C[M, N] = sum_k A(m, k) B(k, n)
  int M, N, K;
  const void* A;
  int64_t lda;
  bool a_kmajor;  // A(m,k) = A[m*lda + k] (true) or A[k*lda + m] (false)
  const void* B0;
  const void* B1;  // k >= kseg reads B1 at k - kseg (nullptr: single segment)
  int kseg;
  int64_t ldb;
  bool b_kmajor;  // B(k,n) = B[n*ldb + k] (true) or B[k*ldb + n] (false)
  // a K-major operand whose rows hold zeros from K up to the next multiple of 64 (within its
  // leading dimension): its ragged reduction length needs no masking (token-contiguous operands
  // of the weight-gradient GEMMs, written with that padding)
  bool a_kpad, b_kpad;
  // epilogue
  int epi;
  void* C;
  int64_t ldc;
  int accumulate;
  // SwiGLU / GELU epilogue: saved tensors read at row rowmap[m] (nullptr: row m)
  const uint16_t* g;   // gate (SwiGLU) or f (GELU)
  const uint16_t* up;  // SwiGLU only
  int64_t ld_g;
  const int32_t* rowmap;
  uint16_t* out2;      // SwiGLU: dup written at out2 (C gets dgate); GELU: unused
  int64_t ld_out2;
  const char* name;    // label for per-kernel timing (static string)
  // runs beside work on another stream: the default plan then takes whole tiles only (persistent
  // stream-K grids and K-split waves would hold every CU the other stream could use)
  bool concurrent;
};
// Work decomposition of the bf16 GEMMs: 0 = cost model, 1 = whole tiles and K-splits only,
// 2 = stream-K wherever the direct-to-LDS kernel applies, 3 = whole tiles only.
void gemm_set_policy(int policy);
// out[7] = tile rows, tile cols, K-splits, whole tiles, stream-K tiles, grid, direct-to-LDS kernel
void gemm_describe_plan(const GemmProblem& p, int* out);
size_t gemm_bf16_workspace_bytes(const GemmProblem& p);
collider_status gemm_bf16(const GemmProblem& p, void* ws, size_t ws_bytes, hipStream_t s);
collider_status gemm_f32(const GemmProblem& p, hipStream_t s);

// attn.hip
size_t attn_workspace_bytes(const collider_attn_cfg& c, int B, int S, int M_kept);
// rope_ready: the (cos, sin) table in the workspace was already written by attn_rope_prepare
// (on a stream this call's stream has waited for); otherwise attn_bwd writes it first.
// srcmap: when not null, row c of io.q, k, v, o and lse is row srcmap[c] (the full-layout saved
// tensors read through the index); dout and the outputs are compacted either way.
collider_status attn_bwd(const collider_attn_cfg& c, const collider_index& ix,
                         const collider_attn_io& io, void* ws, size_t ws_bytes, hipStream_t s,
                         bool rope_ready = false, const int32_t* srcmap = nullptr);
// Writes the RoPE (cos, sin) table of attn_bwd's workspace (it depends on S and the rotary
// configuration only), so that a caller can build it off the critical path.
collider_status attn_rope_prepare(const collider_attn_cfg& c, const collider_index& ix, void* ws,
                                  size_t ws_bytes, hipStream_t s);

}  // namespace collider
