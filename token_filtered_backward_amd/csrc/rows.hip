// Row-wise kernels: gather / scatter of token rows, the transposed recompute of the weight-gradient
// operands, norm backward, column sums and rotary tables.  All are HBM-bound streaming kernels:
// rows are moved in 16-byte vectors.
//
// Dimension reduction (Collider paper, abstract): the rows of kept tokens are gathered into dense
// [M_kept, C] operands (or read through the index by their consumers); the scatter puts results
// back with filtered rows exactly zero.
#include "internal.h"

#include <algorithm>

namespace collider {

// ------------------------------------------------------------------------------------------
// gather: dst[c] = src[idx[c]], several tensors per launch (blockIdx.y = descriptor)
// ------------------------------------------------------------------------------------------
// Each workgroup moves up to kChunks 16-byte chunks (32 KB): the row indices of its rows are
// staged in LDS first, then every thread issues all of its loads before any store, so that many
// loads are in flight per thread.  One launch covers up to 8 tensors; their workgroups are laid
// out one tensor after another (blk0[i] = first workgroup of tensor i).  (64 KB per workgroup
// gave the 20 MB dY gather of the TinyLlama layer 308 workgroups, 1.2 per CU, so a second round
// of a few; 32 KB took it from 13.4 to 12.7 us and the zero fill from 11.0 to 8.8 us.)
static constexpr int kPerThread = 8;
static constexpr int kChunks = 256 * kPerThread;

struct GatherBatch {
  GatherDesc d[8];
  int blk0[9];
};

__device__ __forceinline__ int rows_per_block(int per_row) {
  return per_row >= kChunks ? 1 : kChunks / per_row;
}

__global__ __launch_bounds__(256) void gather_rows_kernel(GatherBatch batch,
                                                          const int32_t* __restrict__ idx,
                                                          int n_rows) {
  __shared__ int s_row[kChunks];
  // this workgroup's tensor (constant indices only: a runtime index into the by-value batch
  // would copy it to scratch memory)
  GatherDesc d = batch.d[0];
  int blk0 = 0;
#pragma unroll
  for (int k = 1; k < 8; ++k)
    if ((int)blockIdx.x >= batch.blk0[k]) {
      d = batch.d[k];
      blk0 = batch.blk0[k];
    }
  const int per_row = d.row_vec16;
  const int rpb = rows_per_block(per_row > 0 ? per_row : 1);  // same count as the host's
  const int r0 = ((int)blockIdx.x - blk0) * rpb;
  const int nr = min(rpb, n_rows - r0);
  if (nr <= 0) return;
  for (int i = threadIdx.x; i < nr; i += 256) s_row[i] = idx[r0 + i];
  __syncthreads();
  const uint4* __restrict__ src = (const uint4*)d.src;
  uint4* __restrict__ dst = (uint4*)d.dst;
  const int items = nr * per_row;
  // row / column of a chunk: shift and mask for power-of-two row widths (no integer division)
  const bool pow2 = per_row > 0 && (per_row & (per_row - 1)) == 0;
  const int sh = pow2 ? __ffs(per_row) - 1 : 0;
  for (int base = 0; base < items; base += kChunks) {
    uint4 v[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int i = base + threadIdx.x + 256 * u;
      v[u] = make_uint4(0, 0, 0, 0);
      if (i < items) {
        const int rr = pow2 ? i >> sh : i / per_row, c = pow2 ? i & (per_row - 1) : i - rr * per_row;
        v[u] = src[(int64_t)s_row[rr] * d.ld_src + c];
      }
    }
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int i = base + threadIdx.x + 256 * u;
      if (i < items) {
        const int rr = pow2 ? i >> sh : i / per_row, c = pow2 ? i & (per_row - 1) : i - rr * per_row;
        dst[(int64_t)(r0 + rr) * d.ld_dst + c] = v[u];
      }
    }
  }
  if (d.tail_bytes) {  // 4-byte tail words (row bytes not a multiple of 16)
    const int tw = d.tail_bytes >> 2;
    for (int i = threadIdx.x; i < nr * tw; i += 256) {
      const int rr = i / tw, w = i - rr * tw;
      const uint32_t* s32 = (const uint32_t*)(src + (int64_t)s_row[rr] * d.ld_src + per_row);
      uint32_t* d32 = (uint32_t*)(dst + (int64_t)(r0 + rr) * d.ld_dst + per_row);
      d32[w] = s32[w];
    }
  }
}

collider_status launch_gather_rows(const GatherDesc* d, int n_desc, const int32_t* idx, int n_rows,
                                   hipStream_t s) {
  if (n_rows <= 0 || n_desc <= 0) return COLLIDER_OK;
  for (int base = 0; base < n_desc; base += 8) {
    GatherBatch b{};
    const int n = n_desc - base < 8 ? n_desc - base : 8;
    int blocks = 0;
    for (int i = 0; i < 9; ++i) b.blk0[i] = 0x7fffffff;
    for (int i = 0; i < n; ++i) {
      b.d[i] = d[base + i];
      const int pr = d[base + i].row_vec16 > 0 ? d[base + i].row_vec16 : 1;
      const int rpb = pr >= kChunks ? 1 : kChunks / pr;
      b.blk0[i] = blocks;
      blocks += (n_rows + rpb - 1) / rpb;
    }
    b.blk0[n] = blocks;
    COLLIDER_LAUNCH("gather_rows", s,
                    hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks), dim3(256), 0, s, b, idx,
                                       n_rows));
  }
  return last_hip_status();
}

// Row-by-row copy of a [rows, cols] bf16 matrix between leading dimensions (16-byte chunks; cols,
// both leading dimensions and both addresses multiples of 8 elements / 16 bytes).
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint4* __restrict__ src, int64_t ld_src,
                                                        uint4* __restrict__ dst, int64_t ld_dst,
                                                        int rows, int per_row) {
  const int64_t n = (int64_t)rows * per_row;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / per_row, c = i - r * per_row;
    dst[r * ld_dst + c] = src[r * ld_src + c];
  }
}

collider_status launch_copy_rows(const uint16_t* src, int64_t ld_src, uint16_t* dst, int64_t ld_dst,
                                 int rows, int cols, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return COLLIDER_OK;
  if (cols % 8 || ld_src % 8 || ld_dst % 8 || !aligned16(src) || !aligned16(dst))
    return COLLIDER_ERR_UNSUPPORTED;
  const int per_row = cols / 8;
  const int64_t n = (int64_t)rows * per_row;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  COLLIDER_LAUNCH("copy_rows", s,
                  hipLaunchKernelGGL(copy_rows_kernel, dim3(blocks), dim3(256), 0, s, (const uint4*)src,
                                     ld_src / 8, (uint4*)dst, ld_dst / 8, rows, per_row));
  return last_hip_status();
}

// Generic byte-granular gather / scatter (2-byte units) for rows that are not 16-byte multiples.
__global__ void gather_u16_kernel(const uint16_t* __restrict__ src, int64_t ld_src,
                                  uint16_t* __restrict__ dst, int64_t ld_dst,
                                  const int32_t* __restrict__ idx, int n_rows, int row_u16) {
  const int c = blockIdx.x;
  if (c >= n_rows) return;
  const int64_t t = idx[c];
  for (int j = threadIdx.x; j < row_u16; j += blockDim.x) dst[c * ld_dst + j] = src[t * ld_src + j];
}

collider_status launch_gather_bytes(const void* src, int64_t ld_src_b, void* dst, int64_t ld_dst_b,
                                    const int32_t* idx, int n_rows, int row_bytes, hipStream_t s) {
  if (n_rows <= 0) return COLLIDER_OK;
  if (row_bytes % 16 == 0 && ld_src_b % 16 == 0 && ld_dst_b % 16 == 0 && aligned16(src) &&
      aligned16(dst)) {
    GatherDesc d{src, dst, ld_src_b / 16, ld_dst_b / 16, row_bytes / 16, 0};
    return launch_gather_rows(&d, 1, idx, n_rows, s);
  }
  COLLIDER_LAUNCH("gather_rows_u16", s,
                  hipLaunchKernelGGL(gather_u16_kernel, dim3(n_rows), dim3(128), 0, s,
                                     (const uint16_t*)src, ld_src_b / 2, (uint16_t*)dst,
                                     ld_dst_b / 2, idx, n_rows, row_bytes / 2));
  return last_hip_status();
}

// ------------------------------------------------------------------------------------------
// scatter: dst[t] = inv[t] >= 0 ? src[inv[t]] : 0 (or untouched), for every t < M
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scatter_rows_kernel(const uint4* __restrict__ src,
                                                           int64_t ld_src, uint4* __restrict__ dst,
                                                           int64_t ld_dst,
                                                           const int32_t* __restrict__ inv, int M,
                                                           int per_row, int zero_fill) {
  __shared__ int s_inv[kChunks];
  const int rpb = rows_per_block(per_row);
  const int r0 = blockIdx.x * rpb;
  const int nr = min(rpb, M - r0);
  if (nr <= 0) return;
  for (int i = threadIdx.x; i < nr; i += 256) s_inv[i] = inv[r0 + i];
  __syncthreads();
  const int items = nr * per_row;
  const bool pow2 = (per_row & (per_row - 1)) == 0;
  const int sh = pow2 ? __ffs(per_row) - 1 : 0;
  for (int base = 0; base < items; base += kChunks) {
    uint4 v[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int i = base + threadIdx.x + 256 * u;
      v[u] = make_uint4(0, 0, 0, 0);
      if (i < items) {
        const int rr = pow2 ? i >> sh : i / per_row, c = pow2 ? i & (per_row - 1) : i - rr * per_row;
        const int ci = s_inv[rr];
        if (ci >= 0 && zero_fill != 2) v[u] = src[(int64_t)ci * ld_src + c];
      }
    }
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int i = base + threadIdx.x + 256 * u;
      if (i < items) {
        const int rr = pow2 ? i >> sh : i / per_row, c = pow2 ? i & (per_row - 1) : i - rr * per_row;
        const bool kept = s_inv[rr] >= 0;
        if (zero_fill == 2 ? !kept : (zero_fill || kept)) dst[(int64_t)(r0 + rr) * ld_dst + c] = v[u];
      }
    }
  }
}

__global__ void scatter_u16_kernel(const uint16_t* __restrict__ src, int64_t ld_src,
                                   uint16_t* __restrict__ dst, int64_t ld_dst,
                                   const int32_t* __restrict__ inv, int M, int row_u16,
                                   int zero_fill) {
  const int t = blockIdx.x;
  if (t >= M) return;
  const int c = inv[t];
  if (c < 0 && !zero_fill) return;
  if (c >= 0 && zero_fill == 2) return;
  for (int j = threadIdx.x; j < row_u16; j += blockDim.x)
    dst[(int64_t)t * ld_dst + j] = c >= 0 ? src[(int64_t)c * ld_src + j] : (uint16_t)0;
}

collider_status launch_scatter_bytes(const void* src, int64_t ld_src_b, void* dst, int64_t ld_dst_b,
                                     const int32_t* inv, int M, int row_bytes, int zero_fill,
                                     hipStream_t s) {
  if (M <= 0) return COLLIDER_OK;
  if (row_bytes % 16 == 0 && ld_src_b % 16 == 0 && ld_dst_b % 16 == 0 && aligned16(src) &&
      aligned16(dst)) {
    const int pr = row_bytes / 16;
    const int rpb = pr >= kChunks ? 1 : kChunks / pr;
    dim3 grid((M + rpb - 1) / rpb);
    COLLIDER_LAUNCH("scatter_rows", s,
                    hipLaunchKernelGGL(scatter_rows_kernel, grid, dim3(256), 0, s,
                                       (const uint4*)src, ld_src_b / 16, (uint4*)dst,
                                       ld_dst_b / 16, inv, M, row_bytes / 16, zero_fill));
  } else {
    COLLIDER_LAUNCH("scatter_rows_u16", s,
                    hipLaunchKernelGGL(scatter_u16_kernel, dim3(M), dim3(128), 0, s,
                                       (const uint16_t*)src, ld_src_b / 2, (uint16_t*)dst,
                                       ld_dst_b / 2, inv, M, row_bytes / 2, zero_fill));
  }
  return last_hip_status();
}

// ------------------------------------------------------------------------------------------
// activations recomputed from the saved pre-activations
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float silu_f(float g) { return g * fast_sigmoid(g); }
__device__ __forceinline__ float gelu_f(float f) {
  const float c = 0.7978845608028654f, a = 0.044715f;
  const float u = c * (f + a * f * f * f);
  return 0.5f * f * (1.f + fast_tanh(u));
}

// ------------------------------------------------------------------------------------------
// transposed recompute: out[col * ldT + c] = bf16(op(row rowmap[c], col)) for c < rows, 0 for
// rows <= c < ldT.  The operands the weight-gradient GEMMs reduce over tokens (normalised inputs,
// activations, the attention output) come out token-contiguous, so the GEMM reads them with
// 16-byte LDS reads instead of transposing ones.  Ops: COL_COPY (a saved tensor as it is),
// COL_NORM (RMSNorm / LayerNorm with the saved statistics: (x - mean) rstd gamma + beta),
// COL_SWIGLU (silu(gate) up), COL_GELU (gelu_tanh(f)), each in fp32 and rounded to bf16 once.
// A workgroup covers 128 tokens x 128 columns and transposes them through LDS, so that both its
// loads and its stores move whole 256-byte runs: each thread first loads eight 16-byte row chunks
// (tokens 16 e + t, the 16 threads of a token reading the row's 16 consecutive chunks) and applies
// the op in fp32; the bf16 results go to an LDS tile; then each thread reads an 8-token x
// 8-column block of it, transposes it in registers and stores eight 16-byte runs of 8 consecutive
// tokens (the 16 threads of an output row writing its 16 consecutive chunks).  Chunk k of tile
// row t sits at position k ^ (t / 8 mod 16), which keeps both LDS access patterns free of bank
// conflicts.  The four transposes of a TinyLlama-shaped layer (M' = 4916) take 78 us this way;
// loading each thread's 8 x 8 block straight from memory took 91 us with 64-byte load runs and
// 256-byte store runs, 81 us with the two the other way round.
// ------------------------------------------------------------------------------------------
template <int OP>
__global__ __launch_bounds__(256) void cols_recompute_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, const uint16_t* __restrict__ x2,
    const float* __restrict__ mean, const float* __restrict__ rstd, const float* __restrict__ gamma,
    const float* __restrict__ beta, const int32_t* __restrict__ rowmap, int rows, int C,
    uint16_t* __restrict__ out, int64_t ldT) {
  __shared__ uint4 tile[128 * 16];  // [token][16-byte chunk], chunks swizzled by token / 8
  const int tok0 = blockIdx.x * 128, colb = blockIdx.y * 128;
  // load phase: tokens tok0 + 16 e + tr, columns col .. col + 7
  const int tr = threadIdx.x >> 4, ch = threadIdx.x & 15;
  const int col = colb + ch * 8;
  const bool col_ok = col < C;
  float g[8] = {}, bt[8] = {};
  if constexpr (OP == COL_NORM) {
    if (col_ok) {
      const float4 g0 = ((const float4*)(gamma + col))[0], g1 = ((const float4*)(gamma + col))[1];
      g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w; g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
      if (beta) {
        const float4 b0 = ((const float4*)(beta + col))[0], b1 = ((const float4*)(beta + col))[1];
        bt[0] = b0.x; bt[1] = b0.y; bt[2] = b0.z; bt[3] = b0.w; bt[4] = b1.x; bt[5] = b1.y; bt[6] = b1.z; bt[7] = b1.w;
      }
    }
  }
  int64_t r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = tok0 + 16 * e + tr;
    r[e] = (c < rows && col_ok) ? (rowmap ? rowmap[c] : c) : -1;
  }
  uint4 v[8], v2[8];
  float mu[8], rs[8];  // row statistics (COL_NORM), loaded with the rows rather than at their use
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = r[e] >= 0 ? *(const uint4*)(x + r[e] * ld_x + col) : make_uint4(0, 0, 0, 0);
    if constexpr (OP == COL_SWIGLU)
      v2[e] = r[e] >= 0 ? *(const uint4*)(x2 + r[e] * ld_x + col) : make_uint4(0, 0, 0, 0);
    if constexpr (OP == COL_NORM) {
      const int64_t rr = r[e] >= 0 ? r[e] : 0;
      mu[e] = mean ? mean[rr] : 0.f;
      rs[e] = rstd[rr];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (r[e] >= 0) {
      if constexpr (OP == COL_COPY) {
        u = v[e];
      } else {
        const uint32_t w[4] = {v[e].x, v[e].y, v[e].z, v[e].w};
        uint32_t o[4];
        if constexpr (OP == COL_NORM) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o[i] = pack2bf((bflo(w[i]) - mu[e]) * rs[e] * g[2 * i] + bt[2 * i],
                           (bfhi(w[i]) - mu[e]) * rs[e] * g[2 * i + 1] + bt[2 * i + 1]);
        } else if constexpr (OP == COL_SWIGLU) {
          const uint32_t w2[4] = {v2[e].x, v2[e].y, v2[e].z, v2[e].w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o[i] = pack2bf(silu_f(bflo(w[i])) * bflo(w2[i]), silu_f(bfhi(w[i])) * bfhi(w2[i]));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = pack2bf(gelu_f(bflo(w[i])), gelu_f(bfhi(w[i])));
        }
        u = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    const int t = 16 * e + tr;
    tile[t * 16 + (ch ^ ((t >> 3) & 15))] = u;
  }
  __syncthreads();
  // store phase: tokens c0 .. c0+7 of columns col0 .. col0+7
  const int tb = threadIdx.x & 15, cb = threadIdx.x >> 4;
  const int c0 = tok0 + tb * 8, col0 = colb + cb * 8;
  if (c0 >= ldT || col0 >= C) return;
  uint4 u[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) u[e] = tile[(tb * 8 + e) * 16 + (cb ^ tb)];
  // transpose: t[j] holds column col0 + j of tokens c0 .. c0+7 (two tokens per dword)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t d[4];
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const uint32_t lo = ((const uint32_t*)&u[2 * pr])[j >> 1];
      const uint32_t hi = ((const uint32_t*)&u[2 * pr + 1])[j >> 1];
      d[pr] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    if (col0 + j < C) *(uint4*)(out + (int64_t)(col0 + j) * ldT + c0) = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

collider_status launch_cols_recompute(int op, const uint16_t* x, int64_t ld_x, const uint16_t* x2,
                                      const float* mean, const float* rstd, const float* gamma,
                                      const float* beta, const int32_t* rowmap, int rows, int C,
                                      uint16_t* out, int64_t ldT, hipStream_t s) {
  if (ldT <= 0 || C <= 0) return COLLIDER_OK;
  if (C % 8 || ldT % 8 || ld_x % 8 || ldT < rows) return COLLIDER_ERR_UNSUPPORTED;
  dim3 grid((unsigned)((ldT + 127) / 128), (unsigned)((C + 127) / 128)), block(256);
#define CR_CASE(OPV)                                                                          \
  case OPV:                                                                                   \
    COLLIDER_LAUNCH("cols_recompute", s,                                                      \
                    hipLaunchKernelGGL(cols_recompute_kernel<OPV>, grid, block, 0, s, x, ld_x, x2, \
                                       mean, rstd, gamma, beta, rowmap, rows, C, out, ldT));  \
    break;
  switch (op) {
    CR_CASE(COL_COPY) CR_CASE(COL_NORM) CR_CASE(COL_SWIGLU) CR_CASE(COL_GELU)
    default:
      return COLLIDER_ERR_UNSUPPORTED;
  }
#undef CR_CASE
  return last_hip_status();
}

// ------------------------------------------------------------------------------------------
// norm backward + residual, in two kernels:
//   xhat = (x - mean) * rstd (mean = 0 for RMSNorm), g = dxn * gamma,
//   RMSNorm:   dx = rstd * (g - xhat * mean(g * xhat))
//   LayerNorm: dx = rstd * (g - mean(g) - xhat * mean(g * xhat))
//   out = dres + dx (bf16)                          norm_bwd_kernel, on the activation-gradient path
//   dgamma = sum_rows dxn * xhat, dbeta = sum_rows dxn    norm_grad_parts_kernel + colsum_parts,
//                                                    which nothing on that path waits for
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Read-only stand-ins for absent optional inputs of norm_bwd_kernel (no row limit: INT_MAX; no
// mean: 0), so that its loads need no branch.
static __device__ const int32_t kNoRowLimit = 0x7fffffff;
static __device__ const float kZeroMean = 0.f;

// One wavefront per row (4 rows per workgroup), the row in registers (NV 8-element vectors per
// lane, H <= 512 * NV); all of a row's loads are issued together and nothing is kept across rows,
// so that many wavefronts per SIMD hide the loads' latency.  The compacted rows (dxn, dres) go out
// first and the row of x, which needs the index lookup, after them; the kept-count limit is loaded
// beside them and only decides the store, so no load waits on another except x on its index.
template <int NV>
__global__ __launch_bounds__(256) void norm_bwd_kernel(
    const uint16_t* __restrict__ dxn, const uint16_t* __restrict__ dres,
    const uint16_t* __restrict__ x, const float* __restrict__ mean, const float* __restrict__ rstd,
    const float* __restrict__ gamma, const int32_t* __restrict__ rowmap, int rows, int H,
    uint16_t* __restrict__ dx, int dx_full, const int32_t* __restrict__ row_limit) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + wave;
  if (c >= rows) return;
  // rows at or past the device's kept count map to filtered positions (an index built with a
  // wrong announced count): their full-layout rows belong to the zero fill alone (checked at the
  // store; rowmap has an entry for every token, so the loads below stay in bounds)
  // (an ordinary vector load, not a scalar one, so that nothing waits for it before the stores;
  // vectors past the row's end are loaded from its last vector and left unused: no branch splits
  // the loads, whose waits the compiler would otherwise put at each branch)
  typedef __attribute__((address_space(1))) const int32_t gi32;  // global (not flat) loads
  const int lim = *(gi32*)(row_limit ? row_limit : &kNoRowLimit);
  const int nvec = H >> 3;
  const int map_v = *(gi32*)(rowmap ? rowmap + c : &kNoRowLimit);
  uint4 dv[NV], xv[NV], rv[NV];
  float4 ga[NV], gb[NV];  // gamma of this lane's columns, loaded once with the rows
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = min(lane + 64 * i, nvec - 1);
    dv[i] = ((const uint4*)(dxn + (int64_t)c * H))[v];
    rv[i] = ((const uint4*)(dres + (int64_t)c * H))[v];
    ga[i] = ((const float4*)gamma)[2 * v];
    gb[i] = ((const float4*)gamma)[2 * v + 1];
  }
  const int64_t r = rowmap ? map_v : c;
#pragma unroll
  for (int i = 0; i < NV; ++i) xv[i] = ((const uint4*)(x + r * H))[min(lane + 64 * i, nvec - 1)];
  const float mu = *(__attribute__((address_space(1))) const float*)(mean ? mean + r : &kZeroMean);
  const float rs = rstd[r];
  float s_g = 0.f, s_gx = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = lane + 64 * i;
    if (v < nvec) {
      const float4 g0 = ga[i], g1 = gb[i];
      const float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const uint32_t dw[4] = {dv[i].x, dv[i].y, dv[i].z, dv[i].w};
      const uint32_t xw[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float d = (j & 1) ? bfhi(dw[j >> 1]) : bflo(dw[j >> 1]);
        const float xh = (((j & 1) ? bfhi(xw[j >> 1]) : bflo(xw[j >> 1])) - mu) * rs;
        const float gv = d * gm[j];
        s_g += gv;
        s_gx += gv * xh;
      }
    }
  }
  s_g = wave_sum(s_g) / (float)H;
  s_gx = wave_sum(s_gx) / (float)H;
  if (!mean) s_g = 0.f;
  if (c >= lim) return;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = lane + 64 * i;
    if (v < nvec) {
      const float4 g0 = ga[i], g1 = gb[i];
      const float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const uint32_t dw[4] = {dv[i].x, dv[i].y, dv[i].z, dv[i].w};
      const uint32_t xw[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
      const uint32_t rw[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
      uint32_t ow[4];
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2) {
        const float g_a = bflo(dw[j2]) * gm[2 * j2], g_b = bfhi(dw[j2]) * gm[2 * j2 + 1];
        const float x_a = (bflo(xw[j2]) - mu) * rs, x_b = (bfhi(xw[j2]) - mu) * rs;
        const float a0 = bflo(rw[j2]) + rs * (g_a - s_g - x_a * s_gx);
        const float a1 = bfhi(rw[j2]) + rs * (g_b - s_g - x_b * s_gx);
        ow[j2] = pack2bf(a0, a1);
      }
      ((uint4*)(dx + (dx_full ? r : (int64_t)c) * H))[v] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
  }
}

// Rows longer than 4096 elements (hidden > 4096): the same computation, in the same per-lane order,
// in two sweeps over the row - the sums, then the output - the second re-reading the row that the
// first has just brought into L2, so that no row has to fit in registers.
__global__ __launch_bounds__(256) void norm_bwd_long_kernel(
    const uint16_t* __restrict__ dxn, const uint16_t* __restrict__ dres,
    const uint16_t* __restrict__ x, const float* __restrict__ mean, const float* __restrict__ rstd,
    const float* __restrict__ gamma, const int32_t* __restrict__ rowmap, int rows, int H,
    uint16_t* __restrict__ dx, int dx_full, const int32_t* __restrict__ row_limit) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + wave;
  if (c >= rows) return;
  const int nvec = H >> 3;
  const int64_t r = rowmap ? rowmap[c] : c;
  const float mu = mean ? mean[r] : 0.f;
  const float rs = rstd[r];
  const uint4* drow = (const uint4*)(dxn + (int64_t)c * H);
  const uint4* xrow = (const uint4*)(x + r * H);
  const uint4* rrow = (const uint4*)(dres + (int64_t)c * H);
  float s_g = 0.f, s_gx = 0.f;
  for (int v = lane; v < nvec; v += 64) {
    const float4 g0 = ((const float4*)gamma)[2 * v], g1 = ((const float4*)gamma)[2 * v + 1];
    const float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const uint4 dv = drow[v], xv = xrow[v];
    const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w}, xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float d = (j & 1) ? bfhi(dw[j >> 1]) : bflo(dw[j >> 1]);
      const float xh = (((j & 1) ? bfhi(xw[j >> 1]) : bflo(xw[j >> 1])) - mu) * rs;
      const float gv = d * gm[j];
      s_g += gv;
      s_gx += gv * xh;
    }
  }
  s_g = wave_sum(s_g) / (float)H;
  s_gx = wave_sum(s_gx) / (float)H;
  if (!mean) s_g = 0.f;
  // rows at or past the device's kept count: their full-layout rows belong to the zero fill alone
  if (row_limit && c >= *row_limit) return;
  for (int v = lane; v < nvec; v += 64) {
    const float4 g0 = ((const float4*)gamma)[2 * v], g1 = ((const float4*)gamma)[2 * v + 1];
    const float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const uint4 dv = drow[v], xv = xrow[v], rv = rrow[v];
    const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w}, xw[4] = {xv.x, xv.y, xv.z, xv.w};
    const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
    uint32_t ow[4];
#pragma unroll
    for (int j2 = 0; j2 < 4; ++j2) {
      const float g_a = bflo(dw[j2]) * gm[2 * j2], g_b = bfhi(dw[j2]) * gm[2 * j2 + 1];
      const float x_a = (bflo(xw[j2]) - mu) * rs, x_b = (bfhi(xw[j2]) - mu) * rs;
      const float a0 = bflo(rw[j2]) + rs * (g_a - s_g - x_a * s_gx);
      const float a1 = bfhi(rw[j2]) + rs * (g_b - s_g - x_b * s_gx);
      ow[j2] = pack2bf(a0, a1);
    }
    ((uint4*)(dx + (dx_full ? r : (int64_t)c) * H))[v] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
}

// Partial column sums of dxn * xhat (and of dxn, LN) over one chunk of rows: workgroup
// (column block cb, part p) covers 512 columns (8 per lane) and rows [p * rpp, (p + 1) * rpp), the
// 4 wavefronts taking every fourth row; their sums are combined in a fixed order, so the result
// is deterministic.  part_*[p, col].
template <bool LN>
__global__ __launch_bounds__(256) void norm_grad_parts_kernel(
    const uint16_t* __restrict__ dxn, const uint16_t* __restrict__ x, const float* __restrict__ mean,
    const float* __restrict__ rstd, const int32_t* __restrict__ rowmap, int rows, int H, int rpp,
    float* __restrict__ part_dgamma, float* __restrict__ part_dbeta) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = blockIdx.x * 512 + lane * 8;
  const bool on = col < H;
  const int r0 = blockIdx.y * rpp, r1 = min(rows, r0 + rpp);
  float ag[8], ab[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) ag[j] = ab[j] = 0.f;
  // rows c = r0 + wave, + 4, ... in batches of RB: the batch's index lookups, then all of its row
  // and statistics loads, go out before any is used (indices clamped into range instead of
  // branches, which would make the compiler wait at each one); the sums still take the rows in
  // order
  constexpr int RB = 4;
  typedef __attribute__((address_space(1))) const float gf32;
  typedef __attribute__((address_space(1))) const int32_t gi32;
  const int colc = on ? col : 0;
  for (int cb = r0 + wave; cb < r1; cb += 4 * RB) {
    int64_t r[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int c = min(cb + 4 * b, r1 - 1);
      const int m = *(gi32*)(rowmap ? rowmap + c : &kNoRowLimit);  // no branch around the load
      r[b] = rowmap ? m : c;
    }
    uint4 dv[RB], xv[RB];
    float mu[RB], rs[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int c = min(cb + 4 * b, r1 - 1);
      dv[b] = *(const uint4*)(dxn + (int64_t)c * H + colc);
      xv[b] = *(const uint4*)(x + r[b] * H + colc);
      mu[b] = *(gf32*)(mean ? mean + r[b] : &kZeroMean);
      rs[b] = rstd[r[b]];
    }
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if (!on || cb + 4 * b >= r1) continue;
      const uint32_t dw[4] = {dv[b].x, dv[b].y, dv[b].z, dv[b].w};
      const uint32_t xw[4] = {xv[b].x, xv[b].y, xv[b].z, xv[b].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float d = (j & 1) ? bfhi(dw[j >> 1]) : bflo(dw[j >> 1]);
        const float xh = (((j & 1) ? bfhi(xw[j >> 1]) : bflo(xw[j >> 1])) - mu[b]) * rs[b];
        ag[j] += d * xh;
        if constexpr (LN) ab[j] += d;
      }
    }
  }
  __shared__ float red[2][4][512];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    red[0][wave][lane * 8 + j] = ag[j];
    if constexpr (LN) red[1][wave][lane * 8 + j] = ab[j];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 512; e += 256) {
    const int cc = blockIdx.x * 512 + e;
    if (cc >= H) continue;
    part_dgamma[(int64_t)blockIdx.y * H + cc] = ((red[0][0][e] + red[0][1][e]) + red[0][2][e]) + red[0][3][e];
    if constexpr (LN)
      part_dbeta[(int64_t)blockIdx.y * H + cc] = ((red[1][0][e] + red[1][1][e]) + red[1][2][e]) + red[1][3][e];
  }
}

// partial-sum rows of a column sum over `rows` rows (bias gradient): enough to fill the CUs
int colsum_parts_count(int rows) { return rows <= 0 ? 1 : (rows < 1024 ? rows : 1024); }

// partial-sum rows of the gain gradients: enough workgroups (parts x 512-column blocks) to fill
// the CUs, at least 4 rows per part
int norm_grad_parts(int rows, int H) {
  const int blocks = (H + 511) / 512;
  int p = 1024 / blocks;
  p = std::min(p, std::max(1, rows / 4));
  return std::max(1, p);
}

collider_status launch_norm_bwd(const uint16_t* dxn, const uint16_t* dres, const uint16_t* x,
                                const float* mean, const float* rstd, const float* gamma,
                                const int32_t* rowmap, int rows, int H, uint16_t* dx, int dx_full,
                                hipStream_t s, const int32_t* row_limit) {
  if (rows <= 0) return COLLIDER_OK;
  const int nv = (H / 8 + 63) / 64;
  dim3 grid((rows + 3) / 4), block(256);
#define NB_CASE(N)                                                                              \
  case N:                                                                                       \
    COLLIDER_LAUNCH("norm_bwd", s,                                                              \
                    hipLaunchKernelGGL((norm_bwd_kernel<N>), grid, block, 0, s, dxn, dres, x,   \
                                       mean, rstd, gamma, rowmap, rows, H, dx, dx_full,         \
                                       row_limit));                                             \
    break;
  switch (nv) {
    NB_CASE(1) NB_CASE(2) NB_CASE(3) NB_CASE(4) NB_CASE(5) NB_CASE(6) NB_CASE(7) NB_CASE(8)
    default:  // rows longer than 4096
      COLLIDER_LAUNCH("norm_bwd", s,
                      hipLaunchKernelGGL(norm_bwd_long_kernel, grid, block, 0, s, dxn, dres, x, mean,
                                         rstd, gamma, rowmap, rows, H, dx, dx_full, row_limit));
  }
#undef NB_CASE
  return last_hip_status();
}

collider_status launch_norm_grad_parts(const uint16_t* dxn, const uint16_t* x, const float* mean,
                                       const float* rstd, const int32_t* rowmap, int rows, int H,
                                       float* part_dgamma, float* part_dbeta, int n_part,
                                       hipStream_t s) {
  if (rows <= 0) return COLLIDER_OK;
  const int rpp = (rows + n_part - 1) / n_part;
  dim3 grid((H + 511) / 512, n_part), block(256);
  if (part_dbeta)
    COLLIDER_LAUNCH("norm_grad_parts", s,
                    hipLaunchKernelGGL((norm_grad_parts_kernel<true>), grid, block, 0, s, dxn, x,
                                       mean, rstd, rowmap, rows, H, rpp, part_dgamma, part_dbeta));
  else
    COLLIDER_LAUNCH("norm_grad_parts", s,
                    hipLaunchKernelGGL((norm_grad_parts_kernel<false>), grid, block, 0, s, dxn, x,
                                       mean, rstd, rowmap, rows, H, rpp, part_dgamma, part_dbeta));
  return last_hip_status();
}

// out[col] (+)= sum_p parts[p, col], in a fixed order (deterministic): 16 columns per workgroup.
// Thread (l, q) adds parts l, l + 64, l + 128, ... of column quad q (independent loads, one memory
// latency), then the 64 lane sums of each column are combined by a fixed binary tree in LDS.
template <bool VEC>
__global__ __launch_bounds__(256) void colsum_parts_kernel(const float* __restrict__ parts,
                                                           int n_part, int H,
                                                           float* __restrict__ out,
                                                           int accumulate) {
  __shared__ float4 red[64][4];
  const int q = threadIdx.x & 3, l = threadIdx.x >> 2;
  const int col = blockIdx.x * 16 + q * 4;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
  if (col < H) {
    for (int p = l; p < n_part; p += 64) {
      const float* src = parts + (int64_t)p * H + col;
      float4 v;
      if constexpr (VEC) {
        v = *(const float4*)src;
      } else {
        v.x = src[0];
        v.y = col + 1 < H ? src[1] : 0.f;
        v.z = col + 2 < H ? src[2] : 0.f;
        v.w = col + 3 < H ? src[3] : 0.f;
      }
      sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
    }
  }
  red[l][q] = sum;
  __syncthreads();
#pragma unroll
  for (int w = 32; w > 0; w >>= 1) {
    if (l < w) {
      const float4 a = red[l][q], b = red[l + w][q];
      red[l][q] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    }
    __syncthreads();
  }
  if (l == 0 && col < H) {
    const float4 t = red[0][q];
    const float tv[4] = {t.x, t.y, t.z, t.w};
    for (int e = 0; e < 4 && col + e < H; ++e) out[col + e] = accumulate ? out[col + e] + tv[e] : tv[e];
  }
}

collider_status launch_colsum_parts(const float* parts, int n_part, int H, float* out,
                                    int accumulate, hipStream_t s) {
  if (H % 4 == 0)
    COLLIDER_LAUNCH("colsum_parts", s,
                    hipLaunchKernelGGL(colsum_parts_kernel<true>, dim3((H + 15) / 16), dim3(256), 0,
                                       s, parts, n_part, H, out, accumulate));
  else
    COLLIDER_LAUNCH("colsum_parts", s,
                    hipLaunchKernelGGL(colsum_parts_kernel<false>, dim3((H + 15) / 16), dim3(256), 0,
                                       s, parts, n_part, H, out, accumulate));
  return last_hip_status();
}

// column sums of a [rows, cols] matrix (bias gradient): per-block partials then colsum_parts
__global__ void colsum_partial_kernel(const void* __restrict__ x, int64_t ld, int rows, int cols,
                                      int is_bf16, int rows_per_part, float* __restrict__ parts) {
  const int col = blockIdx.y * blockDim.x + threadIdx.x;
  if (col >= cols) return;
  const int r0 = blockIdx.x * rows_per_part, r1 = min(rows, r0 + rows_per_part);
  float s = 0.f;
  for (int r = r0; r < r1; ++r)
    s += is_bf16 ? bf2f(((const uint16_t*)x)[(int64_t)r * ld + col])
                 : ((const float*)x)[(int64_t)r * ld + col];
  parts[(int64_t)blockIdx.x * cols + col] = s;
}

collider_status launch_colsum(const void* x, int64_t ld, int rows, int cols, bool bf16, float* out,
                              int accumulate, float* ws, hipStream_t s) {
  const int n_part = colsum_parts_count(rows);
  const int rpp = rows <= 0 ? 1 : (rows + n_part - 1) / n_part;
  COLLIDER_LAUNCH("colsum_partial", s,
                  hipLaunchKernelGGL(colsum_partial_kernel, dim3(n_part, (cols + 255) / 256),
                                     dim3(256), 0, s, x, ld, rows, cols, (int)bf16, rpp, ws));
  return launch_colsum_parts(ws, n_part, cols, out, accumulate, s);
}

__global__ void fill_f32_kernel(float* p, size_t n, float v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

collider_status launch_fill_f32(float* p, size_t n, float v, hipStream_t s) {
  if (n == 0) return COLLIDER_OK;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  COLLIDER_LAUNCH("fill_f32", s,
                  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p,
                                     n, v));
  return last_hip_status();
}

// cs[s][m] = (cos(s*theta_m), sin(s*theta_m)), theta_m = base^(-2m/rot); angles in double
__global__ void rope_table_kernel(float2* cs, int S, int half, double log_base, int rot) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= S * half) return;
  const int p = i / half, m = i - p * half;
  const double theta = exp(-2.0 * (double)m / (double)rot * log_base);
  double sn, cn;
  sincos((double)p * theta, &sn, &cn);
  cs[i] = make_float2((float)cn, (float)sn);
}

collider_status launch_rope_table(float* cs, int S, int rot, float base, hipStream_t s) {
  const int half = rot / 2;
  if (half == 0) return COLLIDER_OK;
  const int n = S * half;
  COLLIDER_LAUNCH("rope_table", s,
                  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s,
                                     (float2*)cs, S, half, log((double)base), rot));
  return last_hip_status();
}

}  // namespace collider
