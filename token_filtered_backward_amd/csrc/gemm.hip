// Dimension-reduced dense GEMMs (Collider paper, abstract: sparse GEMM becomes a dense GEMM over
// the kept tokens).  C[M, N] = sum_k A(m, k) B(k, n), bf16 operands, fp32 accumulation on CDNA4
// matrix cores (v_mfma_f32_32x32x16_bf16, 64-wide wavefronts).
//
// Operand layouts met by the linear backward (weights [out, in], y = x w^T):
//   dX = dY w    : A = dY (K-contiguous rows), B = w (N-contiguous: B(k, n) = w[k*ldb + n])
//   dW = dY^T X  : A = dY (M-contiguous: A(m, k) = dY[k*lda + m]), B = X (N-contiguous)
// The MFMA wants 8 consecutive k per lane for both operands, so every tile lands in LDS
// k-contiguous: K-major tiles are copied as 16-byte vectors, M/N-major tiles are loaded as 8x8
// blocks (eight 16-byte rows) and transposed in registers before one 16-byte LDS store per row.
// Global loads for tile k+1 are issued before the MFMAs of tile k (double-buffered LDS, one
// barrier per k-tile).  Long reductions with few output tiles (the weight gradients reduce over
// all kept tokens) are split over K; the partials are summed in a fixed order by a second kernel
// that also applies the epilogue, so results are deterministic.
#include <type_traits>

#include "internal.h"

namespace collider {

struct GemmParams {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B0;
  const uint16_t* B1;
  int kseg;
  int64_t ldb;
  int M, N, K;
  int k_split;  // reduction length handled by one split (multiple of the k-tile)
  int tiles_m, tiles_n;
  // epilogue
  void* C;
  int64_t ldc;
  int accumulate;
  float* partial;  // [splits][M][N] when split over K
  const uint16_t* g;
  const uint16_t* up;
  int64_t ld_g;
  const int32_t* rowmap;
  uint16_t* out2;
  int64_t ld_out2;
};

// ------------------------------------------------------------------------------------------
// epilogue: one output element
// ------------------------------------------------------------------------------------------
template <int EPI>
__device__ __forceinline__ void epi_store(const GemmParams& p, int m, int n, float v) {
  if constexpr (EPI == EPI_BF16) {
    ((uint16_t*)p.C)[(int64_t)m * p.ldc + n] = f2bf(v);
  } else if constexpr (EPI == EPI_F32) {
    float* c = (float*)p.C + (int64_t)m * p.ldc + n;
    *c = p.accumulate ? *c + v : v;
  } else if constexpr (EPI == EPI_SWIGLU) {
    // a = silu(gate) * up;  dgate = dA * up * s * (1 + gate * (1 - s)),  dup = dA * silu(gate)
    const int64_t r = p.rowmap ? p.rowmap[m] : m;
    const float g = bf2f(p.g[r * p.ld_g + n]);
    const float u = bf2f(p.up[r * p.ld_g + n]);
    const float s = 1.f / (1.f + __expf(-g));
    ((uint16_t*)p.C)[(int64_t)m * p.ldc + n] = f2bf(v * u * s * (1.f + g * (1.f - s)));
    p.out2[(int64_t)m * p.ld_out2 + n] = f2bf(v * g * s);
  } else {  // EPI_GELU: dF = dA * d/df gelu_tanh(f)
    const int64_t r = p.rowmap ? p.rowmap[m] : m;
    const float f = bf2f(p.g[r * p.ld_g + n]);
    const float c = 0.7978845608028654f, a = 0.044715f;
    const float t = tanhf(c * (f + a * f * f * f));
    const float d = 0.5f * (1.f + t) + 0.5f * f * (1.f - t * t) * c * (1.f + 3.f * a * f * f);
    ((uint16_t*)p.C)[(int64_t)m * p.ldc + n] = f2bf(v * d);
  }
}

// ------------------------------------------------------------------------------------------
// tile loaders (global -> registers -> LDS, k-contiguous LDS rows of BK + 8 elements)
// ------------------------------------------------------------------------------------------
template <int R, int BK, int NT>
struct KMajorTile {  // X(r, k) = X[r*ld + k]
  static constexpr int CPR = BK / 8;
  static constexpr int N = (R * CPR + NT - 1) / NT;
  uint4 v[N];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ X, int64_t ld, int r0, int rlim,
                                       int k0, int klim) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + NT * i;
      const int r = c / CPR, kc = c % CPR;
      const int row = r0 + r, k = k0 + kc * 8;
      if (c < R * CPR && row < rlim && k < klim)
        v[i] = *(const uint4*)(X + (int64_t)row * ld + k);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint16_t* S) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + NT * i;
      if (c < R * CPR) {
        const int r = c / CPR, kc = c % CPR;
        *(uint4*)(S + r * (BK + 8) + kc * 8) = v[i];
      }
    }
  }
};

template <int R, int BK, int NT>
struct MNMajorTile {  // X(r, k) = X[k*ld + r]; 8x8 blocks transposed in registers
  static constexpr int RB = R / 8, KB = BK / 8;
  static constexpr int NBLK = RB * KB;
  static constexpr int N = (NBLK + NT - 1) / NT;
  uint4 v[N][8];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ X, int64_t ld, int r0, int rlim,
                                       int k0, int klim) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int b = threadIdx.x + NT * i;
      const int rb = b % RB, kb = b / RB;
      const int row = r0 + rb * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = k0 + kb * 8 + e;
        if (b < NBLK && row < rlim && k < klim)
          v[i][e] = *(const uint4*)(X + (int64_t)k * ld + row);
        else
          v[i][e] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* S) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int b = threadIdx.x + NT * i;
      if (b < NBLK) {
        const int rb = b % RB, kb = b / RB;
        // v[i][e] holds k = kb*8+e for rows rb*8 .. rb*8+7 (two rows per dword)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int w = j >> 1;
          uint32_t d[4];
#pragma unroll
          for (int pr = 0; pr < 4; ++pr) {
            const uint32_t lo = ((const uint32_t*)&v[i][2 * pr])[w];
            const uint32_t hi = ((const uint32_t*)&v[i][2 * pr + 1])[w];
            d[pr] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
          *(uint4*)(S + (rb * 8 + j) * (BK + 8) + kb * 8) = make_uint4(d[0], d[1], d[2], d[3]);
        }
      }
    }
  }
};

template <int R, int BK, int NT, bool KMAJ>
using TileT = typename std::conditional<KMAJ, KMajorTile<R, BK, NT>, MNMajorTile<R, BK, NT>>::type;

// Map a linear workgroup id to an output tile so that the workgroups one XCD receives (ids
// congruent mod 8 are dispatched to the same XCD) cover a contiguous band of tiles.
__device__ __forceinline__ int xcd_remap(int L, int T) {
  const int per = T / 8;
  if (L < per * 8) return (L % 8) * per + L / 8;
  return L;
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool AK, bool BKM, int EPI>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_bf16_kernel(GemmParams p) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int LDK = BK + 8;
  extern __shared__ __align__(16) uint16_t smem[];
  // stage s: A tile at smem + s*(BM+BN)*LDK, B tile right after it
  auto As = [&](int st) { return smem + st * (BM + BN) * LDK; };
  auto Bs = [&](int st) { return smem + st * (BM + BN) * LDK + BM * LDK; };

  const int T = p.tiles_m * p.tiles_n;
  const int t = xcd_remap(blockIdx.x, T);
  const int tm = t / p.tiles_n, tn = t % p.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int split = blockIdx.z;
  const int kbeg = split * p.k_split;
  const int kend = min(p.K, kbeg + p.k_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  TileT<BM, BK, NT, AK> ta;
  TileT<BN, BK, NT, BKM> tb;

  auto load = [&](int k0) {
    ta.load(p.A, p.lda, m0, p.M, k0, kend);
    const uint16_t* Bp = p.B0;
    int kk0 = k0, klim = kend;
    if (p.B1 && k0 >= p.kseg) {
      Bp = p.B1;
      kk0 -= p.kseg;
      klim -= p.kseg;
    } else if (p.B1) {
      klim = min(klim, p.kseg);
    }
    tb.load(Bp, p.ldb, n0, p.N, kk0, klim);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nk > 0) {
    load(kbeg);
    ta.store(As(0));
    tb.store(Bs(0));
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load(kbeg + (kt + 1) * BK);
    const uint16_t* Ac = As(cur) + (wm * WM + (lane & 31)) * LDK + (lane >> 5) * 8;
    const uint16_t* Bc = Bs(cur) + (wn * WN + (lane & 31)) * LDK + (lane >> 5) * 8;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[TM], bfv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *(const bf16x8*)(Ac + i * 32 * LDK + kk * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfv[j] = *(const bf16x8*)(Bc + j * 32 * LDK + kk * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfv[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      ta.store(As(cur ^ 1));
      tb.store(Bs(cur ^ 1));
    }
    __syncthreads();
  }

  // epilogue: 32x32 accumulator layout - lane holds column (lane & 31), rows
  // 8*(r/4) + 4*(lane/32) + (r%4) for r = 0..15
  const bool partial = gridDim.z > 1;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * WN + j * 32 + (lane & 31);
      if (n >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m >= p.M) continue;
        if (partial)
          p.partial[((int64_t)split * p.M + m) * p.N + n] = acc[i][j][r];
        else
          epi_store<EPI>(p, m, n, acc[i][j][r]);
      }
    }
}

template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmParams p, int splits) {
  const int64_t total = (int64_t)p.M * p.N;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    float s = 0.f;
    for (int k = 0; k < splits; ++k) s += p.partial[k * total + e];
    epi_store<EPI>(p, (int)(e / p.N), (int)(e % p.N), s);
  }
}

// ------------------------------------------------------------------------------------------
// host side: configuration choice and launch
// ------------------------------------------------------------------------------------------
namespace {

constexpr int kCUs = 256;

struct Plan {
  int cfg;  // 0: 256x256 (8 waves), 1: 128x128 (4 waves)
  int bm, bn, splits, k_split;
};

Plan make_plan(const GemmProblem& p) {
  const int BK = 64;
  Plan best{1, 128, 128, 1, BK};
  if (p.K <= 0) return best;  // empty reduction: the kernel stores zeros (or leaves C + 0)
  double best_cost = 1e300;
  for (int cfg = 0; cfg < 2; ++cfg) {
    const int bm = cfg == 0 ? 256 : 128, bn = bm;
    const long tiles = (long)((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
    const int per_cu = cfg == 0 ? 1 : 2;
    const double eff = cfg == 0 ? 1.0 : 0.8;  // relative MFMA efficiency of the tile shape
    for (int splits = 1; splits <= 8; ++splits) {
      int ks = (p.K + splits - 1) / splits;
      ks = (ks + BK - 1) / BK * BK;
      const int real = (p.K + ks - 1) / ks;
      if (real != splits) continue;
      const long wgs = tiles * splits;
      const long waves = (wgs + (long)kCUs * per_cu - 1) / ((long)kCUs * per_cu);
      const double t_tile = (double)bm * bn * ks / eff / per_cu;  // per CU-slot time units
      double cost = waves * t_tile;
      if (splits > 1) cost += (double)splits * p.M * p.N * 8.0 * 4.0;  // partial write + read
      if (cost < best_cost * 0.97) {
        best_cost = cost;
        best = Plan{cfg, bm, bn, splits, ks};
      }
    }
  }
  return best;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI>
collider_status launch_cfg(const GemmParams& gp, const Plan& pl, bool ak, bool bk, const char* name,
                           hipStream_t s) {
  constexpr int BK = 64;
  const int T = gp.tiles_m * gp.tiles_n;
  dim3 grid(T, 1, pl.splits), block(64 * WAVES_M * WAVES_N);
  const size_t lds = 2 * (size_t)(BM + BN) * (BK + 8) * sizeof(uint16_t);
#define GEMM_LAUNCH(AKV, BKV)                                                                   \
  {                                                                                             \
    auto kern = gemm_bf16_kernel<BM, BN, BK, WAVES_M, WAVES_N, AKV, BKV, EPI>;                  \
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
    COLLIDER_LAUNCH(name, s, hipLaunchKernelGGL(kern, grid, block, lds, s, gp));                \
  }
  if (ak && !bk) GEMM_LAUNCH(true, false)
  else if (!ak && !bk) GEMM_LAUNCH(false, false)
  else if (ak && bk) GEMM_LAUNCH(true, true)
  else GEMM_LAUNCH(false, true)
#undef GEMM_LAUNCH
  return last_hip_status();
}

template <int EPI>
collider_status run(const GemmProblem& prob, GemmParams gp, const Plan& pl, hipStream_t s) {
  collider_status st;
  const char* name = prob.name ? prob.name : "gemm_bf16";
  if (pl.cfg == 0)
    st = launch_cfg<256, 256, 2, 4, EPI>(gp, pl, prob.a_kmajor, prob.b_kmajor, name, s);
  else
    st = launch_cfg<128, 128, 2, 2, EPI>(gp, pl, prob.a_kmajor, prob.b_kmajor, name, s);
  if (st != COLLIDER_OK || pl.splits == 1) return st;
  const int64_t total = (int64_t)prob.M * prob.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  COLLIDER_LAUNCH("gemm_splitk_reduce", s,
                  hipLaunchKernelGGL(splitk_reduce_kernel<EPI>, dim3((unsigned)blocks), dim3(256),
                                     0, s, gp, pl.splits));
  return last_hip_status();
}

}  // namespace

size_t gemm_bf16_workspace_bytes(const GemmProblem& p) {
  if (p.M <= 0 || p.N <= 0 || p.K <= 0) return 0;
  const Plan pl = make_plan(p);
  return pl.splits > 1 ? (size_t)pl.splits * p.M * p.N * sizeof(float) : 0;
}

collider_status gemm_bf16(const GemmProblem& prob, void* ws, size_t ws_bytes, hipStream_t s) {
  if (prob.M <= 0 || prob.N <= 0) return COLLIDER_OK;
  const Plan pl = make_plan(prob);
  GemmParams gp{};
  gp.A = (const uint16_t*)prob.A;
  gp.lda = prob.lda;
  gp.B0 = (const uint16_t*)prob.B0;
  gp.B1 = (const uint16_t*)prob.B1;
  gp.kseg = prob.B1 ? prob.kseg : prob.K;
  gp.ldb = prob.ldb;
  gp.M = prob.M;
  gp.N = prob.N;
  gp.K = prob.K;
  gp.k_split = pl.k_split;
  gp.tiles_m = (prob.M + pl.bm - 1) / pl.bm;
  gp.tiles_n = (prob.N + pl.bn - 1) / pl.bn;
  gp.C = prob.C;
  gp.ldc = prob.ldc;
  gp.accumulate = prob.accumulate;
  gp.g = prob.g;
  gp.up = prob.up;
  gp.ld_g = prob.ld_g;
  gp.rowmap = prob.rowmap;
  gp.out2 = prob.out2;
  gp.ld_out2 = prob.ld_out2;
  if (pl.splits > 1) {
    if (!ws || ws_bytes < (size_t)pl.splits * prob.M * prob.N * sizeof(float))
      return COLLIDER_ERR_WORKSPACE;
    gp.partial = (float*)ws;
  }
  switch (prob.epi) {
    case EPI_BF16: return run<EPI_BF16>(prob, gp, pl, s);
    case EPI_F32: return run<EPI_F32>(prob, gp, pl, s);
    case EPI_SWIGLU: return run<EPI_SWIGLU>(prob, gp, pl, s);
    case EPI_GELU: return run<EPI_GELU>(prob, gp, pl, s);
  }
  return COLLIDER_ERR_UNSUPPORTED;
}

// ------------------------------------------------------------------------------------------
// fp32 GEMM (CUDA-core style FMA, 64x64 tiles, 4x4 per thread) for the fp32 linear backward
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                       int ak, const float* __restrict__ B,
                                                       int64_t ldb, int bk, int M, int N, int K,
                                                       float* __restrict__ C, int64_t ldc,
                                                       int accumulate) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      int kk, mm;
      if (ak) { mm = e / 16; kk = e % 16; } else { kk = e / 64; mm = e % 64; }
      const int m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < M && k < K) ? (ak ? A[(int64_t)m * lda + k] : A[(int64_t)k * lda + m]) : 0.f;
      int kb, nn;
      if (bk) { nn = e / 16; kb = e % 16; } else { kb = e / 64; nn = e % 64; }
      const int n = n0 + nn, k2 = k0 + kb;
      Bs[kb][nn] = (n < N && k2 < K) ? (bk ? B[(int64_t)n * ldb + k2] : B[(int64_t)k2 * ldb + n]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < M && n < N) {
        float* c = C + (int64_t)m * ldc + n;
        *c = accumulate ? *c + acc[i][j] : acc[i][j];
      }
    }
}

collider_status gemm_f32(const GemmProblem& p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return COLLIDER_OK;
  dim3 grid((p.N + 63) / 64, (p.M + 63) / 64);
  COLLIDER_LAUNCH("gemm_f32", s,
                  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, (const float*)p.A,
                                     p.lda, (int)p.a_kmajor, (const float*)p.B0, p.ldb,
                                     (int)p.b_kmajor, p.M, p.N, p.K, (float*)p.C, p.ldc,
                                     p.accumulate));
  return last_hip_status();
}

}  // namespace collider
