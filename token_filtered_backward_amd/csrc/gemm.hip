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
#include <atomic>
#include <cstdio>
#include <cstdlib>
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
  int splits;
  int tiles_m, tiles_n;
  int group_m;   // tile rows per group of the direct-to-LDS kernel's tile numbering (tile_coords)
  // work decomposition of the direct-to-LDS kernel: tiles [0, dp_tiles) are whole work items
  // (times `splits` K-splits); tiles [dp_tiles, dp_tiles + sk_tiles) are shared out as one
  // stream-K range of k-tiles per workgroup
  int ipt;       // k-tiles per output tile
  int dp_tiles;
  int sk_tiles;
  float* skp;    // stream-K partial tiles: [2 * gridDim.x][BM * BN], two slots per workgroup
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
    const float s = fast_sigmoid(g);
    ((uint16_t*)p.C)[(int64_t)m * p.ldc + n] = f2bf(v * u * s * (1.f + g * (1.f - s)));
    p.out2[(int64_t)m * p.ld_out2 + n] = f2bf(v * g * s);
  } else {  // EPI_GELU: dF = dA * d/df gelu_tanh(f)
    const int64_t r = p.rowmap ? p.rowmap[m] : m;
    const float f = bf2f(p.g[r * p.ld_g + n]);
    const float c = 0.7978845608028654f, a = 0.044715f;
    const float t = fast_tanh(c * (f + a * f * f * f));
    const float d = 0.5f * (1.f + t) + 0.5f * f * (1.f - t * t) * c * (1.f + 3.f * a * f * f);
    ((uint16_t*)p.C)[(int64_t)m * p.ldc + n] = f2bf(v * d);
  }
}

// Eight consecutive outputs (m, n .. n+7) with 16-byte accesses; n and every leading dimension
// are multiples of 8 and the bases 16-byte aligned (checked on the host).
__device__ __forceinline__ uint4 pack8(const float* v) {
  return make_uint4(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]), pack2bf(v[4], v[5]), pack2bf(v[6], v[7]));
}

__device__ __forceinline__ void unpack8(uint4 u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bflo(w[i]);
    f[2 * i + 1] = bfhi(w[i]);
  }
}

template <int EPI>
__device__ __forceinline__ void epi_store8(const GemmParams& p, int m, int n, const float* v) {
  if constexpr (EPI == EPI_BF16) {
    *(uint4*)((uint16_t*)p.C + (int64_t)m * p.ldc + n) = pack8(v);
  } else if constexpr (EPI == EPI_F32) {
    float4* c = (float4*)((float*)p.C + (int64_t)m * p.ldc + n);
    float4 a = make_float4(v[0], v[1], v[2], v[3]), b = make_float4(v[4], v[5], v[6], v[7]);
    if (p.accumulate) {
      const float4 a0 = c[0], b0 = c[1];
      a.x += a0.x; a.y += a0.y; a.z += a0.z; a.w += a0.w;
      b.x += b0.x; b.y += b0.y; b.z += b0.z; b.w += b0.w;
    }
    c[0] = a;
    c[1] = b;
  } else if constexpr (EPI == EPI_SWIGLU) {
    const int64_t r = p.rowmap ? p.rowmap[m] : m;
    float g[8], u[8], dg[8], du[8];
    unpack8(*(const uint4*)(p.g + r * p.ld_g + n), g);
    unpack8(*(const uint4*)(p.up + r * p.ld_g + n), u);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float s = fast_sigmoid(g[e]);
      dg[e] = v[e] * u[e] * s * (1.f + g[e] * (1.f - s));
      du[e] = v[e] * g[e] * s;
    }
    *(uint4*)((uint16_t*)p.C + (int64_t)m * p.ldc + n) = pack8(dg);
    *(uint4*)(p.out2 + (int64_t)m * p.ld_out2 + n) = pack8(du);
  } else {
    const int64_t r = p.rowmap ? p.rowmap[m] : m;
    float f[8], o[8];
    unpack8(*(const uint4*)(p.g + r * p.ld_g + n), f);
    const float c = 0.7978845608028654f, a = 0.044715f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = fast_tanh(c * (f[e] + a * f[e] * f[e] * f[e]));
      o[e] = v[e] * (0.5f * (1.f + t) + 0.5f * f[e] * (1.f - t * t) * c * (1.f + 3.f * a * f[e] * f[e]));
    }
    *(uint4*)((uint16_t*)p.C + (int64_t)m * p.ldc + n) = pack8(o);
  }
}

__device__ __forceinline__ void store8_partial(const GemmParams& p, int split, int m, int n,
                                               const float* v) {
  float4* d = (float4*)(p.partial + ((int64_t)split * p.M + m) * p.N + n);
  d[0] = make_float4(v[0], v[1], v[2], v[3]);
  d[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// The epilogue's other inputs for GPT groups of 8 outputs (rows mfirst + i * mstep, columns
// n .. n+7): the saved pre-activations (SwiGLU: gate in sa, up in sb; GELU: f in sa) or the fp32
// values being accumulated into (sa, sb = columns n .. n+3, n+4 .. n+7).  All loads of a call are
// issued before any is used, so one memory latency covers the whole batch.
// side_rows gives the source rows (the index lookup, -1 past the edge), side_load issues the row
// loads; the direct-to-LDS kernel looks up the rows one epilogue pass before it loads them, so
// that each pass waits on one memory latency instead of two dependent ones.
template <int EPI, int GPT>
__device__ __forceinline__ void side_rows(const GemmParams& p, int mfirst, int mstep, int n,
                                          int (&r)[GPT]) {
  if constexpr (EPI == EPI_BF16) return;
  if constexpr (EPI == EPI_F32) {
    if (!p.accumulate) return;
  }
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int m = mfirst + i * mstep;
    const bool ok = m < p.M && n < p.N;
    if constexpr (EPI == EPI_F32)
      r[i] = ok ? m : -1;
    else
      r[i] = ok ? (p.rowmap ? p.rowmap[m] : m) : -1;
  }
}

template <int EPI, int GPT>
__device__ __forceinline__ void side_load(const GemmParams& p, const int (&r)[GPT], int n,
                                          uint4 (&sa)[GPT], uint4 (&sb)[GPT]) {
  if constexpr (EPI == EPI_BF16) return;
  if constexpr (EPI == EPI_F32) {
    if (!p.accumulate) return;
  }
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    if (r[i] < 0) continue;
    if constexpr (EPI == EPI_F32) {
      const uint4* c = (const uint4*)((const float*)p.C + (int64_t)r[i] * p.ldc + n);
      sa[i] = c[0];
      sb[i] = c[1];
    } else {
      sa[i] = *(const uint4*)(p.g + (int64_t)r[i] * p.ld_g + n);
      if constexpr (EPI == EPI_SWIGLU) sb[i] = *(const uint4*)(p.up + (int64_t)r[i] * p.ld_g + n);
    }
  }
}

template <int EPI, int GPT>
__device__ __forceinline__ void prefetch_side(const GemmParams& p, int mfirst, int mstep, int n,
                                              uint4 (&sa)[GPT], uint4 (&sb)[GPT]) {
  int r[GPT];
  side_rows<EPI, GPT>(p, mfirst, mstep, n, r);
  side_load<EPI, GPT>(p, r, n, sa, sb);
}

// Final epilogue of 8 outputs with the side inputs already in registers.
template <int EPI>
__device__ __forceinline__ void epi_finish8(const GemmParams& p, int m, int n, const float* v,
                                            uint4 sa, uint4 sb) {
  if constexpr (EPI == EPI_BF16) {
    *(uint4*)((uint16_t*)p.C + (int64_t)m * p.ldc + n) = pack8(v);
  } else if constexpr (EPI == EPI_F32) {
    float4 a = make_float4(v[0], v[1], v[2], v[3]), b = make_float4(v[4], v[5], v[6], v[7]);
    if (p.accumulate) {
      const float4 a0 = __builtin_bit_cast(float4, sa), b0 = __builtin_bit_cast(float4, sb);
      a.x += a0.x; a.y += a0.y; a.z += a0.z; a.w += a0.w;
      b.x += b0.x; b.y += b0.y; b.z += b0.z; b.w += b0.w;
    }
    float4* c = (float4*)((float*)p.C + (int64_t)m * p.ldc + n);
    c[0] = a;
    c[1] = b;
  } else if constexpr (EPI == EPI_SWIGLU) {
    float g[8], u[8], dg[8], du[8];
    unpack8(sa, g);
    unpack8(sb, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float s = fast_sigmoid(g[e]);
      dg[e] = v[e] * u[e] * s * (1.f + g[e] * (1.f - s));
      du[e] = v[e] * g[e] * s;
    }
    *(uint4*)((uint16_t*)p.C + (int64_t)m * p.ldc + n) = pack8(dg);
    *(uint4*)(p.out2 + (int64_t)m * p.ld_out2 + n) = pack8(du);
  } else {
    float f[8], o[8];
    unpack8(sa, f);
    const float c = 0.7978845608028654f, a = 0.044715f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = fast_tanh(c * (f[e] + a * f[e] * f[e] * f[e]));
      o[e] = v[e] * (0.5f * (1.f + t) + 0.5f * f[e] * (1.f - t * t) * c * (1.f + 3.f * a * f[e] * f[e]));
    }
    *(uint4*)((uint16_t*)p.C + (int64_t)m * p.ldc + n) = pack8(o);
  }
}


// ------------------------------------------------------------------------------------------
// tile loaders (global -> registers -> LDS).  LDS tiles are k-contiguous rows of BK + 8 elements:
// the 16-byte pad makes consecutive rows start 36 banks apart, so the 16-byte fragment reads of
// 16 consecutive rows touch every bank once.
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

// X(r, k) = X[k*ld + r]: each thread loads an 8 (k) x 8 (r) block as eight 16-byte rows and
// transposes it in registers into eight k-contiguous 16-byte LDS stores.  The k-block index runs
// fastest over the lanes, so the 8 lanes of a row block write 8 consecutive 16-byte chunks of the
// same LDS row (no bank conflicts) and every load instruction reads whole 128-byte lines.
template <int R, int BK, int NT>
struct MNMajorTile {
  static constexpr int RB = R / 8, KB = BK / 8;
  static constexpr int NBLK = RB * KB;
  static constexpr int N = (NBLK + NT - 1) / NT;
  uint4 v[N][8];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ X, int64_t ld, int r0, int rlim,
                                       int k0, int klim) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int b = threadIdx.x + NT * i;
      const int kb = b % KB, rb = b / KB;
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
        const int kb = b % KB, rb = b / KB;
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

// Map a linear work index to an output tile so that the workgroups one XCD receives (ids
// congruent mod 8 are dispatched to the same XCD) cover a contiguous band of tiles, which share
// their A rows / B columns in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int L, int T) {
  const int per = T / 8;
  if (L < per * 8) return (L % 8) * per + L / 8;
  return L;
}

// Output tile (row, column) of tile number t in the direct-to-LDS kernel's numbering: column by
// column within groups of group_m tile rows, one group after another.  A run of consecutive numbers
// - what the workgroups of one XCD receive (xcd_remap) - then covers a compact block of tile rows
// and columns, so the XCD's L2 serves few distinct A row panels and B column panels at a time
// (row-major numbering gives one XCD a band of whole tile rows, which needs every B column).
__device__ __forceinline__ void tile_coords(const GemmParams& p, int t, int& tm, int& tn) {
  const int per_group = p.group_m * p.tiles_n;
  const int g = t / per_group, first = g * p.group_m;
  const int gm = min(p.group_m, p.tiles_m - first);
  const int w = t - g * per_group;
  tm = first + w % gm;
  tn = w / gm;
}

// One workgroup of 4 wavefronts (2 x 2) computes a BM x BN tile; each wavefront a
// (BM/2) x (BN/2) block as a grid of 32x32 MFMA accumulators.  Larger wave blocks read fewer
// LDS bytes per MFMA: at 128 x 128 the fragment reads need half the LDS bandwidth the MFMAs
// can consume.  Work items (tile, K-split) are walked with a grid stride, so the same kernel
// runs one item per workgroup or persistently.
template <int BM, int BN, int BK, bool AK, bool BKM, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmParams p) {
  constexpr int NT = 256;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int LDK = BK + 8;
  extern __shared__ __align__(16) uint16_t smem[];
  auto As = [&](int st) { return smem + st * (BM + BN) * LDK; };
  auto Bs = [&](int st) { return smem + st * (BM + BN) * LDK + BM * LDK; };

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int T = p.tiles_m * p.tiles_n;
  const int total = T * p.splits;
  const bool partial = p.splits > 1;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int li = xcd_remap(item, total);
    const int split = li / T, t = li % T;
    const int tm = t / p.tiles_n, tn = t % p.tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = split * p.k_split;
    const int kend = min(p.K, kbeg + p.k_split);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

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
}

// ------------------------------------------------------------------------------------------
// Direct-to-LDS GEMM (gfx950).  Tiles travel global -> LDS with 16-byte buffer loads that write
// LDS directly (no staging registers), so NS - 1 k-tiles of depth KT (32 or 64) are in flight
// while one is consumed.  Buffer loads are range checked: rows past the end of an operand (the
// ragged token dimension) arrive as zeros.
// Each operand keeps its global orientation in LDS, XOR-swizzled instead of padded:
//   K-major tile  [R][KT]  2KT-byte rows, 16-byte chunk c of row r stored at c ^ ((r >> 1) & (KT/8 - 1))
//   MN-major tile [KT][R]  2R-byte rows,  chunk c of row k stored at c ^ (4 * (k & 3))
// MFMA fragments come from ds_read_b128 (K-major) or two ds_read_b64_tr_b16 (MN-major): within a
// group of 16 lanes, lane j addresses row k0 + j/4, columns n + 4*(j%4) .. +3, and lane i receives
// rows k0 .. k0+3 of column n + i - exactly the k-contiguous operand layout the MFMA expects.
// Both swizzles make the lane groups the LDS serves together bank-conflict free.
// ------------------------------------------------------------------------------------------
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

template <int KT>
__device__ __forceinline__ int kmaj_off(int r, int c) {
  return r * (2 * KT) + ((c ^ ((r >> 1) & (KT / 8 - 1))) << 4);
}
template <int R>
__device__ __forceinline__ int mnmaj_off(int k, int c) {
  return k * (2 * R) + ((c ^ ((k & 3) << 2)) << 4);
}

// Buffer resource of a raw byte buffer (stride 0): base, num_records = bytes, gfx9 dword 3.
typedef int rsrc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return rsrc_t{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xffffu), (int)bytes, 0x00020000};
}


// Where one operand's k-tile comes from: a buffer resource and a scalar byte offset.  K-major
// operands keep the whole buffer and take the k offset as the scalar offset; their rows, which the
// range check must see, are in the per-lane vector offsets.  MN-major operands (whose rows are k)
// instead advance the resource's base to the k-tile's first row and shorten its range by as much,
// so the per-lane offsets stay fixed and rows past the end still read as zeros.  Both cost a few
// scalar instructions per k-tile and none per load.
struct KSrc {
  rsrc_t rs;
  uint32_t soff;
};
template <bool KMAJ>
__device__ __forceinline__ KSrc ktile_src(const void* base, uint32_t bytes, int64_t ld, int k0) {
  if constexpr (KMAJ) {
    return KSrc{make_rsrc(base, bytes), (uint32_t)k0 * 2u};
  } else {
    const uint64_t adv = (uint64_t)k0 * (uint64_t)ld * 2u;
    return KSrc{make_rsrc((const char*)base + adv, adv < bytes ? bytes - (uint32_t)adv : 0u), 0u};
  }
}

// 16-byte buffer load of each lane straight into LDS (M0 = LDS byte address of the wavefront's
// 1 KB slot, lane i lands at M0 + 16 i; global address = base + voff + soff).  Issued as inline
// assembly: the compiler then inserts no waits of its own (it cannot tell which LDS bytes the copy
// writes and would wait for every outstanding load at each LDS read); completion is tracked
// explicitly with s_waitcnt vmcnt in the k-loop.  An LDS-DMA load reads M0 one wait state after a
// scalar write of M0 at the earliest on this GPU family, hence the s_nop between the two.
__device__ __forceinline__ void dma16(rsrc_t rs, uint32_t m0, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}

// Direct loads of one operand tile, [R x KT] (K-major) or [KT x R] (MN-major) in LDS.  Wave w of
// NW issues loads q = w, w + NW, ...; load q fills LDS bytes [1024 q, 1024 q + 1024) of the tile.
// The per-lane byte offsets (relative to the k-tile's source, see ktile_src) are computed once per
// output tile.
template <int R, bool KMAJ, int KT, int NW>
struct TileDMA {
  static constexpr int NI = R * KT * 2 / 1024, PW = NI / NW;
  static_assert(NI % NW == 0, "every wave issues the same number of loads");
  uint32_t off[PW];
  // mn0: first row (K-major) or first column (MN-major) of the tile in the operand
  __device__ __forceinline__ void init(int64_t ld, int mn0, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int b = (wave + NW * i) * 1024 + lane * 16;
      if constexpr (KMAJ) {
        const int r = b / (2 * KT), pos = (b >> 4) & (KT / 8 - 1);
        const int c = pos ^ ((r >> 1) & (KT / 8 - 1));
        off[i] = (uint32_t)(((int64_t)(mn0 + r) * ld + 8 * c) * 2);
      } else {
        const int k = b / (2 * R), pos = (b % (2 * R)) >> 4;
        const int c = pos ^ ((k & 3) << 2);
        off[i] = (uint32_t)(((int64_t)k * ld + mn0 + 8 * c) * 2);
      }
    }
  }
  // load I (< PW) of this wave; mw = LDS byte address of the wave's first slot in the tile
  template <int I>
  __device__ __forceinline__ void issue_one(const KSrc& s, uint32_t mw) const {
    dma16(s.rs, mw + (uint32_t)I * (uint32_t)(NW * 1024), off[I], s.soff);
  }
};

// Wavefronts per workgroup of the direct-to-LDS kernel: 8 (two per SIMD, so that one wavefront's
// waits are covered by the other's MFMAs) for 256 x 256 tiles, 4 otherwise.
constexpr int lds_waves(int bm, int bn) { return (bm == 256 && bn == 256) ? 8 : 4; }
// Wavefront grid over a BM x BN tile: 2 x (NW / 2) when BM / 2 is a multiple of 32, else 1 x 4
// (BM = 160, 224: each wavefront covers all rows and a quarter of the columns).
constexpr int wave_rows(int bm, int bn) { return (bm % 64 == 0) ? 2 : 1; }
constexpr int wave_cols(int bm, int bn) { return lds_waves(bm, bn) / wave_rows(bm, bn); }

// The loads of one k-tile (A then B) into an LDS stage, one instruction at a time, so that they can
// be spread between MFMAs: a burst of 1 KB loads from every wavefront would queue at the CU's vector
// memory unit and stall the wavefronts' MFMA issue behind it.
template <int BM, int BN, bool AK, bool BKM, int KT>
struct StageLoader {
  using TA = TileDMA<BM, AK, KT, lds_waves(BM, BN)>;
  using TB = TileDMA<BN, BKM, KT, lds_waves(BM, BN)>;
  static constexpr int N = TA::PW + TB::PW;
  const TA& da;
  const TB& db;
  KSrc a, b;
  uint32_t ma, mb;  // LDS byte address of this wavefront's first slot in the A / B tile
  // load q of the k-tile; q is a constant once the caller's loops are unrolled, and the chain of
  // comparisons folds to the one load
  template <int Q = 0>
  __device__ __forceinline__ void issue(int q) const {
    if (q == Q) {
      if constexpr (Q < TA::PW)
        da.template issue_one<Q>(a, ma);
      else
        db.template issue_one<Q - TA::PW>(b, mb);
    } else if constexpr (Q + 1 < N) {
      issue<Q + 1>(q);
    }
  }
};

// Per-lane LDS byte offsets of a wavefront's MFMA fragments (32 rows x 16 k) inside an operand tile,
// computed once per kernel.  K-major tile: the offset depends on the k-step (the swizzle mixes the
// chunk with row bits) but not on the fragment (fragments lie 32 rows apart, a whole number of
// swizzle periods): one offset per k-step, fragment f at + 64 KT f bytes.  MN-major tile: the offset
// depends on the fragment (its columns enter the swizzle) but not on the k-step (16 rows, a whole
// number of periods of the 4-row swizzle): one offset per fragment, k-step kk at + 32 R kk bytes and
// the second four-row read at + 8 R.  Reads then take one address register per offset and a
// constant in the instruction.
//   ds_read_b64_tr_b16 (MN-major): within a group of 16 lanes, lane j addresses row k0 + j/4, columns
//   n + 4*(j%4) .. +3, and lane i receives rows k0 .. k0+3 of column n + i - exactly the
//   k-contiguous operand layout the MFMA expects.
template <int R, bool KMAJ, int KT, int NF>
struct FragOffsets {
  static constexpr int KS = KT / 16, N = KMAJ ? KS : NF;
  uint32_t o[N];
  // rbase: the wavefront's first row (K-major) / column (MN-major) within the tile
  __device__ __forceinline__ void init(int rbase, int lane) {
#pragma unroll
    for (int x = 0; x < N; ++x) {
      if constexpr (KMAJ) {
        o[x] = (uint32_t)kmaj_off<KT>(rbase + (lane & 31), x * 2 + (lane >> 5));
      } else {
        const int g = lane >> 4, j = lane & 15;
        const int col = rbase + x * 32 + 16 * (g & 1) + 4 * (j & 3);
        const int kb = 8 * (g >> 1) + (j >> 2);
        o[x] = (uint32_t)(mnmaj_off<R>(kb, col >> 3) + (col & 7) * 2);
      }
    }
  }
  // the wavefront's address registers for a tile at LDS byte address `tile`: one add each, kept
  // opaque so that the compiler folds every fragment's constant into the instruction's offset field
  // instead of holding one precomputed address per read
  __device__ __forceinline__ void bind(uint32_t tile, uint32_t (&a)[N]) const {
#pragma unroll
    for (int x = 0; x < N; ++x) {
      a[x] = tile + o[x];
      asm volatile("" : "+v"(a[x]));
    }
  }
  __device__ __forceinline__ static bf16x8 read(const uint32_t (&a)[N], int f, int kk) {
    typedef __attribute__((address_space(3))) const char* lds_cptr;
    if constexpr (KMAJ) {
      return *(const __attribute__((address_space(3))) bf16x8*)(lds_cptr)(uintptr_t)(a[kk] + f * 64 * KT);
    } else {
      const uint32_t b = a[f] + kk * 32 * R;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(lds_cptr)(uintptr_t)b);
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(lds_cptr)(uintptr_t)(b + 8 * R));
      typedef short v8s __attribute__((ext_vector_type(8)));
      const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8, both);
    }
  }
};

// s_waitcnt vmcnt(n), other counters unconstrained (gfx9 encoding)
#define VMCNT_WAIT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xf) | (((n) >> 4) << 14) | (0x7 << 4) | (0xf << 8))

// MFMAs of one k-tile (KT / 16 steps of k = 16) from one LDS stage; fragments of step kk+1 are read
// while the MFMAs of step kk run (two register sets), interleaved with them.  With LOAD, the loads of a later k-tile (`ld`)
// go out one instruction at a time between the MFMAs, within the first SPN / SPD of them.
template <int BM, int BN, bool AK, bool BKM, int KT, int SPN, int SPD, bool LOAD>
__device__ __forceinline__ void mma_ktile(
    uint32_t As, uint32_t Bs,
    f32x16 (&acc)[BM / wave_rows(BM, BN) / 32][BN / wave_cols(BM, BN) / 32],
    const FragOffsets<BM, AK, KT, BM / wave_rows(BM, BN) / 32>& fa,
    const FragOffsets<BN, BKM, KT, BN / wave_cols(BM, BN) / 32>& fb,
    const StageLoader<BM, BN, AK, BKM, KT>& ld) {
  constexpr int WGM = wave_rows(BM, BN), WGN = wave_cols(BM, BN);
  constexpr int WM = BM / WGM, WN = BN / WGN, TM = WM / 32, TN = WN / 32, KS = KT / 16;
  constexpr int NQ = StageLoader<BM, BN, AK, BKM, KT>::N, MT = KS * TM * TN;
  static_assert(MT * SPN >= NQ * SPD && SPN <= SPD, "every load gets an MFMA slot");
  using FA = FragOffsets<BM, AK, KT, TM>;
  using FB = FragOffsets<BN, BKM, KT, TN>;
  uint32_t aa[FA::N], ba[FB::N];
  fa.bind(As, aa);
  fb.bind(Bs, ba);
  bf16x8 af[2][TM], bfv[2][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) af[0][i] = FA::read(aa, i, 0);
#pragma unroll
  for (int j = 0; j < TN; ++j) bfv[0][j] = FB::read(ba, j, 0);
  // the next k-step's fragments (A then B, NR reads) go out one at a time between the first half
  // of this k-step's MFMAs: a burst of LDS reads ahead of the MFMAs would hold up MFMA issue
  constexpr int NR = TM + TN;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const int cur = kk & 1;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        acc[i][j] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfv[cur][j], acc[i][j], 0, 0, 0);
        if (kk + 1 < KS) {
          const int l = i * TN + j;  // MFMA number within the k-step
#pragma unroll
          for (int r = 0; r < NR; ++r)
            if ((r * TM * TN) / (2 * NR) == l) {
              __builtin_amdgcn_sched_barrier(0);
              if (r < TM)
                af[cur ^ 1][r] = FA::read(aa, r, kk + 1);
              else
                bfv[cur ^ 1][r - TM] = FB::read(ba, r - TM, kk + 1);
              __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (LOAD) {
          const int n = (kk * TM + i) * TN + j;  // MFMA number within the k-tile
#pragma unroll
          for (int q = 0; q < NQ; ++q)
            if (((q + 1) * MT * SPN) / (NQ * SPD) - 1 == n) {
              __builtin_amdgcn_sched_barrier(0);
              ld.issue(q);
              __builtin_amdgcn_sched_barrier(0);
            }
        }
      }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Work decomposition.  Whole tiles (optionally split over K, partials summed by
// splitk_reduce_kernel) are walked with a grid stride.  When the tile count leaves the last wave of
// workgroups partly idle, the remaining tiles are instead shared out as one contiguous range of
// (tile, k-tile) iterations per workgroup ("stream-K"): every workgroup gets the same number of
// k-tiles.  A tile whose k-range one workgroup covers entirely is finished in place; the pieces of
// a tile shared by several workgroups go to per-workgroup fp32 slots (slot 0: the first piece of a
// workgroup's range, slot 1: its last) and sk_fixup_kernel adds them in k order and runs the
// epilogue.  No workgroup waits on another, and every sum has a fixed order, so results are
// deterministic.
template <int BM, int BN, int KT, bool AK, bool BKM, int EPI, int NS>
__global__ __launch_bounds__(64 * lds_waves(BM, BN)) void gemm_lds_kernel(GemmParams p) {
  constexpr int BK = KT;
  constexpr int NW = lds_waves(BM, BN), NT = 64 * NW;
  constexpr int WGM = wave_rows(BM, BN), WGN = wave_cols(BM, BN);
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wavefront blocks of whole 32 x 32 MFMA tiles");
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  constexpr int LPW = (A_BYTES + B_BYTES) / 1024 / NW;  // load instructions per wave per k-tile
  static_assert(NS <= 3 && LPW * (NS - 2) < 64, "vmcnt range");
  extern __shared__ __align__(16) char lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  // LDS byte address of the dynamic LDS block (the low half of its flat address)
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  // operand buffer sizes in bytes: A has M rows when K-major, K rows when MN-major; B's two
  // segments hold reduction indices [0, kseg) and [kseg, K)
  const uint32_t a_bytes = (uint32_t)((int64_t)(AK ? p.M : p.K) * p.lda * 2);
  const int kseg = p.B1 ? p.kseg : p.K;
  const bool two_seg = p.B1 != nullptr;
  const uint32_t b0_bytes = (uint32_t)((int64_t)(BKM ? p.N : kseg) * p.ldb * 2);
  const uint32_t b1_bytes = (uint32_t)((int64_t)(BKM ? p.N : p.K - kseg) * p.ldb * 2);
  // the loads of the k-tile starting at reduction index k into the LDS stage at byte address st
  auto loader = [&](const TileDMA<BM, AK, KT, NW>& da, const TileDMA<BN, BKM, KT, NW>& db, int k,
                    uint32_t st, bool on) {
    const bool seg1 = two_seg && k >= kseg;
    const uint32_t mw = st + (uint32_t)wave * 1024u;
    return StageLoader<BM, BN, AK, BKM, KT>{
        da, db, ktile_src<AK>(p.A, on ? a_bytes : 0u, p.lda, k),
        seg1 ? ktile_src<BKM>(p.B1, on ? b1_bytes : 0u, p.ldb, k - kseg)
             : ktile_src<BKM>(p.B0, on ? b0_bytes : 0u, p.ldb, k),
        mw, mw + (uint32_t)A_BYTES};
  };
  FragOffsets<BM, AK, KT, TM> fa;
  FragOffsets<BN, BKM, KT, TN> fb;
  fa.init(wm * WM, lane);
  fb.init(wn * WN, lane);

  const int dp_items = p.dp_tiles * p.splits;
  const int kts = p.k_split / BK;  // k-tiles per K-split
  // this workgroup's stream-K range; neighbouring ranges (which share tiles and operand panels)
  // go to workgroups on the same XCD
  const int v = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t n_it = (int64_t)p.sk_tiles * p.ipt;
  const int64_t it_first = (int64_t)v * n_it / gridDim.x;
  const int64_t it_end = (int64_t)(v + 1) * n_it / gridDim.x;
  int64_t it = it_first;
  int item = blockIdx.x;

  for (;;) {
    int t, kt0, kt1, mode, oidx;  // mode 0: final epilogue, 1: K-split partial, 2: stream-K slot
    if (item < dp_items) {
      const int li = xcd_remap(item, dp_items);
      const int split = li / p.dp_tiles;
      t = li % p.dp_tiles;
      kt0 = split * kts;
      kt1 = min(p.ipt, kt0 + kts);
      mode = p.splits > 1 ? 1 : 0;
      oidx = split;
      item += gridDim.x;
    } else if (it < it_end) {
      const int st = (int)(it / p.ipt);
      t = p.dp_tiles + st;
      kt0 = (int)(it - (int64_t)st * p.ipt);
      kt1 = (int)min((int64_t)p.ipt, (int64_t)kt0 + (it_end - it));
      mode = (kt0 == 0 && kt1 == p.ipt) ? 0 : 2;
      oidx = 2 * v + (it == it_first ? 0 : 1);
      it += kt1 - kt0;
    } else {
      break;
    }
    int tm, tn;
    tile_coords(p, t, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = kt1 - kt0;
    const int kbeg = kt0 * BK;
    TileDMA<BM, AK, KT, NW> da;
    TileDMA<BN, BKM, KT, NW> db;
    da.init(p.lda, m0, wave, lane);
    db.init(p.ldb, n0, wave, lane);

    // epilogue layout: the fp32 tile is staged row-major in passes of EROWS rows, then every
    // thread finishes 8 consecutive columns of GPT rows with 16-byte loads / stores
    constexpr int LDE = BN + 8;  // +8 floats: the two lane halves' rows land 32 banks apart
    // rows per pass: a divisor of BM that fits the stage buffers; epilogues with two 16-byte side
    // inputs per 8 outputs take shorter passes (registers)
    constexpr int EROWS_REG = (EPI == EPI_SWIGLU || EPI == EPI_F32 || NW == 8) ? 32 : 64;
    constexpr int EROWS = (BM <= EROWS_REG && BM * LDE * 4 <= NS * STAGE) ? BM
                          : (BM % 64 == 0 && 64 <= EROWS_REG && 64 * LDE * 4 <= NS * STAGE) ? 64 : 32;
    static_assert(BM % EROWS == 0 && EROWS % 32 == 0, "epilogue passes cover whole accumulator blocks");
    static_assert(EROWS * LDE * 4 <= NS * STAGE, "epilogue pass must fit in the stage buffers");
    constexpr int CPR = BN / 8, RSTEP = NT / CPR, GPT = EROWS / RSTEP;
    static_assert(EROWS % RSTEP == 0, "epilogue rows per pass");
    const int cg = threadIdx.x % CPR, rsub = threadIdx.x / CPR;
    const int n = n0 + cg * 8;
    // side inputs of the first epilogue pass (SwiGLU / GELU rows, or C when accumulating) and the
    // source rows of the second pass's: loaded now, so that their latency overlaps the k-loop
    // (loads return in order, so the k-loop's own waits never stop short of them)
    constexpr int NPASS = BM / EROWS;
    uint4 sa[GPT], sb[GPT];
    int rn[GPT];  // source rows of the next pass's side inputs
#pragma unroll
    for (int i = 0; i < GPT; ++i) rn[i] = -1;
    if (mode == 0) {
      prefetch_side<EPI, GPT>(p, m0 + rsub, RSTEP, n, sa, sb);
      if (NPASS > 1) side_rows<EPI, GPT>(p, m0 + EROWS + rsub, RSTEP, n, rn);
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    VMCNT_WAIT(0);
    __syncthreads();  // previous item's readers are done with every stage
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      {
        const auto sl = loader(da, db, kbeg + s * BK, lds0 + s * STAGE, s < nk);
#pragma unroll
        for (int q = 0; q < StageLoader<BM, BN, AK, BKM, KT>::N; ++q) sl.issue(q);
      }
    // k-tile kt + NS - 1 refills the stage read in iteration kt - 1; its loads go out between
    // k-tile kt's MFMAs (within the first half with two stages, the first 3/4 with three).  Past the
    // last k-tile the loads still go out, from a source of range 0: they read nothing and write
    // zeros into a stage no k-tile reads any more, and the k-loop keeps a single MFMA sequence.
    for (int kt = 0; kt < nk; ++kt) {
      VMCNT_WAIT(LPW * (NS - 2));  // tile kt complete (for this wave), then visible to all waves
      __syncthreads();
      const uint32_t As = lds0 + (uint32_t)((kt % NS) * STAGE);
      const auto sl = loader(da, db, kbeg + (kt + NS - 1) * BK, lds0 + ((kt + NS - 1) % NS) * STAGE,
                             kt + NS - 1 < nk);
      mma_ktile<BM, BN, AK, BKM, KT, (NS == 2 ? 1 : 3), (NS == 2 ? 2 : 4), true>(
          As, As + A_BYTES, acc, fa, fb, sl);
    }
    VMCNT_WAIT(0);  // the zero-range loads have landed before the epilogue reuses the stages

    // epilogue through LDS (constants and the first pass's side inputs set up before the k-loop)
    float* E = (float*)lds;
#pragma unroll
    for (int pass = 0; pass < BM / EROWS; ++pass) {
      // side inputs of the next pass go out now (their rows were looked up during the previous
      // pass), and the rows of the pass after it are looked up; both latencies overlap this pass
      uint4 na[GPT], nb[GPT];
      if (pass + 1 < NPASS && mode == 0) {
        side_load<EPI, GPT>(p, rn, n, na, nb);
        if (pass + 2 < NPASS) side_rows<EPI, GPT>(p, m0 + (pass + 2) * EROWS + rsub, RSTEP, n, rn);
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int rb = wm * WM + i * 32;  // first tile row of this 32-row accumulator block
        if (rb / EROWS != pass) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            E[(rb - pass * EROWS + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * LDE + wn * WN +
              j * 32 + (lane & 31)] = acc[i][j][r];
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < GPT; ++i) {
        const int row = rsub + i * RSTEP;
        const int m = m0 + pass * EROWS + row;
        const float4 lo = *(const float4*)(E + row * LDE + cg * 8);
        const float4 hi = *(const float4*)(E + row * LDE + cg * 8 + 4);
        if (mode == 2) {
          float4* d = (float4*)(p.skp + (int64_t)oidx * (BM * BN) + (pass * EROWS + row) * BN + cg * 8);
          d[0] = lo;
          d[1] = hi;
        } else if (m < p.M && n < p.N) {
          const float vv[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          if (mode == 1)
            store8_partial(p, oidx, m, n, vv);
          else
            epi_finish8<EPI>(p, m, n, vv, sa[i], sb[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < GPT; ++i) {
        sa[i] = na[i];
        sb[i] = nb[i];
      }
    }
  }
}

// Stream-K tiles shared by several workgroups: add their slots in k order (workgroup order) and
// run the epilogue.  Grid: (stream-K tiles, BM / 32 row bands); G = the main kernel's grid size.
template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void sk_fixup_kernel(GemmParams p, int G) {
  constexpr int ROWS = 32, CPR = BN / 8, RSTEP = 256 / CPR, GPT = ROWS / RSTEP;
  const int st = blockIdx.x;
  const int64_t n_it = (int64_t)p.sk_tiles * p.ipt;
  const int64_t b = (int64_t)st * p.ipt, e = b + p.ipt;
  // owner(i) = the workgroup whose range [v * n_it / G, (v + 1) * n_it / G) holds iteration i
  const int g0 = (int)(((b + 1) * G + n_it - 1) / n_it - 1);
  const int g1 = (int)((e * G + n_it - 1) / n_it - 1);
  if (g0 == g1) return;  // one workgroup covered the whole tile and finished it
  const int t = p.dp_tiles + st;
  int tm, tn;
  tile_coords(p, t, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int cg = threadIdx.x % CPR, rsub = threadIdx.x / CPR;
  const int n = n0 + cg * 8;
  const int rfirst = blockIdx.y * ROWS + rsub;
  uint4 sa[GPT], sb[GPT];
  prefetch_side<EPI, GPT>(p, m0 + rfirst, RSTEP, n, sa, sb);
  float acc[GPT][8];
#pragma unroll
  for (int i = 0; i < GPT; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[i][q] = 0.f;
  for (int g = g0; g <= g1; ++g) {
    // the tile is slot 1 (last piece) of a range that began in an earlier tile, else slot 0
    const int slot = 2 * g + (((int64_t)g * n_it / G) < b ? 1 : 0);
    const float* src = p.skp + (int64_t)slot * (BM * BN) + cg * 8;
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const float4 lo = *(const float4*)(src + (rfirst + i * RSTEP) * BN);
      const float4 hi = *(const float4*)(src + (rfirst + i * RSTEP) * BN + 4);
      acc[i][0] += lo.x; acc[i][1] += lo.y; acc[i][2] += lo.z; acc[i][3] += lo.w;
      acc[i][4] += hi.x; acc[i][5] += hi.y; acc[i][6] += hi.z; acc[i][7] += hi.w;
    }
  }
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int m = m0 + rfirst + i * RSTEP;
    if (m < p.M && n < p.N) epi_finish8<EPI>(p, m, n, acc[i], sa[i], sb[i]);
  }
}

// Sum of the K-split partials in split order (deterministic), 8 outputs per thread, then the
// epilogue.  N is a multiple of 8.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmParams p, int splits) {
  const int64_t total = (int64_t)p.M * p.N;
  const int64_t groups = total / 8;
  for (int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x; gi < groups;
       gi += (int64_t)gridDim.x * 256) {
    const int64_t e = gi * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < splits; ++k) {
      const float4* src = (const float4*)(p.partial + k * total + e);
      const float4 a = src[0], b = src[1];
      s[0] += a.x; s[1] += a.y; s[2] += a.z; s[3] += a.w;
      s[4] += b.x; s[5] += b.y; s[6] += b.z; s[7] += b.w;
    }
    epi_store8<EPI>(p, (int)(e / p.N), (int)(e % p.N), s);
  }
}

// ------------------------------------------------------------------------------------------
// host side: configuration choice and launch
// ------------------------------------------------------------------------------------------
namespace {

constexpr int kBK = 64;
constexpr int kMaxDevices = 64;

// per host thread: one thread's choice does not change another thread's launches
thread_local int t_policy = 0;

// Raises a kernel's dynamic-LDS limit once per device (the call costs microseconds of host time,
// and every launch would otherwise repeat it).
void set_lds_limit_once(const void* kern, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return;
  }
  const uint64_t bit = 1ull << dev;
  if (done.load(std::memory_order_acquire) & bit) return;
  if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess)
    done.fetch_or(bit, std::memory_order_acq_rel);
}

// Compute units of the current device, read once per device.
int cu_count() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Tile shapes and the time one workgroup spends per 64-deep k-tile on MI355X with the whole chip
// busy, in microseconds, measured on the linear backward's GEMMs: t_k with A K-major (dX: B read
// through the transposing LDS read), t_mn with both operands token-major (dW: both transposed, so
// the narrow tiles are bound by LDS bandwidth).  160 / 192 / 224-row tiles (K-major A only) let a
// ragged token count fill the CUs: with N = 2048, M' = 4916 makes 160 tiles of 256 rows but 248
// of 160.
struct TileCfg {
  int bm, bn;
  double t_k, t_mn;
};
constexpr TileCfg kCfgs[] = {{256, 256, 1.62, 1.80}, {256, 128, 1.01, 1.45}, {128, 256, 1.14, 1.37},
                             {128, 128, 0.69, 0.91}, {160, 256, 1.21, 0.0},  {192, 256, 1.44, 0.0},
                             {224, 256, 1.54, 0.0}};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

// Direct-to-LDS pipeline of each tile shape: k-tile depth KT and stage count NS, within the
// 160 KB of LDS a workgroup may hold (NS * (BM + BN) * KT * 2 bytes).  Every shape keeps 64-deep
// k-tiles: 32-deep ones with four stages for the 192- and 256-row tiles (the same prefetch distance
// in bytes, finer grained) measured 5-15% slower on MI355X, the extra barrier and loop overhead per
// MFMA outweighing the deeper pipeline.
constexpr int lds_kt(int, int) { return 64; }
constexpr int lds_ns(int bm, int bn) {
  return (bn == 256 && (bm == 256 || bm == 224 || bm == 192)) ? 2 : 3;
}

struct Plan {
  int cfg, bm, bn;
  bool lds;        // direct-to-LDS kernel (gemm_lds_kernel) or the register-staged one
  int splits, k_split;
  int dp_tiles, sk_tiles, ipt, grid;
  double cost;     // estimated microseconds
};

// The direct-to-LDS kernel needs whole 64-wide k-tiles along every K-contiguous operand row
// (buffer loads only zero-fill past the end of a buffer) and 32-bit byte offsets.
bool lds_eligible(const GemmProblem& p) {
  const int64_t kpad = ((int64_t)p.K + kBK - 1) / kBK * kBK;
  if (p.a_kmajor && p.K % kBK && !(p.a_kpad && p.lda >= kpad)) return false;
  if (p.b_kmajor && p.K % kBK && !(p.b_kpad && p.ldb >= kpad)) return false;
  if (p.B1 && p.kseg % kBK) return false;
  const int64_t a_rows = p.a_kmajor ? p.M : p.K, b_rows = p.b_kmajor ? p.N : p.K;
  return a_rows * p.lda * 2 < (1ll << 31) && b_rows * p.ldb * 2 < (1ll << 31);
}

// HBM bytes the epilogue moves per output element besides the accumulator.  The plan must not
// depend on `accumulate` (workspace sizes are queried without it), so its extra read is left out.
double epi_bytes(const GemmProblem& p) {
  switch (p.epi) {
    case EPI_BF16: return 2.0;
    case EPI_F32: return 4.0;
    case EPI_SWIGLU: return 8.0;  // gate, up in; dgate, dup out
    default: return 4.0;          // f in, dF out
  }
}

// Cost model (microseconds): waves of workgroups, each running its k-tiles and its epilogue at an
// equal share of HBM bandwidth; K-split partials cost a write and a read-back; stream-K costs two
// partial tiles per workgroup, a fix-up pass over them and one more launch.
Plan make_plan(const GemmProblem& p) {
  const int ncu = cu_count();
  const bool lds = lds_eligible(p);
  int policy = t_policy;
  if (policy == 0 && p.concurrent) policy = 3;
  const double bw = 8.0e6, bw_cu = bw / ncu;  // bytes per microsecond
  const double eb = epi_bytes(p);
  Plan best{};
  best.cost = 1e300;
  if (p.K <= 0) {  // empty reduction: the kernel stores zeros (or leaves C + 0)
    const int T = ((p.M + 127) / 128) * ((p.N + 127) / 128);
    return Plan{3, 128, 128, lds, 1, kBK, T, 0, 0, T, 0.0};
  }
  // tuning override: COLLIDER_GEMM_TILE=<rows>x<cols> restricts the plan to that tile shape
  // wherever it applies
  static const int force_tile = [] {
    const char* e = getenv("COLLIDER_GEMM_TILE");
    int r = 0, c = 0;
    return (e && sscanf(e, "%dx%d", &r, &c) == 2) ? r * 1000 + c : 0;
  }();
  // 256 x 256 only in the direct-to-LDS kernel (staged through registers it would spill)
  for (int pass = 0; pass < 2 && best.cost >= 1e300; ++pass)  // pass 1: the override does not apply
  for (int c = lds ? 0 : 1; c < kNumCfgs; ++c) {
    if (c >= 4 && !(lds && p.a_kmajor)) continue;  // row counts other than 128 / 256: K-major A
    if (pass == 0 && force_tile && force_tile != kCfgs[c].bm * 1000 + kCfgs[c].bn) continue;
    const TileCfg tc = kCfgs[c];
    const int kt = lds ? lds_kt(tc.bm, tc.bn) : kBK;
    const int ipt = (p.K + kt - 1) / kt;  // k-tiles per output tile, in the kernel's k-tile depth
    const double t_it = (p.a_kmajor ? tc.t_k : tc.t_mn) * (lds ? 1.0 : 1.5);
    const int per_cu = (!lds && c == 3) ? 2 : 1;  // LDS-limited residency
    const long tiles = (long)((p.M + tc.bm - 1) / tc.bm) * ((p.N + tc.bn - 1) / tc.bn);
    const double epi_tile = tc.bm * tc.bn * eb / bw_cu, part_tile = tc.bm * tc.bn * 4.0 / bw_cu;
    if (policy != 2 || !lds) {
      for (int splits = 1; splits <= (policy == 3 ? 1 : 8); ++splits) {
        int ks = (p.K + splits - 1) / splits;
        ks = (ks + kBK - 1) / kBK * kBK;
        if ((p.K + ks - 1) / ks != splits) continue;
        const long items = tiles * splits;
        const long slots = (long)ncu * per_cu;
        const long waves = (items + slots - 1) / slots;
        double cost = (double)waves * per_cu * ((ks / kBK) * t_it + (splits > 1 ? part_tile : epi_tile));
        if (splits > 1) cost += ((double)splits * p.M * p.N * 4.0 + (double)p.M * p.N * eb) / bw + 4.0;
        if (cost < best.cost * 0.98)
          best = Plan{c, tc.bm, tc.bn, lds, splits, ks, (int)tiles, 0, ipt, (int)items, cost};
      }
    }
    if (lds && policy != 1 && policy != 3 && (tiles % ncu != 0 || policy == 2)) {
      const long dp = tiles >= 2L * ncu ? (tiles / ncu - 1) * ncu : 0;
      const long sk = tiles - dp;
      const long n_it = sk * ipt;
      const long grid = n_it < ncu ? n_it : ncu;
      const double per_wg = (double)((n_it + grid - 1) / grid) * kt / kBK;
      // A stream-K k-tile costs kSkSlow times a whole tile's: measured on MI355X with 256 x 256
      // tiles, the dX GEMM of the TinyLlama gate/up projection (M' 4916, K 11264) took 273 us + a
      // 57 us fix-up as stream-K (110 k-tiles per workgroup: 2.5 us each) against 186 us in whole
      // 160-row tiles, and the LM head's dh' (K 32000) 0.73 ms against 0.55 ms.
      constexpr double kSkSlow = 1.6;
      const double cost = (double)dp / grid * ((double)ipt * kt / kBK * t_it + epi_tile) + per_wg * t_it * kSkSlow +
                          (double)sk / grid * epi_tile + 2.0 * part_tile +
                          2.0 * grid * tc.bm * tc.bn * 4.0 / bw + 4.0;
      if (cost < best.cost * 0.98)
        best = Plan{c, tc.bm, tc.bn, lds, 1, ipt * kt, (int)dp, (int)sk, ipt, (int)grid, cost};
    }
  }
  return best;
}

size_t plan_workspace(const GemmProblem& p, const Plan& pl) {
  if (pl.sk_tiles > 0) return (size_t)2 * pl.grid * pl.bm * pl.bn * sizeof(float);
  if (pl.splits > 1) return (size_t)pl.splits * p.M * p.N * sizeof(float);
  return 0;
}

template <int BM, int BN, int EPI, bool AK, bool BKM>
collider_status launch_lds(const GemmParams& gp, int grid, const char* name, hipStream_t s) {
  constexpr int KT = lds_kt(BM, BN), NS = lds_ns(BM, BN);
  const size_t lds = (size_t)NS * (BM + BN) * KT * sizeof(uint16_t);
  static_assert(NS * (BM + BN) * KT * 2 <= 160 * 1024, "LDS budget");
  auto kern = gemm_lds_kernel<BM, BN, KT, AK, BKM, EPI, NS>;
  static std::atomic<uint64_t> attr_set{0};  // devices whose LDS limit is raised for this kernel
  set_lds_limit_once((const void*)kern, (int)lds, attr_set);
  COLLIDER_LAUNCH(name, s,
                  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * lds_waves(BM, BN)), lds, s, gp));
  collider_status st = last_hip_status();
  if (st != COLLIDER_OK || gp.sk_tiles == 0) return st;
  COLLIDER_LAUNCH("gemm_sk_fixup", s,
                  hipLaunchKernelGGL((sk_fixup_kernel<BM, BN, EPI>), dim3(gp.sk_tiles, BM / 32),
                                     dim3(256), 0, s, gp, grid));
  return last_hip_status();
}

template <int BM, int BN, int EPI, bool AK, bool BKM>
collider_status launch_one(const GemmParams& gp, const char* name, hipStream_t s) {
  const int total = gp.tiles_m * gp.tiles_n * gp.splits;
  const size_t lds = 2 * (size_t)(BM + BN) * (kBK + 8) * sizeof(uint16_t);
  auto kern = gemm_bf16_kernel<BM, BN, kBK, AK, BKM, EPI>;
  static std::atomic<uint64_t> attr_set{0};
  set_lds_limit_once((const void*)kern, (int)lds, attr_set);
  COLLIDER_LAUNCH(name, s, hipLaunchKernelGGL(kern, dim3(total), dim3(256), lds, s, gp));
  return last_hip_status();
}

// Layout / epilogue combinations the linear backward uses: dX GEMMs (A K-major, B N-major) with a
// bf16 / SwiGLU / GELU epilogue; dW GEMMs (both operands token-major) with an fp32 epilogue.  Tile
// shapes exist where their operand layouts do: MN-major tiles of 128 or 256 rows, register-staged
// kernels for 128 / 256 shapes below 256 x 256.
template <int BM, int BN>
collider_status launch_cfg(const GemmParams& gp, const GemmProblem& pr, const Plan& pl,
                           const char* name, hipStream_t s) {
  constexpr bool kStaged = (BM == 128 || BM == 256) && !(BM == 256 && BN == 256);
  constexpr bool kMnA = BM % 128 == 0;
  if (pr.a_kmajor && !pr.b_kmajor) {
    switch (pr.epi) {
      case EPI_BF16:
        if (pl.lds) return launch_lds<BM, BN, EPI_BF16, true, false>(gp, pl.grid, name, s);
        if constexpr (kStaged) return launch_one<BM, BN, EPI_BF16, true, false>(gp, name, s);
        break;
      case EPI_SWIGLU:
        if (pl.lds) return launch_lds<BM, BN, EPI_SWIGLU, true, false>(gp, pl.grid, name, s);
        if constexpr (kStaged) return launch_one<BM, BN, EPI_SWIGLU, true, false>(gp, name, s);
        break;
      case EPI_GELU:
        if (pl.lds) return launch_lds<BM, BN, EPI_GELU, true, false>(gp, pl.grid, name, s);
        if constexpr (kStaged) return launch_one<BM, BN, EPI_GELU, true, false>(gp, name, s);
        break;
    }
  } else if (pr.a_kmajor && pr.b_kmajor) {
    // activation gradients with weights stored [in, out] (each weight row K-contiguous): both
    // operands read with 16-byte LDS reads
    switch (pr.epi) {
      case EPI_BF16:
        if (pl.lds) return launch_lds<BM, BN, EPI_BF16, true, true>(gp, pl.grid, name, s);
        if constexpr (kStaged) return launch_one<BM, BN, EPI_BF16, true, true>(gp, name, s);
        break;
      case EPI_SWIGLU:
        if (pl.lds) return launch_lds<BM, BN, EPI_SWIGLU, true, true>(gp, pl.grid, name, s);
        if constexpr (kStaged) return launch_one<BM, BN, EPI_SWIGLU, true, true>(gp, name, s);
        break;
      case EPI_GELU:
        if (pl.lds) return launch_lds<BM, BN, EPI_GELU, true, true>(gp, pl.grid, name, s);
        if constexpr (kStaged) return launch_one<BM, BN, EPI_GELU, true, true>(gp, name, s);
        break;
    }
  } else if (!pr.a_kmajor && !pr.b_kmajor && pr.epi == EPI_F32) {
    if constexpr (kMnA) {
      if (pl.lds) return launch_lds<BM, BN, EPI_F32, false, false>(gp, pl.grid, name, s);
      if constexpr (kStaged) return launch_one<BM, BN, EPI_F32, false, false>(gp, name, s);
    }
  }
  // weight gradients with one token-contiguous operand (the transposed normalised input /
  // activation): A = X^T (weights [in, out]) or B = X^T (weights [out, in]); direct-to-LDS only
  if (pr.epi == EPI_F32 && pl.lds) {
    if (pr.a_kmajor && !pr.b_kmajor) return launch_lds<BM, BN, EPI_F32, true, false>(gp, pl.grid, name, s);
    if constexpr (kMnA)
      if (!pr.a_kmajor && pr.b_kmajor) return launch_lds<BM, BN, EPI_F32, false, true>(gp, pl.grid, name, s);
  }
  return COLLIDER_ERR_UNSUPPORTED;
}

template <int EPI>
collider_status launch_reduce(const GemmParams& gp, const GemmProblem& prob, int splits,
                              hipStream_t s) {
  const int64_t total = (int64_t)prob.M * prob.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  COLLIDER_LAUNCH("gemm_splitk_reduce", s,
                  hipLaunchKernelGGL(splitk_reduce_kernel<EPI>, dim3((unsigned)blocks), dim3(256),
                                     0, s, gp, splits));
  return last_hip_status();
}

// Tile rows per group of the tile numbering (tile_coords): the power of two that makes the block
// of tiles one XCD runs at a time (about 32, one per CU) read the fewest operand bytes per k-step,
// gm row panels of A (bm rows each) plus ceil(c / gm) column panels of B (bn columns each).
int tile_group_rows(int tiles_m, int tiles_n, int bm, int bn) {
  const int total = tiles_m * tiles_n;
  const int c = std::max(1, std::min(32, (total + 7) / 8));
  int best = 1;
  double best_cost = 1e30;
  for (int gm = 1; gm <= tiles_m; gm *= 2) {
    // c consecutive tiles: within one group, min(gm, c) rows x ceil(c / gm) columns; past a
    // group's gm * tiles_n tiles, whole groups of every column
    const int per_group = gm * tiles_n;
    const int rows = c <= per_group ? std::min(gm, c)
                                    : std::min(tiles_m, gm * ((c + per_group - 1) / per_group));
    const int cols = c <= per_group ? (c + gm - 1) / gm : tiles_n;
    const double cost = (double)rows * bm + (double)cols * bn;
    if (cost < best_cost) {
      best_cost = cost;
      best = gm;
    }
  }
  return best;
}

}  // namespace

void gemm_set_policy(int policy) { t_policy = policy; }

void gemm_describe_plan(const GemmProblem& p, int* out) {
  const Plan pl = make_plan(p);
  const int v[7] = {pl.bm, pl.bn, pl.splits, pl.dp_tiles, pl.sk_tiles, pl.grid, pl.lds ? 1 : 0};
  for (int i = 0; i < 7; ++i) out[i] = v[i];
}

size_t gemm_bf16_workspace_bytes(const GemmProblem& p) {
  if (p.M <= 0 || p.N <= 0 || p.K <= 0) return 0;
  return plan_workspace(p, make_plan(p));
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
  gp.splits = pl.splits;
  gp.tiles_m = (prob.M + pl.bm - 1) / pl.bm;
  gp.tiles_n = (prob.N + pl.bn - 1) / pl.bn;
  gp.group_m = tile_group_rows(gp.tiles_m, gp.tiles_n, pl.bm, pl.bn);
  gp.ipt = pl.ipt;
  gp.dp_tiles = pl.dp_tiles;
  gp.sk_tiles = pl.sk_tiles;
  gp.C = prob.C;
  gp.ldc = prob.ldc;
  gp.accumulate = prob.accumulate;
  gp.g = prob.g;
  gp.up = prob.up;
  gp.ld_g = prob.ld_g;
  gp.rowmap = prob.rowmap;
  gp.out2 = prob.out2;
  gp.ld_out2 = prob.ld_out2;
  const size_t need = plan_workspace(prob, pl);
  if (need) {
    if (!ws || ws_bytes < need) return COLLIDER_ERR_WORKSPACE;
    if (pl.sk_tiles > 0)
      gp.skp = (float*)ws;
    else
      gp.partial = (float*)ws;
  }
  // every stream-K workgroup must own at least one k-tile (the fix-up reads each owner's slot),
  // and the work items must cover every tile exactly once
  if (pl.sk_tiles > 0 && ((int64_t)pl.sk_tiles * pl.ipt < pl.grid || pl.splits != 1))
    return COLLIDER_ERR_UNSUPPORTED;
  if (pl.dp_tiles + pl.sk_tiles != gp.tiles_m * gp.tiles_n) return COLLIDER_ERR_UNSUPPORTED;
  const char* name = prob.name ? prob.name : "gemm_bf16";
  static const bool verbose = getenv("COLLIDER_GEMM_PLANS") != nullptr;
  if (verbose)
    fprintf(stderr,
            "[collider] %s M=%d N=%d K=%d tile=%dx%d splits=%d dp_tiles=%d sk_tiles=%d grid=%d "
            "est=%.1fus %s\n",
            name, prob.M, prob.N, prob.K, pl.bm, pl.bn, pl.splits, pl.dp_tiles, pl.sk_tiles,
            pl.grid, pl.cost, pl.lds ? "lds" : "staged");
  collider_status st;
  switch (pl.cfg) {
    case 0:
      if (!pl.lds) return COLLIDER_ERR_UNSUPPORTED;
      st = launch_cfg<256, 256>(gp, prob, pl, name, s);
      break;
    case 1: st = launch_cfg<256, 128>(gp, prob, pl, name, s); break;
    case 2: st = launch_cfg<128, 256>(gp, prob, pl, name, s); break;
    case 4: st = launch_cfg<160, 256>(gp, prob, pl, name, s); break;
    case 5: st = launch_cfg<192, 256>(gp, prob, pl, name, s); break;
    case 6: st = launch_cfg<224, 256>(gp, prob, pl, name, s); break;
    default: st = launch_cfg<128, 128>(gp, prob, pl, name, s); break;
  }
  if (st != COLLIDER_OK || pl.splits == 1) return st;
  switch (prob.epi) {
    case EPI_BF16: return launch_reduce<EPI_BF16>(gp, prob, pl.splits, s);
    case EPI_F32: return launch_reduce<EPI_F32>(gp, prob, pl.splits, s);
    case EPI_SWIGLU: return launch_reduce<EPI_SWIGLU>(gp, prob, pl.splits, s);
    default: return launch_reduce<EPI_GELU>(gp, prob, pl.splits, s);
  }
}


// ------------------------------------------------------------------------------------------
// fp32 GEMM (vector-ALU FMA, 64x64 tiles, 4x4 outputs per thread) for the fp32 linear backward
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
