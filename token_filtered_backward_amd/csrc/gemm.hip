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
      const float s = 1.f / (1.f + __expf(-g[e]));
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
      const float t = tanhf(c * (f[e] + a * f[e] * f[e] * f[e]));
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
// LDS directly (no staging registers), so 3 k-tiles can be in flight.  Buffer loads are range
// checked: rows past the end of an operand (the ragged token dimension) arrive as zeros.
// Each operand keeps its global orientation in LDS, XOR-swizzled instead of padded:
//   K-major tile  [R][64]  128-byte rows, 16-byte chunk c of row r stored at c ^ ((r >> 1) & 7)
//   MN-major tile [64][R]  2R-byte rows,  chunk c of row k stored at c ^ (4 * (k & 3))
// MFMA fragments come from ds_read_b128 (K-major) or two ds_read_b64_tr_b16 (MN-major): within a
// group of 16 lanes, lane j addresses row k0 + j/4, columns n + 4*(j%4) .. +3, and lane i receives
// rows k0 .. k0+3 of column n + i - exactly the k-contiguous operand layout the MFMA expects.
// Both swizzles make the 16-lane (K-major) and 32-lane (MN-major) read groups bank-conflict free.
// ------------------------------------------------------------------------------------------
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int kmaj_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }
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

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// 16-byte buffer load of each lane straight into LDS (M0 = LDS base of the wave, lane i lands at
// M0 + 16*i).  Issued as inline assembly: the compiler then inserts no waits for it of its own
// (it cannot tell which LDS bytes the copy writes and would wait for every outstanding load at
// each LDS read); completion is tracked explicitly with s_waitcnt vmcnt in the k-loop.
__device__ __forceinline__ void dma16(rsrc_t rs, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rs)
               : "memory", "m0");
}

// Issue the direct loads of one [R x 64] (K-major) or [64 x R] (MN-major) tile; wave w issues
// instructions w, w+4, ...  `row0` is the first tile row (token or feature index of the operand
// rows), `col0` the first column.  Byte offsets are relative to the buffer base.
template <int R, bool KMAJ>
__device__ __forceinline__ void issue_tile(rsrc_t rs, int64_t ld, int row0, int col0,
                                           char* lds_tile, int wave, int lane) {
  constexpr int NI = R * 64 * 2 / 1024;
#pragma unroll
  for (int q = wave; q < NI; q += 4) {
    const int b = q * 1024 + lane * 16;
    uint32_t off;
    if constexpr (KMAJ) {
      const int r = b >> 7, pos = (b >> 4) & 7;
      const int c = pos ^ ((r >> 1) & 7);
      off = (uint32_t)(((int64_t)(row0 + r) * ld + col0 + 8 * c) * 2);
    } else {
      const int k = b / (2 * R), pos = (b % (2 * R)) >> 4;
      const int c = pos ^ ((k & 3) << 2);
      off = (uint32_t)(((int64_t)(row0 + k) * ld + col0 + 8 * c) * 2);
    }
    dma16(rs, lds_addr(lds_tile + q * 1024), off);
  }
}

// 32x32x16 operand fragment: rows rbase .. rbase+31 (M or N index), k = kk*16 .. +15
template <int R, bool KMAJ>
__device__ __forceinline__ bf16x8 read_frag(const char* lds_tile, int rbase, int kk, int lane) {
  if constexpr (KMAJ) {
    const int r = rbase + (lane & 31), c = kk * 2 + (lane >> 5);
    return *(const bf16x8*)(lds_tile + kmaj_off(r, c));
  } else {
    const int g = lane >> 4, j = lane & 15;
    const int col = rbase + 16 * (g & 1) + 4 * (j & 3);
    const int kb = kk * 16 + 8 * (g >> 1) + (j >> 2);
    const int c = col >> 3, within = (col & 7) * 2;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (v4s __attribute__((address_space(3)))*)(lds_tile + mnmaj_off<R>(kb, c) + within));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (v4s __attribute__((address_space(3)))*)(lds_tile + mnmaj_off<R>(kb + 4, c) + within));
    typedef short v8s __attribute__((ext_vector_type(8)));
    const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, both);
  }
}

// Loads of one k-tile (A then B) into one LDS stage.  B may come in two row segments (B0 for
// k < kseg, B1 after); a 64-row k-tile never straddles them.
template <int BM, int BN, bool AK, bool BKM>
__device__ __forceinline__ void issue_stage(rsrc_t ra, rsrc_t rb0, rsrc_t rb1, int64_t lda, int64_t ldb,
                                            int kseg, bool two_seg, int m0, int n0, int k0,
                                            char* stage, int wave, int lane) {
  if constexpr (AK)
    issue_tile<BM, true>(ra, lda, m0, k0, stage, wave, lane);
  else
    issue_tile<BM, false>(ra, lda, k0, m0, stage, wave, lane);
  const bool seg1 = two_seg && k0 >= kseg;
  const int kb = seg1 ? k0 - kseg : k0;
  char* bst = stage + BM * 64 * 2;
  if (seg1) {
    if constexpr (BKM)
      issue_tile<BN, true>(rb1, ldb, n0, kb, bst, wave, lane);
    else
      issue_tile<BN, false>(rb1, ldb, kb, n0, bst, wave, lane);
  } else {
    if constexpr (BKM)
      issue_tile<BN, true>(rb0, ldb, n0, kb, bst, wave, lane);
    else
      issue_tile<BN, false>(rb0, ldb, kb, n0, bst, wave, lane);
  }
}

// s_waitcnt vmcnt(n), other counters unconstrained (gfx9 encoding)
#define VMCNT_WAIT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xf) | (((n) >> 4) << 14) | (0x7 << 4) | (0xf << 8))

// MFMAs of one k-tile (4 steps of k = 16) from one LDS stage; fragments of step kk+1 are read
// while the MFMAs of step kk run (two register sets).
template <int BM, int BN, bool AK, bool BKM>
__device__ __forceinline__ void mma_ktile(const char* As, const char* Bs,
                                          f32x16 (&acc)[BM / 64][BN / 64], int wm, int wn,
                                          int lane) {
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  bf16x8 af[2][TM], bfv[2][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) af[0][i] = read_frag<BM, AK>(As, wm * WM + i * 32, 0, lane);
#pragma unroll
  for (int j = 0; j < TN; ++j) bfv[0][j] = read_frag<BN, BKM>(Bs, wn * WN + j * 32, 0, lane);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int cur = kk & 1;
    if (kk + 1 < 4) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[cur ^ 1][i] = read_frag<BM, AK>(As, wm * WM + i * 32, kk + 1, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfv[cur ^ 1][j] = read_frag<BN, BKM>(Bs, wn * WN + j * 32, kk + 1, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfv[cur][j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int BM, int BN, bool AK, bool BKM, int EPI, int NS>
__global__ __launch_bounds__(256) void gemm_lds_kernel(GemmParams p) {
  constexpr int BK = 64;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  constexpr int LPW = (A_BYTES + B_BYTES) / 1024 / 4;  // load instructions per wave per k-tile
  extern __shared__ __align__(16) char lds[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int T = p.tiles_m * p.tiles_n;
  const int total = T * p.splits;
  const bool partial = p.splits > 1;
  // operand buffers: rows of A are tokens (K-major A: M rows; MN-major A: K rows)
  const rsrc_t ra = make_rsrc(p.A, (uint32_t)((int64_t)(AK ? p.M : p.K) * p.lda * 2));
  const int kseg = p.B1 ? p.kseg : p.K;
  const bool two_seg = p.B1 != nullptr;
  const rsrc_t rb0 = make_rsrc(p.B0, (uint32_t)((int64_t)kseg * p.ldb * 2));
  const rsrc_t rb1 =
      make_rsrc(p.B1 ? p.B1 : p.B0, (uint32_t)((int64_t)(p.B1 ? p.K - kseg : 0) * p.ldb * 2));

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int li = xcd_remap(item, total);
    const int split = li / T, t = li % T;
    const int tm = t / p.tiles_n, tn = t % p.tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = split * p.k_split;
    const int kend = min(p.K, kbeg + p.k_split);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

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
      if (s < nk)
        issue_stage<BM, BN, AK, BKM>(ra, rb0, rb1, p.lda, p.ldb, kseg, two_seg, m0, n0,
                                     kbeg + s * BK, lds + s * STAGE, wave, lane);
    for (int kt = 0; kt < nk; ++kt) {
      // tile kt complete (for this wave), then visible to all waves
      if (kt + NS - 2 < nk) {
        VMCNT_WAIT(LPW * (NS - 2));
      } else {
        VMCNT_WAIT(0);
      }
      __syncthreads();
      if (kt + NS - 1 < nk)  // refills the stage read in iteration kt-1
        issue_stage<BM, BN, AK, BKM>(ra, rb0, rb1, p.lda, p.ldb, kseg, two_seg, m0, n0,
                                     kbeg + (kt + NS - 1) * BK, lds + ((kt + NS - 1) % NS) * STAGE,
                                     wave, lane);
      const char* As = lds + (kt % NS) * STAGE;
      mma_ktile<BM, BN, AK, BKM>(As, As + A_BYTES, acc, wm, wn, lane);
    }

    // epilogue through LDS: the fp32 tile is staged row-major in passes of EROWS rows, then every
    // thread finishes 8 consecutive columns of a row with 16-byte loads / stores (one row lookup
    // per 8 outputs)
    constexpr int LDE = BN + 8;  // +8 floats: the two lane halves' rows land 32 banks apart
    constexpr int EROWS = (BM * LDE * 4 <= NS * STAGE) ? BM : ((64 * LDE * 4 <= NS * STAGE) ? 64 : 32);
    static_assert(EROWS * LDE * 4 <= NS * STAGE, "epilogue pass must fit in the stage buffers");
    float* E = (float*)lds;
#pragma unroll
    for (int pass = 0; pass < BM / EROWS; ++pass) {
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
      for (int c = threadIdx.x; c < EROWS * (BN / 8); c += 256) {
        const int row = c / (BN / 8), col = (c % (BN / 8)) * 8;
        const int m = m0 + pass * EROWS + row, n = n0 + col;
        if (m >= p.M || n >= p.N) continue;
        const float4 lo = *(const float4*)(E + row * LDE + col);
        const float4 hi = *(const float4*)(E + row * LDE + col + 4);
        const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        if (partial)
          store8_partial(p, split, m, n, v);
        else
          epi_store8<EPI>(p, m, n, v);
      }
    }
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

constexpr int kCUs = 256;
constexpr int kBK = 64;

struct TileCfg {
  int bm, bn, per_cu;  // workgroups resident per CU (LDS-limited)
  double eff;          // relative MFMA efficiency of the tile shape (LDS bytes per MFMA)
};
constexpr TileCfg kCfgs[] = {{256, 256, 1, 1.00}, {256, 128, 1, 0.80}, {128, 256, 1, 0.80},
                             {128, 128, 2, 0.55}};

struct Plan {
  int cfg, bm, bn, splits, k_split;
  bool lds;  // direct-to-LDS kernel (gemm_lds_kernel) or the register-staged one
};

// The direct-to-LDS kernel needs whole 64-wide k-tiles along every K-contiguous operand row
// (buffer loads only zero-fill past the end of a buffer) and 32-bit byte offsets.
bool lds_eligible(const GemmProblem& p) {
  if (p.a_kmajor && p.K % kBK) return false;
  if (p.b_kmajor && p.K % kBK) return false;
  if (p.B1 && p.kseg % kBK) return false;
  const int64_t a_rows = p.a_kmajor ? p.M : p.K, b_rows = p.b_kmajor ? p.N : p.K;
  return a_rows * p.lda * 2 < (1ll << 31) && b_rows * p.ldb * 2 < (1ll << 31);
}

Plan make_plan(const GemmProblem& p) {
  const bool lds = lds_eligible(p);
  Plan best{3, 128, 128, 1, kBK, lds};
  if (p.K <= 0) return best;  // empty reduction: the kernel stores zeros (or leaves C + 0)
  double best_cost = 1e300;
  // 256 x 256 only in the direct-to-LDS kernel (staged through registers it would spill)
  for (int c = lds ? 0 : 1; c < 4; ++c) {
    TileCfg tc = kCfgs[c];
    if (lds && c == 3) tc.per_cu = 1;  // three 32 KB stages
    if (lds && (c == 1 || c == 2)) tc.eff = 0.85;
    const long tiles = (long)((p.M + tc.bm - 1) / tc.bm) * ((p.N + tc.bn - 1) / tc.bn);
    for (int splits = 1; splits <= 8; ++splits) {
      int ks = (p.K + splits - 1) / splits;
      ks = (ks + kBK - 1) / kBK * kBK;
      if ((p.K + ks - 1) / ks != splits) continue;
      const long items = tiles * splits;
      const long slots = (long)kCUs * tc.per_cu;
      const long waves = (items + slots - 1) / slots;
      // one wave: every resident workgroup computes a bm x bn x ks tile; a CU shares its
      // throughput between its per_cu workgroups
      double cost = (double)waves * tc.per_cu * tc.bm * tc.bn * ks / tc.eff;
      // split partials: written once, read once by the reduction (in MFMA-time units)
      if (splits > 1) cost += (double)splits * p.M * p.N * 8.0 * 64.0 / kCUs;
      if (cost < best_cost * 0.98) {
        best_cost = cost;
        best = Plan{c, tc.bm, tc.bn, splits, ks, lds};
      }
    }
  }
  return best;
}

template <int BM, int BN, int EPI, bool AK, bool BKM>
collider_status launch_lds(const GemmParams& gp, const char* name, hipStream_t s) {
  constexpr int NS = (BM == 256 && BN == 256) ? 2 : 3;
  const int total = gp.tiles_m * gp.tiles_n * gp.splits;
  const size_t lds = (size_t)NS * (BM + BN) * kBK * sizeof(uint16_t);
  auto kern = gemm_lds_kernel<BM, BN, AK, BKM, EPI, NS>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  COLLIDER_LAUNCH(name, s, hipLaunchKernelGGL(kern, dim3(total), dim3(256), lds, s, gp));
  return last_hip_status();
}

template <int BM, int BN, int EPI, bool AK, bool BKM>
collider_status launch_one(const GemmParams& gp, const char* name, hipStream_t s) {
  const int total = gp.tiles_m * gp.tiles_n * gp.splits;
  const size_t lds = 2 * (size_t)(BM + BN) * (kBK + 8) * sizeof(uint16_t);
  auto kern = gemm_bf16_kernel<BM, BN, kBK, AK, BKM, EPI>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  COLLIDER_LAUNCH(name, s, hipLaunchKernelGGL(kern, dim3(total), dim3(256), lds, s, gp));
  return last_hip_status();
}

// Layout / epilogue combinations the linear backward uses: dX GEMMs (A K-major, B N-major) with a
// bf16 / SwiGLU / GELU epilogue; dW GEMMs (both operands token-major) with an fp32 epilogue.
template <int BM, int BN>
collider_status launch_cfg(const GemmParams& gp, const GemmProblem& pr, bool lds, const char* name,
                           hipStream_t s) {
  if (pr.a_kmajor && !pr.b_kmajor) {
    switch (pr.epi) {
      case EPI_BF16:
        return lds ? launch_lds<BM, BN, EPI_BF16, true, false>(gp, name, s)
                   : launch_one<BM, BN, EPI_BF16, true, false>(gp, name, s);
      case EPI_SWIGLU:
        return lds ? launch_lds<BM, BN, EPI_SWIGLU, true, false>(gp, name, s)
                   : launch_one<BM, BN, EPI_SWIGLU, true, false>(gp, name, s);
      case EPI_GELU:
        return lds ? launch_lds<BM, BN, EPI_GELU, true, false>(gp, name, s)
                   : launch_one<BM, BN, EPI_GELU, true, false>(gp, name, s);
    }
  } else if (!pr.a_kmajor && !pr.b_kmajor && pr.epi == EPI_F32) {
    return lds ? launch_lds<BM, BN, EPI_F32, false, false>(gp, name, s)
               : launch_one<BM, BN, EPI_F32, false, false>(gp, name, s);
  }
  return COLLIDER_ERR_UNSUPPORTED;
}

// 256 x 256 exists only as a direct-to-LDS kernel (the register-staged one would spill)
template <int BM, int BN>
collider_status launch_cfg_lds(const GemmParams& gp, const GemmProblem& pr, const char* name,
                               hipStream_t s) {
  if (pr.a_kmajor && !pr.b_kmajor) {
    switch (pr.epi) {
      case EPI_BF16: return launch_lds<BM, BN, EPI_BF16, true, false>(gp, name, s);
      case EPI_SWIGLU: return launch_lds<BM, BN, EPI_SWIGLU, true, false>(gp, name, s);
      case EPI_GELU: return launch_lds<BM, BN, EPI_GELU, true, false>(gp, name, s);
    }
  } else if (!pr.a_kmajor && !pr.b_kmajor && pr.epi == EPI_F32) {
    return launch_lds<BM, BN, EPI_F32, false, false>(gp, name, s);
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
  gp.splits = pl.splits;
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
  const char* name = prob.name ? prob.name : "gemm_bf16";
  static const bool verbose = getenv("COLLIDER_GEMM_PLANS") != nullptr;
  if (verbose)
    fprintf(stderr, "[collider] %s M=%d N=%d K=%d tile=%dx%d splits=%d %s\n", name, prob.M, prob.N,
            prob.K, pl.bm, pl.bn, pl.splits, pl.lds ? "lds" : "staged");
  collider_status st;
  switch (pl.cfg) {
    case 0:
      if (!pl.lds) return COLLIDER_ERR_UNSUPPORTED;
      st = launch_cfg_lds<256, 256>(gp, prob, name, s);
      break;
    case 1: st = launch_cfg<256, 128>(gp, prob, pl.lds, name, s); break;
    case 2: st = launch_cfg<128, 256>(gp, prob, pl.lds, name, s); break;
    default: st = launch_cfg<128, 128>(gp, prob, pl.lds, name, s); break;
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
