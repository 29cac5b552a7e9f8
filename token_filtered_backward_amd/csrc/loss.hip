// Loss side of the filtered backward (Collider paper, Figure 2(b): the per-token training loss
// decides which tokens are filtered, and a filtered token's loss is dropped, so it sends no
// gradient into the LM head, the layers or the token embedding):
//   ce_loss_kernel          per-token cross-entropy loss of every token (the score to rank by)
//   select_topk_kernel      per-token scores -> keep mask (the n_keep largest scores kept)
//   ce_grad_kernel          dlogits' = scale * (softmax(logits') - onehot(label')) over kept rows
//   embed_*_kernel          dE[v] = sum of dx over the kept tokens with id v, in token order
// The LM head's two reduced GEMMs reuse the bf16 GEMM (gemm.hip).
#include <atomic>
#include <mutex>

#include <algorithm>
#include <type_traits>

#include "internal.h"

namespace collider {

// ------------------------------------------------------------------------------------------
// top-k selection: one workgroup, radix select on 32-bit order-preserving keys
// ------------------------------------------------------------------------------------------
// Larger score -> larger key; -0.0 ranks as +0.0; NaN ranks below every number (key 0, below
// -inf's 0x007fffff).
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (x != x) return 0u;
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

constexpr int kSelThreads = 1024;

// keep[t] = 1 for the n_keep tokens of largest score (equal scores: lower t first), else 0.
// Four passes pick the threshold key byte by byte from the top (a 256-bin histogram of the keys
// that match the bytes chosen so far); a last pass keeps every key above the threshold and the
// first `need` keys equal to it in token order (a block-wide running count).
// CACHE: the scores of M <= kSelThreads * kSelCached tokens are loaded once, all loads in flight,
// and kept in registers through the passes.  (Re-reading them every pass into one shared
// histogram took 24 us for 8192 tokens; this form takes 19 us.)
constexpr int kSelCached = 8;
template <bool CACHE>
__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(const float* __restrict__ score,
                                                                  int M, int n_keep,
                                                                  uint8_t* __restrict__ keep) {
  // a histogram per wavefront (atomics of different wavefronts never collide; most keys share
  // their top bytes, and one shared histogram serialised every atomic of the pass on a few bins)
  __shared__ uint32_t hist[kSelThreads / 64][256];
  __shared__ uint32_t s_sel[2];
  __shared__ uint32_t s_wsum[kSelThreads / 64];
  __shared__ uint32_t s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n_keep <= 0 || n_keep >= M) {
    const uint8_t v = n_keep <= 0 ? 0 : 1;
    for (int t = tid; t < M; t += kSelThreads) keep[t] = v;
    return;
  }
  uint32_t kc[CACHE ? kSelCached : 1];
  if constexpr (CACHE) {
#pragma unroll
    for (int q = 0; q < kSelCached; ++q) {
      const int t = tid + kSelThreads * q;
      kc[q] = t < M ? score_key(score[t]) : 0u;
    }
  }
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)n_keep;
  for (int d = 3; d >= 0; --d) {
    for (int i = tid; i < 256 * (kSelThreads / 64); i += kSelThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    // a thread adds its run of equal bins with one atomic (a wavefront's lanes still share bins)
    uint32_t cur = 0u, run = 0u;
    auto count = [&](uint32_t k) {
      if ((k & pmask) != prefix) return;
      const uint32_t b = (k >> (8 * d)) & 255u;
      if (run && b != cur) {
        atomicAdd(&hist[wave][cur], run);
        run = 0u;
      }
      cur = b;
      ++run;
    };
    if constexpr (CACHE) {
#pragma unroll
      for (int q = 0; q < kSelCached; ++q)
        if (tid + kSelThreads * q < M) count(kc[q]);
    } else {
      for (int t = tid; t < M; t += kSelThreads) count(score_key(score[t]));
    }
    if (run) atomicAdd(&hist[wave][cur], run);
    __syncthreads();
    if (tid < 256) {  // the wavefronts' histograms summed into the first
      uint32_t tot = 0;
#pragma unroll
      for (int w = 0; w < kSelThreads / 64; ++w) tot += hist[w][tid];
      hist[0][tid] = tot;
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 255 - 4l - q (q = 0..3), i.e. the bins in descending order
      uint32_t loc[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        loc[q] = hist[0][255 - 4 * lane - q];
        sum += loc[q];
      }
      uint32_t incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      const uint32_t excl = incl - sum;
      if (excl < need && need <= incl) {  // exactly one lane: the total is at least `need`
        uint32_t acc = excl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (acc + loc[q] >= need) {
            s_sel[0] = (uint32_t)(255 - 4 * lane - q);
            s_sel[1] = need - acc;
            break;
          }
          acc += loc[q];
        }
      }
    }
    __syncthreads();
    prefix |= s_sel[0] << (8 * d);
    need = s_sel[1];
    pmask |= 255u << (8 * d);
    __syncthreads();  // s_sel is rewritten by the next pass
  }
  // prefix is now the threshold key T; keep keys > T and the first `need` keys == T
  const uint32_t T = prefix;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  constexpr int PER = 8;
  for (int base = 0; base < M; base += kSelThreads * PER) {
    const int t0 = base + tid * PER;
    uint32_t kk[PER], eq = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      kk[q] = t0 + q < M ? score_key(score[t0 + q]) : 0u;
      eq += (t0 + q < M && kk[q] == T) ? 1u : 0u;
    }
    uint32_t incl = eq;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    uint32_t before = s_carry + incl - eq;
    for (int w = 0; w < wave; ++w) before += s_wsum[w];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      if (t0 + q >= M) break;
      bool kp = kk[q] > T;
      if (kk[q] == T) {
        kp = before < need;
        ++before;
      }
      keep[t0 + q] = kp ? 1 : 0;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t tot = 0;
      for (int w = 0; w < kSelThreads / 64; ++w) tot += s_wsum[w];
      s_carry += tot;
    }
    __syncthreads();
  }
}

collider_status launch_select_topk(const float* score, int M, int n_keep, uint8_t* keep,
                                   hipStream_t s) {
  if (M <= 0) return COLLIDER_OK;
  if (M <= kSelThreads * kSelCached)
    COLLIDER_LAUNCH("select_topk", s,
                    hipLaunchKernelGGL(select_topk_kernel<true>, dim3(1), dim3(kSelThreads), 0, s, score,
                                       M, n_keep, keep));
  else
    COLLIDER_LAUNCH("select_topk", s,
                    hipLaunchKernelGGL(select_topk_kernel<false>, dim3(1), dim3(kSelThreads), 0, s, score,
                                       M, n_keep, keep));
  return last_hip_status();
}

// ------------------------------------------------------------------------------------------
// top-k selection over many workgroups (large token counts): the same radix select, the same
// result bit for bit.  Each pass is two launches: every workgroup histograms the keys of its
// contiguous chunk of tokens that match the bytes chosen so far (sel_hist_kernel), then one
// workgroup adds the histograms in workgroup order and picks the next byte (sel_choose_kernel).
// After the fourth pass every workgroup counts the keys equal to the threshold in its chunk
// (sel_eqcount_kernel), and the last launch writes the mask: keys above the threshold, and the
// first `need` equal keys in token order, each workgroup starting from the equal keys of the
// chunks before its own (sel_mark_kernel).  Workspace (uint32, 16-byte aligned): the state
// {prefix, byte mask, need} in 4 words, Gp words of equal-key counts (one per workgroup; Gp = the
// workgroup count rounded up to 4), then the histograms bin-major ([256][Gp]), so that the
// choosing workgroup reads each bin's counts with 16-byte loads, four threads per bin.  (Workgroup-major histograms read one count per load and
// per thread made the four choosing launches take most of the selection's time.)
// ------------------------------------------------------------------------------------------
constexpr int kSelMT = 256;          // threads per workgroup
constexpr int kSelSub = 4096;        // tokens per workgroup and step (16 per thread)
constexpr int kSelMaxGroups = 2048;  // chunks grow past M / 2048 tokens instead

struct SelPlan {
  int groups, chunk;  // workgroups, tokens per workgroup (a multiple of kSelSub)
};
SelPlan sel_plan(int M) {
  const int64_t subs = ((int64_t)M + kSelSub - 1) / kSelSub;
  const int64_t per = (subs + kSelMaxGroups - 1) / kSelMaxGroups;  // sub-chunks per workgroup
  const int chunk = (int)(per * kSelSub);
  return SelPlan{(int)(((int64_t)M + chunk - 1) / chunk), chunk};
}

__global__ __launch_bounds__(kSelMT) void sel_hist_kernel(const float* __restrict__ score, int M,
                                                          int chunk, int d,
                                                          uint32_t* __restrict__ ws, int G) {
  __shared__ uint32_t hist[kSelMT / 64][256];
  const int tid = threadIdx.x, wave = tid >> 6;
  // the bytes chosen by the earlier passes (none before the first)
  const uint32_t prefix = d == 3 ? 0u : ws[0], pmask = d == 3 ? 0u : ws[1];
  for (int i = tid; i < 256 * (kSelMT / 64); i += kSelMT) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int64_t t0 = (int64_t)blockIdx.x * chunk;
  const int64_t t1 = min((int64_t)M, t0 + chunk);
  uint32_t cur = 0u, run = 0u;  // a run of equal bins is added with one atomic
  for (int64_t base = t0; base < t1; base += kSelSub) {
    uint32_t k[kSelSub / kSelMT];
#pragma unroll
    for (int q = 0; q < kSelSub / kSelMT; ++q) {
      const int64_t t = base + tid + kSelMT * q;
      k[q] = t < t1 ? score_key(score[t]) : 0u;
    }
#pragma unroll
    for (int q = 0; q < kSelSub / kSelMT; ++q) {
      if (base + tid + kSelMT * q >= t1 || (k[q] & pmask) != prefix) continue;
      const uint32_t b = (k[q] >> (8 * d)) & 255u;
      if (run && b != cur) {
        atomicAdd(&hist[wave][cur], run);
        run = 0u;
      }
      cur = b;
      ++run;
    }
  }
  if (run) atomicAdd(&hist[wave][cur], run);
  __syncthreads();
  uint32_t tot = 0;
#pragma unroll
  for (int w = 0; w < kSelMT / 64; ++w) tot += hist[w][tid];
  const int Gp = (G + 3) & ~3;
  ws[4 + Gp + (int64_t)tid * Gp + blockIdx.x] = tot;
}

__global__ __launch_bounds__(1024) void sel_choose_kernel(uint32_t* __restrict__ ws, int G, int d,
                                                          int n_keep) {
  __shared__ uint32_t part[4][256];
  __shared__ uint32_t tot[256];
  __shared__ uint32_t s_sel[2];
  const int tid = threadIdx.x, lane = tid & 63;
  {  // bin tid / 4: its counts summed by four threads, 4 workgroups per 16-byte load
    const int bin = tid >> 2, q = tid & 3, Gp = (G + 3) & ~3;
    const uint32_t* row = ws + 4 + Gp + (int64_t)bin * Gp;  // 16-byte aligned (Gp = 0 mod 4)
    uint32_t t = 0;
#pragma unroll 8
    for (int v = q; v < Gp / 4; v += 4) {
      const uint4 c = *(const uint4*)(row + 4 * v);
      const int g = 4 * v;
      t += c.x + (g + 1 < G ? c.y : 0u) + (g + 2 < G ? c.z : 0u) + (g + 3 < G ? c.w : 0u);
    }
    part[q][bin] = t;
  }
  const uint32_t need = d == 3 ? (uint32_t)n_keep : ws[2];
  __syncthreads();
  if (tid < 256) tot[tid] = part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid];
  __syncthreads();
  if (tid < 64) {
    // lane l holds bins 255 - 4l - q (q = 0..3), i.e. the bins in descending order
    uint32_t loc[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      loc[q] = tot[255 - 4 * lane - q];
      sum += loc[q];
    }
    uint32_t incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    const uint32_t excl = incl - sum;
    if (excl < need && need <= incl) {  // exactly one lane: the total is at least `need`
      uint32_t acc = excl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (acc + loc[q] >= need) {
          s_sel[0] = (uint32_t)(255 - 4 * lane - q);
          s_sel[1] = need - acc;
          break;
        }
        acc += loc[q];
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    const uint32_t prefix = d == 3 ? 0u : ws[0], pmask = d == 3 ? 0u : ws[1];
    ws[0] = prefix | (s_sel[0] << (8 * d));
    ws[1] = pmask | (255u << (8 * d));
    ws[2] = s_sel[1];
  }
}

// keys equal to the threshold in each workgroup's chunk
__global__ __launch_bounds__(kSelMT) void sel_eqcount_kernel(const float* __restrict__ score, int M,
                                                             int chunk, uint32_t* __restrict__ ws) {
  __shared__ uint32_t s_w[kSelMT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t T = ws[0];
  const int64_t t0 = (int64_t)blockIdx.x * chunk;
  const int64_t t1 = min((int64_t)M, t0 + chunk);
  uint32_t n = 0;
  for (int64_t t = t0 + tid; t < t1; t += kSelMT) n += score_key(score[t]) == T ? 1u : 0u;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off, 64);
  if (lane == 0) s_w[wave] = n;
  __syncthreads();
  if (tid == 0) {
    uint32_t tot = 0;
#pragma unroll
    for (int w = 0; w < kSelMT / 64; ++w) tot += s_w[w];
    ws[4 + blockIdx.x] = tot;
  }
}

__global__ __launch_bounds__(kSelMT) void sel_mark_kernel(const float* __restrict__ score, int M,
                                                          int chunk, const uint32_t* __restrict__ ws,
                                                          uint8_t* __restrict__ keep) {
  constexpr int PER = kSelSub / kSelMT;  // consecutive tokens per thread and step
  __shared__ uint32_t s_w[kSelMT / 64];
  __shared__ uint32_t s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t T = ws[0], need = ws[2];
  // equal keys in the chunks before this one, summed in a fixed order
  uint32_t before_g = 0;
  for (int g = tid; g < (int)blockIdx.x; g += kSelMT) before_g += ws[4 + g];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) before_g += __shfl_xor(before_g, off, 64);
  if (lane == 0) s_w[wave] = before_g;
  __syncthreads();
  if (tid == 0) {
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < kSelMT / 64; ++w) c += s_w[w];
    s_carry = c;
  }
  __syncthreads();
  const int64_t t0 = (int64_t)blockIdx.x * chunk;
  const int64_t t1 = min((int64_t)M, t0 + chunk);
  for (int64_t base = t0; base < t1; base += kSelSub) {
    const int64_t tb = base + (int64_t)tid * PER;
    uint32_t kk[PER], eq = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      kk[q] = tb + q < t1 ? score_key(score[tb + q]) : 0u;
      eq += (tb + q < t1 && kk[q] == T) ? 1u : 0u;
    }
    uint32_t incl = eq;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    __syncthreads();  // s_w is rewritten
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    uint32_t before = s_carry + incl - eq;
    for (int w = 0; w < wave; ++w) before += s_w[w];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      if (tb + q >= t1) break;
      bool kp = kk[q] > T;
      if (kk[q] == T) {
        kp = before < need;
        ++before;
      }
      keep[tb + q] = kp ? 1 : 0;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t tot = 0;
#pragma unroll
      for (int w = 0; w < kSelMT / 64; ++w) tot += s_w[w];
      s_carry += tot;
    }
  }
}

// keep[t] = v for every t (nothing or everything kept)
__global__ __launch_bounds__(256) void sel_fill_kernel(uint8_t* __restrict__ keep, int64_t M,
                                                       uint8_t v) {
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < M; t += (int64_t)gridDim.x * 256)
    keep[t] = v;
}

size_t select_workspace_bytes(int M) {
  if (M <= kSelThreads * kSelCached) return 0;
  const SelPlan pl = sel_plan(M);
  const int64_t Gp = (pl.groups + 3) & ~3;
  return (size_t)(4 + Gp + Gp * 256) * sizeof(uint32_t);
}

collider_status launch_select_topk_multi(const float* score, int M, int n_keep, uint8_t* keep,
                                         uint32_t* ws, hipStream_t s) {
  if (M <= 0) return COLLIDER_OK;
  if (M <= kSelThreads * kSelCached) return launch_select_topk(score, M, n_keep, keep, s);
  if (n_keep <= 0 || n_keep >= M) {
    const int blocks = (int)std::min<int64_t>(((int64_t)M + 255) / 256, 4096);
    COLLIDER_LAUNCH("select_fill", s,
                    hipLaunchKernelGGL(sel_fill_kernel, dim3(blocks), dim3(256), 0, s, keep, (int64_t)M,
                                       (uint8_t)(n_keep <= 0 ? 0 : 1)));
    return last_hip_status();
  }
  const SelPlan pl = sel_plan(M);
  for (int d = 3; d >= 0; --d) {
    COLLIDER_LAUNCH("select_hist", s,
                    hipLaunchKernelGGL(sel_hist_kernel, dim3(pl.groups), dim3(kSelMT), 0, s, score, M,
                                       pl.chunk, d, ws, pl.groups));
    COLLIDER_LAUNCH("select_choose", s,
                    hipLaunchKernelGGL(sel_choose_kernel, dim3(1), dim3(1024), 0, s, ws, pl.groups, d,
                                       n_keep));
  }
  COLLIDER_LAUNCH("select_eqcount", s,
                  hipLaunchKernelGGL(sel_eqcount_kernel, dim3(pl.groups), dim3(kSelMT), 0, s, score, M,
                                     pl.chunk, ws));
  COLLIDER_LAUNCH("select_mark", s,
                  hipLaunchKernelGGL(sel_mark_kernel, dim3(pl.groups), dim3(kSelMT), 0, s, score, M,
                                     pl.chunk, ws, keep));
  return last_hip_status();
}

// ------------------------------------------------------------------------------------------
// cross-entropy gradient over the kept rows: one workgroup per row
// ------------------------------------------------------------------------------------------
constexpr float kLog2eF = 1.4426950408889634f;

struct MaxSum {
  float m, s;  // running max of z * log2(e) and sum of 2^(z log2(e) - m)
};
// An empty state (no finite logit seen yet) has m = -inf and s = 0; merging it must not form
// exp2(-inf - (-inf)) = exp2(NaN), so either side being empty returns the other.
__device__ __forceinline__ MaxSum ms_merge(MaxSum a, MaxSum b) {
  if (a.m == -INFINITY) return b;
  if (b.m == -INFINITY) return a;
  const float m = fmaxf(a.m, b.m);
  return MaxSum{m, a.s * __builtin_amdgcn_exp2f(a.m - m) + b.s * __builtin_amdgcn_exp2f(b.m - m)};
}
__device__ __forceinline__ MaxSum ms_add8(MaxSum a, uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float z[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[2 * i] = bflo(w[i]) * kLog2eF;
    z[2 * i + 1] = bfhi(w[i]) * kLog2eF;
  }
  float m8 = z[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) m8 = fmaxf(m8, z[i]);
  const float m = fmaxf(a.m, m8);
  if (m == -INFINITY) return a;  // every logit so far is -inf (masked entries): nothing to add
  float s = a.m == -INFINITY ? 0.f : a.s * __builtin_amdgcn_exp2f(a.m - m);
#pragma unroll
  for (int i = 0; i < 8; ++i) s += __builtin_amdgcn_exp2f(z[i] - m);
  return MaxSum{m, s};
}

// RV > 0: the row stays in registers (RV 16-byte vectors per thread, V <= 2048 RV); RV == 0: the
// row is read twice (the second read mostly from cache).
template <int RV>
__global__ __launch_bounds__(256) void ce_grad_kernel(const uint16_t* __restrict__ logits,
                                                      int64_t ld, const int32_t* __restrict__ labels,
                                                      const int32_t* __restrict__ rowmap, int V,
                                                      float scale, uint16_t* __restrict__ dl,
                                                      int64_t ldd) {
  __shared__ MaxSum s_ms[4];
  const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = rowmap ? rowmap[c] : c;
  const int nvec = V >> 3;
  const uint4* src = (const uint4*)(logits + t * ld);
  uint4* dst = (uint4*)(dl + (int64_t)c * ldd);
  MaxSum ms{-INFINITY, 0.f};
  uint4 row[RV > 0 ? RV : 1];
  if constexpr (RV > 0) {
    // the row's loads go out before the label is looked at, so that they need not wait for it
#pragma unroll
    for (int j = 0; j < RV; ++j) {
      const int i = tid + 256 * j;
      row[j] = i < nvec ? src[i] : make_uint4(0, 0, 0, 0);
    }
  }
  const int y = labels[t];
  if (y < 0 || y >= V) {  // no target: no loss, no gradient
    for (int i = tid; i < nvec; i += 256) dst[i] = make_uint4(0, 0, 0, 0);
    return;
  }
  if constexpr (RV > 0) {
#pragma unroll
    for (int j = 0; j < RV; ++j)
      if (tid + 256 * j < nvec) ms = ms_add8(ms, row[j]);
  } else {
    for (int i = tid; i < nvec; i += 256) ms = ms_add8(ms, src[i]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
    ms = ms_merge(ms, MaxSum{__shfl_xor(ms.m, off, 64), __shfl_xor(ms.s, off, 64)});
  if (lane == 0) s_ms[wave] = ms;
  __syncthreads();
  ms = s_ms[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) ms = ms_merge(ms, s_ms[w]);
  const float m = ms.m, sc = scale / ms.s;
  auto grad8 = [&](int i, uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float g[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      g[2 * e] = __builtin_amdgcn_exp2f(bflo(w[e]) * kLog2eF - m) * sc;
      g[2 * e + 1] = __builtin_amdgcn_exp2f(bfhi(w[e]) * kLog2eF - m) * sc;
    }
    const int d = y - 8 * i;
    if (d >= 0 && d < 8) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e == d) g[e] -= scale;
    }
    dst[i] = make_uint4(pack2bf(g[0], g[1]), pack2bf(g[2], g[3]), pack2bf(g[4], g[5]),
                        pack2bf(g[6], g[7]));
  };
  if constexpr (RV > 0) {
#pragma unroll
    for (int j = 0; j < RV; ++j)
      if (tid + 256 * j < nvec) grad8(tid + 256 * j, row[j]);
  } else {
    for (int i = tid; i < nvec; i += 256) grad8(i, src[i]);
  }
}

collider_status launch_ce_grad(const uint16_t* logits, int64_t ld, const int32_t* labels,
                               const int32_t* rowmap, int rows, int V, float scale, uint16_t* dl,
                               int64_t ldd, hipStream_t s) {
  if (rows <= 0) return COLLIDER_OK;
  const int nvec = V / 8;
  if (nvec <= 256 * 16)
    COLLIDER_LAUNCH("ce_grad", s, hipLaunchKernelGGL(ce_grad_kernel<16>, dim3(rows), dim3(256), 0, s,
                                                     logits, ld, labels, rowmap, V, scale, dl, ldd));
  else if (nvec <= 256 * 32)
    COLLIDER_LAUNCH("ce_grad", s, hipLaunchKernelGGL(ce_grad_kernel<32>, dim3(rows), dim3(256), 0, s,
                                                     logits, ld, labels, rowmap, V, scale, dl, ldd));
  else
    COLLIDER_LAUNCH("ce_grad", s, hipLaunchKernelGGL(ce_grad_kernel<0>, dim3(rows), dim3(256), 0, s,
                                                     logits, ld, labels, rowmap, V, scale, dl, ldd));
  return last_hip_status();
}

// ------------------------------------------------------------------------------------------
// per-token cross-entropy loss over every token: loss_t = logsumexp(z_t) - z_t[y_t] (0 without a
// target).  It is the score backward token filtering ranks tokens by (Figure 2(b)).  One
// workgroup per row, the row read once.  Rows of up to NV * 2048 logits are loaded whole into
// registers first (every load of the row in flight at once, together with the label's own logit);
// longer rows (NV = 0) stream through four 16-byte vectors per thread at a time.  Each thread
// folds its vectors in the same order either way, so the result does not depend on the path.
// ------------------------------------------------------------------------------------------
template <int NV>
__global__ __launch_bounds__(256) void ce_loss_kernel(const uint16_t* __restrict__ logits, int64_t ld,
                                                      const int32_t* __restrict__ labels, int V,
                                                      float* __restrict__ loss) {
  __shared__ MaxSum s_ms[4];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int y = labels[t];
  if (y < 0 || y >= V) {
    if (tid == 0) loss[t] = 0.f;
    return;
  }
  const int nvec = V >> 3;
  const uint16_t* row = logits + t * ld;
  const uint4* src = (const uint4*)row;
  float zy = 0.f;
  if (tid == 0) zy = bf2f(row[y]);
  MaxSum ms{-INFINITY, 0.f};
  if constexpr (NV > 0) {
    uint4 v[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      v[u] = make_uint4(0, 0, 0, 0);
      if (tid + 256 * u < nvec) v[u] = src[tid + 256 * u];
    }
#pragma unroll
    for (int u = 0; u < NV; ++u)
      if (tid + 256 * u < nvec) ms = ms_add8(ms, v[u]);
  } else {
    int i = tid;
    for (; i + 3 * 256 < nvec; i += 4 * 256) {
      const uint4 a = src[i], b = src[i + 256], c = src[i + 512], d = src[i + 768];
      ms = ms_add8(ms_add8(ms_add8(ms_add8(ms, a), b), c), d);
    }
    for (; i < nvec; i += 256) ms = ms_add8(ms, src[i]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
    ms = ms_merge(ms, MaxSum{__shfl_xor(ms.m, off, 64), __shfl_xor(ms.s, off, 64)});
  if (lane == 0) s_ms[wave] = ms;
  __syncthreads();
  if (tid == 0) {
    ms = s_ms[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) ms = ms_merge(ms, s_ms[w]);
    // log-sum-exp in natural-log units: (m + log2 s) ln 2, m and s in base-2 units
    const float lse = (ms.m + __builtin_amdgcn_logf(ms.s)) * 0.6931471805599453f;
    loss[t] = lse - zy;
  }
}

collider_status launch_ce_loss(const uint16_t* logits, int64_t ld, const int32_t* labels, int M, int V,
                               float* loss, hipStream_t s) {
  if (M <= 0) return COLLIDER_OK;
  const int nvec = V >> 3;
  if (nvec <= 256 * 8) {
    COLLIDER_LAUNCH("ce_loss", s, hipLaunchKernelGGL(ce_loss_kernel<8>, dim3(M), dim3(256), 0, s,
                                                     logits, ld, labels, V, loss));
  } else if (nvec <= 256 * 16) {
    COLLIDER_LAUNCH("ce_loss", s, hipLaunchKernelGGL(ce_loss_kernel<16>, dim3(M), dim3(256), 0, s,
                                                     logits, ld, labels, V, loss));
  } else if (nvec <= 256 * 32) {
    COLLIDER_LAUNCH("ce_loss", s, hipLaunchKernelGGL(ce_loss_kernel<32>, dim3(M), dim3(256), 0, s,
                                                     logits, ld, labels, V, loss));
  } else {
    COLLIDER_LAUNCH("ce_loss", s, hipLaunchKernelGGL(ce_loss_kernel<0>, dim3(M), dim3(256), 0, s,
                                                     logits, ld, labels, V, loss));
  }
  return last_hip_status();
}

// ------------------------------------------------------------------------------------------
// embedding gradient: kept tokens bucketed by id (stable counting sort), then one wavefront per
// vocabulary row sums its bucket's dx rows in token order.  No float atomics: every sum has a
// fixed order.
// ------------------------------------------------------------------------------------------
__global__ void fill_i32_kernel(int32_t* __restrict__ p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// id of kept token c (-1 when outside [0, V): such tokens have no embedding row)
__device__ __forceinline__ int kept_id(const int32_t* ids, const int32_t* idx, int c, int V) {
  const int id = ids[idx[c]];
  return (id >= 0 && id < V) ? id : -1;
}

__global__ void embed_count_kernel(const int32_t* __restrict__ ids, const int32_t* __restrict__ idx,
                                   int rows, int V, int32_t* __restrict__ cnt) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= rows) return;
  const int id = kept_id(ids, idx, c, V);
  if (id >= 0) atomicAdd(&cnt[id], 1);  // integer counts: the same totals in any order
}

// off[v] = sum of cnt[u] for u < v, off[V] = total.  One workgroup of 1024 threads walks the ids
// in tiles of kScanTile: the tile is loaded into LDS with coalesced reads, thread i scans its 16
// consecutive entries there, a block scan of the thread sums (plus the carry of earlier tiles) gives
// each run's start, and the offsets go back out coalesced.
constexpr int kScanTile = 16384;
__global__ __launch_bounds__(1024) void embed_scan_kernel(const int32_t* __restrict__ cnt, int V,
                                                          int32_t* __restrict__ off) {
  // each thread scans 16 consecutive counts in registers (16-byte loads and stores where the tile
  // is whole), the threads' sums are scanned across the block, and tiles carry their totals on.
  // (Through an LDS tile read with a 16-element stride per thread the scan took 21 us for
  // V = 32000: a 16-way bank conflict on every access.)
  __shared__ int32_t s_w[16];
  __shared__ int32_t s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int PER = kScanTile / 1024;
  static_assert(PER == 16, "four 16-byte vectors per thread");
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < V; base += kScanTile) {
    const int i0 = base + tid * PER;
    int v[PER];
    if (i0 + PER <= V) {
#pragma unroll
      for (int q = 0; q < PER / 4; ++q) {
        const int4 c4 = *(const int4*)(cnt + i0 + 4 * q);
        v[4 * q] = c4.x; v[4 * q + 1] = c4.y; v[4 * q + 2] = c4.z; v[4 * q + 3] = c4.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < PER; ++q) v[q] = i0 + q < V ? cnt[i0 + q] : 0;
    }
    int sum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) sum += v[q];
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    int run = s_carry + incl - sum;
    for (int w = 0; w < wave; ++w) run += s_w[w];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int x = v[q];
      v[q] = run;
      run += x;
    }
    if (i0 + PER <= V) {
#pragma unroll
      for (int q = 0; q < PER / 4; ++q)
        *(int4*)(off + i0 + 4 * q) = make_int4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    } else {
#pragma unroll
      for (int q = 0; q < PER; ++q)
        if (i0 + q < V) off[i0 + q] = v[q];
    }
    __syncthreads();  // every thread has read s_carry and s_w
    if (tid == 1023) s_carry = run;  // the tile's last run ends at the tile's total
    __syncthreads();
  }
  if (tid == 0) off[V] = s_carry;
}

// sorted[off[id] + r] = c, r = number of kept tokens before c with the same id (stable).  One
// workgroup walks the kept tokens in chunks of 1024: a token's rank inside its chunk comes from the
// chunk's ids in LDS (four ids per LDS read), its rank across earlier chunks from cursor[id], which
// is raised once the whole chunk has read it.  LDS_CURSOR: the cursors live in LDS (V <= 32768);
// otherwise in global memory (an atomic read and add per token and chunk).
constexpr int kCursorLds = 32768;
template <bool LDS_CURSOR>
__global__ __launch_bounds__(1024) void embed_place_kernel(const int32_t* __restrict__ ids,
                                                           const int32_t* __restrict__ idx, int rows,
                                                           int V, const int32_t* __restrict__ off,
                                                           int32_t* cursor,
                                                           int32_t* __restrict__ sorted) {
  extern __shared__ __align__(16) int32_t s_dyn[];
  __shared__ __align__(16) int32_t s_id[1024];
  const int tid = threadIdx.x;
  if constexpr (LDS_CURSOR) {
    for (int i = tid; i < V; i += 1024) s_dyn[i] = 0;
    __syncthreads();
  }
  for (int base = 0; base < rows; base += 1024) {
    const int c = base + tid;
    const int id = c < rows ? kept_id(ids, idx, c, V) : -1;
    s_id[tid] = id;
    __syncthreads();
    if (id >= 0) {
      int r = 0;
      const int4* s4 = (const int4*)s_id;
      for (int j4 = 0; j4 < (tid >> 2); ++j4) {
        const int4 q = s4[j4];
        r += (q.x == id) + (q.y == id) + (q.z == id) + (q.w == id);
      }
      for (int j = tid & ~3; j < tid; ++j) r += s_id[j] == id ? 1 : 0;
      int cur;
      if constexpr (LDS_CURSOR)
        cur = s_dyn[id];
      else
        cur = __hip_atomic_load(&cursor[id], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sorted[off[id] + cur + r] = c;
    }
    __syncthreads();  // every token of the chunk has read its cursor before any update
    if (id >= 0) {
      if constexpr (LDS_CURSOR)
        atomicAdd(&s_dyn[id], 1);
      else
        atomicAdd(&cursor[id], 1);
    }
    if constexpr (!LDS_CURSOR) __threadfence();
    __syncthreads();
  }
}

// The same placement spread over workgroups, one per chunk of kEmbChunk kept tokens.  A token's
// place is off[id] + (tokens with its id in earlier chunks) + (tokens with its id earlier in its
// own chunk).  The middle term comes from per-chunk id histograms (integer atomics: the counts,
// not their order, are what is kept) summed over the chunks in order, a pass that also yields
// every id's count for the offsets (the separate counting pass and its clearing are not needed:
// 20 us less on Zipf-distributed ids, whose frequent ids made that pass's atomics collide); the
// last term from the chunk's ids in LDS, as above.  Used when the histograms (chunks x V ints)
// fit the workspace.
constexpr int kEmbChunk = 1024;

__global__ __launch_bounds__(kEmbChunk) void embed_hist_kernel(const int32_t* __restrict__ ids,
                                                                const int32_t* __restrict__ idx,
                                                                int rows, int V,
                                                                int32_t* __restrict__ hist) {
  int32_t* h = hist + (int64_t)blockIdx.x * V;
  for (int v = threadIdx.x; v < V; v += kEmbChunk) h[v] = 0;
  __syncthreads();
  const int c = blockIdx.x * kEmbChunk + threadIdx.x;
  const int id = c < rows ? kept_id(ids, idx, c, V) : -1;
  if (id >= 0) atomicAdd(&h[id], 1);
}

// Per id, over the chunks in order: each chunk's count becomes the number of the id's tokens in
// the chunks before it, and the total is the id's count (the offsets' scan reads it; no separate
// counting pass).
__global__ __launch_bounds__(256) void embed_hist_prefix_kernel(int V, int chunks,
                                                                int32_t* __restrict__ hist,
                                                                int32_t* __restrict__ cnt) {
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= V) return;
  int acc = 0;
  for (int j = 0; j < chunks; ++j) {
    const int64_t e = (int64_t)j * V + v;
    const int t = hist[e];
    hist[e] = acc;
    acc += t;
  }
  cnt[v] = acc;
}

__global__ __launch_bounds__(kEmbChunk) void embed_place_chunks_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ idx, int rows, int V,
    const int32_t* __restrict__ off, const int32_t* __restrict__ hist, int32_t* __restrict__ sorted) {
  __shared__ __align__(16) int32_t s_id[kEmbChunk];
  const int tid = threadIdx.x;
  const int c = blockIdx.x * kEmbChunk + tid;
  const int id = c < rows ? kept_id(ids, idx, c, V) : -1;
  s_id[tid] = id;
  __syncthreads();
  if (id < 0) return;
  int r = 0;
  const int4* s4 = (const int4*)s_id;
  for (int j4 = 0; j4 < (tid >> 2); ++j4) {
    const int4 q = s4[j4];
    r += (q.x == id) + (q.y == id) + (q.z == id) + (q.w == id);
  }
  for (int j = tid & ~3; j < tid; ++j) r += s_id[j] == id ? 1 : 0;
  sorted[off[id] + hist[(int64_t)blockIdx.x * V + id] + r] = c;
}

// dE[v, c0 .. c0+511] (+)= sum over j < off[v+1] - off[v] of dx[row(sorted[off[v] + j]), ...]: one
// wavefront per vocabulary row and 512-column block, 8 columns per lane; rows with no kept token
// are skipped (zeroed before by embed_zero_kernel, or left as they are when accumulating).  Every
// column adds its tokens in token order, up to 16 row loads in flight before their additions.
// The column blocks and the batched loads keep an id that many tokens share (natural text puts a
// tenth of its tokens on its most frequent id) from serialising the kernel on one wavefront: one
// wavefront per row, loading one token row at a time, took 26 us on uniform ids and 1382 us on
// Zipf-distributed ids (690 kept tokens on the most frequent id) for the TinyLlama shapes; this
// form takes 32 and 81 us, with the same sums bit for bit.  (Writing the zero rows here, a few KB per
// wavefront, took the 32000 x 2048 fp32 gradient 80 us.)
constexpr int kRowsumCols = 512, kRowsumBatch = 16;
__global__ __launch_bounds__(256) void embed_rowsum_kernel(const uint16_t* __restrict__ dx,
                                                           int64_t ld, const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ off,
                                                           const int32_t* __restrict__ sorted, int V,
                                                           int H, float* __restrict__ dE,
                                                           int accumulate) {
  const int ncb = (H + kRowsumCols - 1) / kRowsumCols;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (gw >= (int64_t)V * ncb) return;
  const int v = (int)(gw / ncb), cb = (int)(gw - (int64_t)v * ncb);
  const int b = off[v], n = off[v + 1] - b;
  if (n == 0) return;  // the row is zero already (or keeps its value when accumulating)
  const int col = cb * kRowsumCols + lane * 8;
  const bool on = col < H;
  const int lcol = on ? col : 0;  // lanes past H load a valid column and drop it
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](uint4 u) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bflo(w[e]);
      acc[2 * e + 1] += bfhi(w[e]);
    }
  };
  for (int j0 = 0; j0 < n; j0 += 64) {
    // the source rows of up to 64 tokens, looked up by the lanes together
    const int nj = min(64, n - j0);
    int rl = 0;
    if (lane < nj) {
      const int c = sorted[b + j0 + lane];
      rl = idx ? idx[c] : c;
    }
    // every load of a batch is issued before the first addition (the loads are unconditional:
    // a load under a condition is compiled as a branch with its own wait); the additions keep
    // token order.  Batches of 16 while they fill, then of 4, then the last 1-3 tokens together
    int j = 0;  // uniform over the wavefront
    auto batch = [&](auto nb) {
      constexpr int NB = decltype(nb)::value;
      uint4 u[NB];
#pragma unroll
      for (int q = 0; q < NB; ++q)
        u[q] = *(const uint4*)(dx + (int64_t)__shfl(rl, j + q, 64) * ld + lcol);
#pragma unroll
      for (int q = 0; q < NB; ++q) add(u[q]);
      j += NB;
    };
    while (j + kRowsumBatch <= nj) batch(std::integral_constant<int, kRowsumBatch>{});
    while (j + 4 <= nj) batch(std::integral_constant<int, 4>{});
    if (nj - j == 3) batch(std::integral_constant<int, 3>{});
    else if (nj - j == 2) batch(std::integral_constant<int, 2>{});
    else if (nj - j == 1) batch(std::integral_constant<int, 1>{});
  }
  if (!on) return;
  float4* o = (float4*)(dE + (int64_t)v * H + col);
  float4 a = make_float4(acc[0], acc[1], acc[2], acc[3]), c4 = make_float4(acc[4], acc[5], acc[6], acc[7]);
  if (accumulate) {
    const float4 p0 = o[0], p1 = o[1];
    a.x += p0.x; a.y += p0.y; a.z += p0.z; a.w += p0.w;
    c4.x += p1.x; c4.y += p1.y; c4.z += p1.z; c4.w += p1.w;
  }
  o[0] = a;
  o[1] = c4;
}

// dE = 0 in 16-byte stores (the rows of ids no token has stay so; embed_rowsum_kernel writes the
// others)
__global__ __launch_bounds__(256) void embed_zero_kernel(float4* __restrict__ p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Raises embed_place_kernel<true>'s dynamic-LDS limit to the cursor array's size, once per device.
static bool place_lds_limit_set() {
  static std::atomic<uint64_t> done{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  const uint64_t bit = 1ull << dev;
  if (done.load(std::memory_order_acquire) & bit) return true;
  if (hipFuncSetAttribute((const void*)embed_place_kernel<true>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, kCursorLds * 4) != hipSuccess)
    return false;
  done.fetch_or(bit, std::memory_order_acq_rel);
  return true;
}

// ------------------------------------------------------------------------------------------
// Scratch of the allocation-free embedding gradient: the counting sort's counts, offsets,
// cursors and sorted token list for up to kEmbScratchMaxV vocabulary rows and kEmbScratchMaxRows
// kept tokens (7 MiB per GPU, held until the process ends).  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the device address of each
// GPU's copy is looked up once per device with hipGetSymbolAddress and used from then on.
// ------------------------------------------------------------------------------------------
constexpr int kEmbScratchInts = 3 * kEmbScratchMaxV + 1 + kEmbScratchMaxRows;
static __device__ __align__(256) int32_t scratch[kEmbScratchInts];

collider_status embedding_scratch(int32_t** cnt, int32_t** off, int32_t** cursor, int32_t** sorted) {
  static std::mutex mu;
  static int32_t* ptr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return COLLIDER_ERR_HIP;
  int32_t* base = nullptr;
  {
    std::lock_guard<std::mutex> lk(mu);
    if (!ptr[dev]) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return COLLIDER_ERR_HIP;
      ptr[dev] = (int32_t*)p;
    }
    base = ptr[dev];
  }
  *cnt = base;
  *off = base + kEmbScratchMaxV;
  *cursor = base + 2 * kEmbScratchMaxV + 1;
  *sorted = base + 3 * kEmbScratchMaxV + 1;
  return COLLIDER_OK;
}

int embedding_hist_chunks(int rows, int V) {
  const int64_t chunks = ((int64_t)rows + kEmbChunk - 1) / kEmbChunk;
  return (chunks >= 2 && chunks * V <= kEmbHistMax) ? (int)chunks : 0;
}

collider_status launch_embedding_bwd(const uint16_t* dx, int64_t ld, int dx_compact,
                                     const int32_t* ids, const int32_t* idx, int rows, int V, int H,
                                     float* dE, int accumulate, int32_t* cnt, int32_t* off,
                                     int32_t* cursor, int32_t* sorted, hipStream_t s,
                                     int32_t* hist) {
  const int chunks = hist ? embedding_hist_chunks(rows, V) : 0;
  if (chunks > 0) {
    // per-chunk histograms, their running sums per id (which also give the counts), the offsets,
    // then every token's place: the id's offset, its tokens in earlier chunks, its rank in its own
    COLLIDER_LAUNCH("embed_place", s,
                    hipLaunchKernelGGL(embed_hist_kernel, dim3(chunks), dim3(kEmbChunk), 0, s, ids, idx,
                                       rows, V, hist));
    COLLIDER_LAUNCH("embed_place", s,
                    hipLaunchKernelGGL(embed_hist_prefix_kernel, dim3((V + 255) / 256), dim3(256), 0, s,
                                       V, chunks, hist, cnt));
    COLLIDER_LAUNCH("embed_scan", s,
                    hipLaunchKernelGGL(embed_scan_kernel, dim3(1), dim3(1024), 0, s, cnt, V, off));
    COLLIDER_LAUNCH("embed_place", s,
                    hipLaunchKernelGGL(embed_place_chunks_kernel, dim3(chunks), dim3(kEmbChunk), 0, s,
                                       ids, idx, rows, V, off, hist, sorted));
  } else {
    COLLIDER_LAUNCH("embed_fill", s,
                    hipLaunchKernelGGL(fill_i32_kernel, dim3((V + 255) / 256), dim3(256), 0, s, cnt, V, 0));
    COLLIDER_LAUNCH("embed_fill", s,
                    hipLaunchKernelGGL(fill_i32_kernel, dim3((V + 255) / 256), dim3(256), 0, s, cursor, V, 0));
    if (rows > 0)
      COLLIDER_LAUNCH("embed_count", s,
                      hipLaunchKernelGGL(embed_count_kernel, dim3((rows + 255) / 256), dim3(256), 0, s,
                                         ids, idx, rows, V, cnt));
    COLLIDER_LAUNCH("embed_scan", s,
                    hipLaunchKernelGGL(embed_scan_kernel, dim3(1), dim3(1024), 0, s, cnt, V, off));
    if (rows > 0 && V <= kCursorLds) {
      if (!place_lds_limit_set()) return COLLIDER_ERR_HIP;
      COLLIDER_LAUNCH("embed_place", s,
                      hipLaunchKernelGGL(embed_place_kernel<true>, dim3(1), dim3(1024), V * 4, s, ids,
                                         idx, rows, V, off, cursor, sorted));
    } else if (rows > 0) {
      COLLIDER_LAUNCH("embed_place", s,
                      hipLaunchKernelGGL(embed_place_kernel<false>, dim3(1), dim3(1024), 0, s, ids, idx,
                                         rows, V, off, cursor, sorted));
    }
  }
  if (!accumulate) {
    const int64_t n4 = (int64_t)V * H / 4;
    const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 8192);
    COLLIDER_LAUNCH("embed_zero", s,
                    hipLaunchKernelGGL(embed_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                                       (float4*)dE, n4));
  }
  COLLIDER_LAUNCH("embed_rowsum", s,
                  hipLaunchKernelGGL(embed_rowsum_kernel,
                                     dim3((unsigned)(((int64_t)V * ((H + kRowsumCols - 1) / kRowsumCols) + 3) / 4)),
                                     dim3(256), 0, s, dx, ld,
                                     dx_compact ? nullptr : idx, off, sorted, V, H, dE, accumulate));
  return last_hip_status();
}

}  // namespace collider
