// Mask -> index: stable stream compaction of the per-token keep mask.
//
// Backward token filtering decides per token whether its loss is kept (Collider paper, Figure 2(b));
// the kept tokens are the rows the dimension-reduced dense GEMMs run over (abstract).  One
// workgroup of 1024 threads (16 wavefronts) walks the mask in chunks of 8 tokens per thread:
// wavefront prefix sums via shuffles, then an LDS scan over the 16 wavefront totals.  The mask is
// small (bytes per token) and the work latency-bound, so one workgroup avoids a multi-kernel scan.
#include "internal.h"

namespace collider {

static constexpr int kThreads = 1024;
static constexpr int kPer = 8;
static constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int n = __shfl_up(v, off, 64);
    if (lane >= off) v += n;
  }
  return v;
}

// Exclusive scan of one int per thread over the block; also returns the block total.
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = wave_incl_scan(v);
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kWaves ? s_wave[lane] : 0;
    int wi = wave_incl_scan(w);
    if (lane < kWaves) s_wave[lane] = wi - w;  // exclusive wave offsets
    if (lane == kWaves - 1) s_wave[kWaves] = wi;
  }
  __syncthreads();
  int r = s_wave[wave] + incl - v;
  *total = s_wave[kWaves];
  __syncthreads();  // s_wave is reused by the next call
  return r;
}

__global__ __launch_bounds__(kThreads) void build_index_kernel(const uint8_t* __restrict__ keep,
                                                               int B, int S,
                                                               int32_t* __restrict__ idx,
                                                               int32_t* __restrict__ inv,
                                                               int32_t* __restrict__ cu,
                                                               int32_t* __restrict__ count) {
  __shared__ int s_wave[kWaves + 1];
  const int M = B * S;
  // pass 1: number of kept tokens (needed to place the filtered positions after the kept ones)
  int local = 0;
  for (int t = threadIdx.x; t < M; t += kThreads) local += keep[t] != 0;
  int total = 0;
  (void)block_excl_scan(local, &total, s_wave);
  const int n_kept = total;
  // pass 2: chunked exclusive scan and scatter
  int before = 0;  // kept tokens before the current chunk
  for (int base = 0; base < M; base += kThreads * kPer) {
    const int t0 = base + threadIdx.x * kPer;
    unsigned bits = 0;
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int t = t0 + e;
      const bool k = (t < M) && keep[t] != 0;
      bits |= (unsigned)k << e;
      cnt += k;
    }
    int chunk_total = 0;
    int pre = before + block_excl_scan(cnt, &chunk_total, s_wave);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int t = t0 + e;
      if (t >= M) break;
      if (t % S == 0) cu[t / S] = pre;
      if ((bits >> e) & 1u) {
        idx[pre] = t;
        inv[t] = pre;
        ++pre;
      } else {
        idx[n_kept + (t - pre)] = t;
        inv[t] = -1;
      }
    }
    before += chunk_total;
  }
  if (threadIdx.x == 0) {
    cu[B] = n_kept;
    count[0] = n_kept;
  }
}

collider_status launch_build_index(const uint8_t* keep, int B, int S, int32_t* idx, int32_t* inv,
                                   int32_t* cu, int32_t* count, hipStream_t s) {
  COLLIDER_LAUNCH("build_index", s,
                  hipLaunchKernelGGL(build_index_kernel, dim3(1), dim3(kThreads), 0, s, keep, B, S,
                                     idx, inv, cu, count));
  return last_hip_status();
}

}  // namespace collider
