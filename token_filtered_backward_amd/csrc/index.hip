// Mask -> index: stable stream compaction of the per-token keep mask.
//
// Backward token filtering decides per token whether its loss is kept (Collider paper, Figure 2(b));
// the kept tokens are the rows the dimension-reduced dense GEMMs run over (abstract).  A workgroup
// of 1024 threads (16 wavefronts) walks the mask in chunks of 8 tokens per thread: wavefront prefix
// sums via shuffles, then an LDS scan over the 16 wavefront totals.  Masks up to 16384 tokens take
// one workgroup (the work is latency-bound); longer ones are split over up to 64 workgroups, each of
// which finds its starting position by counting the kept tokens before its range itself.
#include "internal.h"

namespace collider {

static constexpr int kThreads = 1024;
static constexpr int kPer = 8;
static constexpr int kWaves = kThreads / 64;
// masks up to kMwMin tokens: one workgroup (a few microseconds of latency, no gain from more);
// longer masks: up to kMwGrid workgroups, each with a range of the mask
static constexpr int64_t kMwMin = 16384;
static constexpr int kMwGrid = 64;

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

// 8 mask bytes of tokens t0 .. t0+7 as a bit mask (bit e: token t0 + e kept); tokens >= M count
// as filtered.  One 8-byte load when the whole group exists and the address allows it.
__device__ __forceinline__ unsigned load_bits(const uint8_t* __restrict__ keep, int t0, int M) {
  unsigned bits = 0;
  if (t0 + 8 <= M && ((uintptr_t)(keep + t0) & 7) == 0) {
    const uint2 w = *(const uint2*)(keep + t0);
    const uint32_t lo = w.x, hi = w.y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bits |= (unsigned)(((lo >> (8 * e)) & 0xffu) != 0) << e;
      bits |= (unsigned)(((hi >> (8 * e)) & 0xffu) != 0) << (e + 4);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (t0 + e < M) bits |= (unsigned)(keep[t0 + e] != 0) << e;
  }
  return bits;
}

// Writes idx / inv / cu for tokens t0 .. t0+7, whose first kept token gets compacted position pre.
// Compacted positions at or past lim are left out of inv and cu (lim = the count the caller
// announced; INT_MAX when it announced none), so that no consumer sized for lim rows ever indexes
// past them.
__device__ __forceinline__ void scatter_group(unsigned bits, int t0, int pre, int n_kept, int M, int S,
                                              int lim, int32_t* __restrict__ idx,
                                              int32_t* __restrict__ inv, int32_t* __restrict__ cu) {
  int iv[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int t = t0 + e;
    const bool k = (bits >> e) & 1u;
    iv[e] = (k && pre < lim) ? pre : -1;
    if (t < M) {
      if (t % S == 0) cu[t / S] = min(pre, lim);
      if (k)
        idx[pre] = t;
      else
        idx[n_kept + (t - pre)] = t;
    }
    pre += k;
  }
  if (t0 + 8 <= M && ((uintptr_t)(inv + t0) & 15) == 0) {
    ((int4*)(inv + t0))[0] = make_int4(iv[0], iv[1], iv[2], iv[3]);
    ((int4*)(inv + t0))[1] = make_int4(iv[4], iv[5], iv[6], iv[7]);
  } else {
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (t0 + e < M) inv[t0 + e] = iv[e];
  }
}

// Multi-workgroup form for long masks: workgroup g owns tokens [g*T, min(M, (g+1)*T)), T a multiple
// of kChunkMW.  It needs the number of kept tokens before its range (its first compacted position)
// and in the whole mask (the filtered positions' offset); rather than exchange partial counts
// through memory (which would need scratch the call does not have), every workgroup counts them
// itself in one sweep over the mask (1 byte per token, served by L2 after the first workgroups).
// Then it scans its range chunk by chunk like the single-workgroup kernel.
constexpr int kThreadsMW = kThreads;
constexpr int kChunkMW = kThreadsMW * kPer;  // 8192 tokens per scan step

__device__ __forceinline__ int count_kept_16(const uint8_t* __restrict__ keep, int t0, int M) {
  // kept tokens among t0 .. t0+15 (t0 a multiple of 16)
  if (t0 + 16 <= M && ((uintptr_t)(keep + t0) & 15) == 0) {
    const uint4 w = *(const uint4*)(keep + t0);
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
    int n = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < 4; ++b) n += ((v[i] >> (8 * b)) & 0xffu) != 0;
    return n;
  }
  int n = 0;
  for (int e = 0; e < 16 && t0 + e < M; ++e) n += keep[t0 + e] != 0;
  return n;
}

__device__ __forceinline__ int block_sum_mw(int v, int* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if (lane == 0) s_wave[wave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kThreadsMW / 64; ++w) t += s_wave[w];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kThreadsMW) void build_index_mw_kernel(
    const uint8_t* __restrict__ keep, int B, int S, int T, int32_t* __restrict__ idx,
    int32_t* __restrict__ inv, int32_t* __restrict__ cu, int32_t* __restrict__ count, int expect,
    int32_t* __restrict__ mismatch) {
  __shared__ int s_wave[kWaves + 1];
  const int M = B * S;
  const int lim = expect >= 0 ? expect : 0x7fffffff;
  const int g0 = blockIdx.x * T, g1 = min(M, g0 + T);
  // kept tokens before this range and in the whole mask (16 tokens per thread per step, eight
  // steps' loads in flight)
  int before = 0, all = 0;
#pragma unroll 8
  for (int t = threadIdx.x * 16; t < M; t += kThreadsMW * 16) {
    const int n = count_kept_16(keep, t, M);
    all += n;
    before += t < g0 ? n : 0;
  }
  before = block_sum_mw(before, s_wave);
  const int n_kept = block_sum_mw(all, s_wave);
  for (int base = g0; base < g1; base += kChunkMW) {
    const int t0 = base + threadIdx.x * kPer;
    const unsigned bits = t0 < g1 ? load_bits(keep, t0, g1) : 0u;
    int chunk_total = 0;
    const int pre = before + block_excl_scan(__popc(bits), &chunk_total, s_wave);
    if (t0 < g1) scatter_group(bits, t0, pre, n_kept, g1, S, lim, idx, inv, cu);
    before += chunk_total;
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
    cu[B] = min(n_kept, lim);
    count[0] = n_kept;
    if (mismatch) mismatch[0] = (expect >= 0 && n_kept != expect) ? 1 : 0;
  }
}

__global__ __launch_bounds__(kThreads) void build_index_kernel(const uint8_t* __restrict__ keep,
                                                               int B, int S,
                                                               int32_t* __restrict__ idx,
                                                               int32_t* __restrict__ inv,
                                                               int32_t* __restrict__ cu,
                                                               int32_t* __restrict__ count,
                                                               int expect,
                                                               int32_t* __restrict__ mismatch) {
  __shared__ int s_wave[kWaves + 1];
  const int M = B * S;
  const int lim = expect >= 0 ? expect : 0x7fffffff;
  constexpr int CHUNK = kThreads * kPer;
  int n_kept;
  if (M <= CHUNK) {
    // one chunk: the scan of the only chunk also gives the total
    const int t0 = threadIdx.x * kPer;
    const unsigned bits = load_bits(keep, t0, M);
    int total = 0;
    const int pre = block_excl_scan(__popc(bits), &total, s_wave);
    n_kept = total;
    scatter_group(bits, t0, pre, n_kept, M, S, lim, idx, inv, cu);
  } else {
    // pass 1: number of kept tokens (the filtered positions are placed after the kept ones)
    int local = 0;
    for (int t0 = threadIdx.x * kPer; t0 < M; t0 += CHUNK) local += __popc(load_bits(keep, t0, M));
    int total = 0;
    (void)block_excl_scan(local, &total, s_wave);
    n_kept = total;
    // pass 2: chunked exclusive scan and scatter
    int before = 0;  // kept tokens before the current chunk
    for (int base = 0; base < M; base += CHUNK) {
      const int t0 = base + threadIdx.x * kPer;
      const unsigned bits = load_bits(keep, t0, M);
      int chunk_total = 0;
      const int pre = before + block_excl_scan(__popc(bits), &chunk_total, s_wave);
      scatter_group(bits, t0, pre, n_kept, M, S, lim, idx, inv, cu);
      before += chunk_total;
    }
  }
  if (threadIdx.x == 0) {
    cu[B] = min(n_kept, lim);
    count[0] = n_kept;
    if (mismatch) mismatch[0] = (expect >= 0 && n_kept != expect) ? 1 : 0;
  }
}

collider_status launch_build_index(const uint8_t* keep, int B, int S, int32_t* idx, int32_t* inv,
                                   int32_t* cu, int32_t* count, int expect, int32_t* mismatch,
                                   hipStream_t s) {
  const int64_t M = (int64_t)B * S;
  if (M <= kMwMin) {
    COLLIDER_LAUNCH("build_index", s,
                    hipLaunchKernelGGL(build_index_kernel, dim3(1), dim3(kThreads), 0, s, keep, B, S,
                                       idx, inv, cu, count, expect, mismatch));
  } else {
    // ranges of whole 8192-token scan steps, at most kMwGrid workgroups (each also sweeps the
    // whole mask once for its counts)
    const int64_t chunks = (M + kChunkMW - 1) / kChunkMW;
    const int64_t per = (chunks + kMwGrid - 1) / kMwGrid;
    const int T = (int)(per * kChunkMW);
    const int grid = (int)((M + T - 1) / T);
    COLLIDER_LAUNCH("build_index", s,
                    hipLaunchKernelGGL(build_index_mw_kernel, dim3(grid), dim3(kThreadsMW), 0, s, keep,
                                       B, S, T, idx, inv, cu, count, expect, mismatch));
  }
  return last_hip_status();
}

}  // namespace collider
