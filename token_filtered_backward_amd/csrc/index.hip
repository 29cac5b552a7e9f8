// Mask -> index: stable stream compaction of the per-token keep mask.
//
// Backward token filtering decides per token whether its loss is kept (Collider paper, Figure 2(b));
// the kept tokens are the rows the dimension-reduced dense GEMMs run over (abstract).  Each
// workgroup owns a range of the mask and walks it in scan steps of 8 tokens per thread: wavefront
// prefix sums via shuffles, then an LDS scan over the wavefront totals.  The call has no scratch
// memory to exchange partial counts through, so every workgroup counts the kept tokens before its
// range and in the whole mask itself (1 byte per token, served by L2 after the first workgroups).
// The token ids of a scan step are placed in LDS in their compacted order (kept ones, then the
// filtered ones) and written out as two contiguous runs of idx, so that the stores coalesce.
#include "internal.h"

namespace collider {

static constexpr int kPer = 8;
// masks up to kSmallMax tokens: workgroups of 256 threads, one 2048-token scan step each; longer
// masks: up to kBigGrid workgroups of 1024 threads, each over a range of whole 8192-token scan
// steps (at 65536 tokens 8 such workgroups built the index in 8.0 us against 9.2 us for 32 of the
// small ones, whose count sweeps then take two memory round trips)
static constexpr int64_t kSmallMax = 16384;
static constexpr int kBigGrid = 64;

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int n = __shfl_up(v, off, 64);
    if (lane >= off) v += n;
  }
  return v;
}

// Exclusive scan of one int per thread over the block of NT threads; also returns the block total.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* s_wave) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = wave_incl_scan(v);
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < NW ? s_wave[lane] : 0;
    int wi = wave_incl_scan(w);
    if (lane < NW) s_wave[lane] = wi - w;  // exclusive wave offsets
    if (lane == NW - 1) s_wave[NW] = wi;
  }
  __syncthreads();
  int r = s_wave[wave] + incl - v;
  *total = s_wave[NW];
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

// Writes inv and cu for tokens t0 .. t0+7 (t0 < M), whose first kept token gets compacted position
// pre, and places their ids at their compacted slots of the scan step in LDS: kept token number k of
// the step at loc[k], filtered token number f at loc[n_step_kept + f] (lpre / lpos: kept tokens and
// tokens of the step before t0).  Compacted positions at or past lim are left out of inv and cu
// (lim = the count the caller announced; INT_MAX when it announced none), so that no consumer sized
// for lim rows ever indexes past them.
__device__ __forceinline__ void place_group(unsigned bits, int t0, int pre, int lpre, int lpos,
                                            int n_step_kept, int M, int S, int lim, int32_t* loc,
                                            int32_t* __restrict__ inv, int32_t* __restrict__ cu) {
  int iv[kPer];
  int r = t0 % S;  // position of token t0 in its sequence
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int t = t0 + e;
    const bool k = (bits >> e) & 1u;
    iv[e] = (k && pre < lim) ? pre : -1;
    if (t < M) {
      if (r == 0) cu[t / S] = min(pre, lim);
      loc[k ? lpre : n_step_kept + (lpos + e - lpre)] = t;
    }
    r = r + 1 == S ? 0 : r + 1;
    pre += k;
    lpre += k;
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

// Workgroup g of NT threads owns tokens [g T, min(M, (g + 1) T)), T a multiple of the scan step
// NT * 8.
template <int NT>
__global__ __launch_bounds__(NT) void build_index_kernel(const uint8_t* __restrict__ keep, int B,
                                                         int S, int T, int32_t* __restrict__ idx,
                                                         int32_t* __restrict__ inv,
                                                         int32_t* __restrict__ cu,
                                                         int32_t* __restrict__ count, int expect,
                                                         int32_t* __restrict__ mismatch) {
  constexpr int NW = NT / 64, STEP = NT * kPer;
  __shared__ int s_wave[NW + 1];
  __shared__ int2 s_pair[NW];
  __shared__ int32_t loc[STEP];
  const int M = B * S;
  const int lim = expect >= 0 ? expect : 0x7fffffff;
  const int g0 = blockIdx.x * T, g1 = min(M, g0 + T);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the first scan step's mask bytes go out with the count sweep's
  unsigned bits = g0 + (int)threadIdx.x * kPer < g1 ? load_bits(keep, g0 + threadIdx.x * kPer, g1) : 0u;
  // kept tokens before this range and in the whole mask (16 tokens per thread per step, eight
  // steps' loads in flight)
  int before = 0, n_kept = 0;
#pragma unroll 8
  for (int t = threadIdx.x * 16; t < M; t += NT * 16) {
    const int n = count_kept_16(keep, t, M);
    n_kept += n;
    before += t < g0 ? n : 0;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    before += __shfl_xor(before, off, 64);
    n_kept += __shfl_xor(n_kept, off, 64);
  }
  if (lane == 0) s_pair[wave] = make_int2(before, n_kept);
  __syncthreads();
  before = 0;
  n_kept = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    before += s_pair[w].x;
    n_kept += s_pair[w].y;
  }
  for (int base = g0; base < g1; base += STEP) {
    const int t0 = base + threadIdx.x * kPer;
    if (base != g0) bits = t0 < g1 ? load_bits(keep, t0, g1) : 0u;
    int step_kept = 0;
    const int lpre = block_excl_scan<NT>(__popc(bits), &step_kept, s_wave);
    if (t0 < g1)
      place_group(bits, t0, before + lpre, lpre, threadIdx.x * kPer, step_kept, g1, S, lim, loc, inv, cu);
    __syncthreads();
    // kept ids to idx[before ..), filtered ids to idx[n_kept + filtered tokens before this step ..)
    const int n_step = min(STEP, g1 - base);
    const int fdst = n_kept + (base - before) - step_kept;
    for (int j = threadIdx.x; j < n_step; j += NT) idx[(j < step_kept ? before : fdst) + j] = loc[j];
    before += step_kept;
    __syncthreads();  // loc is reused by the next scan step
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
    cu[B] = min(n_kept, lim);
    count[0] = n_kept;
    if (mismatch) mismatch[0] = (expect >= 0 && n_kept != expect) ? 1 : 0;
  }
}

collider_status launch_build_index(const uint8_t* keep, int B, int S, int32_t* idx, int32_t* inv,
                                   int32_t* cu, int32_t* count, int expect, int32_t* mismatch,
                                   hipStream_t s) {
  const int64_t M = (int64_t)B * S;
  if (M <= kSmallMax) {
    constexpr int NT = 256, STEP = NT * kPer;
    const int grid = (int)((M + STEP - 1) / STEP);
    COLLIDER_LAUNCH("build_index", s,
                    hipLaunchKernelGGL(build_index_kernel<NT>, dim3(grid), dim3(NT), 0, s, keep, B, S,
                                       STEP, idx, inv, cu, count, expect, mismatch));
  } else {
    // ranges of whole scan steps, at most kBigGrid workgroups (each also sweeps the whole mask once
    // for its counts)
    constexpr int NT = 1024, STEP = NT * kPer;
    const int64_t steps = (M + STEP - 1) / STEP;
    const int64_t per = (steps + kBigGrid - 1) / kBigGrid;
    const int T = (int)(per * STEP);
    const int grid = (int)((M + T - 1) / T);
    COLLIDER_LAUNCH("build_index", s,
                    hipLaunchKernelGGL(build_index_kernel<NT>, dim3(grid), dim3(NT), 0, s, keep, B, S,
                                       T, idx, inv, cu, count, expect, mismatch));
  }
  return last_hip_status();
}

}  // namespace collider
