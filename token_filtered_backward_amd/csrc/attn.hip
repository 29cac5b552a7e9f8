// Filtered attention backward (Collider paper, Figures 3 and 5): the softmax activation P of
// filtered tokens is removed in the attention backward, so G_V = P~^T G_O and the Q/K gradients
// stay row-sparse.  After compaction every key of the compacted sequence is kept, so removing the
// filtered columns of P is the same as running a causal, variable-length attention backward over
// the kept rows only, with the forward's log-sum-exp (over all keys) kept as the normaliser.
//
// Three kernels, all on CDNA4 bf16 MFMA 32x32x16 with fp32 accumulation, P recomputed from Q, K:
//  1. attn_dq   (query-block outer, 4 wavefronts x 32 queries): with dmode FILTERED it first sweeps
//     the kept keys to form D~_i = sum_j P_ij dP_ij; with FULL it forms D_i = dO_i . O_i.  It then
//     sweeps the keys again for dQ = tau * dS K, applies the rotary backward and stores bf16 dq.
//     It computes S^T = K Q^T so that each lane owns one query: its lse and D are scalars, and the
//     S^T accumulator registers are directly the A operand of dS K.
//  2. attn_dkv  (key-block outer, 4 wavefronts x 32 keys): S = Q K^T so each lane owns one key and
//     the P / dS accumulators are directly the A operands of P^T dO and dS^T Q.  A workgroup sums
//     over a slice of the query heads sharing its KV head; slices go to fp32 partial buffers.
//  3. attn_dkv_finalize: sums the slices in a fixed order, applies the rotary backward to dK and
//     stores bf16 dk, dv.
// Operands that need the token index as the MFMA reduction index (K in dS K, Q and dO in the key
// kernel) are kept twice in LDS: row-major and transposed.
#include "internal.h"

namespace collider {

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  int64_t ld_q, ld_k, ld_v, ld_o, ld_do;
  const float* lse;
  int64_t ld_lse;
  const int32_t* cu;
  const int32_t* idx;
  int M_kept, S, nq, nkv, G, HS;
  float scale, scale_log2;
  int rot;
  const float2* rope;  // [S][rot/2] (cos, sin)
  float* Dbuf;         // [M_kept][nq]
  float* dkp;          // [HS][M_kept][nkv][D]
  float* dvp;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int64_t ld_dq, ld_dk, ld_dv;
};

static constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

__device__ __forceinline__ bf16x8 zero_frag() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.f;
  return z;
}

__device__ __forceinline__ bf16x8 to_frag(const float* v8) {
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = (__bf16)v8[e];
  return a;
}

// 8 values of a transposed LDS tile: row `d`, token columns base+4h+{0..3} and base+8+4h+{0..3}
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* T, int ldt, int d, int base, int hl) {
  const uint2 lo = *(const uint2*)(T + d * ldt + base + 4 * hl);
  const uint2 hi = *(const uint2*)(T + d * ldt + base + 8 + 4 * hl);
  uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
  return __builtin_bit_cast(bf16x8, u);
}

// Cooperative copy of a [64 x D] token tile into LDS (row-major, and transposed if T != nullptr).
template <int D, int ROWS, int LDR, int LDT>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ src, int64_t ld, int col0,
                                          int row0, int nrows, uint16_t* R, uint16_t* T) {
  constexpr int CPR = D / 8;
  for (int c = threadIdx.x; c < ROWS * CPR; c += 256) {
    const int r = c / CPR, dc = c % CPR;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row0 + r < nrows) v = *(const uint4*)(src + (int64_t)(row0 + r) * ld + col0 + dc * 8);
    *(uint4*)(R + r * LDR + dc * 8) = v;
    if (T) {
      const uint16_t* e = (const uint16_t*)&v;
#pragma unroll
      for (int i = 0; i < 8; ++i) T[(dc * 8 + i) * LDT + r] = e[i];
    }
  }
}

// ------------------------------------------------------------------------------------------
// 1. dQ (and D) kernel
// ------------------------------------------------------------------------------------------
template <int D, bool FULLD>
__global__ __launch_bounds__(256) void attn_dq_kernel(AttnParams p) {
  constexpr int BQ = 128, BKV = 64, LDR = D + 8, LDT = BKV + 8, KK = D / 16, DT = D / 32;
  constexpr int LDE = D + 4;  // fp32 epilogue tile [BQ][LDE] reuses the same LDS
  constexpr int KV_ELEMS = 2 * BKV * LDR + D * LDT, EPI_ELEMS = BQ * LDE * 2;
  __shared__ __align__(16) uint16_t smem[KV_ELEMS > EPI_ELEMS ? KV_ELEMS : EPI_ELEMS];
  uint16_t* Ks = smem;
  uint16_t* Vs = smem + BKV * LDR;
  uint16_t* Kt = smem + 2 * BKV * LDR;
  const int b = blockIdx.z, h = blockIdx.y, g = h / p.G;
  const int cs = p.cu ? min(p.cu[b], p.M_kept) : b * p.S;
  const int nb = p.cu ? max(0, min(p.cu[b + 1], p.M_kept) - cs) : p.S;
  const int nqb = (nb + BQ - 1) / BQ;
  if ((int)blockIdx.x >= nqb) return;
  const int q0 = (nqb - 1 - (int)blockIdx.x) * BQ;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hl = lane >> 5, l32 = lane & 31;
  const int iq = q0 + wave * 32 + l32;
  const bool qvalid = iq < nb;
  const uint16_t* kseq = p.k + (int64_t)cs * p.ld_k;  // rows of this sequence
  const uint16_t* vseq = p.v + (int64_t)cs * p.ld_v;

  bf16x8 qf[KK], dof[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (qvalid) {
      qf[kk] = *(const bf16x8*)(p.q + (int64_t)(cs + iq) * p.ld_q + h * D + kk * 16 + hl * 8);
      dof[kk] = *(const bf16x8*)(p.dout + (int64_t)(cs + iq) * p.ld_do + h * D + kk * 16 + hl * 8);
    } else {
      qf[kk] = zero_frag();
      dof[kk] = zero_frag();
    }
  }
  const float lse2 = qvalid ? p.lse[(int64_t)(cs + iq) * p.ld_lse + h] * kLog2e : 0.f;
  const int kv_end = min(nb, q0 + BQ);
  const int nkvb = (kv_end + BKV - 1) / BKV;

  float Dv = 0.f;
  if constexpr (FULLD) {
    float part = 0.f;
    if (qvalid) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 of = *(const bf16x8*)(p.o + (int64_t)(cs + iq) * p.ld_o + h * D + kk * 16 + hl * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) part += (float)of[e] * (float)dof[kk][e];
      }
    }
    Dv = part + __shfl_xor(part, 32, 64);
  } else {
    // pass 1: D~_i = sum over kept keys j <= i of P_ij dP_ij
    float dacc = 0.f;
    for (int kb = 0; kb < nkvb; ++kb) {
      __syncthreads();
      load_tile<D, BKV, LDR, LDT>(kseq, p.ld_k, g * D, kb * BKV, nb, Ks, nullptr);
      load_tile<D, BKV, LDR, LDT>(vseq, p.ld_v, g * D, kb * BKV, nb, Vs, nullptr);
      __syncthreads();
#pragma unroll
      for (int jt = 0; jt < BKV / 32; ++jt) {
        f32x16 st, dpt;
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = dpt[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 ka = *(const bf16x8*)(Ks + (jt * 32 + l32) * LDR + kk * 16 + hl * 8);
          const bf16x8 va = *(const bf16x8*)(Vs + (jt * 32 + l32) * LDR + kk * 16 + hl * 8);
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], st, 0, 0, 0);
          dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, dof[kk], dpt, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kb * BKV + jt * 32 + acc_row(r, lane);
          const float pr = (qvalid && j <= iq) ? exp2f(st[r] * p.scale_log2 - lse2) : 0.f;
          dacc += pr * dpt[r];
        }
      }
    }
    Dv = dacc + __shfl_xor(dacc, 32, 64);
  }
  if (hl == 0 && qvalid) p.Dbuf[(int64_t)(cs + iq) * p.nq + h] = Dv;

  // pass 2: dQ = sum_j dS_ij K_j
  f32x16 dqa[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[t][r] = 0.f;
  for (int kb = 0; kb < nkvb; ++kb) {
    __syncthreads();
    load_tile<D, BKV, LDR, LDT>(kseq, p.ld_k, g * D, kb * BKV, nb, Ks, Kt);
    load_tile<D, BKV, LDR, LDT>(vseq, p.ld_v, g * D, kb * BKV, nb, Vs, nullptr);
    __syncthreads();
#pragma unroll
    for (int jt = 0; jt < BKV / 32; ++jt) {
      f32x16 st, dpt;
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = dpt[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 ka = *(const bf16x8*)(Ks + (jt * 32 + l32) * LDR + kk * 16 + hl * 8);
        const bf16x8 va = *(const bf16x8*)(Vs + (jt * 32 + l32) * LDR + kk * 16 + hl * 8);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], st, 0, 0, 0);
        dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, dof[kk], dpt, 0, 0, 0);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = kb * BKV + jt * 32 + acc_row(r, lane);
        const float pr = (qvalid && j <= iq) ? exp2f(st[r] * p.scale_log2 - lse2) : 0.f;
        ds[r] = pr * (dpt[r] - Dv);
      }
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        const bf16x8 a = to_frag(ds + 8 * step);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const bf16x8 bk = tr_frag(Kt, LDT, t * 32 + l32, jt * 32 + 16 * step, hl);
          dqa[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bk, dqa[t], 0, 0, 0);
        }
      }
    }
  }

  // epilogue: tau * dQ through LDS (fp32), rotary backward, bf16 store
  __syncthreads();
  float* E = (float*)smem;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      E[(wave * 32 + acc_row(r, lane)) * LDE + t * 32 + l32] = dqa[t][r] * p.scale;
  __syncthreads();
  const int half = p.rot >> 1;
  for (int c = threadIdx.x; c < BQ * (D / 8); c += 256) {
    const int row = c / (D / 8), c0 = (c % (D / 8)) * 8;
    const int i = q0 + row;
    if (i >= nb) continue;
    float out[8];
    const float* er = E + row * LDE;
    if (c0 < p.rot) {
      const int pos = (p.idx ? p.idx[cs + i] : cs + i) % p.S;
      const bool lower = c0 < half;
      const int m0 = lower ? c0 : c0 - half;
      const int pc = lower ? c0 + half : c0 - half;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 t = p.rope[(int64_t)pos * half + m0 + e];
        const float x = er[c0 + e], y = er[pc + e];
        out[e] = lower ? x * t.x + y * t.y : x * t.x - y * t.y;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = er[c0 + e];
    }
    uint4 w = make_uint4(pack2bf(out[0], out[1]), pack2bf(out[2], out[3]), pack2bf(out[4], out[5]),
                         pack2bf(out[6], out[7]));
    *(uint4*)(p.dq + (int64_t)(cs + i) * p.ld_dq + h * D + c0) = w;
  }
}

// ------------------------------------------------------------------------------------------
// 2. dK / dV kernel
// ------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_dkv_kernel(AttnParams p) {
  constexpr int BKV = 128, BQ = 64, LDR = D + 8, LDT = BQ + 8, KK = D / 16, DT = D / 32;
  __shared__ __align__(16) uint16_t Qs[BQ * LDR];
  __shared__ __align__(16) uint16_t Qt[D * LDT];
  __shared__ __align__(16) uint16_t Os[BQ * LDR];
  __shared__ __align__(16) uint16_t Ot[D * LDT];
  __shared__ __align__(16) float Ls[BQ];
  __shared__ __align__(16) float Ds[BQ];
  const int b = blockIdx.z, g = blockIdx.y / p.HS, hs = blockIdx.y % p.HS;
  const int cs = p.cu ? min(p.cu[b], p.M_kept) : b * p.S;
  const int nb = p.cu ? max(0, min(p.cu[b + 1], p.M_kept) - cs) : p.S;
  const int nkb = (nb + BKV - 1) / BKV;
  if ((int)blockIdx.x >= nkb) return;
  const int k0 = blockIdx.x * BKV;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hl = lane >> 5, l32 = lane & 31;
  const int jk = k0 + wave * 32 + l32;  // this lane's key (S column)
  const bool kvalid = jk < nb;
  const uint16_t* qseq = p.q + (int64_t)cs * p.ld_q;  // rows of this sequence
  const uint16_t* doseq = p.dout + (int64_t)cs * p.ld_do;

  bf16x8 kf[KK], vf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (kvalid) {
      kf[kk] = *(const bf16x8*)(p.k + (int64_t)(cs + jk) * p.ld_k + g * D + kk * 16 + hl * 8);
      vf[kk] = *(const bf16x8*)(p.v + (int64_t)(cs + jk) * p.ld_v + g * D + kk * 16 + hl * 8);
    } else {
      kf[kk] = zero_frag();
      vf[kk] = zero_frag();
    }
  }
  f32x16 dka[DT], dva[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[t][r] = dva[t][r] = 0.f;

  const int GH = p.G / p.HS;
  const int nqb = (nb + BQ - 1) / BQ;
  for (int hh = 0; hh < GH; ++hh) {
    const int h = g * p.G + hs * GH + hh;
    for (int qb = k0 / BQ; qb < nqb; ++qb) {
      const int i0 = qb * BQ;
      __syncthreads();
      load_tile<D, BQ, LDR, LDT>(qseq, p.ld_q, h * D, i0, nb, Qs, Qt);
      load_tile<D, BQ, LDR, LDT>(doseq, p.ld_do, h * D, i0, nb, Os, Ot);
      if (threadIdx.x < BQ) {
        const int i = i0 + threadIdx.x;
        Ls[threadIdx.x] = i < nb ? p.lse[(int64_t)(cs + i) * p.ld_lse + h] * kLog2e : 0.f;
        Ds[threadIdx.x] = i < nb ? p.Dbuf[(int64_t)(cs + i) * p.nq + h] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < BQ / 32; ++it) {
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 qa = *(const bf16x8*)(Qs + (it * 32 + l32) * LDR + kk * 16 + hl * 8);
          const bf16x8 oa = *(const bf16x8*)(Os + (it * 32 + l32) * LDR + kk * 16 + hl * 8);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[kk], dp, 0, 0, 0);
        }
        float pr[16], ds[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int ib = it * 32 + 8 * r4 + 4 * hl;  // 4 consecutive queries
          const float4 l4 = *(const float4*)(Ls + ib);
          const float4 d4 = *(const float4*)(Ds + ib);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 4 * r4 + q;
            const int i = i0 + ib + q;
            const float pv = (kvalid && i < nb && jk <= i) ? exp2f(s[r] * p.scale_log2 - lv[q]) : 0.f;
            pr[r] = pv;
            ds[r] = pv * (dp[r] - dvv[q]);
          }
        }
#pragma unroll
        for (int step = 0; step < 2; ++step) {
          const bf16x8 ap = to_frag(pr + 8 * step);
          const bf16x8 as = to_frag(ds + 8 * step);
#pragma unroll
          for (int t = 0; t < DT; ++t) {
            const bf16x8 bo = tr_frag(Ot, LDT, t * 32 + l32, it * 32 + 16 * step, hl);
            const bf16x8 bq = tr_frag(Qt, LDT, t * 32 + l32, it * 32 + 16 * step, hl);
            dva[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap, bo, dva[t], 0, 0, 0);
            dka[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as, bq, dka[t], 0, 0, 0);
          }
        }
      }
    }
  }
  // partial slices: [HS][M_kept][nkv][D]
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = k0 + wave * 32 + acc_row(r, lane);
      if (j < nb) {
        const int64_t off = (((int64_t)hs * p.M_kept + cs + j) * p.nkv + g) * D + t * 32 + l32;
        p.dkp[off] = dka[t][r] * p.scale;
        p.dvp[off] = dva[t][r];
      }
    }
}

// ------------------------------------------------------------------------------------------
// 3. finalize: ordered sum over head slices, rotary backward on dK, bf16 stores
// ------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_dkv_finalize_kernel(AttnParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + wave;  // (row, kv head)
  if (item >= p.M_kept * p.nkv) return;
  const int c = item / p.nkv, g = item % p.nkv;
  const int half = p.rot >> 1;
  const int64_t slice = (int64_t)p.M_kept * p.nkv * D;
  const int64_t base = ((int64_t)c * p.nkv + g) * D;
  int pos = 0;
  if (p.rot) pos = (p.idx ? p.idx[c] : c) % p.S;
  for (int m = lane; m < D; m += 64) {
    float xk = 0.f, yk = 0.f, xv = 0.f;
    const bool rotated = m < p.rot;
    const int pm = m < half ? m + half : m - half;
    for (int s = 0; s < p.HS; ++s) {
      xk += p.dkp[s * slice + base + m];
      xv += p.dvp[s * slice + base + m];
      if (rotated) yk += p.dkp[s * slice + base + pm];
    }
    float out = xk;
    if (rotated) {
      const float2 t = p.rope[(int64_t)pos * half + (m < half ? m : m - half)];
      out = m < half ? xk * t.x + yk * t.y : xk * t.x - yk * t.y;
    }
    p.dk[(int64_t)c * p.ld_dk + g * D + m] = f2bf(out);
    p.dv[(int64_t)c * p.ld_dv + g * D + m] = f2bf(xv);
  }
}

// ------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------
static int choose_hs(const collider_attn_cfg& c, int B, int M_kept) {
  const int G = c.n_q_heads / c.n_kv_heads;
  const long kblocks = (long)(M_kept + 127) / 128 + B;
  for (int hs = 1; hs <= G; ++hs) {
    if (G % hs) continue;
    if (kblocks * c.n_kv_heads * hs >= 1024) return hs;
  }
  return G;
}

struct AttnWs {
  float* D;
  float* dkp;
  float* dvp;
  float* rope;
  size_t bytes;
};

static AttnWs carve_attn(const collider_attn_cfg& c, int B, int S, int M_kept, void* base) {
  Carver cv(base);
  AttnWs w;
  const int hs = choose_hs(c, B, M_kept);
  w.D = cv.take<float>((size_t)M_kept * c.n_q_heads);
  w.dkp = cv.take<float>((size_t)hs * M_kept * c.n_kv_heads * c.head_dim);
  w.dvp = cv.take<float>((size_t)hs * M_kept * c.n_kv_heads * c.head_dim);
  w.rope = cv.take<float>((size_t)S * (c.rot_dims > 0 ? c.rot_dims : 2));
  w.bytes = cv.bytes();
  return w;
}

size_t attn_workspace_bytes(const collider_attn_cfg& c, int B, int S, int M_kept) {
  return carve_attn(c, B, S, M_kept, nullptr).bytes;
}

collider_status attn_bwd(const collider_attn_cfg& c, const collider_index& ix,
                         const collider_attn_io& io, void* ws, size_t ws_bytes, hipStream_t s) {
  const int B = ix.B, S = ix.S, Mk = ix.M_kept;
  if (Mk <= 0) return COLLIDER_OK;
  AttnWs w = carve_attn(c, B, S, Mk, ws);
  if (ws_bytes < w.bytes) return COLLIDER_ERR_WORKSPACE;
  AttnParams p{};
  p.q = (const uint16_t*)io.q;
  p.k = (const uint16_t*)io.k;
  p.v = (const uint16_t*)io.v;
  p.o = (const uint16_t*)io.o;
  p.dout = (const uint16_t*)io.dout;
  p.ld_q = io.ld_q;
  p.ld_k = io.ld_k;
  p.ld_v = io.ld_v;
  p.ld_o = io.ld_o;
  p.ld_do = io.ld_do;
  p.lse = io.lse;
  p.ld_lse = io.ld_lse;
  p.cu = ix.cu_seqlens;
  p.idx = ix.idx;
  p.M_kept = Mk;
  p.S = S;
  p.nq = c.n_q_heads;
  p.nkv = c.n_kv_heads;
  p.G = c.n_q_heads / c.n_kv_heads;
  p.HS = choose_hs(c, B, Mk);
  p.scale = c.softmax_scale > 0.f ? c.softmax_scale : 1.f / sqrtf((float)c.head_dim);
  p.scale_log2 = p.scale * kLog2e;
  p.rot = c.rot_dims;
  p.rope = (const float2*)w.rope;
  p.Dbuf = w.D;
  p.dkp = w.dkp;
  p.dvp = w.dvp;
  p.dq = (uint16_t*)io.dq;
  p.dk = (uint16_t*)io.dk;
  p.dv = (uint16_t*)io.dv;
  p.ld_dq = io.ld_dq;
  p.ld_dk = io.ld_dk;
  p.ld_dv = io.ld_dv;

  collider_status st = COLLIDER_OK;
  if (c.rot_dims > 0) {
    st = launch_rope_table(w.rope, S, c.rot_dims, c.rope_base, s);
    if (st != COLLIDER_OK) return st;
  }
  const bool full = c.dmode == COLLIDER_ATTN_D_FULL;
  dim3 gq((S + 127) / 128, c.n_q_heads, B), gk((S + 127) / 128, c.n_kv_heads * p.HS, B);
  const int fin_blocks = (Mk * c.n_kv_heads + 3) / 4;
  if (c.head_dim == 64) {
    if (full)
      COLLIDER_LAUNCH("attn_dq", s, hipLaunchKernelGGL((attn_dq_kernel<64, true>), gq, dim3(256), 0, s, p));
    else
      COLLIDER_LAUNCH("attn_dq", s, hipLaunchKernelGGL((attn_dq_kernel<64, false>), gq, dim3(256), 0, s, p));
    COLLIDER_LAUNCH("attn_dkv", s, hipLaunchKernelGGL(attn_dkv_kernel<64>, gk, dim3(256), 0, s, p));
    COLLIDER_LAUNCH("attn_dkv_finalize", s,
                    hipLaunchKernelGGL(attn_dkv_finalize_kernel<64>, dim3(fin_blocks), dim3(256), 0, s, p));
  } else {
    if (full)
      COLLIDER_LAUNCH("attn_dq", s, hipLaunchKernelGGL((attn_dq_kernel<128, true>), gq, dim3(256), 0, s, p));
    else
      COLLIDER_LAUNCH("attn_dq", s, hipLaunchKernelGGL((attn_dq_kernel<128, false>), gq, dim3(256), 0, s, p));
    COLLIDER_LAUNCH("attn_dkv", s, hipLaunchKernelGGL(attn_dkv_kernel<128>, gk, dim3(256), 0, s, p));
    COLLIDER_LAUNCH("attn_dkv_finalize", s,
                    hipLaunchKernelGGL(attn_dkv_finalize_kernel<128>, dim3(fin_blocks), dim3(256), 0, s, p));
  }
  return last_hip_status();
}

}  // namespace collider
