// Filtered attention backward (Collider paper, Figures 3 and 5): the softmax activation P of
// filtered tokens is removed in the attention backward, so G_V = P~^T G_O and the Q/K gradients
// stay row-sparse.  After compaction every key of the compacted sequence is kept, so removing the
// filtered columns of P is the same as running a causal, variable-length attention backward over
// the kept rows only, with the forward's log-sum-exp (over all keys) kept as the normaliser.
//
// Three kernels, all on CDNA4 bf16 MFMA 32x32x16 with fp32 accumulation, P recomputed from Q, K:
//  1. attn_dq   (query-block outer, 4 wavefronts x 32 queries): one sweep over the kept keys for
//     dQ = tau * dS K.  With dmode FULL the row term D_i = dO_i . O_i is known before the sweep;
//     with FILTERED the sweep also forms D~_i = sum_j P_ij dP_ij and the products that let dQ be
//     finished from it afterwards (see the kernel).  It applies the rotary backward, stores bf16 dq
//     and the row term for the dK/dV kernel.
//     It computes S^T = K Q^T so that each lane owns one query: its lse and D are scalars, and the
//     S^T accumulator registers are directly the A operand of dS K.
//  2. attn_dkv  (key-block outer, 4 wavefronts x 32 keys): S = Q K^T so each lane owns one key and
//     the P / dS accumulators are directly the A operands of P^T dO and dS^T Q.  A workgroup sums
//     over a slice of the query heads sharing its KV head; slices go to fp32 partial buffers.
//  3. attn_dkv_finalize: sums the slices in a fixed order, applies the rotary backward to dK and
//     stores bf16 dk, dv.  With a single slice (one query head per KV head, or few keys) the dK/dV
//     kernel does this itself from an LDS copy of its tile, and writes no partials.
// Token tiles [64 rows x D] live in LDS once, row-major (XOR-swizzled chunks for D = 64, padded
// rows for D = 128).  Operands that need the token index as the MFMA reduction index (K in dS K;
// Q and dO in P^T dO and dS^T Q) are read with
// ds_read_b64_tr_b16: within a group of 16 lanes, lane j addresses row k0 + j/4 at columns
// n + 4*(j%4) and lane i receives rows k0 .. k0+3 of column n + i.  The row order of the two
// transpose reads per fragment follows the 32x32 accumulator layout (rows 8*(r/4) + 4*(lane/32) +
// r%4), so the P / dS registers feed the MFMA without any data movement.  The next tile is fetched
// into registers while the MFMAs of the current one run (two LDS buffers, one barrier per tile).
// Inside the layer the kernels read q, k, v, o and lse of the full token layout through the index
// (row idx[c] for compacted row c), looked up a tile ahead of the loads that use them.
#include <cstdlib>

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
  // row of compacted token c in q, k, v, o and lse: srcmap[c] (the full-layout saved tensors read
  // through the index), or c when null (compacted inputs); dout, the outputs and Dbuf are compacted
  const int32_t* srcmap;
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

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

// 2^x with the hardware instruction alone: results below the smallest normal flush to 0, which is
// what a softmax probability that small should be.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// [64 x D] bf16 token tile in LDS, row-major.
// D = 64: 128-byte rows whose 16-byte chunks sit at chunk ^ swz(r), so that both read patterns are
// free of bank conflicts (64 banks of 4 bytes) - a 16-byte fragment read (16 lanes, 16 consecutive
// rows, one chunk) and a transpose read (32 lanes, 4 consecutive rows, 4 consecutive chunks) - and
// so are the tile stores: swz takes distinct values on the 8 even and on the 8 odd rows of any 16,
// and its bit 2 differs between rows r and r + 2 for r = 0, 1 mod 4.  A padded pitch left the
// transpose reads 2-way conflicted; the swizzle took the dQ kernel from 108 to 104 us (TinyLlama
// layer, 40%).
// D = 128: padded 304-byte rows (76 banks): 16 consecutive rows of a fragment read start on
// distinct 4-bank groups.  The same swizzle (4 bits) measured 10% slower there: the extra address
// arithmetic outweighed the conflicts it removed.
template <int D>
struct TokTile {
  static constexpr int ROWB = D == 64 ? 128 : 304;  // bytes per row
  static constexpr int BYTES = 64 * ROWB;
  static constexpr int NV = 64 * (D / 8) / 256;      // 16-byte chunks per thread
  static __device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
  // byte offset of byte `b` of row r
  static __device__ __forceinline__ int off(int r, int b) {
    if constexpr (D == 64) return r * ROWB + ((((b >> 4) ^ swz(r))) << 4) + (b & 15);
    return r * ROWB + b;
  }
};

__device__ __forceinline__ int64_t src_row(const AttnParams& p, int c) {
  return p.srcmap ? (int64_t)p.srcmap[c] : (int64_t)c;
}

// Source rows of this thread's 16-byte chunks of a 64-row tile (tile rows row0 .. row0+63 of a
// sequence starting at compacted row `base`; -1 past its nrows rows), looked up through `map` -
// one tile ahead of the loads that use them, so that the lookup's latency is hidden.  The rows stay
// 32-bit until a load uses them: widening them here would make the wavefront wait for the lookup
// (and for every load issued before it, the prefetch of the current tile included) at once.
template <int D>
struct TileRows {
  int32_t r[TokTile<D>::NV];
  __device__ __forceinline__ void set(const int32_t* __restrict__ map, int base, int row0, int nrows) {
#pragma unroll
    for (int i = 0; i < TokTile<D>::NV; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int rr = row0 + c / (D / 8);
      int v = -1;
      if (rr < nrows) v = map ? map[base + rr] : base + rr;
      r[i] = v;
    }
  }
};

template <int D>
struct TileRegs {
  uint4 v[TokTile<D>::NV];
  // rows row0 .. row0+63 of `src` (row stride ld elements), columns col0 .. col0+D-1
  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int64_t ld, int col0,
                                       int row0, int nrows) {
#pragma unroll
    for (int i = 0; i < TokTile<D>::NV; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int r = c / (D / 8), dc = c % (D / 8);
      v[i] = (row0 + r < nrows) ? *(const uint4*)(src + (int64_t)(row0 + r) * ld + col0 + dc * 8)
                                : make_uint4(0, 0, 0, 0);
    }
  }
  // the tile whose rows `t` lists
  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int64_t ld, int col0,
                                       const TileRows<D>& t) {
#pragma unroll
    for (int i = 0; i < TokTile<D>::NV; ++i) {
      const int dc = (threadIdx.x + 256 * i) % (D / 8);
      v[i] = t.r[i] >= 0 ? *(const uint4*)(src + (int64_t)t.r[i] * ld + col0 + dc * 8)
                         : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(char* T) const {
#pragma unroll
    for (int i = 0; i < TokTile<D>::NV; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int r = c / (D / 8), dc = c % (D / 8);
      *(uint4*)(T + TokTile<D>::off(r, dc * 16)) = v[i];
    }
  }
};

// A/B operand with the head dimension as the reduction index: rows rbase .. rbase+31,
// d = kk*16 .. kk*16+15 (16-byte read per lane)
template <int D>
__device__ __forceinline__ bf16x8 frag_rows(const char* T, int rbase, int kk, int lane) {
  return *(const bf16x8*)(T + TokTile<D>::off(rbase + (lane & 31), (kk * 16 + (lane >> 5) * 8) * 2));
}

// B operand with the token index as the reduction index: 16 tokens tbase .. tbase+15 in the
// accumulator row order (lane half h, element 4c+e <-> token tbase + 8c + 4h + e), columns
// dbase .. dbase+31 (lane & 31)
template <int D>
__device__ __forceinline__ bf16x8 frag_tr(const char* T, int tbase, int dbase, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int col = dbase + 16 * (g & 1) + 4 * (j & 3);
  const int row = tbase + 4 * (g >> 1) + (j >> 2);
  const char* a0 = T + TokTile<D>::off(row, col * 2);
  const char* a1 = T + TokTile<D>::off(row + 8, col * 2);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)a0);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)a1);
  const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// ------------------------------------------------------------------------------------------
// 1. dQ (and D) kernel
// ------------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void score_tiles(const char* Ks, const char* Vs, const bf16x8* qf,
                                            const bf16x8* dof, int jt, int lane, f32x16& st,
                                            f32x16& dpt) {
  constexpr int KK = D / 16;
#pragma unroll
  for (int r = 0; r < 16; ++r) st[r] = dpt[r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const bf16x8 ka = frag_rows<D>(Ks, jt * 32, kk, lane);
    const bf16x8 va = frag_rows<D>(Vs, jt * 32, kk, lane);
    st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], st, 0, 0, 0);
    dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, dof[kk], dpt, 0, 0, 0);
  }
}

// One sweep over the kept keys of the query block.  dS_ij = P_ij (dP_ij - D_i) needs the row term
// D_i before any of it can be formed.  With D = dO . O (FULLD) it is known up front.  With the
// filtered row term D~_i = sum_j P_ij dP_ij (a sum over the same sweep) the kernel instead uses,
// for a per-query constant c_i known up front,
//   sum_j dS_ij K_j = sum_j P_ij (dP_ij - c_i) K_j  -  (D~_i - c_i) sum_j P_ij K_j,
// accumulating both products and D~ in the one sweep (each score exponentiated once instead of
// twice) and combining them at the end.  c_i = dO_i . O_i, the full softmax's row term: it equals
// D~_i when no causal key of query i is filtered, so the correction stays small and the bf16
// operands of the first product are the usual dS values.  Without O (it is optional for the
// filtered row term) c_i = 0.
template <int D, bool FULLD>
__global__ __launch_bounds__(256, D == 64 ? (FULLD ? 3 : 2) : 1) void attn_dq_kernel(AttnParams p) {
  constexpr int BQ = 128, BKV = 64, KK = D / 16, DT = D / 32;
  constexpr int TB = TokTile<D>::BYTES;
  constexpr int LDE = D + 4;  // fp32 epilogue tile [BQ][LDE] reuses the same LDS
  constexpr int KV_BYTES = 4 * TB, EPI_BYTES = BQ * LDE * 4;
  constexpr int CORR_OFF = KV_BYTES > EPI_BYTES ? KV_BYTES : EPI_BYTES;
  // + the per-query correction D~ - c of the filtered row term, [BQ] floats
  __shared__ __align__(16) char smem[CORR_OFF + (FULLD ? 0 : BQ * 4)];
  // buffers: K in smem + buf*2*TB, V right after it
  // grid (head, sequence, block rank): blocks are dispatched x-fastest, so every sequence's and
  // head's largest query block (the last one, which sees the most keys) starts first
  const int b = blockIdx.y, h = blockIdx.x, g = h / p.G;
  const int cs = p.cu ? min(p.cu[b], p.M_kept) : b * p.S;
  const int nb = p.cu ? max(0, min(p.cu[b + 1], p.M_kept) - cs) : p.S;
  const int nqb = (nb + BQ - 1) / BQ;
  if ((int)blockIdx.z >= nqb) return;
  const int q0 = (nqb - 1 - (int)blockIdx.z) * BQ;
  const int lane = threadIdx.x & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int iq = q0 + wave * 32 + l32;
  const bool qvalid = iq < nb;
  const int qw = q0 + wave * 32;     // first query of this wave
  const bool qall = qw + 31 < nb;    // all 32 queries of the wave exist
  const int jlim = qw < nb ? min(qw + 31, nb - 1) : -1;  // last key any query of the wave sees
  const int64_t qrow = qvalid ? src_row(p, cs + iq) : 0;  // this lane's query in q, o, lse

  bf16x8 qf[KK], dof[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (qvalid) {
      qf[kk] = *(const bf16x8*)(p.q + qrow * p.ld_q + h * D + kk * 16 + hl * 8);
      dof[kk] = *(const bf16x8*)(p.dout + (int64_t)(cs + iq) * p.ld_do + h * D + kk * 16 + hl * 8);
    } else {
      qf[kk] = zero_frag();
      dof[kk] = zero_frag();
    }
  }
  const float lse2 = qvalid ? p.lse[qrow * p.ld_lse + h] * kLog2e : 0.f;
  const int kv_end = min(nb, q0 + BQ);
  const int nkvb = (kv_end + BKV - 1) / BKV;
  TileRegs<D> rk, rv;
  TileRows<D> tkv;  // rows of the next K / V tile

  // cref = c_i = dO_i . O_i (this lane's query; both lane halves hold the full sum)
  float cref = 0.f;
  if (p.o && qvalid) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 of = *(const bf16x8*)(p.o + qrow * p.ld_o + h * D + kk * 16 + hl * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) cref += (float)of[e] * (float)dof[kk][e];
    }
  }
  cref += __shfl_xor(cref, 32, 64);

  // dqa = sum_j P_ij (dP_ij - c_i) K_j; dqb = sum_j P_ij K_j (filtered row term only)
  f32x16 dqa[DT], dqb[FULLD ? 1 : DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[t][r] = 0.f;
  if constexpr (!FULLD) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqb[t][r] = 0.f;
  }
  float dacc = 0.f;  // this lane's part of D~_i = sum_j P_ij dP_ij
  tkv.set(p.srcmap, cs, 0, nb);
  rk.load(p.k, p.ld_k, g * D, tkv);
  rv.load(p.v, p.ld_v, g * D, tkv);
  if (nkvb > 1) tkv.set(p.srcmap, cs, BKV, nb);
  rk.store(smem);
  rv.store(smem + TB);
  __syncthreads();
  for (int kb = 0; kb < nkvb; ++kb) {
    const char* Ks = smem + (kb & 1) * 2 * TB;
    if (kb + 1 < nkvb) {
      rk.load(p.k, p.ld_k, g * D, tkv);
      rv.load(p.v, p.ld_v, g * D, tkv);
      if (kb + 2 < nkvb) tkv.set(p.srcmap, cs, (kb + 2) * BKV, nb);
    }
#pragma unroll
    for (int jt = 0; jt < BKV / 32; ++jt) {
      // 32 keys past every valid query of this wave: all masked, nothing to add (wave-uniform)
      if (kb * BKV + jt * 32 > jlim) continue;
      f32x16 st, dpt;
      score_tiles<D>(Ks, Ks + TB, qf, dof, jt, lane, st, dpt);
      float pr[16], x[16];
      if (kb * BKV + jt * 32 + 31 <= qw && qall) {  // below the diagonal: no mask
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pr[r] = fast_exp2(fmaf(st[r], p.scale_log2, -lse2));
          x[r] = pr[r] * (dpt[r] - cref);
          if constexpr (!FULLD) dacc = fmaf(pr[r], dpt[r], dacc);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kb * BKV + jt * 32 + acc_row(r, lane);
          pr[r] = (qvalid && j <= iq) ? fast_exp2(fmaf(st[r], p.scale_log2, -lse2)) : 0.f;
          x[r] = pr[r] * (dpt[r] - cref);
          if constexpr (!FULLD) dacc = fmaf(pr[r], dpt[r], dacc);
        }
      }
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        const bf16x8 a = to_frag(x + 8 * step);
        bf16x8 ap;
        if constexpr (!FULLD) ap = to_frag(pr + 8 * step);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const bf16x8 bk = frag_tr<D>(Ks, jt * 32 + 16 * step, t * 32, lane);
          dqa[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bk, dqa[t], 0, 0, 0);
          if constexpr (!FULLD) dqb[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap, bk, dqb[t], 0, 0, 0);
        }
      }
    }
    if (kb + 1 < nkvb) {
      char* nx = smem + ((kb + 1) & 1) * 2 * TB;
      rk.store(nx);
      rv.store(nx + TB);
    }
    __syncthreads();
  }
  float Dv = cref;
  if constexpr (!FULLD) {
    Dv = dacc + __shfl_xor(dacc, 32, 64);
    if (hl == 0) ((float*)(smem + CORR_OFF))[wave * 32 + l32] = Dv - cref;
  }
  if (hl == 0 && qvalid) p.Dbuf[(int64_t)(cs + iq) * p.nq + h] = Dv;
  if constexpr (!FULLD) {
    __syncthreads();  // the corrections of the wave's 32 queries are in LDS
    // dQ accumulator rows are queries acc_row(r, lane): D~ - c of row r comes from LDS
    const float* corr = (const float*)(smem + CORR_OFF) + wave * 32;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 c4 = *(const float4*)(corr + 8 * r4 + 4 * hl);
      const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) dqa[t][4 * r4 + q] = fmaf(-cv[q], dqb[t][4 * r4 + q], dqa[t][4 * r4 + q]);
    }
  }

  // epilogue: tau * dQ through LDS (fp32), rotary backward, bf16 store
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
    const bool one_side = c0 + 8 <= half || (c0 >= half && c0 + 8 <= p.rot);
    if (c0 < p.rot && one_side) {
      // rotate-half pairs (m, m + rot/2) for m < rot/2, the 8 columns all in one half: their
      // partners and table entries are 8 consecutive values too (vector reads)
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
    } else if (c0 < p.rot) {
      // the general case: rot/2 or rot falls inside this group of 8 (columns from rot on pass
      // through), paired per element
      const int pos = (p.idx ? p.idx[cs + i] : cs + i) % p.S;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = c0 + e;
        const float x = er[col];
        if (col < p.rot) {
          const bool lower = col < half;
          const float2 t = p.rope[(int64_t)pos * half + (lower ? col : col - half)];
          const float y = er[lower ? col + half : col - half];
          out[e] = lower ? x * t.x + y * t.y : x * t.x - y * t.y;
        } else {
          out[e] = x;
        }
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
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void attn_dkv_kernel(AttnParams p) {
  constexpr int BKV = 128, BQ = 64, KK = D / 16, DT = D / 32;
  constexpr int TB = TokTile<D>::BYTES;
  constexpr int BUF = 2 * TB + 2 * BQ * 4;  // Q tile, dO tile, lse*log2e, D
  // with a single head slice the epilogue stages the fp32 dK and dV tiles ([BKV][LDF] each) here
  constexpr int LDF = D + 4;
  constexpr int STAGE = 2 * BKV * LDF * 4;
  __shared__ __align__(16) char smem[2 * BUF > STAGE ? 2 * BUF : STAGE];
  // grid (kv head x head slice, sequence, key block): the first key blocks, which see the most
  // queries, are dispatched first
  const int b = blockIdx.y, g = blockIdx.x / p.HS, hs = blockIdx.x % p.HS;
  const int cs = p.cu ? min(p.cu[b], p.M_kept) : b * p.S;
  const int nb = p.cu ? max(0, min(p.cu[b + 1], p.M_kept) - cs) : p.S;
  const int nkb = (nb + BKV - 1) / BKV;
  if ((int)blockIdx.z >= nkb) return;
  const int k0 = blockIdx.z * BKV;
  const int lane = threadIdx.x & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int jk = k0 + wave * 32 + l32;  // this lane's key (S column)
  const bool kvalid = jk < nb;
  const int kw = k0 + wave * 32;     // first key of this wave
  const bool kall = kw + 31 < nb;    // all 32 keys of the wave exist
  const uint16_t* doseq = p.dout + (int64_t)cs * p.ld_do;  // compacted rows of this sequence
  const int64_t krow = kvalid ? src_row(p, cs + jk) : 0;     // this lane's key in k, v

  bf16x8 kf[KK], vf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (kvalid) {
      kf[kk] = *(const bf16x8*)(p.k + krow * p.ld_k + g * D + kk * 16 + hl * 8);
      vf[kk] = *(const bf16x8*)(p.v + krow * p.ld_v + g * D + kk * 16 + hl * 8);
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
  const int qb0 = k0 / BQ;
  const int per_head = nqb - qb0;
  const int n_iter = GH * per_head;  // (head, query block) pairs, head-major
  TileRegs<D> rq, ro;
  float sl = 0.f, sd = 0.f;
  // source rows of the Q tile and of the lse entry (threads < BQ) the next fetch reads, looked up
  // one iteration ahead of it
  TileRows<D> tq;
  int32_t lrow = -1;  // 32-bit until used, as in TileRows
  auto rows_of = [&](int it) {
    const int i0 = (qb0 + it % per_head) * BQ;
    tq.set(p.srcmap, cs, i0, nb);
    lrow = -1;
    if (threadIdx.x < BQ && i0 + (int)threadIdx.x < nb) {
      const int c = cs + i0 + (int)threadIdx.x;
      lrow = p.srcmap ? p.srcmap[c] : c;
    }
  };
  auto fetch = [&](int it) {
    const int h = g * p.G + hs * GH + it / per_head;
    const int i0 = (qb0 + it % per_head) * BQ;
    rq.load(p.q, p.ld_q, h * D, tq);
    ro.load(doseq, p.ld_do, h * D, i0, nb);
    // raw values: scaling them here would make the wavefront wait for these loads, and for the
    // tile loads above them, before the current tile's work
    if (threadIdx.x < BQ) {
      const int i = i0 + threadIdx.x;
      sl = 0.f;
      sd = 0.f;
      if (lrow >= 0) sl = p.lse[(int64_t)lrow * p.ld_lse + h];
      if (i < nb) sd = p.Dbuf[(int64_t)(cs + i) * p.nq + h];
    }
  };
  auto put = [&](int buf) {
    char* base = smem + buf * BUF;
    rq.store(base);
    ro.store(base + TB);
    if (threadIdx.x < BQ) {
      ((float*)(base + 2 * TB))[threadIdx.x] = sl * kLog2e;
      ((float*)(base + 2 * TB + BQ * 4))[threadIdx.x] = -sd;  // -D: the dP accumulator's start
    }
  };

  if (n_iter > 0) {
    rows_of(0);
    fetch(0);
    if (n_iter > 1) rows_of(1);
    put(0);
  }
  __syncthreads();
  for (int it = 0; it < n_iter; ++it) {
    const char* base = smem + (it & 1) * BUF;
    const char* Qs = base;
    const char* Os = base + TB;
    const float* Ls = (const float*)(base + 2 * TB);
    const float* Ds = Ls + BQ;
    const int i0 = (qb0 + it % per_head) * BQ;
    if (it + 1 < n_iter) {
      fetch(it + 1);
      if (it + 2 < n_iter) rows_of(it + 2);
    }
#pragma unroll
    for (int t2 = 0; t2 < BQ / 32; ++t2) {
      // 32 queries that all precede every key of this wave, or none of which exists: all masked,
      // nothing to add (wave-uniform)
      if (i0 + t2 * 32 + 31 < kw || i0 + t2 * 32 >= nb) continue;
      // dP accumulates onto -D_i (rows of the tile are queries 8*r4 + 4*hl + q), so that it comes
      // out of the MFMAs as dP - D
      f32x16 s, dp;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 d4 = *(const float4*)(Ds + t2 * 32 + 8 * r4 + 4 * hl);
        dp[4 * r4] = d4.x;
        dp[4 * r4 + 1] = d4.y;
        dp[4 * r4 + 2] = d4.z;
        dp[4 * r4 + 3] = d4.w;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 qa = frag_rows<D>(Qs, t2 * 32, kk, lane);
        const bf16x8 oa = frag_rows<D>(Os, t2 * 32, kk, lane);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[kk], dp, 0, 0, 0);
      }
      float pr[16], ds[16];
      float lv[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 l4 = *(const float4*)(Ls + t2 * 32 + 8 * r4 + 4 * hl);
        lv[4 * r4] = l4.x;
        lv[4 * r4 + 1] = l4.y;
        lv[4 * r4 + 2] = l4.z;
        lv[4 * r4 + 3] = l4.w;
      }
      // every query of this 32-block is valid and after every key of the wave: no mask
      if ((i0 + t2 * 32 >= kw + 31) && (i0 + t2 * 32 + 31 < nb) && kall) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pr[r] = fast_exp2(fmaf(s[r], p.scale_log2, -lv[r]));
          ds[r] = pr[r] * dp[r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = i0 + t2 * 32 + acc_row(r, lane);
          const float pv = (kvalid && i < nb && jk <= i) ? fast_exp2(fmaf(s[r], p.scale_log2, -lv[r])) : 0.f;
          pr[r] = pv;
          ds[r] = pv * dp[r];
        }
      }
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        const bf16x8 ap = to_frag(pr + 8 * step);
        const bf16x8 as = to_frag(ds + 8 * step);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const bf16x8 bo = frag_tr<D>(Os, t2 * 32 + 16 * step, t * 32, lane);
          const bf16x8 bq = frag_tr<D>(Qs, t2 * 32 + 16 * step, t * 32, lane);
          dva[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap, bo, dva[t], 0, 0, 0);
          dka[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as, bq, dka[t], 0, 0, 0);
        }
      }
    }
    if (it + 1 < n_iter) put((it + 1) & 1);
    __syncthreads();
  }
  if (p.HS == 1) {
    // the whole dK / dV of these keys: scale, rotary backward and bf16 stores here, through LDS
    // (each thread then takes 4 consecutive columns of a row, as the finalize kernel does)
    __syncthreads();  // every wavefront is done with the Q / dO tiles
    float* Ek = (float*)smem;
    float* Ev = Ek + BKV * LDF;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wave * 32 + acc_row(r, lane);
        Ek[row * LDF + t * 32 + l32] = dka[t][r] * p.scale;
        Ev[row * LDF + t * 32 + l32] = dva[t][r];
      }
    __syncthreads();
    const int half = p.rot >> 1;
    for (int q = threadIdx.x; q < BKV * (D / 4); q += 256) {
      const int row = q / (D / 4), m0 = (q % (D / 4)) * 4;
      const int j = k0 + row;
      if (j >= nb) continue;
      const float* ek = Ek + row * LDF;
      const float4 x4 = *(const float4*)(ek + m0);
      const float4 v4 = *(const float4*)(Ev + row * LDF + m0);
      const float xk[4] = {x4.x, x4.y, x4.z, x4.w};
      float out[4] = {x4.x, x4.y, x4.z, x4.w};
      if (m0 < p.rot) {
        const int pos = (p.idx ? p.idx[cs + j] : cs + j) % p.S;
        const float2* tab = p.rope + (int64_t)pos * half;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + e;
          if (m >= p.rot) continue;
          const bool lower = m < half;
          const float2 r = tab[lower ? m : m - half];
          const float y = ek[lower ? m + half : m - half];
          out[e] = lower ? xk[e] * r.x + y * r.y : xk[e] * r.x - y * r.y;
        }
      }
      const int64_t o = (int64_t)(cs + j);
      *(uint2*)(p.dk + o * p.ld_dk + g * D + m0) = make_uint2(pack2bf(out[0], out[1]), pack2bf(out[2], out[3]));
      *(uint2*)(p.dv + o * p.ld_dv + g * D + m0) = make_uint2(pack2bf(v4.x, v4.y), pack2bf(v4.z, v4.w));
    }
    return;
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
// Each thread finishes 4 consecutive columns of one row's [nkv x D] dK and dV: 16-byte loads of
// every slice (consecutive threads read consecutive 16-byte pieces of the row), the rotary partner
// columns (m +- rot/2 of the same head) read the same way when the 4 columns lie in one half and
// rot/2 is a multiple of 4, else element by element.  (One wavefront per row and head with 4-byte
// loads took 40 us for the Phi-1.5-shaped layer, 32 kv heads.)
template <int D>
__global__ __launch_bounds__(256) void attn_dkv_finalize_kernel(AttnParams p) {
  const int W = p.nkv * D;  // columns of a row
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)p.M_kept * (W / 4)) return;
  const int c = (int)(t / (W / 4));
  const int col = (int)(t % (W / 4)) * 4;  // first of this thread's columns within the row
  const int g = col / D, m0 = col % D;       // kv head and head column
  const int half = p.rot >> 1;
  const int64_t slice = (int64_t)p.M_kept * W;
  const int64_t base = (int64_t)c * W + col;
  float xk[4] = {0.f, 0.f, 0.f, 0.f}, xv[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.HS; ++s) {
    const float4 k4 = *(const float4*)(p.dkp + s * slice + base);
    const float4 v4 = *(const float4*)(p.dvp + s * slice + base);
    xk[0] += k4.x; xk[1] += k4.y; xk[2] += k4.z; xk[3] += k4.w;
    xv[0] += v4.x; xv[1] += v4.y; xv[2] += v4.z; xv[3] += v4.w;
  }
  float out[4] = {xk[0], xk[1], xk[2], xk[3]};
  if (m0 < p.rot) {
    const int pos = (p.idx ? p.idx[c] : c) % p.S;
    const float2* tab = p.rope + (int64_t)pos * half;
    const bool vec = (half & 3) == 0 && (m0 + 4 <= half || (m0 >= half && m0 + 4 <= p.rot));
    if (vec) {
      const bool lower = m0 < half;
      const int pm = lower ? m0 + half : m0 - half;
      float yk[4] = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < p.HS; ++s) {
        const float4 y4 = *(const float4*)(p.dkp + s * slice + (int64_t)c * W + g * D + pm);
        yk[0] += y4.x; yk[1] += y4.y; yk[2] += y4.z; yk[3] += y4.w;
      }
      const int tm = lower ? m0 : m0 - half;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 r = tab[tm + e];
        out[e] = lower ? xk[e] * r.x + yk[e] * r.y : xk[e] * r.x - yk[e] * r.y;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + e;
        if (m >= p.rot) continue;
        const bool lower = m < half;
        const int pm = lower ? m + half : m - half;
        float yk = 0.f;
        for (int s = 0; s < p.HS; ++s) yk += p.dkp[s * slice + (int64_t)c * W + g * D + pm];
        const float2 r = tab[lower ? m : m - half];
        out[e] = lower ? xk[e] * r.x + yk * r.y : xk[e] * r.x - yk * r.y;
      }
    }
  }
  *(uint2*)(p.dk + (int64_t)c * p.ld_dk + col) = make_uint2(pack2bf(out[0], out[1]), pack2bf(out[2], out[3]));
  *(uint2*)(p.dv + (int64_t)c * p.ld_dv + col) = make_uint2(pack2bf(xv[0], xv[1]), pack2bf(xv[2], xv[3]));
}

// ------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------
// Head slices of the dK / dV kernel.  Each slice adds a partial dK / dV buffer that the finalize
// kernel reads back, so the fewest slices that keep the GPU busy win: the fewest that give
// `target` workgroups, or fewer when short sequences allow - at least 512 workgroups, with the
// longest workgroup (the first key block of a sequence: its heads times the query tiles after it)
// at most 96 query-tile iterations.  Measured (TinyLlama-shaped layer, 40%): at S = 2048, 4
// slices instead of 8 took the finalize from 20.6 to 13.4 us with the dK/dV kernel unchanged; at
// S = 8192 (B = 2), 2 slices instead of 4 (308 iterations for the longest workgroup) made the
// dK/dV kernel 0.52 -> 0.65 ms.  COLLIDER_ATTN_MIN_WG overrides the target (tuning).
static int choose_hs(const collider_attn_cfg& c, int B, int S, int M_kept) {
  static const long target = [] {
    const char* e = getenv("COLLIDER_ATTN_MIN_WG");
    const long v = e ? atol(e) : 0;
    return v > 0 ? v : 1024L;
  }();
  const int G = c.n_q_heads / c.n_kv_heads;
  const long kblocks = (long)(M_kept + 127) / 128 + B;
  const long qtiles = (long)(std::min(S, M_kept) + 63) / 64;  // of the longest sequence, at most
  int hs_target = G;
  for (int hs = 1; hs <= G; ++hs) {
    if (G % hs) continue;
    if (kblocks * c.n_kv_heads * hs >= target) {
      hs_target = hs;
      break;
    }
  }
  for (int hs = 1; hs < hs_target; ++hs) {
    if (G % hs) continue;
    if (kblocks * c.n_kv_heads * hs >= 512 && (long)(G / hs) * qtiles <= 96) return hs;
  }
  return hs_target;
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
  const int hs = choose_hs(c, B, S, M_kept);
  w.D = cv.take<float>((size_t)M_kept * c.n_q_heads);
  // partial dK / dV slices (a single slice is finished inside the dK / dV kernel)
  const size_t part = hs > 1 ? (size_t)hs * M_kept * c.n_kv_heads * c.head_dim : 0;
  w.dkp = cv.take<float>(part);
  w.dvp = cv.take<float>(part);
  w.rope = cv.take<float>((size_t)S * (c.rot_dims > 0 ? c.rot_dims : 2));
  w.bytes = cv.bytes();
  return w;
}

size_t attn_workspace_bytes(const collider_attn_cfg& c, int B, int S, int M_kept) {
  return carve_attn(c, B, S, M_kept, nullptr).bytes;
}

collider_status attn_rope_prepare(const collider_attn_cfg& c, const collider_index& ix, void* ws,
                                  size_t ws_bytes, hipStream_t s) {
  if (ix.M_kept <= 0 || c.rot_dims <= 0) return COLLIDER_OK;
  AttnWs w = carve_attn(c, ix.B, ix.S, ix.M_kept, ws);
  if (ws_bytes < w.bytes) return COLLIDER_ERR_WORKSPACE;
  return launch_rope_table(w.rope, ix.S, c.rot_dims, c.rope_base, s);
}

collider_status attn_bwd(const collider_attn_cfg& c, const collider_index& ix,
                         const collider_attn_io& io, void* ws, size_t ws_bytes, hipStream_t s,
                         bool rope_ready, const int32_t* srcmap) {
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
  p.srcmap = srcmap;
  p.M_kept = Mk;
  p.S = S;
  p.nq = c.n_q_heads;
  p.nkv = c.n_kv_heads;
  p.G = c.n_q_heads / c.n_kv_heads;
  p.HS = choose_hs(c, B, S, Mk);
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
  if (c.rot_dims > 0 && !rope_ready) {
    st = launch_rope_table(w.rope, S, c.rot_dims, c.rope_base, s);
    if (st != COLLIDER_OK) return st;
  }
  const bool full = c.dmode == COLLIDER_ATTN_D_FULL;
  dim3 gq(c.n_q_heads, B, (S + 127) / 128), gk(c.n_kv_heads * p.HS, B, (S + 127) / 128);
  const int fin_blocks = (int)(((int64_t)Mk * c.n_kv_heads * c.head_dim / 4 + 255) / 256);
  if (c.head_dim == 64) {
    if (full)
      COLLIDER_LAUNCH("attn_dq", s, hipLaunchKernelGGL((attn_dq_kernel<64, true>), gq, dim3(256), 0, s, p));
    else
      COLLIDER_LAUNCH("attn_dq", s, hipLaunchKernelGGL((attn_dq_kernel<64, false>), gq, dim3(256), 0, s, p));
    COLLIDER_LAUNCH("attn_dkv", s, hipLaunchKernelGGL(attn_dkv_kernel<64>, gk, dim3(256), 0, s, p));
    if (p.HS > 1)
      COLLIDER_LAUNCH("attn_dkv_finalize", s,
                      hipLaunchKernelGGL(attn_dkv_finalize_kernel<64>, dim3(fin_blocks), dim3(256), 0, s, p));
  } else {
    if (full)
      COLLIDER_LAUNCH("attn_dq", s, hipLaunchKernelGGL((attn_dq_kernel<128, true>), gq, dim3(256), 0, s, p));
    else
      COLLIDER_LAUNCH("attn_dq", s, hipLaunchKernelGGL((attn_dq_kernel<128, false>), gq, dim3(256), 0, s, p));
    COLLIDER_LAUNCH("attn_dkv", s, hipLaunchKernelGGL(attn_dkv_kernel<128>, gk, dim3(256), 0, s, p));
    if (p.HS > 1)
      COLLIDER_LAUNCH("attn_dkv_finalize", s,
                      hipLaunchKernelGGL(attn_dkv_finalize_kernel<128>, dim3(fin_blocks), dim3(256), 0, s, p));
  }
  return last_hip_status();
}

}  // namespace collider
