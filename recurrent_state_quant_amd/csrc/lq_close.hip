// LeapQuant window close, fused last-token close, initial split and
// dequantize for gfx950: one 256-thread workgroup per state.
#include "lq_decode_one.h"

namespace lq {

// ---------------------------------------------------------------------------
// Window close and initial quantization: 256 threads (4 waves) per state.
//
// The rebuilt fp32 state lives in MFMA accumulators.  Wave w owns the rows
// of half h = w & 1 (64h .. 64h+63) and the columns of half ch = w >> 1
// (64ch .. 64ch+63) as 4 x 4 tiles of 16 x 16 (tile ct holds columns
// 64ch + 16ct .. +15).  Lane l (lr = l >> 4, lc = l & 15) holds, for each of
// its 4 columns 64ch + 16ct + lc, the 16 rows 64h + 16rt + 4lr + v (rt, v =
// 0..3), which are slots 16lr .. 16lr+15 of that column's segment in the
// code layout: codes are read and written as one 16-byte access per column,
// and one wave instruction covers 16 adjacent column segments (1 KiB of
// whole cache lines).
//   acc  = Gamma (deQ + comps)    (window of <= kChunk records: the MFMAs
//                                  accumulate onto it)
//   acc += K_w U                  (v_mfma_f32_16x16x4_f32 over the records,
//                                  newest chunk first: the decays are
//                                  running products)
// with K_w[i][row] = rho_i[row] k~_i[row].  Longer windows start from zero
// and add the boundary term after the last chunk.  Each record chunk is
// staged in LDS with 128-bit loads issued by all 256 threads before the
// first LDS write.
// Then (split_state): row norms, top-r rank selection, extraction, column
// absmax (smoothing scale), per-row absmax and int8 codes.  Row reductions
// combine the two column-half waves through LDS.
// ---------------------------------------------------------------------------
constexpr int kChunk = 16;  // records staged in LDS per MFMA pass

// Code byte B of `word` from x = q * inv (|x| <= 127): adding 1.5 * 2^23
// rounds x to the nearest integer, ties to even, and leaves that integer's
// two's-complement low byte in the low byte of the sum's bit pattern; the
// SDWA form of the add writes exactly that byte into byte B of `word` and
// keeps the other three.
template <int B>
__device__ __forceinline__ void pack_code(uint32_t &word, float x) {
  static_assert(B >= 0 && B < 4, "byte index");
  const float magic = 12582912.0f;
  if (B == 0)
    asm volatile("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
                 : "+v"(word) : "v"(x), "v"(magic));
  else if (B == 1)
    asm volatile("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
                 : "+v"(word) : "v"(x), "v"(magic));
  else if (B == 2)
    asm volatile("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
                 : "+v"(word) : "v"(x), "v"(magic));
  else
    asm volatile("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
                 : "+v"(word) : "v"(x), "v"(magic));
}

__device__ __forceinline__ float f4get(const float4 &x, int i) {
  return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
}

// Signed byte B of `word` as a float: one SDWA convert (the compiler
// otherwise extracts the byte with a shift or bit-field extract first).
template <int B>
__device__ __forceinline__ float sbyte_to_f32(uint32_t word) {
  static_assert(B >= 0 && B < 4, "byte index");
  float r;
  if (B == 0)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(word));
  else if (B == 1)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(word));
  else if (B == 2)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(word));
  else
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(word));
  return r;
}
// signed byte v of `word` (v a constant once loops are unrolled)
__device__ __forceinline__ float sbyte_to_f32(uint32_t word, int v) {
  return v == 0 ? sbyte_to_f32<0>(word) : v == 1 ? sbyte_to_f32<1>(word) : v == 2 ? sbyte_to_f32<2>(word)
                                                                        : sbyte_to_f32<3>(word);
}
__device__ __forceinline__ uint32_t u4get(const uint4 &x, int i) {
  return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
}

struct SplitLds {    // LDS used by the split (a6-a8), shared by both kernels
  float *part;       // [2][D] per column half: row norms^2, later row absmax
                     // (with red: [D], the rows' totals)
  int *sel;          // [D] compensator slot of a row or -1
  float *cmx;        // [8][D] column-max partials
  float *sig;        // [D] 1 / s_j
  float *inv;        // [D] 127 / m_i (0 for zero or extracted rows)
  // dense compensator tokens only, [16][D] each
  float *dq;         // keys K (row c: k_c)
  float *dw;         // W = K S (row c: w_c)
  float *dy;         // Y = S W^T (row c: column c of Y)
  // optional [D][kRedRow]: every lane's row partials, reduced by one thread
  // per row (in place of a DPP reduction chain per row and lane group)
  float *red;
};
// Row stride of the transposed partials: column half ch and lane lc at
// ch * 16 + lc; 36 puts the four rows 4 apart that one store instruction
// writes in distinct banks.
constexpr int kRedRow = 36;

constexpr float kMgsDrop = 2e-2f;  // relative projected norm at or below which a key is dropped

// Dense compensator tokens of the state in acc (r >= 1), after the top-r
// rows have set one-hot keys in L.dq: `iters` rounds of subspace iteration
// K <- MGS(S S^T K), then W = K S (w_c = S^T k_c), the keys and values
// written out, and the residual S - sum_c k_c w_c^T left in acc.  Partial
// sums of the two row halves (W) and of the two column halves (Y) meet in
// LDS: one half stores into a free [16][D] array, then all threads add.
__device__ __forceinline__ void dense_comp_split(floatx4 (&acc)[4][4], const SplitLds &L, float *comp_key,
                                                 float *comp_val, size_t s, int r, int iters) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int lr = lane >> 4, lc = lane & 15;
  const int h = w & 1, ch = w >> 1;
  const int rbase = 64 * h + 4 * lr;
  const int col0 = 64 * ch + lc;
  // dst[e] += src[e] for the r rows of [16][D] arrays, all threads
  auto add_halves = [&](float *dst, const float *src) {
    for (int e = tid; e < r * (D / 4); e += 256) {
      float4 x = reinterpret_cast<float4 *>(dst)[e];
      const float4 y = reinterpret_cast<const float4 *>(src)[e];
      x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
      reinterpret_cast<float4 *>(dst)[e] = x;
    }
  };
  for (int it = 0;; ++it) {
    // ---- W = K S: each lane sums its 16 rows of the half, lanes 16 and 32
    // apart hold the half's other rows; halves meet in dw (h = 0) + dy (h = 1)
    float *wdst = h == 0 ? L.dw : L.dy;
    for (int c = 0; c < r; ++c) {
      float pw[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float4 k4 = *reinterpret_cast<const float4 *>(L.dq + c * D + rbase + 16 * rt);
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) pw[ct] = fmaf(f4get(k4, v), acc[rt][ct][v], pw[ct]);
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        pw[ct] += __shfl_xor(pw[ct], 16);
        pw[ct] += __shfl_xor(pw[ct], 32);
      }
      if (lr == 0) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) wdst[c * D + col0 + 16 * ct] = pw[ct];
      }
    }
    __syncthreads();
    add_halves(L.dw, L.dy);
    __syncthreads();
    if (it == iters) break;
    // ---- Y = S W^T: each lane sums its 4 columns, the 16 lanes of a DPP
    // row hold the half's other columns; halves meet in dy (ch = 0) + dq
    // (ch = 1: the keys are not read again this round)
    float *ydst = ch == 0 ? L.dy : L.dq;
    for (int c = 0; c < r; ++c) {
      float wv[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) wv[ct] = L.dw[c * D + col0 + 16 * ct];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        float y[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float x = 0.f;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) x = fmaf(acc[rt][ct][v], wv[ct], x);
          y[v] = row16_sum(x);
        }
        if (lc == 0)
          *reinterpret_cast<float4 *>(ydst + c * D + rbase + 16 * rt) = make_float4(y[0], y[1], y[2], y[3]);
      }
    }
    __syncthreads();
    add_halves(L.dy, L.dq);
    __syncthreads();
    // ---- K = MGS(Y) on wave 0: lane l holds rows 2l and 2l+1
    if (w == 0) {
      for (int c = 0; c < r; ++c) {
        float2 v = *reinterpret_cast<const float2 *>(L.dy + c * D + 2 * lane);
        const float n0 = sqrtf(wave_sum(v.x * v.x + v.y * v.y));
        for (int c2 = 0; c2 < c; ++c2) {
          const float2 q = *reinterpret_cast<const float2 *>(L.dq + c2 * D + 2 * lane);
          const float d = wave_sum(q.x * v.x + q.y * v.y);
          v.x = fmaf(-d, q.x, v.x);
          v.y = fmaf(-d, q.y, v.y);
        }
        const float nv = sqrtf(wave_sum(v.x * v.x + v.y * v.y));
        const bool keep = nv > 0.f && nv > kMgsDrop * n0;
        *reinterpret_cast<float2 *>(L.dq + c * D + 2 * lane) =
            keep ? make_float2(v.x / nv, v.y / nv) : make_float2(0.f, 0.f);
      }
    }
    __syncthreads();
  }
  // ---- keys and values out; residual S - sum_c k_c w_c^T
  for (int e = tid; e < r * (D / 4); e += 256) {
    reinterpret_cast<float4 *>(comp_key + s * r * D)[e] = reinterpret_cast<const float4 *>(L.dq)[e];
    reinterpret_cast<float4 *>(comp_val + s * r * D)[e] = reinterpret_cast<const float4 *>(L.dw)[e];
  }
  for (int c = 0; c < r; ++c) {
    float wv[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) wv[ct] = L.dw[c * D + col0 + 16 * ct];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const float4 k4 = *reinterpret_cast<const float4 *>(L.dq + c * D + rbase + 16 * rt);
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rt][ct][v] = fmaf(-f4get(k4, v), wv[ct], acc[rt][ct][v]);
    }
  }
}

// a6-a8 on the fp32 state held in acc: row norms, top-r extraction (writes
// comp_idx, comp_val; with DENSE the dense tokens started from those rows,
// also comp_key), smoothing scales (col_scale), row scales (row_scale) and
// int8 codes, all for state s.  Ends with every LDS array consumed.
template <bool DENSE, bool TRED = false>
__device__ __forceinline__ void split_state(floatx4 (&acc)[4][4], const SplitLds &L, int8_t *codes,
                                            float *row_scale, float *col_scale, int32_t *comp_idx,
                                            float *comp_val, float *comp_key, size_t s, int r, int iters,
                                            unsigned flags) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int lr = lane >> 4, lc = lane & 15;
  const int h = w & 1, ch = w >> 1;
  const int rbase = 64 * h + 4 * lr;  // row of (rt, v) = rbase + 16 rt + v
  const int col0 = 64 * ch + lc;  // column of ct = col0 + 16 ct
  // ---- a6 row L2 norms (squared, fp32; two column-half partials, or with
  // L.red every lane's partials summed by one thread per row)
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float q = 0.f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) q = fmaf(acc[rt][ct][v], acc[rt][ct][v], q);
      if (TRED) {
        L.red[(rbase + 16 * rt + v) * kRedRow + 16 * ch + lc] = q;
      } else {
        q = row16_sum(q);
        if (lc == 0) L.part[ch * D + rbase + 16 * rt + v] = q;
      }
    }
  if (TRED) {
    __syncthreads();
    if (tid < D) {
      const float4 *pr = reinterpret_cast<const float4 *>(L.red + tid * kRedRow);
      float4 x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = pr[e];
      float t[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = (x[e].x + x[e].y) + (x[e].z + x[e].w);
      L.part[tid] = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
    }
  }
  if (tid < D) L.sel[tid] = -1;
  if (DENSE)
    for (int e = tid; e < r * D; e += 256) L.dq[e] = 0.f;
  __syncthreads();
  if (w == 0 && r > 0) {
    // iterative argmax on wave 0: lane l holds rows 2l and 2l+1; each round
    // takes the largest remaining norm, ties to the lower row index
    float n0 = TRED ? L.part[2 * lane] : L.part[2 * lane] + L.part[D + 2 * lane];
    float n1 = TRED ? L.part[2 * lane + 1] : L.part[2 * lane + 1] + L.part[D + 2 * lane + 1];
    for (int c = 0; c < r; ++c) {
      const bool pick1 = n1 > n0;  // equal norms keep the lower row
      const float best = pick1 ? n1 : n0;
      const float m = row16_max(best);
      const float mx = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0)),
                                   __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16))),
                             fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32)),
                                   __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48))));
      const unsigned long long hit = __ballot(best == mx && best >= 0.f);
      int wl, odd;
      if (hit) {
        wl = __ffsll((long long)hit) - 1;
        odd = __builtin_amdgcn_readlane((int)pick1, wl);
      } else {
        // only reachable with NaN norms: take the lowest row not yet picked
        const unsigned long long f0 = __ballot(n0 != -1.f), f1 = __ballot(n1 != -1.f);
        wl = __ffsll((long long)(f0 | f1)) - 1;
        odd = ((f0 >> wl) & 1ull) ? 0 : 1;
      }
      const int wrow = 2 * wl + odd;
      if (lane == wl) {
        if (odd) n1 = -1.f; else n0 = -1.f;
      }
      if (lane == 0) {
        if (DENSE) L.dq[c * D + wrow] = 1.f;  // one-hot start key
        else L.sel[wrow] = c;
        comp_idx[s * r + c] = wrow;
      }
    }
  }
  __syncthreads();

  // ---- extraction and a7 column absmax of the residual.  Extracted rows
  // are written out and zeroed in the lanes that hold them (a branch that
  // most waves skip), so they drop out of the column maxima and get row
  // scale 0 (hence codes 0) below.  DENSE: the dense tokens leave the
  // residual S - sum_c k_c w_c^T instead.
  if constexpr (DENSE) {
    if (r > 0) dense_comp_split(acc, L, comp_key, comp_val, s, r, iters);
  } else {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int4 sl4 = *reinterpret_cast<const int4 *>(L.sel + rbase + 16 * rt);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int sel = v == 0 ? sl4.x : v == 1 ? sl4.y : v == 2 ? sl4.z : sl4.w;
      if (sel >= 0) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) comp_val[(s * r + sel) * D + col0 + 16 * ct] = acc[rt][ct][v];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rt][ct][v] = 0.f;
      }
    }
  }
  }
  float cm[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    float m = 0.f;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) m = fmaxf(m, fabsf(acc[rt][ct][v]));
    cm[ct] = m;
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) L.cmx[(4 * h + lr) * D + col0 + 16 * ct] = cm[ct];
  __syncthreads();
  // per-column and per-row finishing work: with TRED on waves 2 and 3 (the
  // row norms and the top-r selection ran on waves 0 and 1), so that every
  // SIMD gets a share
  int fin = threadIdx.x;  // a fresh copy: values derived earlier would be kept live
  asm volatile("" : "+v"(fin));
  if (TRED) fin -= D;
  if ((unsigned)fin < (unsigned)D) {
    float m = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) m = fmaxf(m, L.cmx[g * D + fin]);
    const float sc = (flags & 1u) ? 1.f : (m > 0.f ? m : 1.f);
    col_scale[s * D + fin] = sc;
    L.sig[fin] = 1.f / sc;  // sigma_j, correctly rounded
  }
  __syncthreads();

  // ---- a8 smoothed residual q = R * sigma (in place), per-row absmax
  {
    float sig[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) sig[ct] = L.sig[col0 + 16 * ct];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float m = 0.f;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          acc[rt][ct][v] = acc[rt][ct][v] * sig[ct];
          m = fmaxf(m, fabsf(acc[rt][ct][v]));
        }
        if (TRED) {
          L.red[(rbase + 16 * rt + v) * kRedRow + 16 * ch + lc] = m;
        } else {
          m = row16_max_nn(m);
          if (lc == 0) L.part[ch * D + rbase + 16 * rt + v] = m;
        }
      }
  }
  __syncthreads();
  if ((unsigned)fin < (unsigned)D) {
    // row scale and its reciprocal, once per row (correctly rounded)
    float m;
    if (TRED) {
      const float4 *pr = reinterpret_cast<const float4 *>(L.red + fin * kRedRow);
      m = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 x = pr[e];
        m = fmaxf(m, fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w)));
      }
    } else {
      m = fmaxf(L.part[fin], L.part[D + fin]);
    }
    float a = 0.f, inv = 0.f;
    if (m > 0.f && L.sel[fin] < 0) {
      a = m / 127.f;
      inv = 127.f / m;
    }
    row_scale[s * D + fin] = a;
    L.inv[fin] = inv;
  }
  __syncthreads();
  // codes: rne(q * inv), one v_add_f32 per code (see pack_code); the
  // product is rounded on its own: no contraction into an FMA.
  {
    float4 iv[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) iv[rt] = *reinterpret_cast<const float4 *>(L.inv + rbase + 16 * rt);
    // the store offset from a fresh copy of the thread index: derived
    // values kept live from the kernel's start would cost registers
    int t2 = threadIdx.x;
    asm volatile("" : "+v"(t2));
    const int coff = ((t2 >> 6) & 1) * 8192 + (64 * (t2 >> 7) + (t2 & 15)) * 64 + 16 * ((t2 >> 4) & 3);
    int8_t *cdst = codes + s * D * D + coff;  // + 1024 ct
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma clang fp contract(off)
      uint32_t wd[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        wd[rt] = 0u;
        pack_code<0>(wd[rt], acc[rt][ct][0] * iv[rt].x);
        pack_code<1>(wd[rt], acc[rt][ct][1] * iv[rt].y);
        pack_code<2>(wd[rt], acc[rt][ct][2] * iv[rt].z);
        pack_code<3>(wd[rt], acc[rt][ct][3] * iv[rt].w);
      }
      __builtin_nontemporal_store(vu4{wd[0], wd[1], wd[2], wd[3]},
                                  reinterpret_cast<vu4 *>(cdst + ct * 1024));
    }
  }
}

// ---- a9: split a caller fp32 state (one workgroup per state)
template <bool DENSE>
__global__ __launch_bounds__(256) void quantize_kernel(const CloseArgs A) {
  const size_t s = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int lr = lane >> 4, lc = lane & 15;
  const int h = w & 1, ch = w >> 1;
  __shared__ float sh_part[2 * D], sh_sig[D];
  __shared__ __attribute__((aligned(16))) float sh_inv[D];
  __shared__ __attribute__((aligned(16))) int sh_sel[D];
  __shared__ __attribute__((aligned(16))) float sh_cmx[8 * D];
  __shared__ __attribute__((aligned(16))) float sh_dq[DENSE ? 16 * D : 4];
  __shared__ __attribute__((aligned(16))) float sh_dw[DENSE ? 16 * D : 4];
  __shared__ __attribute__((aligned(16))) float sh_dy[DENSE ? 16 * D : 4];
  __shared__ __attribute__((aligned(16))) float sh_red[DENSE ? 4 : D * kRedRow];
  floatx4 acc[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 64 * h + 16 * rt + 4 * lr + v;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        acc[rt][ct][v] = __builtin_nontemporal_load(A.S_in + (s * D + row) * D + 64 * ch + 16 * ct + lc);
    }
  const SplitLds L{sh_part, sh_sel, sh_cmx, sh_sig, sh_inv, sh_dq, sh_dw, sh_dy, DENSE ? nullptr : sh_red};
  split_state<DENSE, !DENSE>(acc, L, A.codes, A.row_scale, A.col_scale, A.comp_idx, A.comp_val, A.comp_key, s,
                             A.r, A.iters, A.flags);
}

// ---- a5-a8: window close, one workgroup per state.  With FUSED the
// workgroup first decodes the window's last token t from the rebuilt fp32
// state: the decay chain starts at alpha_t, so the accumulators hold
// D_t S_{t-1}; then z = (D_t S_{t-1})^T k_t = S_{t-1}^T b_t and
// (D_t S_{t-1})^T q_t = S_{t-1}^T (alpha_t q_t), u_t = v_t - z_b,
// o_t = z_q + (k~_t . q_t) u_t, and S_t = D_t S_{t-1} + k~_t u_t^T is split.
// KDA row closes are held to 128 VGPRs (4 waves per SIMD; their LDS fits 4
// workgroups per CU with the split's column maxima in the dead gate array):
// 12% faster than 3 workgroups per CU.
template <bool KDA, bool FUSED, bool DENSE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KDA && !DENSE ? 4 : 1))) void close_kernel(const CloseArgs A) {
  // the state: this workgroup's, or the listed slot of a compacted launch
  int slot = blockIdx.x;
  if (A.slots) {
    slot = A.slots[blockIdx.x];
    if ((unsigned)slot >= (unsigned)A.n) return;
  }
  const size_t s = slot;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int lr = lane >> 4, lc = lane & 15;
  const int h = w & 1, ch = w >> 1;
  const int rbase = 64 * h + 4 * lr;
  const int col0 = 64 * ch + lc;  // column of ct = col0 + 16 ct
  const int r = A.r, p = A.p;
  // per-slot record counts (continuous batching); a slot outside the valid
  // range is left untouched.  FUSED: len is the last token's position t.
  const int len = A.lens ? A.lens[s] : A.len;
  if (FUSED ? (len < 0 || len >= p) : (len < 1 || len > p)) return;
  if (A.only_last && len != p - 1) return;
  const size_t rec0 = s * p;

  __shared__ __attribute__((aligned(16))) float sh_K[kChunk * D];
  __shared__ __attribute__((aligned(16))) float sh_U[kChunk * D];
  __shared__ __attribute__((aligned(16))) float sh_g[KDA ? kChunk * D : kChunk];
  __shared__ __attribute__((aligned(16))) float sh_a[D];
  __shared__ __attribute__((aligned(16))) float sh_ag[D];  // a_i * Gamma_i
  __shared__ __attribute__((aligned(16))) float sh_gam[D];
  __shared__ __attribute__((aligned(16))) float sh_s[D];
  __shared__ __attribute__((aligned(16))) int sh_cslot[D];  // compensator slot of a row or -1
  __shared__ __attribute__((aligned(16))) float sh_comp[16 * D];  // compensator rows w_c
  // FUSED: the last token's k, q, k~ per row, u per column, k~ . q per wave
  __shared__ __attribute__((aligned(16))) float sh_tk[FUSED ? D : 4], sh_tq[FUSED ? D : 4];
  __shared__ __attribute__((aligned(16))) float sh_tkt[FUSED ? D : 4], sh_tu[FUSED ? D : 4];
  __shared__ float sh_kq[2];
  __shared__ float sh_part[2 * D], sh_sig[D];
  __shared__ __attribute__((aligned(16))) float sh_inv[D];
  __shared__ __attribute__((aligned(16))) int sh_sel[D];
  // column-max partials of the split; KDA: in the per-row gate array, dead by then
  __shared__ __attribute__((aligned(16))) float sh_cmx[KDA ? 4 : 8 * D];

  // this lane's code segments and the boundary state's scales, issued
  // first; the scales reach LDS with the first record chunk, so that no
  // wait separates these loads from the records'
  const int8_t *csrc = A.codes + s * D * D + h * 8192 + col0 * 64 + 16 * lr;
  uint4 cw[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) cw[ct] = ldu4(csrc + ct * 1024);
  float a_row = 0.f, s_col = 0.f;
  if (tid < D) {
    a_row = A.row_scale[s * D + tid];
    s_col = A.col_scale[s * D + tid];
    sh_cslot[tid] = -1;
  }

  floatx4 acc[4][4];
  // acc (+)= Gamma ((c (a Gamma)) s + compensator rows); Gamma from sh_gam
  auto add_boundary = [&](bool first) {
    float sv[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) sv[ct] = sh_s[col0 + 16 * ct];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const float4 ag4 = *reinterpret_cast<const float4 *>(sh_ag + rbase + 16 * rt);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float ag = f4get(ag4, v);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const float x = (float)(int8_t)(u4get(cw[ct], rt) >> (8 * v)) * (ag * sv[ct]);
          acc[rt][ct][v] = first ? x : acc[rt][ct][v] + x;
        }
      }
    }
    // compensator rows: the lanes holding row idx_c add Gamma_idx * w_c
    // (sh_cslot maps a row to its compensator slot or -1); dense tokens
    // join the contraction instead
    if (DENSE) return;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int4 cs4 = *reinterpret_cast<const int4 *>(sh_cslot + rbase + 16 * rt);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int c = v == 0 ? cs4.x : v == 1 ? cs4.y : v == 2 ? cs4.z : cs4.w;
        if (c >= 0) {
          const float G = sh_gam[rbase + 16 * rt + v];
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            acc[rt][ct][v] = fmaf(G, sh_comp[c * D + col0 + 16 * ct], acc[rt][ct][v]);
        }
      }
    }
  };

  // stage records lo .. hi-1 in LDS (zero-padded to a multiple of 4) and
  // fold the decays into K: sh_K[j] *= P, P *= gate_j, newest first.
  // FUSED: the first call also stages the last token's k, q, k~ (rows) and
  // v (columns), and starts the decay chain at alpha_t.
  float P = 1.f;  // running decay product for row tid (tid < D)
  auto stage = [&](int lo, int hi, bool first) {
    const int cnt = hi - lo, cnt4 = (cnt + 3) & ~3;
    __syncthreads();
    {
      // kChunk * D / 4 = 512 float4 per array: two per thread, all loads
      // of the chunk issued before the first LDS write
      static_assert(kChunk * D / 4 == 512, "staging assumes two float4 per thread");
      const float *su = A.buf_u + (rec0 + lo) * D;
      const float *sk = A.buf_k + (rec0 + lo) * D;
      const float *sg = A.buf_gate + (rec0 + lo) * D;
      float4 *du = reinterpret_cast<float4 *>(sh_U);
      float4 *dk = reinterpret_cast<float4 *>(sh_K);
      float4 *dg = reinterpret_cast<float4 *>(sh_g);
      const int nvec = cnt * (D / 4), npad = cnt4 * (D / 4);
      const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
      const int e0 = tid, e1 = tid + 256;
      // the compensator rows (r * 32 float4) come with the first chunk;
      // rows 8 .. r-1 (r > 8 only) follow it
      const int ncv = (first && !DENSE) ? r * (D / 4) : 0;
      float4 c0 = z4;
      if (e0 < ncv) c0 = ld4(A.comp_val + s * r * D + 4 * e0);
      float tk = 0.f, tq = 0.f, tv = 0.f, tx = 0.f, ta = 1.f;
      if (FUSED && first && tid < D) {
        tk = A.k[s * D + tid];
        tq = A.q[s * D + tid];
        tv = A.v[s * D + tid];
        // beta_t in even lanes and GDN's alpha_t in odd lanes: a lane-indexed
        // vector load, broadcast once the record loads are issued (as scalar
        // loads they would be waited for before those issue); KDA reads
        // alpha_t per row
        tx = *((lane & 1) ? A.alpha + (KDA ? s * D + tid : s) : A.beta + s);
        if (KDA) ta = A.alpha[s * D + tid];
      }
      float4 u0 = z4, u1 = z4, k0 = z4, k1 = z4, g0 = z4, g1 = z4;
      if (e0 < nvec) {
        u0 = ld4(su + 4 * e0);
        k0 = ld4(sk + 4 * e0);
        if (KDA) g0 = ld4(sg + 4 * e0);
      }
      if (e1 < nvec) {
        u1 = ld4(su + 4 * e1);
        k1 = ld4(sk + 4 * e1);
        if (KDA) g1 = ld4(sg + 4 * e1);
      }
      float gsc = 1.f;
      if (!KDA && tid < cnt) gsc = A.buf_gate[rec0 + lo + tid];
      if (e0 < npad) {
        du[e0] = u0;
        dk[e0] = k0;
        if (KDA && e0 < nvec) dg[e0] = g0;
      }
      if (e1 < npad) {
        du[e1] = u1;
        dk[e1] = k1;
        if (KDA && e1 < nvec) dg[e1] = g1;
      }
      if (!KDA && tid < cnt) sh_g[tid] = gsc;
      float4 *dc = reinterpret_cast<float4 *>(sh_comp);
      if (e0 < ncv) dc[e0] = c0;
      if (e1 < ncv) dc[e1] = ld4(A.comp_val + s * r * D + 4 * e1);
      if (first && tid < D) {
        sh_a[tid] = a_row;
        sh_s[tid] = s_col;
      }
      if (FUSED && first && tid < D) {
        const float tb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tx), 0));
        P = KDA ? ta : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tx), 1));
        sh_tk[tid] = (A.flags & 2u) ? 0.f : tk;  // b_t = 0 without the delta correction
        sh_tq[tid] = tq;
        sh_tkt[tid] = tb * tk;
        sh_tu[tid] = tv;  // v_t; replaced by u_t after the decode
      }
    }
    __syncthreads();
    if (tid < D) {
      for (int j = cnt - 1; j >= 0; --j) {
        sh_K[j * D + tid] *= P;
        P *= KDA ? sh_g[j * D + tid] : sh_g[j];
      }
    }
  };
  // acc += K_w U over the staged records
  auto contract = [&](int cnt) {
    const int cnt4 = (cnt + 3) & ~3;
    for (int ks = 0; ks < cnt4 / 4; ++ks) {
      const int kr = 4 * ks + lr;
      float a[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) a[rt] = sh_K[kr * D + 64 * h + 16 * rt + lc];
      float bb[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) bb[ct] = sh_U[kr * D + col0 + 16 * ct];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rt], bb[ct], acc[rt][ct], 0, 0, 0);
    }
  };
  auto set_gamma = [&]() {
    if (tid < D) {
      sh_gam[tid] = P;
      sh_ag[tid] = sh_a[tid] * P;
    }
    if (!DENSE && tid < r) {
      // comp_idx entries outside [0, dk) are ignored
      const int idx = A.comp_idx[s * r + tid];
      if ((unsigned)idx < (unsigned)D) sh_cslot[idx] = tid;
    }
    if (FUSED && tid < D) {
      const float kq = wave_sum(sh_tkt[tid] * sh_tq[tid]);  // waves 0 and 1, all lanes active
      if (lane == 0) sh_kq[w] = kq;
    }
    __syncthreads();
  };

  if (len <= kChunk) {
    // one chunk: Gamma is known before the contraction, so the boundary
    // term initialises the accumulators
    stage(0, len, true);
    set_gamma();
    add_boundary(true);
    contract(len);
  } else {
    // newest chunk first; the accumulators start at zero after its staging
    stage(len - kChunk, len, true);
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
    contract(kChunk);
    for (int hi = len - kChunk; hi > 0; hi -= kChunk) {
      const int lo = hi > kChunk ? hi - kChunk : 0;
      stage(lo, hi, false);
      __syncthreads();
      contract(hi - lo);
    }
    set_gamma();
    add_boundary(false);
  }
  if (DENSE && r > 0) {
    // dense compensator tokens: r more records of the contraction, written
    // before the window's first token: K column Gamma * k_c, U row w_c
    __syncthreads();  // every wave is done with the staged records
    {
      const int r4 = (r + 3) & ~3;
      float4 *dk = reinterpret_cast<float4 *>(sh_K);
      float4 *du = reinterpret_cast<float4 *>(sh_U);
      for (int e = tid; e < r4 * (D / 4); e += 256) {
        const int c = e >> 5, i4 = e & 31;
        float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), ww = kk;
        if (c < r) {
          kk = ld4(A.comp_key + (s * r + c) * D + 4 * i4);
          ww = ld4(A.comp_val + (s * r + c) * D + 4 * i4);
          const float4 g = *reinterpret_cast<const float4 *>(sh_gam + 4 * i4);
          kk.x *= g.x; kk.y *= g.y; kk.z *= g.z; kk.w *= g.w;
        }
        dk[e] = kk;
        du[e] = ww;
      }
    }
    __syncthreads();
    contract(r);
  }
  if (FUSED) {
    // z = acc^T k_t and acc^T q_t: each lane sums its 16 rows for its 4
    // columns; the 8 (row half, lane group) partials meet in LDS
    float zb[4] = {0.f, 0.f, 0.f, 0.f}, zq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const float4 k4 = *reinterpret_cast<const float4 *>(sh_tk + rbase + 16 * rt);
      const float4 q4 = *reinterpret_cast<const float4 *>(sh_tq + rbase + 16 * rt);
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          zb[ct] = fmaf(acc[rt][ct][v], f4get(k4, v), zb[ct]);
          zq[ct] = fmaf(acc[rt][ct][v], f4get(q4, v), zq[ct]);
        }
    }
    __syncthreads();  // every wave is done with sh_K
    float2 *zp = reinterpret_cast<float2 *>(sh_K);  // [8][D]
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) zp[(4 * h + lr) * D + col0 + 16 * ct] = make_float2(zb[ct], zq[ct]);
    __syncthreads();
    if (tid < D) {
      float b = 0.f, q = 0.f;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const float2 x = zp[g * D + tid];
        b += x.x;
        q += x.y;
      }
      const float u = sh_tu[tid] - b;
      __builtin_nontemporal_store(fmaf(sh_kq[0] + sh_kq[1], u, q), A.o + s * D + tid);
      sh_tu[tid] = u;
    }
    __syncthreads();
    // S_t = D_t S_{t-1} + k~_t u_t^T
    float uu[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) uu[ct] = sh_tu[col0 + 16 * ct];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const float4 kt4 = *reinterpret_cast<const float4 *>(sh_tkt + rbase + 16 * rt);
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rt][ct][v] = fmaf(f4get(kt4, v), uu[ct], acc[rt][ct][v]);
    }
  }
  // every read of this state's compensator rows is done before the split
  // overwrites them
  __syncthreads();
  const SplitLds L{sh_part, sh_sel, KDA ? sh_g : sh_cmx, sh_sig, sh_inv, sh_K, sh_U, sh_comp};
  split_state<DENSE>(acc, L, A.codes, A.row_scale, A.col_scale, A.comp_idx, A.comp_val, A.comp_key, s, r,
                     A.iters, A.flags);
}

// ---------------------------------------------------------------------------
// Window close for windows of at most 16 records with compensator rows
// (r <= 8): the form every full window of length 16 takes.  Same state
// layout, split and results as close_kernel; the rebuild's contraction K_w U
// runs on the bf16 matrix path instead of the fp32 one, which on gfx950
// occupies the SIMD for 32 cycles per 16x16x4 step and does not overlap the
// split's vector work.
//
// Each fp32 operand x is split into three bf16 parts, x = hi + mid + lo
// (each part the round-to-nearest-even bf16 of what the previous parts leave;
// the split is exact), and K_w U is accumulated in fp32 from the six cross
// products whose size is at least 2^-16 of |K||U|: hh + mh + hm + mm + hl +
// lh.  The dropped products mid.lo, lo.mid and lo.lo are below 2^-24 of
// |K_i||U_i| each, the size of one fp32 rounding of the product.  16 records
// of three parts fill the K = 32 slots of three v_mfma_f32_16x16x32_bf16 per
// output tile:
//   [Kh | Km] x [Uh ; Uh],   [Kh | Km] x [Um ; Um],   [Kh | Kl] x [Ul ; Uh]
// (48 matrix instructions of 16 cycles per wave instead of 64 of 32).
//
// Staging: threads 0..127 own key row i = tid: they load k~_j[i] of every
// record and the gates, fold the decays in registers (K_w[j][i] = rho_j[i]
// k~_j[i], newest record first, the chain starting at alpha_t for the fused
// last token) and write the row's parts; threads 128..255 own value column
// c = tid - 128 and write the parts of u_j[c].  Parts are stored transposed,
// [row][record] per part, so that each matrix operand is one 16-byte LDS
// read per lane: lane (i, kb) of an operand holds records 8 (kb & 1) .. +7
// of row (column) i of the part that k-block kb takes.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float fx2_t __attribute__((ext_vector_type(2)));

// the bf16 pair nearest to (x, y) (ties to even), as one 32-bit word
__device__ __forceinline__ uint32_t bf16_pair(float x, float y) {
  const bf16x2_t h = __builtin_convertvector((fx2_t){x, y}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}
// three-part split of (x, y): hi, mid, lo pairs; x = hi.x + mid.x + lo.x exactly
__device__ __forceinline__ void split3(float x, float y, uint32_t &hi, uint32_t &mid, uint32_t &lo) {
  hi = bf16_pair(x, y);
  x -= __uint_as_float(hi << 16);
  y -= __uint_as_float(hi & 0xFFFF0000u);
  mid = bf16_pair(x, y);
  x -= __uint_as_float(mid << 16);
  y -= __uint_as_float(mid & 0xFFFF0000u);
  lo = bf16_pair(x, y);
}

constexpr int kSplitRecs = 16;  // records per row of a split operand

// LDS of one close16 workgroup, carved from one buffer (byte offsets)
template <bool FUSED>
struct Close16Lds {
  static constexpr int kOps = 0;                                  // [2][3][D][16] bf16 split operands
  static constexpr int kAg = kOps + 2 * 3 * D * kSplitRecs * 2;   // [D] a_i * Gamma_i
  static constexpr int kGam = kAg + D * 4;                        // [D] Gamma_i
  static constexpr int kS = kGam + D * 4;                         // [D] s_j
  static constexpr int kCslot = kS + D * 4;                       // [D] compensator slot of a row or -1
  static constexpr int kComp = kCslot + D * 4;                    // [8][D] compensator rows
  static constexpr int kTok = kComp + 8 * D * 4;                  // FUSED: tk, tq, tkt, tu [D] each
  static constexpr int kKq = kTok + (FUSED ? 4 * D : 16) * 4;     // [2] (padded to 16 bytes)
  static constexpr int kPart = kKq + 16;                          // [2][D]
  static constexpr int kSig = kPart + 2 * D * 4;                  // [D]
  static constexpr int kInv = kSig + D * 4;                       // [D]
  static constexpr int kSel = kInv + D * 4;                       // [D]
  static constexpr int kBytes = kSel + D * 4;
  static_assert(2 * 3 * D * kSplitRecs * 2 >= (D * kRedRow + 8 * D) * 4, "scratch for the split's partials");
};

// The LDS arrays of one close16 workgroup
struct Close16Ptrs {
  uint16_t (*ops)[3][D][kSplitRecs];
  float *ag, *gam, *s;
  int *cslot;
  float *comp, *tk, *tq, *tkt, *tu, *kq, *part, *sig, *inv;
  int *sel;
};

// The arrays carved from one buffer of Close16Lds<FUSED>::kBytes
template <bool FUSED>
__device__ __forceinline__ Close16Ptrs close16_carve(uint8_t *smem) {
  using Lo = Close16Lds<FUSED>;
  Close16Ptrs P;
  P.ops = reinterpret_cast<uint16_t (*)[3][D][kSplitRecs]>(smem + Lo::kOps);
  P.ag = reinterpret_cast<float *>(smem + Lo::kAg);
  P.gam = reinterpret_cast<float *>(smem + Lo::kGam);
  P.s = reinterpret_cast<float *>(smem + Lo::kS);
  P.cslot = reinterpret_cast<int *>(smem + Lo::kCslot);
  P.comp = reinterpret_cast<float *>(smem + Lo::kComp);
  P.tk = reinterpret_cast<float *>(smem + Lo::kTok);
  P.tq = P.tk + (FUSED ? D : 4);
  P.tkt = P.tq + (FUSED ? D : 4);
  P.tu = P.tkt + (FUSED ? D : 4);
  P.kq = reinterpret_cast<float *>(smem + Lo::kKq);
  P.part = reinterpret_cast<float *>(smem + Lo::kPart);
  P.sig = reinterpret_cast<float *>(smem + Lo::kSig);
  P.inv = reinterpret_cast<float *>(smem + Lo::kInv);
  P.sel = reinterpret_cast<int *>(smem + Lo::kSel);
  return P;
}

// One workgroup per state (or listed slot): the close of p <= 16 records
// (FUSED: decoding the window's last token first), body in
// lq_close16_body.inc.
template <bool KDA, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void close16_kernel(const CloseArgs A) {
  int slot = blockIdx.x;
  if (A.slots) {
    slot = A.slots[blockIdx.x];
    if ((unsigned)slot >= (unsigned)A.n) return;
  }
  const int len = A.lens ? A.lens[slot] : A.len;
  if (FUSED ? (len < 0 || len >= A.p) : (len < 1 || len > A.p)) return;
  if (A.only_last && len != A.p - 1) return;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Close16Lds<FUSED>::kBytes];
  const size_t s = slot;
  const Close16Ptrs P = close16_carve<FUSED>(smem);
#include "lq_close16_body.inc"
}

// ---------------------------------------------------------------------------
// A continuous-batching token in one launch: count workgroups decode and
// close the listed slots whose window ends at this token (the fused close
// above, one workgroup per slot), the others decode four slots each (one
// wave per slot, the one-wave decode step with its own LDS) for every slot
// at positions 0 .. p-2.  The closes no longer form a launch of their own
// whose length is one workgroup's lifetime; they run among the decode
// steps, which keep memory busy around them.
// ---------------------------------------------------------------------------
// GDN: 127 VGPRs and 40,448 bytes of LDS, four workgroups per CU; KDA's
// decode body needs 154 VGPRs (three).
template <bool KDA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KDA ? 3 : 4))) void mixed_kernel(const MixedArgs M) {
  constexpr int kBytes = Close16Lds<true>::kBytes > 4 * kDecodeLdsBytes ? Close16Lds<true>::kBytes
                                                                          : 4 * kDecodeLdsBytes;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kBytes];
  // The close workgroups are spread evenly through the first half of the
  // grid (dispatch order): close i sits at position floor(i Tc / nc) of
  // the first Tc = max(T / 2, nc) of the T workgroups, so that about nc / Tc
  // of the resident workgroups are closes (VALU work) among decode steps
  // (memory streams), and the last closes (a close workgroup lives several
  // times as long as a decode step) finish before the decode steps do:
  // spread over the whole grid they extended the launch's tail (0.86 of
  // lockstep against 0.90).  Workgroup b < Tc is a close iff
  // ceil((b + 1) nc / Tc) > ceil(b nc / Tc); closes before it: ceil(b nc /
  // Tc), all nc of them from Tc on.
  const long long nc = M.c.n_launch;
  const long long T = gridDim.x, b = blockIdx.x;
  const long long Tc = T / 2 > nc ? T / 2 : nc;  // closes within the first half of the grid
  const long long before = b < Tc ? (b * nc + Tc - 1) / Tc : nc;
  const long long upto = b < Tc ? ((b + 1) * nc + Tc - 1) / Tc : nc;
  if (upto > before) {
    const int slot = M.c.slots[before];
    if ((unsigned)slot >= (unsigned)M.c.n) return;
    const int len = M.c.lens[slot];
    if (len != M.c.p - 1) return;
    const CloseArgs &A = M.c;
    const size_t s = slot;
    constexpr bool FUSED = true;
    const Close16Ptrs P = close16_carve<true>(smem);
#include "lq_close16_body.inc"
  } else {
    // whole waves leave here; the wave-local decode has no workgroup barrier
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
    const int s = 4 * (int)(b - before) + w;
    if (s >= M.d.n) return;
    const int t = M.d.pos[s];
    if (t < 0 || t >= M.d.p - 1) return;
    uint8_t *base = smem + w * kDecodeLdsBytes;
    float2 *gy = reinterpret_cast<float2 *>(base);
    float2 *hh = gy + D;
    float2 *hc = hh + 64;
    float *red = reinterpret_cast<float *>(hc + 16);
    // z and the digits share the record dots' transpose buffer
    const DecodeLds Ls{gy, hh, hc, reinterpret_cast<float2 *>(red), reinterpret_cast<uint8_t *>(red) + D * 8, red};
    const DecodeArgs &A = M.d;
    const int lane = threadIdx.x & 63;
    constexpr bool DENSE = false, WAVE = true, LONG = false;  // p <= 16
#include "lq_decode_body.inc"
  }
}

// Windows the bf16-split close takes: row compensators (r <= 8) and 4 to 16
// tokens.  Shorter windows take the fp32 close, whose contraction is sized
// to the record count, where the split's is a fixed 16-record tile: at
// p = 1 (the per-token baseline) that made the whole step 12% slower; at
// p = 4 the two closes run even.
static bool close16_covers(const CloseArgs &c) {
  return c.comp_key == nullptr && c.p >= 4 && c.p <= kSplitRecs && c.r <= 8;
}

// The single launch covers the windows the bf16 close takes, on slabs above
// kSmallSlab, where the decode steps it runs are the ones
// leapquant_decode_step_slots runs (the one-wave kernel): both forms then
// run the same kernels' code and give identical results.
bool mixed_supported(const CloseArgs &c) { return close16_covers(c) && c.n > kSmallSlab; }

hipError_t launch_mixed(const MixedArgs &a, bool kda, hipStream_t stream) {
  const int nd = (a.d.n + 3) / 4;
  const dim3 grid(a.c.n_launch + nd);
  if (kda)
    hipLaunchKernelGGL(mixed_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(mixed_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dequantize: S_out = deQ(codes, a, s) + compensator rows (fp32).  Thread
// (half hh, column j) reads the 64 code bytes of its column segment and
// writes column j of rows 64hh .. 64hh+63; the row scales and compensator
// data are staged in LDS once per state.
// ---------------------------------------------------------------------------
template <bool DENSE>
__global__ __launch_bounds__(256) void dequant_kernel(const DequantArgs A) {
  const size_t s = blockIdx.x;
  const int tid = threadIdx.x;
  const int j = tid & (D - 1), hh = tid >> 7;  // column j, row half hh
  const int r = A.r;
  __shared__ float sh_a[D];                      // row scales
  __shared__ int sh_cs[DENSE ? 1 : D];           // compensator slot of a row or -1
  __shared__ float sh_key[DENSE ? 16 * D : 1];   // dense keys [c][row]
  __shared__ float sh_val[16 * D];               // compensator rows [c][col]
  // every load first: this thread's 64 codes (4 x 16 bytes of one column
  // half), its column scale, then the per-state side data
  const uint4 *src = reinterpret_cast<const uint4 *>(A.codes + s * D * D + hh * 8192 + j * 64);
  uint4 cq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) cq[q] = src[q];
  const float sj = A.col_scale[s * D + j];
  if (tid < D) {
    sh_a[tid] = A.row_scale[s * D + tid];
    if (!DENSE) sh_cs[tid] = -1;
  }
  for (int e = tid; e < r * D; e += 256) {
    sh_val[e] = A.comp_val[s * r * D + e];
    if (DENSE) sh_key[e] = A.comp_key[s * r * D + e];
  }
  __syncthreads();
  if (!DENSE && tid < r) {
    const int idx = A.comp_idx[s * r + tid];  // entries outside [0, dk) are ignored
    if ((unsigned)idx < (unsigned)D) sh_cs[idx] = tid;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int slot = 16 * q + e;
      const int row = 64 * hh + code_slot(slot);  // the slot map is its own inverse
      const uint32_t wd = u4get(cq[q], e >> 2);
      float x = (float)(int8_t)(wd >> (8 * (e & 3))) * sh_a[row] * sj;
      if (DENSE) {
        for (int c = 0; c < r; ++c) x = fmaf(sh_key[c * D + row], sh_val[c * D + j], x);
      } else {
        const int c = sh_cs[row];
        if (c >= 0) x += sh_val[c * D + j];
      }
      A.S_out[(s * D + row) * D + j] = x;
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <bool FUSED>
hipError_t launch_close(const CloseArgs &a, bool kda, hipStream_t stream) {
  const dim3 grid(a.slots ? a.n_launch : a.n);
  const bool dense = a.comp_key != nullptr;
  if (close16_covers(a)) {
    if (kda)
      hipLaunchKernelGGL((close16_kernel<true, FUSED>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((close16_kernel<false, FUSED>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (kda && dense)
    hipLaunchKernelGGL((close_kernel<true, FUSED, true>), grid, dim3(256), 0, stream, a);
  else if (kda)
    hipLaunchKernelGGL((close_kernel<true, FUSED, false>), grid, dim3(256), 0, stream, a);
  else if (dense)
    hipLaunchKernelGGL((close_kernel<false, FUSED, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((close_kernel<false, FUSED, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_window_close(const CloseArgs &a, bool kda, hipStream_t stream) {
  return launch_close<false>(a, kda, stream);
}

hipError_t launch_decode_close(const CloseArgs &a, bool kda, hipStream_t stream) {
  return launch_close<true>(a, kda, stream);
}

hipError_t launch_quantize_state(const CloseArgs &a, hipStream_t stream) {
  if (a.comp_key)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3(a.n), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs &a, hipStream_t stream) {
  if (a.comp_key)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3(a.n), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lq
