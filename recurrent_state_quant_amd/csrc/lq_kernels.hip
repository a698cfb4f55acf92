// LeapQuant decode-path kernels for gfx950 (CDNA4, wave64).
//
// Pages cited (by title and section):
//   [EL] "LeapQuant: Efficient Linear Attention with Accurate Recurrent State
//        Quantization": Abstract, Figure 2, Figure 4, Appendix Table 4.
//   [TM] "LeapQuant trims the memory burden of linear-attention models":
//        "Quantize less often, protect the outliers".
//
// State layout per state s (dk = dv = 128):
//   codes     int8  [128][128] row-major (row = key channel i, col = value j)
//   row_scale fp32  [128] a_i,  col_scale fp32 [128] s_j
//   comp_idx  int32 [r],        comp_val  fp32 [r][128]
//   buffer    buf_gate [p] or [p][128], buf_k [p][128], buf_u [p][128]
//
// Windowed form used by the decode step (exact algebra of the recurrence of
// [EL] Table 4 started from the boundary state B and replayed through the
// buffered records; decays are plain products, no division):
//   Gamma = d_{t-1} ... d_0,   rho_i = d_{t-1} ... d_{i+1}   (per key row)
//   S_{t-1}^T y = B^T (Gamma * y) + sum_{i<t} u_i (k~_i . (rho_i * y))
//   B^T x       = s * (c^T (a * x)) + sum_c w_c x[idx_c]
//   u_t = v_t - S_{t-1}^T (alpha_t * k_t),
//   o_t = S_{t-1}^T (alpha_t * q_t) + (k~_t . q_t) u_t
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lq_kernels.h"

namespace lq {

constexpr int D = 128;  // dk == dv == 128

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float2 ld2(const float *p) {
  return *reinterpret_cast<const float2 *>(p);
}
__device__ __forceinline__ void st2(float *p, float2 v) {
  *reinterpret_cast<float2 *>(p) = v;
}

// DPP lane permutes (gfx9 encodings): quad_perm, row_half_mirror, row_mirror.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum / max over the 16 lanes of a DPP row; every lane of the row gets it.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror: the other quad of the half-row
  x += dpp<0x140>(x);  // row_mirror: the other half-row
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// ---------------------------------------------------------------------------
// Decode step: one wave per state.
//
// Lane l owns key rows / value columns 2l and 2l+1 for the vector work.  For
// the int8 GEMV it owns the 16-byte column chunk cc = l & 7 of rows
// rg + 8m (rg = l >> 3, m = 0..15): each of the 16 loads of the wave reads 8
// full rows (1 KiB, fully coalesced 128-bit loads) and both vectors
// (Gamma*alpha*k and Gamma*alpha*q, scaled by a_i) are accumulated from one
// pass over the codes.
// ---------------------------------------------------------------------------
constexpr int kRedStride = 33;   // padded row of the transposed partials
constexpr int kGemvStride = 260; // padded row of the GEMV partials (16B aligned)

template <bool KDA>
__global__ __launch_bounds__(64) void decode_step_kernel(const DecodeArgs A) {
  const int s = blockIdx.x;
  const int lane = threadIdx.x;
  const int t = A.t, p = A.p, r = A.r;

  __shared__ float2 sh_w[D];   // a_i * Gamma_i * (y_b, y_q)_i
  __shared__ float2 sh_gy[D];  // Gamma_i * (y_b, y_q)_i
  __shared__ float2 sh_h[64];  // record weights (h_b, h_q)
  __shared__ __attribute__((aligned(16))) float sh_red[64 * kRedStride];

  // ---- a3 stream first: the 16 KiB of int8 codes of this state
  const int cc = lane & 7, rg = lane >> 3;
  const uint4 *csrc =
      reinterpret_cast<const uint4 *>(A.codes + (size_t)s * D * D) + rg * 8 + cc;
  uint4 cv[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) cv[m] = csrc[m * 64];

  // ---- a1 token prep
  const size_t vo = (size_t)s * D + 2 * lane;
  const float2 kk = ld2(A.k + vo);
  const float2 qq = ld2(A.q + vo);
  const float2 vv = ld2(A.v + vo);
  const float bt = A.beta[s];
  float2 al;
  if (KDA) {
    al = ld2(A.alpha + vo);
  } else {
    const float a = A.alpha[s];
    al = make_float2(a, a);
  }
  const float2 kt = make_float2(bt * kk.x, bt * kk.y);
  const float2 yb = make_float2(al.x * kk.x, al.y * kk.y);
  const float2 yq = make_float2(al.x * qq.x, al.y * qq.y);
  const float kq = wave_sum(kt.x * qq.x + kt.y * qq.y);

  // ---- a2 history: suffix decay products and record dot products,
  // records visited from the newest (i = t-1) to the oldest.
  const size_t rec0 = (size_t)s * p;
  float Pg = 1.f;                   // GDN: rho_i (uniform)
  float2 Pk = make_float2(1.f, 1.f);  // KDA: rho_i for rows 2l, 2l+1
  for (int hi = t - 1; hi >= 0; hi -= 16) {
    const int cnt = hi + 1 < 16 ? hi + 1 : 16;
    for (int j = 0; j < cnt; ++j) {
      const int i = hi - j;
      const float2 ki = ld2(A.buf_k + (rec0 + i) * D + 2 * lane);
      float hb, hq;
      if (KDA) {
        const float2 kr = make_float2(ki.x * Pk.x, ki.y * Pk.y);
        hb = kr.x * yb.x + kr.y * yb.y;
        hq = kr.x * yq.x + kr.y * yq.y;
        const float2 g = ld2(A.buf_gate + (rec0 + i) * D + 2 * lane);
        Pk.x *= g.x;
        Pk.y *= g.y;
      } else {
        hb = (ki.x * yb.x + ki.y * yb.y) * Pg;
        hq = (ki.x * yq.x + ki.y * yq.y) * Pg;
        Pg *= A.buf_gate[rec0 + i];
      }
      sh_red[lane * kRedStride + 2 * j] = hb;
      sh_red[lane * kRedStride + 2 * j + 1] = hq;
    }
    __syncthreads();
    // transpose-reduce: value v = lane & 31 summed over one half of the lanes
    const int v = lane & 31, half = lane >> 5;
    float acc = 0.f;
    if (v < 2 * cnt) {
#pragma unroll 8
      for (int m = 0; m < 32; ++m) {
        const int src = 32 * half + ((m + 16 * half) & 31);
        acc += sh_red[src * kRedStride + v];
      }
    }
    acc += __shfl_xor(acc, 32);
    if (lane < 2 * cnt) {
      const int i = hi - (lane >> 1);
      reinterpret_cast<float *>(&sh_h[i])[lane & 1] = acc;
    }
    __syncthreads();
  }

  // ---- GEMV weights: a_i * Gamma_i * y_i
  {
    const float2 ar = ld2(A.row_scale + vo);
    const float2 G = KDA ? Pk : make_float2(Pg, Pg);
    const float2 gb = make_float2(G.x * yb.x, G.y * yb.y);
    const float2 gq = make_float2(G.x * yq.x, G.y * yq.y);
    sh_gy[2 * lane] = make_float2(gb.x, gq.x);
    sh_gy[2 * lane + 1] = make_float2(gb.y, gq.y);
    sh_w[2 * lane] = make_float2(ar.x * gb.x, ar.x * gq.x);
    sh_w[2 * lane + 1] = make_float2(ar.y * gb.y, ar.y * gq.y);
  }
  __syncthreads();

  // ---- a3 int8 GEMV: both vectors from one pass over the codes
  float accb[16], accq[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) accb[j] = accq[j] = 0.f;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const float2 w = sh_w[rg + 8 * m];
    const uint32_t wd[4] = {cv[m].x, cv[m].y, cv[m].z, cv[m].w};
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float c = (float)(int8_t)(wd[q4] >> (8 * b));
        accb[4 * q4 + b] = fmaf(c, w.x, accb[4 * q4 + b]);
        accq[4 * q4 + b] = fmaf(c, w.y, accq[4 * q4 + b]);
      }
    }
  }
  // reduce over the 8 row groups through LDS
  {
    float4 *dst = reinterpret_cast<float4 *>(sh_red + rg * kGemvStride + 16 * cc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[j] = make_float4(accb[4 * j], accb[4 * j + 1], accb[4 * j + 2], accb[4 * j + 3]);
      dst[32 + j] = make_float4(accq[4 * j], accq[4 * j + 1], accq[4 * j + 2], accq[4 * j + 3]);
    }
  }
  __syncthreads();
  float2 zb = make_float2(0.f, 0.f), zq = make_float2(0.f, 0.f);
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const float2 pb = *reinterpret_cast<const float2 *>(sh_red + g * kGemvStride + 2 * lane);
    const float2 pq = *reinterpret_cast<const float2 *>(sh_red + g * kGemvStride + 128 + 2 * lane);
    zb.x += pb.x; zb.y += pb.y;
    zq.x += pq.x; zq.y += pq.y;
  }

  // ---- a4 combine: column scales, compensator rows, buffered records
  {
    const float2 sc = ld2(A.col_scale + vo);
    zb.x *= sc.x; zb.y *= sc.y;
    zq.x *= sc.x; zq.y *= sc.y;
  }
  for (int c = 0; c < r; ++c) {
    const int idx = A.comp_idx[(size_t)s * r + c];
    if ((unsigned)idx < (unsigned)D) {
      const float2 g = sh_gy[idx];
      const float2 w = ld2(A.comp_val + ((size_t)s * r + c) * D + 2 * lane);
      zb.x = fmaf(w.x, g.x, zb.x); zb.y = fmaf(w.y, g.x, zb.y);
      zq.x = fmaf(w.x, g.y, zq.x); zq.y = fmaf(w.y, g.y, zq.y);
    }
  }
  for (int i = 0; i < t; ++i) {
    const float2 u = ld2(A.buf_u + (rec0 + i) * D + 2 * lane);
    const float2 h = sh_h[i];
    zb.x = fmaf(u.x, h.x, zb.x); zb.y = fmaf(u.y, h.x, zb.y);
    zq.x = fmaf(u.x, h.y, zq.x); zq.y = fmaf(u.y, h.y, zq.y);
  }
  const float2 ut = make_float2(vv.x - zb.x, vv.y - zb.y);
  const float2 ot = make_float2(fmaf(kq, ut.x, zq.x), fmaf(kq, ut.y, zq.y));
  st2(A.o + vo, ot);
  st2(A.buf_u + (rec0 + t) * D + 2 * lane, ut);
  st2(A.buf_k + (rec0 + t) * D + 2 * lane, kt);
  if (KDA) {
    st2(A.buf_gate + (rec0 + t) * D + 2 * lane, al);
  } else if (lane == 0) {
    A.buf_gate[rec0 + t] = al.x;
  }
}

// ---------------------------------------------------------------------------
// Window close / quantize: one 256-thread workgroup (4 waves) per state.
//
// The rebuilt fp32 state lives in MFMA accumulators.  Wave w owns rows
// 32w .. 32w+31 as two 16-row tiles; the 16 columns of tile ct map to value
// columns 8c'+ct, so lane l holds 8 rows (32w + 16rt + 4(l>>4) + v) x 8
// contiguous columns (8(l&15) .. +7): codes are read and written as 8-byte
// row segments, 16 lanes covering one 128-byte row.
//   S_len = Gamma * (deQ + comps)  (accumulator init)
//         + K_w U                  (v_mfma_f32_16x16x4_f32, K = records)
// with K_w[i][row] = rho_i[row] k~_i[row].
// Then: row L2 norms (DPP row reductions), top-r rank selection, extraction,
// column absmax (smoothing scale), per-row absmax and int8 codes.
// ---------------------------------------------------------------------------
constexpr int kChunk = 32;  // records staged in LDS per MFMA pass

template <bool KDA, bool FROM_FP32>
__global__ __launch_bounds__(256) void close_kernel(const CloseArgs A) {
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int lr = lane >> 4, lc = lane & 15;
  const int r = A.r;

  __shared__ __attribute__((aligned(16))) float sh_K[kChunk * D];
  __shared__ __attribute__((aligned(16))) float sh_U[kChunk * D];
  __shared__ float sh_G[D];
  __shared__ float sh_a[D];
  __shared__ __attribute__((aligned(16))) float sh_s[D];
  __shared__ float sh_norm[D];
  __shared__ int sh_sel[D];
  __shared__ int sh_oidx[16];
  __shared__ float sh_cm[4 * D];

  floatx4 acc[2][8];

  if (FROM_FP32) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 32 * w + 16 * rt + 4 * lr + v;
        const float4 *src =
            reinterpret_cast<const float4 *>(A.S_in + ((size_t)s * D + row) * D + 8 * lc);
        const float4 x0 = src[0], x1 = src[1];
        acc[rt][0][v] = x0.x; acc[rt][1][v] = x0.y; acc[rt][2][v] = x0.z; acc[rt][3][v] = x0.w;
        acc[rt][4][v] = x1.x; acc[rt][5][v] = x1.y; acc[rt][6][v] = x1.z; acc[rt][7][v] = x1.w;
      }
  } else {
    const int len = A.len, p = A.p;
    const size_t rec0 = (size_t)s * p;
    if (tid < D) {
      sh_a[tid] = A.row_scale[(size_t)s * D + tid];
      sh_s[tid] = A.col_scale[(size_t)s * D + tid];
      // Gamma for row tid: product of all len decays
      float P = 1.f;
      for (int i = len - 1; i >= 0; --i)
        P *= KDA ? A.buf_gate[(rec0 + i) * D + tid] : A.buf_gate[rec0 + i];
      sh_G[tid] = P;
    }
    if (tid < r) sh_oidx[tid] = A.comp_idx[(size_t)s * r + tid];
    __syncthreads();

    // accumulator init: Gamma * (c a s + compensator rows)
    float sv[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) sv[ct] = sh_s[8 * lc + ct];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 32 * w + 16 * rt + 4 * lr + v;
        const uint2 cw =
            *reinterpret_cast<const uint2 *>(A.codes + ((size_t)s * D + row) * D + 8 * lc);
        const float a = sh_a[row], G = sh_G[row];
        float x[8];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          x[b] = (float)(int8_t)(cw.x >> (8 * b)) * a * sv[b];
          x[4 + b] = (float)(int8_t)(cw.y >> (8 * b)) * a * sv[4 + b];
        }
        for (int c = 0; c < r; ++c) {
          if (sh_oidx[c] == row) {
            const float4 *wp = reinterpret_cast<const float4 *>(
                A.comp_val + ((size_t)s * r + c) * D + 8 * lc);
            const float4 w0 = wp[0], w1 = wp[1];
            x[0] += w0.x; x[1] += w0.y; x[2] += w0.z; x[3] += w0.w;
            x[4] += w1.x; x[5] += w1.y; x[6] += w1.z; x[7] += w1.w;
          }
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[rt][ct][v] = x[ct] * G;
      }

    // K_w U over the buffered records, kChunk records per LDS pass
    for (int c0 = 0; c0 < len; c0 += kChunk) {
      const int cnt = len - c0 < kChunk ? len - c0 : kChunk;
      const int cnt4 = (cnt + 3) & ~3;
      __syncthreads();
      {
        const float4 *su = reinterpret_cast<const float4 *>(A.buf_u + (rec0 + c0) * D);
        float4 *du = reinterpret_cast<float4 *>(sh_U);
        for (int e = tid; e < cnt4 * (D / 4); e += 256)
          du[e] = e < cnt * (D / 4) ? su[e] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if (tid < D) {
        // rho_i for row tid, i from the newest record down
        float P = 1.f;
        for (int i = len - 1; i >= c0; --i) {
          if (i < c0 + cnt) sh_K[(i - c0) * D + tid] = P * A.buf_k[(rec0 + i) * D + tid];
          P *= KDA ? A.buf_gate[(rec0 + i) * D + tid] : A.buf_gate[rec0 + i];
        }
        for (int i = cnt; i < cnt4; ++i) sh_K[i * D + tid] = 0.f;
      }
      __syncthreads();
      for (int ks = 0; ks < cnt4 / 4; ++ks) {
        const int kr = 4 * ks + lr;
        const float a0 = sh_K[kr * D + 32 * w + lc];
        const float a1 = sh_K[kr * D + 32 * w + 16 + lc];
        const float4 b0 = *reinterpret_cast<const float4 *>(sh_U + kr * D + 8 * lc);
        const float4 b1 = *reinterpret_cast<const float4 *>(sh_U + kr * D + 8 * lc + 4);
        const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          acc[0][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, bb[ct], acc[0][ct], 0, 0, 0);
          acc[1][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, bb[ct], acc[1][ct], 0, 0, 0);
        }
      }
    }
  }

  // ---- a6 row L2 norms and top-r selection
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float q = 0.f;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) q = fmaf(acc[rt][ct][v], acc[rt][ct][v], q);
      q = row16_sum(q);
      if (lc == 0) sh_norm[32 * w + 16 * rt + 4 * lr + v] = q;
    }
  __syncthreads();
  if (tid < D) {
    const float ni = sh_norm[tid];
    int rank = 0;
    for (int j = 0; j < D; ++j) {
      const float nj = sh_norm[j];
      rank += (nj > ni) || (nj == ni && j < tid);
    }
    const int sel = rank < r ? rank : -1;
    sh_sel[tid] = sel;
    if (sel >= 0) A.comp_idx[(size_t)s * r + sel] = tid;
  }
  __syncthreads();

  // ---- extraction and a7 column absmax of the residual
  float cm[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) cm[ct] = 0.f;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 32 * w + 16 * rt + 4 * lr + v;
      const int sel = sh_sel[row];
      if (sel >= 0) {
        float4 *wp = reinterpret_cast<float4 *>(A.comp_val + ((size_t)s * r + sel) * D + 8 * lc);
        wp[0] = make_float4(acc[rt][0][v], acc[rt][1][v], acc[rt][2][v], acc[rt][3][v]);
        wp[1] = make_float4(acc[rt][4][v], acc[rt][5][v], acc[rt][6][v], acc[rt][7][v]);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[rt][ct][v] = 0.f;
      }
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) cm[ct] = fmaxf(cm[ct], fabsf(acc[rt][ct][v]));
    }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    cm[ct] = fmaxf(cm[ct], __shfl_xor(cm[ct], 16));
    cm[ct] = fmaxf(cm[ct], __shfl_xor(cm[ct], 32));
  }
  if (lr == 0) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) sh_cm[w * D + 8 * lc + ct] = cm[ct];
  }
  __syncthreads();
  if (tid < D) {
    const float m = fmaxf(fmaxf(sh_cm[tid], sh_cm[D + tid]), fmaxf(sh_cm[2 * D + tid], sh_cm[3 * D + tid]));
    const float sc = (A.flags & 1u) ? 1.f : (m > 0.f ? m : 1.f);
    A.col_scale[(size_t)s * D + tid] = sc;
    sh_s[tid] = 1.f / sc;  // sigma_j, correctly rounded
  }
  __syncthreads();

  // ---- a8 per-row absmax and int8 codes
  float sig[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) sig[ct] = sh_s[8 * lc + ct];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 32 * w + 16 * rt + 4 * lr + v;
      float qv[8];
      float m = 0.f;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        qv[ct] = acc[rt][ct][v] * sig[ct];
        m = fmaxf(m, fabsf(qv[ct]));
      }
      m = row16_max(m);
      float a = 0.f, inv = 0.f;
      if (m > 0.f) {
        a = m / 127.f;
        inv = 127.f / m;
      }
      uint32_t pk[2] = {0u, 0u};
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        float x = rintf(qv[ct] * inv);
        x = fminf(fmaxf(x, -127.f), 127.f);
        const uint32_t byte = (uint32_t)((int)x) & 0xFFu;
        pk[ct >> 2] |= byte << (8 * (ct & 3));
      }
      *reinterpret_cast<uint2 *>(A.codes + ((size_t)s * D + row) * D + 8 * lc) =
          make_uint2(pk[0], pk[1]);
      if (lc == 0) A.row_scale[(size_t)s * D + row] = a;
    }
}

// ---------------------------------------------------------------------------
// Dequantize: S_out = deQ(codes, a, s) + compensator rows (fp32)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequant_kernel(const DequantArgs A) {
  const int s = blockIdx.x;
  const int row = threadIdx.x >> 1, h = threadIdx.x & 1;
  const float a = A.row_scale[(size_t)s * D + row];
  const int8_t *cr = A.codes + ((size_t)s * D + row) * D + 64 * h;
  const float *sc = A.col_scale + (size_t)s * D + 64 * h;
  float *out = A.S_out + ((size_t)s * D + row) * D + 64 * h;
  for (int j4 = 0; j4 < 16; ++j4) {
    const uint32_t cw = *reinterpret_cast<const uint32_t *>(cr + 4 * j4);
    const float4 s4 = *reinterpret_cast<const float4 *>(sc + 4 * j4);
    float4 x;
    x.x = (float)(int8_t)(cw) * a * s4.x;
    x.y = (float)(int8_t)(cw >> 8) * a * s4.y;
    x.z = (float)(int8_t)(cw >> 16) * a * s4.z;
    x.w = (float)(int8_t)(cw >> 24) * a * s4.w;
    for (int c = 0; c < A.r; ++c) {
      if (A.comp_idx[(size_t)s * A.r + c] == row) {
        const float4 w4 = *reinterpret_cast<const float4 *>(
            A.comp_val + ((size_t)s * A.r + c) * D + 64 * h + 4 * j4);
        x.x += w4.x; x.y += w4.y; x.z += w4.z; x.w += w4.w;
      }
    }
    *reinterpret_cast<float4 *>(out + 4 * j4) = x;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_decode_step(const DecodeArgs &a, bool kda, hipStream_t stream) {
  if (kda)
    hipLaunchKernelGGL(decode_step_kernel<true>, dim3(a.n), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_step_kernel<false>, dim3(a.n), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_window_close(const CloseArgs &a, bool kda, hipStream_t stream) {
  if (kda)
    hipLaunchKernelGGL((close_kernel<true, false>), dim3(a.n), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((close_kernel<false, false>), dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_quantize_state(const CloseArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((close_kernel<false, true>), dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(dequant_kernel, dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lq
