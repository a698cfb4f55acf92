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

typedef float vf2 __attribute__((ext_vector_type(2)));
typedef float vf4 __attribute__((ext_vector_type(4)));
typedef unsigned int vu2 __attribute__((ext_vector_type(2)));
typedef unsigned int vu4 __attribute__((ext_vector_type(4)));

// Streaming (nontemporal) accesses: every state array is touched once per
// launch and the working set of a launch is far larger than the caches, so
// loads and stores bypass cache retention (measured on MI355X: ~7.1 TB/s
// for nontemporal 16-byte streaming reads against ~6.3 TB/s for plain ones).
__device__ __forceinline__ float2 ld2(const float *p) {
  const vf2 t = __builtin_nontemporal_load(reinterpret_cast<const vf2 *>(p));
  return make_float2(t.x, t.y);
}
__device__ __forceinline__ float4 ld4(const float *p) {
  const vf4 t = __builtin_nontemporal_load(reinterpret_cast<const vf4 *>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint4 ldu4(const void *p) {
  const vu4 t = __builtin_nontemporal_load(reinterpret_cast<const vu4 *>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint2 ldu2(const void *p) {
  const vu2 t = __builtin_nontemporal_load(reinterpret_cast<const vu2 *>(p));
  return make_uint2(t.x, t.y);
}
__device__ __forceinline__ void st2(float *p, float2 v) {
  __builtin_nontemporal_store(vf2{v.x, v.y}, reinterpret_cast<vf2 *>(p));
}
__device__ __forceinline__ void st4(float *p, float4 v) {
  __builtin_nontemporal_store(vf4{v.x, v.y, v.z, v.w}, reinterpret_cast<vf4 *>(p));
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
//
// Memory-level parallelism: every load a phase needs is issued before the
// phase waits on any of them.  The token inputs, the newest kRecChunk
// records' k~ and gates, the first compensator rows and the whole code
// stream are in flight before the first wait; the records' u rows are
// issued after the record dots and arrive during the GEMV.  Record t's k~
// and gate depend only on the inputs and are stored as soon as they are
// known: stores left to the end of a wave hold it (and its registers) until
// they drain, which measurably lowers the streaming rate.
// ---------------------------------------------------------------------------
constexpr int kRecChunk = 16;    // records in flight per chunk
constexpr int kCompEarly = 4;    // compensator rows loaded with the records
constexpr int kRedStride = 33;   // odd row stride of the transposed partials: no bank conflicts
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

  const size_t vo = (size_t)s * D + 2 * lane;
  const size_t rec0 = (size_t)s * p;

  // ---- issue: token inputs, the newest record chunk, early compensators
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
  int hi = t;
  int lo = hi > kRecChunk ? hi - kRecChunk : 0;
  float2 kr[kRecChunk], gr[kRecChunk];
  float gs[kRecChunk];
  auto load_chunk = [&](int lo_, int cnt_) {
#pragma unroll
    for (int j = 0; j < kRecChunk; ++j) {
      if (j < cnt_) {
        const size_t rr = (rec0 + lo_ + j) * D + 2 * lane;
        kr[j] = ld2(A.buf_k + rr);
        if (KDA) gr[j] = ld2(A.buf_gate + rr);
        else gs[j] = A.buf_gate[rec0 + lo_ + j];
      }
    }
  };
  load_chunk(lo, hi - lo);
  int cidx[kCompEarly];
  float2 cw[kCompEarly];
#pragma unroll
  for (int c = 0; c < kCompEarly; ++c) {
    if (c < r) {
      cidx[c] = A.comp_idx[(size_t)s * r + c];
      cw[c] = ld2(A.comp_val + ((size_t)s * r + c) * D + 2 * lane);
    }
  }
  // ---- issue: the 16 KiB of int8 codes of this state
  const int cc = lane & 7, rg = lane >> 3;
  const uint4 *csrc =
      reinterpret_cast<const uint4 *>(A.codes + (size_t)s * D * D) + rg * 8 + cc;
  uint4 cv[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) cv[m] = ldu4(csrc + m * 64);

  // ---- a1 token prep; append k~_t and the gate of record t
  const float2 kt = make_float2(bt * kk.x, bt * kk.y);
  const float2 yb = make_float2(al.x * kk.x, al.y * kk.y);
  const float2 yq = make_float2(al.x * qq.x, al.y * qq.y);
  st2(A.buf_k + (rec0 + t) * D + 2 * lane, kt);
  if (KDA) {
    st2(A.buf_gate + (rec0 + t) * D + 2 * lane, al);
  } else if (lane == 0) {
    A.buf_gate[rec0 + t] = al.x;
  }
  const float kq = wave_sum(kt.x * qq.x + kt.y * qq.y);

  // ---- a2 history, newest records first: suffix decays rho_i and record
  // dots h_i = k~_i . (rho_i * y) for both vectors
  float Pg = 1.f;                     // GDN: rho (uniform)
  float2 Pk = make_float2(1.f, 1.f);  // KDA: rho for rows 2l, 2l+1
  while (hi > 0) {
    const int cnt = hi - lo;
#pragma unroll
    for (int j = kRecChunk - 1; j >= 0; --j) {
      if (j < cnt) {
        float hb, hq;
        if (KDA) {
          const float2 kw = make_float2(kr[j].x * Pk.x, kr[j].y * Pk.y);
          hb = kw.x * yb.x + kw.y * yb.y;
          hq = kw.x * yq.x + kw.y * yq.y;
          Pk.x *= gr[j].x;
          Pk.y *= gr[j].y;
        } else {
          hb = (kr[j].x * yb.x + kr[j].y * yb.y) * Pg;
          hq = (kr[j].x * yq.x + kr[j].y * yq.y) * Pg;
          Pg *= gs[j];
        }
        sh_red[lane * kRedStride + 2 * j] = hb;
        sh_red[lane * kRedStride + 2 * j + 1] = hq;
      }
    }
    __syncthreads();
    // transpose-reduce: value v = lane & 31 summed over one half of the lanes
    {
      const int v = lane & 31, half = lane >> 5;
      float acc = 0.f;
      if (v < 2 * cnt) {
#pragma unroll 8
        for (int m = 0; m < 32; ++m) acc += sh_red[(32 * half + m) * kRedStride + v];
      }
      acc += __shfl_xor(acc, 32);
      if (lane < 2 * cnt) reinterpret_cast<float *>(&sh_h[lo + (lane >> 1)])[lane & 1] = acc;
    }
    __syncthreads();
    hi = lo;
    lo = hi > kRecChunk ? hi - kRecChunk : 0;
    if (hi > 0) load_chunk(lo, hi - lo);
  }
  // U of the newest chunk, in flight during the GEMV
  const int ulo = t > kRecChunk ? t - kRecChunk : 0;
  float2 ur[kRecChunk];
#pragma unroll
  for (int j = 0; j < kRecChunk; ++j)
    if (j < t - ulo) ur[j] = ld2(A.buf_u + (rec0 + ulo + j) * D + 2 * lane);

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
  // (sum_i u_i h_i: the newest chunk from registers, older ones streamed)
  {
    const float2 sc = ld2(A.col_scale + vo);
    zb.x *= sc.x; zb.y *= sc.y;
    zq.x *= sc.x; zq.y *= sc.y;
  }
#pragma unroll
  for (int c = 0; c < kCompEarly; ++c) {
    if (c < r && (unsigned)cidx[c] < (unsigned)D) {
      const float2 g = sh_gy[cidx[c]];
      zb.x = fmaf(cw[c].x, g.x, zb.x); zb.y = fmaf(cw[c].y, g.x, zb.y);
      zq.x = fmaf(cw[c].x, g.y, zq.x); zq.y = fmaf(cw[c].y, g.y, zq.y);
    }
  }
  for (int c = kCompEarly; c < r; ++c) {
    const int idx = A.comp_idx[(size_t)s * r + c];
    if ((unsigned)idx < (unsigned)D) {
      const float2 g = sh_gy[idx];
      const float2 w = ld2(A.comp_val + ((size_t)s * r + c) * D + 2 * lane);
      zb.x = fmaf(w.x, g.x, zb.x); zb.y = fmaf(w.y, g.x, zb.y);
      zq.x = fmaf(w.x, g.y, zq.x); zq.y = fmaf(w.y, g.y, zq.y);
    }
  }
  {
    float2 zub = make_float2(0.f, 0.f), zuq = make_float2(0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kRecChunk; ++j) {
      if (j < t - ulo) {
        const float2 h = sh_h[ulo + j];
        zub.x = fmaf(ur[j].x, h.x, zub.x); zub.y = fmaf(ur[j].y, h.x, zub.y);
        zuq.x = fmaf(ur[j].x, h.y, zuq.x); zuq.y = fmaf(ur[j].y, h.y, zuq.y);
      }
    }
    for (int i = 0; i < ulo; ++i) {
      const float2 u = ld2(A.buf_u + (rec0 + i) * D + 2 * lane);
      const float2 h = sh_h[i];
      zub.x = fmaf(u.x, h.x, zub.x); zub.y = fmaf(u.y, h.x, zub.y);
      zuq.x = fmaf(u.x, h.y, zuq.x); zuq.y = fmaf(u.y, h.y, zuq.y);
    }
    zb.x += zub.x; zb.y += zub.y;
    zq.x += zuq.x; zq.y += zuq.y;
  }
  const float2 ut = make_float2(vv.x - zb.x, vv.y - zb.y);
  const float2 ot = make_float2(fmaf(kq, ut.x, zq.x), fmaf(kq, ut.y, zq.y));
  st2(A.o + vo, ot);
  st2(A.buf_u + (rec0 + t) * D + 2 * lane, ut);
}

// ---------------------------------------------------------------------------
// Window close and initial quantization: 256 threads (4 waves) per state.
//
// The fp32 state lives in MFMA accumulator registers.  Wave w owns rows
// 32w .. 32w+31 as two 16-row tiles; the 16 columns of tile ct map to value
// columns 8c'+ct, so lane l holds 8 rows (32w + 16rt + 4(l>>4) + v) x 8
// contiguous columns (8(l&15) .. +7): codes are read and written as 8-byte
// row segments, 16 lanes covering one 128-byte row.
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

struct SplitLds {    // LDS used by the split (a6-a8), shared by both kernels
  float *norm;       // [D] row norms^2, later row absmax
  int *sel;          // [D] compensator slot of a row or -1
  float *cmx;        // [16 * D] column-max partials
  float *sig;        // [D] 1 / s_j
  float *inv;        // [D] 127 / m_i (0 for zero or extracted rows)
};

// a6-a8 on the fp32 state held in acc: row norms, top-r extraction (writes
// comp_idx, comp_val), smoothing scales (col_scale), row scales (row_scale)
// and int8 codes, all for state s.  Ends with every LDS array consumed.
__device__ __forceinline__ void split_state(floatx4 (&acc)[2][8], const SplitLds &L, int8_t *codes,
                                            float *row_scale, float *col_scale, int32_t *comp_idx,
                                            float *comp_val, size_t s, int r, unsigned flags) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int lr = lane >> 4, lc = lane & 15;
  // ---- a6 row L2 norms (squared, fp32) and top-r selection
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float q = 0.f;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) q = fmaf(acc[rt][ct][v], acc[rt][ct][v], q);
      q = row16_sum(q);
      if (lc == 0) L.norm[32 * w + 16 * rt + 4 * lr + v] = q;
    }
  if (tid < D) L.sel[tid] = -1;
  __syncthreads();
  if (w == 0 && r > 0) {
    // iterative argmax on wave 0: lane l holds rows 2l and 2l+1; each round
    // takes the largest remaining norm, ties to the lower row index
    float n0 = L.norm[2 * lane], n1 = L.norm[2 * lane + 1];
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
        L.sel[wrow] = c;
        comp_idx[s * r + c] = wrow;
      }
    }
  }
  __syncthreads();

  // ---- extraction and a7 column absmax of the residual.  Extracted rows
  // are not zeroed in registers: they are left out of the column maxima
  // here and get row scale 0 (hence codes 0) below.
  float cm[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) cm[ct] = 0.f;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 32 * w + 16 * rt + 4 * lr + v;
      const int sel = L.sel[row];
      if (sel >= 0) {
        float *wp = comp_val + (s * r + sel) * D + 8 * lc;
        st4(wp, make_float4(acc[rt][0][v], acc[rt][1][v], acc[rt][2][v], acc[rt][3][v]));
        st4(wp + 4, make_float4(acc[rt][4][v], acc[rt][5][v], acc[rt][6][v], acc[rt][7][v]));
      }
      const float keep = sel < 0 ? 1.f : 0.f;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) cm[ct] = fmaxf(cm[ct], fabsf(acc[rt][ct][v]) * keep);
    }
  {
    float4 *dst = reinterpret_cast<float4 *>(L.cmx + (4 * w + lr) * D + 8 * lc);
    dst[0] = make_float4(cm[0], cm[1], cm[2], cm[3]);
    dst[1] = make_float4(cm[4], cm[5], cm[6], cm[7]);
  }
  __syncthreads();
  if (tid < D) {
    float m = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) m = fmaxf(m, L.cmx[g * D + tid]);
    const float sc = (flags & 1u) ? 1.f : (m > 0.f ? m : 1.f);
    col_scale[s * D + tid] = sc;
    L.sig[tid] = 1.f / sc;  // sigma_j, correctly rounded
  }
  __syncthreads();

  // ---- a8 smoothed residual q = R * sigma (in place), per-row absmax
  {
    float sig[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) sig[ct] = L.sig[8 * lc + ct];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float m = 0.f;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          acc[rt][ct][v] = acc[rt][ct][v] * sig[ct];
          m = fmaxf(m, fabsf(acc[rt][ct][v]));
        }
        m = row16_max(m);
        if (lc == 0) L.norm[32 * w + 16 * rt + 4 * lr + v] = m;
      }
  }
  __syncthreads();
  if (tid < D) {
    // row scale and its reciprocal, once per row (correctly rounded)
    const float m = L.norm[tid];
    float a = 0.f, inv = 0.f;
    if (m > 0.f && L.sel[tid] < 0) {
      a = m / 127.f;
      inv = 127.f / m;
    }
    row_scale[s * D + tid] = a;
    L.inv[tid] = inv;
  }
  __syncthreads();
  // codes: rne(q * inv), one v_add_f32 per code (see pack_code); the
  // product is rounded on its own: no contraction into an FMA.
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
#pragma clang fp contract(off)
      const int row = 32 * w + 16 * rt + 4 * lr + v;
      const float inv = L.inv[row];
      uint32_t w0 = 0u, w1 = 0u;
      pack_code<0>(w0, acc[rt][0][v] * inv);
      pack_code<1>(w0, acc[rt][1][v] * inv);
      pack_code<2>(w0, acc[rt][2][v] * inv);
      pack_code<3>(w0, acc[rt][3][v] * inv);
      pack_code<0>(w1, acc[rt][4][v] * inv);
      pack_code<1>(w1, acc[rt][5][v] * inv);
      pack_code<2>(w1, acc[rt][6][v] * inv);
      pack_code<3>(w1, acc[rt][7][v] * inv);
      __builtin_nontemporal_store(vu2{w0, w1},
                                  reinterpret_cast<vu2 *>(codes + (s * D + row) * D + 8 * lc));
    }
}

// ---- a9: split a caller fp32 state (one workgroup per state)
__global__ __launch_bounds__(256) void quantize_kernel(const CloseArgs A) {
  const size_t s = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int lr = lane >> 4, lc = lane & 15;
  __shared__ float sh_norm[D], sh_sig[D], sh_inv[D];
  __shared__ int sh_sel[D];
  __shared__ __attribute__((aligned(16))) float sh_cmx[16 * D];
  floatx4 acc[2][8];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 32 * w + 16 * rt + 4 * lr + v;
      const float *src = A.S_in + (s * D + row) * D + 8 * lc;
      const float4 x0 = ld4(src), x1 = ld4(src + 4);
      acc[rt][0][v] = x0.x; acc[rt][1][v] = x0.y; acc[rt][2][v] = x0.z; acc[rt][3][v] = x0.w;
      acc[rt][4][v] = x1.x; acc[rt][5][v] = x1.y; acc[rt][6][v] = x1.z; acc[rt][7][v] = x1.w;
    }
  const SplitLds L{sh_norm, sh_sel, sh_cmx, sh_sig, sh_inv};
  split_state(acc, L, A.codes, A.row_scale, A.col_scale, A.comp_idx, A.comp_val, s, A.r, A.flags);
}

// ---- a5-a8: window close, one workgroup per state.
//   acc  = Gamma (c (a s)) + Gamma comps   (window of <= kChunk records:
//                                          the MFMAs accumulate onto it)
//   acc += K_w U                           (v_mfma_f32_16x16x4_f32 over the
//                                          records, newest chunk first: the
//                                          decays are running products)
// with K_w[i][row] = rho_i[row] k~_i[row].  Longer windows start from zero
// and add the boundary term after the last chunk.  Each record chunk is
// staged in LDS with 128-bit loads issued by all 256 threads before the
// first LDS write.
template <bool KDA>
__global__ __launch_bounds__(256) void close_kernel(const CloseArgs A) {
  const size_t s = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int lr = lane >> 4, lc = lane & 15;
  const int r = A.r, len = A.len, p = A.p;
  const size_t rec0 = s * p;

  __shared__ __attribute__((aligned(16))) float sh_K[kChunk * D];
  __shared__ __attribute__((aligned(16))) float sh_U[kChunk * D];
  __shared__ __attribute__((aligned(16))) float sh_g[KDA ? kChunk * D : kChunk];
  __shared__ float sh_a[D], sh_gam[D];
  __shared__ __attribute__((aligned(16))) float sh_s[D];
  __shared__ int sh_oidx[16];
  __shared__ float sh_norm[D], sh_sig[D], sh_inv[D];
  __shared__ int sh_sel[D];
  __shared__ __attribute__((aligned(16))) float sh_cmx[16 * D];

  // boundary-state side data and this lane's code segments, issued first
  if (tid < D) {
    sh_a[tid] = A.row_scale[s * D + tid];
    sh_s[tid] = A.col_scale[s * D + tid];
  }
  if (tid < r) sh_oidx[tid] = A.comp_idx[s * r + tid];
  uint2 cw[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 32 * w + 16 * rt + 4 * lr + v;
      cw[rt][v] = ldu2(A.codes + (s * D + row) * D + 8 * lc);
    }

  floatx4 acc[2][8];
  // acc += Gamma ((c (a Gamma)) s + compensator rows); Gamma from sh_gam
  auto add_boundary = [&](bool first) {
    float sv[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) sv[ct] = sh_s[8 * lc + ct];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 32 * w + 16 * rt + 4 * lr + v;
        const float G = sh_gam[row];
        const float aG = sh_a[row] * G;
        float x[8];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          x[b] = (float)(int8_t)(cw[rt][v].x >> (8 * b)) * (aG * sv[b]);
          x[4 + b] = (float)(int8_t)(cw[rt][v].y >> (8 * b)) * (aG * sv[4 + b]);
        }
        for (int c = 0; c < r; ++c) {
          if (sh_oidx[c] == row) {
            const float *wp = A.comp_val + (s * r + c) * D + 8 * lc;
            const float4 w0 = ld4(wp), w1 = ld4(wp + 4);
            x[0] = fmaf(G, w0.x, x[0]); x[1] = fmaf(G, w0.y, x[1]);
            x[2] = fmaf(G, w0.z, x[2]); x[3] = fmaf(G, w0.w, x[3]);
            x[4] = fmaf(G, w1.x, x[4]); x[5] = fmaf(G, w1.y, x[5]);
            x[6] = fmaf(G, w1.z, x[6]); x[7] = fmaf(G, w1.w, x[7]);
          }
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[rt][ct][v] = first ? x[ct] : acc[rt][ct][v] + x[ct];
      }
  };

  // stage records lo .. hi-1 in LDS (zero-padded to a multiple of 4) and
  // fold the decays into K: sh_K[j] *= P, P *= gate_j, newest first
  float P = 1.f;  // running decay product for row tid (tid < D)
  auto stage = [&](int lo, int hi) {
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
  };

  if (len <= kChunk) {
    // one chunk: Gamma is known before the contraction, so the boundary
    // term initialises the accumulators
    stage(0, len);
    if (tid < D) sh_gam[tid] = P;
    __syncthreads();
    add_boundary(true);
    contract(len);
  } else {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) acc[rt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int hi = len; hi > 0; hi -= kChunk) {
      const int lo = hi > kChunk ? hi - kChunk : 0;
      stage(lo, hi);
      __syncthreads();
      contract(hi - lo);
    }
    if (tid < D) sh_gam[tid] = P;
    __syncthreads();
    add_boundary(false);
  }
  // every read of this state's compensator rows is done before the split
  // overwrites them
  __syncthreads();
  const SplitLds L{sh_norm, sh_sel, sh_cmx, sh_sig, sh_inv};
  split_state(acc, L, A.codes, A.row_scale, A.col_scale, A.comp_idx, A.comp_val, s, r, A.flags);
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
    hipLaunchKernelGGL(close_kernel<true>, dim3(a.n), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(close_kernel<false>, dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_quantize_state(const CloseArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(quantize_kernel, dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(dequant_kernel, dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lq
