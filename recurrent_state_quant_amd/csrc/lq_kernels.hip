// LeapQuant decode-path kernels for gfx950 (CDNA4, wave64).
//
// Pages cited (by title and section):
//   [EL] "LeapQuant: Efficient Linear Attention with Accurate Recurrent State
//        Quantization": Abstract, Figure 2, Figure 4, Appendix Table 4.
//   [TM] "LeapQuant trims the memory burden of linear-attention models":
//        "Quantize less often, protect the outliers".
//
// State layout per state s (dk = dv = 128):
//   codes     int8  16 KiB, column-major in two 64-row halves: code (i, j) at
//                   byte (i >> 6) * 8192 + j * 64 + slot(i & 63), with
//                   slot(x) = (x & 0x0C) << 2 | (x & 0x30) >> 2 | (x & 3)
//                   (the two 2-bit fields above the lowest two swapped)
//   row_scale fp32  [128] a_i,  col_scale fp32 [128] s_j
//   comp_idx  int32 [r],        comp_val  fp32 [r][128]
//   buffer    buf_gate [p] or [p][128], buf_k [p][128], buf_u [p][128]
// The code layout serves both kernels with 16-byte accesses: in the decode
// GEMV one lane's 16 bytes are the 16 rows of one column that an int8 MFMA
// lane consumes, and in the window close they are the 16 rows of one column
// that one lane holds in its MFMA accumulators.
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
// Every pattern used reads a lane that exists, so bound_ctrl is irrelevant;
// setting it lets the compiler fold the move into the consuming operation.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);
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
// Max of non-negative floats (or +NaN) over a DPP row: for such values the
// IEEE order is the order of the bit patterns as integers, and an integer
// max folds into one DPP instruction per step.
__device__ __forceinline__ float row16_max_nn(float x) {
  int v = __float_as_int(x);
  v = max(v, dppi<0xB1>(v));
  v = max(v, dppi<0x4E>(v));
  v = max(v, dppi<0x141>(v));
  v = max(v, dppi<0x140>(v));
  return __int_as_float(v);
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
// Lane l owns key rows / value columns 2l and 2l+1 for the vector work.
//
// The int8 GEMV z = c^T W for the two weight vectors W = a * Gamma * y
// (y = alpha*k and alpha*q) runs on v_mfma_i32_16x16x64_i8 and is exact in
// integers: each weight vector is scaled by a power of two 2^e so that
// |W 2^e| < 2^30, rounded to an integer x_i (an error of at most 2^-31 of
// the vector's largest entry, below fp32 rounding of that entry), and x_i is
// split into four signed base-256 digits d0..d3 (x = d0 + 2^8 d1 + 2^16 d2 +
// 2^24 d3, each in [-128, 127]).  The MFMA's A operand holds the 8 digit
// rows (2 vectors x 4 digits; rows 8..15 are zero), its B operand the
// codes: lane (g = l >> 4, n = l & 15) loads, for row half kb and column
// tile nt, the 16 bytes of column 16nt + n at slots 16g .. 16g+15, which is
// exactly the B layout of the instruction (one 128-bit load per operand,
// 1 KiB contiguous per wave load).  The A lane holds the digits of the same
// 16 slots, written to LDS by slot.  Integer sums per digit are bounded by
// 128 * 128 * 127 < 2^21, combined in fp32 and scaled back by 2^-e.
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

typedef int v4i __attribute__((ext_vector_type(4)));

// slot of row i & 63 inside its column segment (see the state layout)
__device__ __forceinline__ int code_slot(int x) {
  return ((x & 0x0C) << 2) | ((x & 0x30) >> 2) | (x & 3);
}

// max over the wave of non-negative floats
__device__ __forceinline__ float wave_max_nn(float x) {
  int v = __float_as_int(row16_max_nn(x));
  v = max(v, __shfl_xor(v, 16));
  v = max(v, __shfl_xor(v, 32));
  return __int_as_float(v);
}

// Signed base-256 digits of x (|x| < 2^30): byte k of the result is the
// low byte of x_k, where x_0 = x and x_{k+1} = (x_k + 128) >> 8, so that
// x = sum_k 2^(8k) * sext(byte k).
__device__ __forceinline__ uint32_t digits4(int x0) {
  const int x1 = (x0 + 128) >> 8;
  const int x2 = (x1 + 128) >> 8;
  const int x3 = (x2 + 128) >> 8;
  const uint32_t lo = __builtin_amdgcn_perm((uint32_t)x1, (uint32_t)x0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm((uint32_t)x3, (uint32_t)x2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

template <bool KDA, bool DENSE>
__global__ __launch_bounds__(64) void decode_step_kernel(const DecodeArgs A) {
  const int s = blockIdx.x;
  const int lane = threadIdx.x;
  const int p = A.p, r = A.r;
  // per-slot positions (continuous batching): out-of-range slots are idle
  const int t = A.pos ? A.pos[s] : A.t;
  if (t < 0 || t >= p) return;

  __shared__ float2 sh_gy[D];  // Gamma_i * (y_b, y_q)_i
  __shared__ float2 sh_h[64];  // record weights (h_b, h_q)
  __shared__ float2 sh_hc[DENSE ? 16 : 1];  // dense compensator weights (h_b, h_q)
  __shared__ float2 sh_z[D];   // GEMV result (z_b, z_q) per column
  __shared__ __attribute__((aligned(16))) uint8_t sh_dig[8 * 2 * 64];  // [vector*4+digit][half][slot]
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
  float2 ck[DENSE ? kCompEarly : 1];  // dense keys, rows 2l and 2l+1
#pragma unroll
  for (int c = 0; c < kCompEarly; ++c) {
    if (c < r) {
      if constexpr (DENSE) ck[c] = ld2(A.comp_key + ((size_t)s * r + c) * D + 2 * lane);
      else cidx[c] = A.comp_idx[(size_t)s * r + c];
      cw[c] = ld2(A.comp_val + ((size_t)s * r + c) * D + 2 * lane);
    }
  }
  const float2 ar = ld2(A.row_scale + vo);
  // ---- issue: the 16 KiB of int8 codes, as the MFMA B operands
  const int n16 = lane & 15, g = lane >> 4;
  const uint8_t *cbase =
      reinterpret_cast<const uint8_t *>(A.codes) + (size_t)s * D * D + n16 * 64 + 16 * g;
  v4i cv[2][8];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const uint4 x = ldu4(cbase + kb * 8192 + nt * 1024);
      cv[kb][nt] = v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
    }

  // ---- a1 token prep; append k~_t and the gate of record t
  const float2 kt = make_float2(bt * kk.x, bt * kk.y);
  // b_t = alpha_t * k_t, or 0 for the recurrences without the delta
  // correction (flag bit 1)
  const float2 yb = (A.flags & 2u) ? make_float2(0.f, 0.f) : make_float2(al.x * kk.x, al.y * kk.y);
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
  // ---- dense compensator tokens: records written before the window's
  // first token (decay Gamma), weights h_c = k_c . (Gamma * y)
  if constexpr (DENSE) {
    const float2 G = KDA ? Pk : make_float2(Pg, Pg);
    const float2 gb = make_float2(G.x * yb.x, G.y * yb.y);
    const float2 gq = make_float2(G.x * yq.x, G.y * yq.y);
    float *red = sh_red + lane * kRedStride;
#pragma unroll
    for (int c = 0; c < kCompEarly; ++c) {
      if (c < r) {
        red[2 * c] = ck[c].x * gb.x + ck[c].y * gb.y;
        red[2 * c + 1] = ck[c].x * gq.x + ck[c].y * gq.y;
      }
    }
    for (int c = kCompEarly; c < r; ++c) {
      const float2 kc = ld2(A.comp_key + ((size_t)s * r + c) * D + 2 * lane);
      red[2 * c] = kc.x * gb.x + kc.y * gb.y;
      red[2 * c + 1] = kc.x * gq.x + kc.y * gq.y;
    }
    __syncthreads();
    {
      const int v = lane & 31, half = lane >> 5;
      float acc = 0.f;
      if (v < 2 * r) {
#pragma unroll 8
        for (int m = 0; m < 32; ++m) acc += sh_red[(32 * half + m) * kRedStride + v];
      }
      acc += __shfl_xor(acc, 32);
      if (lane < 2 * r) reinterpret_cast<float *>(&sh_hc[lane >> 1])[lane & 1] = acc;
    }
    __syncthreads();
  }
  // U of the newest chunk, in flight during the GEMV
  const int ulo = t > kRecChunk ? t - kRecChunk : 0;
  float2 ur[kRecChunk];
#pragma unroll
  for (int j = 0; j < kRecChunk; ++j)
    if (j < t - ulo) ur[j] = ld2(A.buf_u + (rec0 + ulo + j) * D + 2 * lane);

  // ---- GEMV weights W = a_i Gamma_i y_i as integers with a power-of-two
  // scale per vector, split into digits and written to LDS by slot
  int eb, eq;  // W * 2^eb, W * 2^eq are below 2^30 in magnitude
  {
    const float2 G = KDA ? Pk : make_float2(Pg, Pg);
    const float2 gb = make_float2(G.x * yb.x, G.y * yb.y);
    const float2 gq = make_float2(G.x * yq.x, G.y * yq.y);
    sh_gy[2 * lane] = make_float2(gb.x, gq.x);
    sh_gy[2 * lane + 1] = make_float2(gb.y, gq.y);
    const float wb0 = ar.x * gb.x, wb1 = ar.y * gb.y;
    const float wq0 = ar.x * gq.x, wq1 = ar.y * gq.y;
    const float mb = wave_max_nn(fmaxf(fabsf(wb0), fabsf(wb1)));
    const float mq = wave_max_nn(fmaxf(fabsf(wq0), fabsf(wq1)));
    // max < 2^frexp_exp(max), so W * 2^(30 - exp) < 2^30 (exact scaling)
    eb = 30 - __builtin_amdgcn_frexp_expf(mb);
    eq = 30 - __builtin_amdgcn_frexp_expf(mq);
    const uint32_t db0 = digits4(__float2int_rn(ldexpf(wb0, eb)));
    const uint32_t db1 = digits4(__float2int_rn(ldexpf(wb1, eb)));
    const uint32_t dq0 = digits4(__float2int_rn(ldexpf(wq0, eq)));
    const uint32_t dq1 = digits4(__float2int_rn(ldexpf(wq1, eq)));
    // rows 2l and 2l+1 sit in adjacent slots of the same half
    const int kb = lane >> 5, sl = code_slot((2 * lane) & 63);
    uint16_t *dst = reinterpret_cast<uint16_t *>(sh_dig + kb * 64 + sl);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t sel = 0x0c0c0400u + 0x00000101u * d;  // byte d of each
      dst[(d * 2) * 32] = (uint16_t)__builtin_amdgcn_perm(db1, db0, sel);
      dst[((4 + d) * 2) * 32] = (uint16_t)__builtin_amdgcn_perm(dq1, dq0, sel);
    }
  }
  __syncthreads();

  // ---- a3 int8 GEMV on MFMA: both vectors, all four digits
  {
    const int m = lane & 15;
    v4i da[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint4 x = *reinterpret_cast<const uint4 *>(sh_dig + ((m & 7) * 2 + kb) * 64 + 16 * g);
      da[kb] = m < 8 ? v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w} : v4i{0, 0, 0, 0};
    }
    const int e = g == 0 ? eb : eq;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(da[0], cv[0][nt], v4i{0, 0, 0, 0}, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(da[1], cv[1][nt], acc, 0, 0, 0);
      // lane (g, n16) holds digits 0..3 of vector g for column 16nt + n16
      if (g < 2) {
        const float zs = fmaf((float)acc.w, 16777216.f,
                              fmaf((float)acc.z, 65536.f, fmaf((float)acc.y, 256.f, (float)acc.x)));
        reinterpret_cast<float *>(&sh_z[16 * nt + n16])[g] = ldexpf(zs, -e);
      }
    }
  }
  __syncthreads();
  float2 zb, zq;
  {
    const float2 z0 = sh_z[2 * lane], z1 = sh_z[2 * lane + 1];
    zb = make_float2(z0.x, z1.x);
    zq = make_float2(z0.y, z1.y);
  }

  // ---- a4 combine: column scales, compensator rows, buffered records
  // (sum_i u_i h_i: the newest chunk from registers, older ones streamed)
  {
    const float2 sc = ld2(A.col_scale + vo);
    zb.x *= sc.x; zb.y *= sc.y;
    zq.x *= sc.x; zq.y *= sc.y;
  }
  if constexpr (DENSE) {
#pragma unroll
    for (int c = 0; c < kCompEarly; ++c) {
      if (c < r) {
        const float2 gg = sh_hc[c];
        zb.x = fmaf(cw[c].x, gg.x, zb.x); zb.y = fmaf(cw[c].y, gg.x, zb.y);
        zq.x = fmaf(cw[c].x, gg.y, zq.x); zq.y = fmaf(cw[c].y, gg.y, zq.y);
      }
    }
    for (int c = kCompEarly; c < r; ++c) {
      const float2 gg = sh_hc[c];
      const float2 w = ld2(A.comp_val + ((size_t)s * r + c) * D + 2 * lane);
      zb.x = fmaf(w.x, gg.x, zb.x); zb.y = fmaf(w.y, gg.x, zb.y);
      zq.x = fmaf(w.x, gg.y, zq.x); zq.y = fmaf(w.y, gg.y, zq.y);
    }
  } else {
#pragma unroll
    for (int c = 0; c < kCompEarly; ++c) {
      if (c < r && (unsigned)cidx[c] < (unsigned)D) {
        const float2 gg = sh_gy[cidx[c]];
        zb.x = fmaf(cw[c].x, gg.x, zb.x); zb.y = fmaf(cw[c].y, gg.x, zb.y);
        zq.x = fmaf(cw[c].x, gg.y, zq.x); zq.y = fmaf(cw[c].y, gg.y, zq.y);
      }
    }
    for (int c = kCompEarly; c < r; ++c) {
      const int idx = A.comp_idx[(size_t)s * r + c];
      if ((unsigned)idx < (unsigned)D) {
        const float2 gg = sh_gy[idx];
        const float2 w = ld2(A.comp_val + ((size_t)s * r + c) * D + 2 * lane);
        zb.x = fmaf(w.x, gg.x, zb.x); zb.y = fmaf(w.y, gg.x, zb.y);
        zq.x = fmaf(w.x, gg.y, zq.x); zq.y = fmaf(w.y, gg.y, zq.y);
      }
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

// Decode step for small slabs, two waves per state: wave w owns key rows
// 64w .. 64w+63 (code half w) for the record dots and the GEMV, and value
// columns 64w .. 64w+63 for the combine.  Each wave scales its half of the
// weights by its own power of two; the halves' GEMV results and record dots
// meet in fp32 through LDS.  A slab of n states is n workgroups of two
// waves: with n <= 4,096 this fills the chip where one wave per state would
// not (measured: +5% at 2,048 states, +18% for KDA at 4,096), while at
// 8,192 states and more the one-wave kernel is faster (1.6%).
template <bool KDA, bool DENSE>
__global__ __launch_bounds__(128) void decode_step2_kernel(const DecodeArgs A) {
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int p = A.p, r = A.r;
  const int t = A.pos ? A.pos[s] : A.t;
  if (t < 0 || t >= p) return;
  const int row = 64 * w + lane;  // key row (history, weights)
  const int col = 64 * w + lane;  // value column (combine)

  __shared__ float2 sh_gy[D];           // Gamma_i * (y_b, y_q)_i
  __shared__ float2 sh_hp[2][64];       // per-wave partial record dots
  __shared__ float2 sh_hcp[2][DENSE ? 16 : 1];  // per-wave partial dense compensator dots
  __shared__ float2 sh_z[2][D];         // per-wave GEMV partials (z_b, z_q)
  __shared__ float sh_kq[2];
  __shared__ __attribute__((aligned(16))) uint8_t sh_dig[2][8 * 64];  // [wave][vector*4+digit][slot]
  __shared__ __attribute__((aligned(16))) float sh_red[2][32 * kRedStride];

  const size_t so = (size_t)s * D;
  const size_t rec0 = (size_t)s * p;

  // ---- issue: token inputs, records, early compensators, codes of half w
  const float kk = A.k[so + row], qq = A.q[so + row];
  const float vv = A.v[so + col];
  const float bt = A.beta[s];
  const float al = KDA ? A.alpha[so + row] : A.alpha[s];
  int hi = t;
  int lo = hi > kRecChunk ? hi - kRecChunk : 0;
  float kr[kRecChunk], gr[kRecChunk];
  auto load_chunk = [&](int lo_, int cnt_) {
#pragma unroll
    for (int j = 0; j < kRecChunk; ++j) {
      if (j < cnt_) {
        kr[j] = A.buf_k[(rec0 + lo_ + j) * D + row];
        gr[j] = KDA ? A.buf_gate[(rec0 + lo_ + j) * D + row] : A.buf_gate[rec0 + lo_ + j];
      }
    }
  };
  load_chunk(lo, hi - lo);
  int cidx[kCompEarly];
  float cw[kCompEarly];
  float ck[DENSE ? kCompEarly : 1];  // dense keys at this lane's row
#pragma unroll
  for (int c = 0; c < kCompEarly; ++c) {
    if (c < r) {
      if constexpr (DENSE) ck[c] = A.comp_key[((size_t)s * r + c) * D + row];
      else cidx[c] = A.comp_idx[(size_t)s * r + c];
      cw[c] = A.comp_val[((size_t)s * r + c) * D + col];
    }
  }
  const float ar = A.row_scale[so + row];
  const int n16 = lane & 15, g = lane >> 4;
  const uint8_t *cbase =
      reinterpret_cast<const uint8_t *>(A.codes) + (size_t)s * D * D + w * 8192 + n16 * 64 + 16 * g;
  v4i cv[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const uint4 x = ldu4(cbase + nt * 1024);
    cv[nt] = v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
  }

  // ---- a1 token prep; append k~_t and the gate of record t
  const float kt = bt * kk;
  const float yb = (A.flags & 2u) ? 0.f : al * kk, yq = al * qq;
  A.buf_k[(rec0 + t) * D + row] = kt;
  if (KDA) A.buf_gate[(rec0 + t) * D + row] = al;
  else if (tid == 0) A.buf_gate[rec0 + t] = al;
  {
    const float kqw = wave_sum(kt * qq);
    if (lane == 0) sh_kq[w] = kqw;
  }

  // ---- a2 history over this wave's rows, partial dots through LDS
  float P = 1.f;
  float *red = sh_red[w];
  while (hi > 0) {
    const int cnt = hi - lo;
#pragma unroll
    for (int j = kRecChunk - 1; j >= 0; --j) {
      if (j < cnt) {
        const float kw = kr[j] * P;
        float hb = kw * yb, hq = kw * yq;
        hb += dpp<0xB1>(hb);  // pairs of rows
        hq += dpp<0xB1>(hq);
        if ((lane & 1) == 0) {
          red[(lane >> 1) * kRedStride + 2 * j] = hb;
          red[(lane >> 1) * kRedStride + 2 * j + 1] = hq;
        }
        P *= gr[j];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {
      const int v = lane & 31, half = lane >> 5;
      float acc = 0.f;
      if (v < 2 * cnt) {
#pragma unroll 8
        for (int m = 0; m < 16; ++m) acc += red[(16 * half + m) * kRedStride + v];
      }
      acc += __shfl_xor(acc, 32);
      if (lane < 2 * cnt) reinterpret_cast<float *>(&sh_hp[w][lo + (lane >> 1)])[lane & 1] = acc;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    hi = lo;
    lo = hi > kRecChunk ? hi - kRecChunk : 0;
    if (hi > 0) load_chunk(lo, hi - lo);
  }
  // ---- dense compensator tokens: records written before the window's
  // first token (decay Gamma); this wave's partial k_c . (Gamma * y)
  if constexpr (DENSE) {
    const float gb = P * yb, gq = P * yq;
    auto put = [&](int c, float kc) {
      float hb = kc * gb, hq = kc * gq;
      hb += dpp<0xB1>(hb);  // pairs of rows
      hq += dpp<0xB1>(hq);
      if ((lane & 1) == 0) {
        red[(lane >> 1) * kRedStride + 2 * c] = hb;
        red[(lane >> 1) * kRedStride + 2 * c + 1] = hq;
      }
    };
#pragma unroll
    for (int c = 0; c < kCompEarly; ++c)
      if (c < r) put(c, ck[c]);
    for (int c = kCompEarly; c < r; ++c) put(c, A.comp_key[((size_t)s * r + c) * D + row]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {
      const int v = lane & 31, half = lane >> 5;
      float acc = 0.f;
      if (v < 2 * r) {
#pragma unroll 8
        for (int m = 0; m < 16; ++m) acc += red[(16 * half + m) * kRedStride + v];
      }
      acc += __shfl_xor(acc, 32);
      if (lane < 2 * r) reinterpret_cast<float *>(&sh_hcp[w][lane >> 1])[lane & 1] = acc;
    }
  }
  // u rows of this wave's columns, in flight during the GEMV
  const int ulo = t > kRecChunk ? t - kRecChunk : 0;
  float ur[kRecChunk];
#pragma unroll
  for (int j = 0; j < kRecChunk; ++j)
    if (j < t - ulo) ur[j] = A.buf_u[(rec0 + ulo + j) * D + col];

  // ---- GEMV weights of this half: power-of-two scale per wave and vector
  int eb, eq;
  {
    const float gb = P * yb, gq = P * yq;
    sh_gy[row] = make_float2(gb, gq);
    const float wb = ar * gb, wq = ar * gq;
    eb = 30 - __builtin_amdgcn_frexp_expf(wave_max_nn(fabsf(wb)));
    eq = 30 - __builtin_amdgcn_frexp_expf(wave_max_nn(fabsf(wq)));
    const uint32_t db = digits4(__float2int_rn(ldexpf(wb, eb)));
    const uint32_t dq = digits4(__float2int_rn(ldexpf(wq, eq)));
    const int sl = code_slot(lane);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      sh_dig[w][d * 64 + sl] = (uint8_t)(db >> (8 * d));
      sh_dig[w][(4 + d) * 64 + sl] = (uint8_t)(dq >> (8 * d));
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  {
    const int m = lane & 15;
    const uint4 x = *reinterpret_cast<const uint4 *>(&sh_dig[w][(m & 7) * 64 + 16 * g]);
    const v4i da = m < 8 ? v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w} : v4i{0, 0, 0, 0};
    const int e = g == 0 ? eb : eq;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(da, cv[nt], v4i{0, 0, 0, 0}, 0, 0, 0);
      if (g < 2) {
        const float zs = fmaf((float)acc.w, 16777216.f,
                              fmaf((float)acc.z, 65536.f, fmaf((float)acc.y, 256.f, (float)acc.x)));
        reinterpret_cast<float *>(&sh_z[w][16 * nt + n16])[g] = ldexpf(zs, -e);
      }
    }
  }
  __syncthreads();
  float zb, zq;
  {
    const float2 z0 = sh_z[0][col], z1 = sh_z[1][col];
    zb = z0.x + z1.x;
    zq = z0.y + z1.y;
  }
  {
    const float sc = A.col_scale[so + col];
    zb *= sc;
    zq *= sc;
  }
  if constexpr (DENSE) {
#pragma unroll
    for (int c = 0; c < kCompEarly; ++c) {
      if (c < r) {
        const float2 h0 = sh_hcp[0][c], h1 = sh_hcp[1][c];
        zb = fmaf(cw[c], h0.x + h1.x, zb);
        zq = fmaf(cw[c], h0.y + h1.y, zq);
      }
    }
    for (int c = kCompEarly; c < r; ++c) {
      const float2 h0 = sh_hcp[0][c], h1 = sh_hcp[1][c];
      const float wv = A.comp_val[((size_t)s * r + c) * D + col];
      zb = fmaf(wv, h0.x + h1.x, zb);
      zq = fmaf(wv, h0.y + h1.y, zq);
    }
  } else {
#pragma unroll
    for (int c = 0; c < kCompEarly; ++c) {
      if (c < r && (unsigned)cidx[c] < (unsigned)D) {
        const float2 gg = sh_gy[cidx[c]];
        zb = fmaf(cw[c], gg.x, zb);
        zq = fmaf(cw[c], gg.y, zq);
      }
    }
    for (int c = kCompEarly; c < r; ++c) {
      const int idx = A.comp_idx[(size_t)s * r + c];
      if ((unsigned)idx < (unsigned)D) {
        const float2 gg = sh_gy[idx];
        const float wv = A.comp_val[((size_t)s * r + c) * D + col];
        zb = fmaf(wv, gg.x, zb);
        zq = fmaf(wv, gg.y, zq);
      }
    }
  }
  {
    float zub = 0.f, zuq = 0.f;
#pragma unroll
    for (int j = 0; j < kRecChunk; ++j) {
      if (j < t - ulo) {
        const float2 h0 = sh_hp[0][ulo + j], h1 = sh_hp[1][ulo + j];
        zub = fmaf(ur[j], h0.x + h1.x, zub);
        zuq = fmaf(ur[j], h0.y + h1.y, zuq);
      }
    }
    for (int i = 0; i < ulo; ++i) {
      const float u = A.buf_u[(rec0 + i) * D + col];
      const float2 h0 = sh_hp[0][i], h1 = sh_hp[1][i];
      zub = fmaf(u, h0.x + h1.x, zub);
      zuq = fmaf(u, h0.y + h1.y, zuq);
    }
    zb += zub;
    zq += zuq;
  }
  const float ut = vv - zb;
  __builtin_nontemporal_store(fmaf(sh_kq[0] + sh_kq[1], ut, zq), A.o + so + col);
  __builtin_nontemporal_store(ut, A.buf_u + (rec0 + t) * D + col);
}

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
__device__ __forceinline__ uint32_t u4get(const uint4 &x, int i) {
  return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
}

struct SplitLds {    // LDS used by the split (a6-a8), shared by both kernels
  float *part;       // [2][D] per column half: row norms^2, later row absmax
  int *sel;          // [D] compensator slot of a row or -1
  float *cmx;        // [8][D] column-max partials
  float *sig;        // [D] 1 / s_j
  float *inv;        // [D] 127 / m_i (0 for zero or extracted rows)
  // dense compensator tokens only, [16][D] each
  float *dq;         // keys K (row c: k_c)
  float *dw;         // W = K S (row c: w_c)
  float *dy;         // Y = S W^T (row c: column c of Y)
};

constexpr float kMgsDrop = 1e-3f;  // relative projected norm at or below which a key is dropped

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
template <bool DENSE>
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
  // ---- a6 row L2 norms (squared, fp32; two column-half partials)
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float q = 0.f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) q = fmaf(acc[rt][ct][v], acc[rt][ct][v], q);
      q = row16_sum(q);
      if (lc == 0) L.part[ch * D + rbase + 16 * rt + v] = q;
    }
  if (tid < D) L.sel[tid] = -1;
  if (DENSE)
    for (int e = tid; e < r * D; e += 256) L.dq[e] = 0.f;
  __syncthreads();
  if (w == 0 && r > 0) {
    // iterative argmax on wave 0: lane l holds rows 2l and 2l+1; each round
    // takes the largest remaining norm, ties to the lower row index
    float n0 = L.part[2 * lane] + L.part[D + 2 * lane];
    float n1 = L.part[2 * lane + 1] + L.part[D + 2 * lane + 1];
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
  if (tid < D) {
    float m = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) m = fmaxf(m, L.cmx[g * D + tid]);
    const float sc = (flags & 1u) ? 1.f : (m > 0.f ? m : 1.f);
    col_scale[s * D + tid] = sc;
    L.sig[tid] = 1.f / sc;  // sigma_j, correctly rounded
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
        m = row16_max_nn(m);
        if (lc == 0) L.part[ch * D + rbase + 16 * rt + v] = m;
      }
  }
  __syncthreads();
  if (tid < D) {
    // row scale and its reciprocal, once per row (correctly rounded)
    const float m = fmaxf(L.part[tid], L.part[D + tid]);
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
  {
    float4 iv[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) iv[rt] = *reinterpret_cast<const float4 *>(L.inv + rbase + 16 * rt);
    int8_t *cdst = codes + s * D * D + h * 8192 + col0 * 64 + 16 * lr;  // + 1024 ct
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
  const SplitLds L{sh_part, sh_sel, sh_cmx, sh_sig, sh_inv, sh_dq, sh_dw, sh_dy};
  split_state<DENSE>(acc, L, A.codes, A.row_scale, A.col_scale, A.comp_idx, A.comp_val, A.comp_key, s,
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
  const size_t s = blockIdx.x;
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

  // boundary-state side data and this lane's code segments, issued first
  if (tid < D) {
    sh_a[tid] = A.row_scale[s * D + tid];
    sh_s[tid] = A.col_scale[s * D + tid];
  }
  if (tid < D) sh_cslot[tid] = -1;
  const int8_t *csrc = A.codes + s * D * D + h * 8192 + col0 * 64 + 16 * lr;
  uint4 cw[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) cw[ct] = ldu4(csrc + ct * 1024);

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
      float tk = 0.f, tq = 0.f, tv = 0.f, tb = 0.f;
      if (FUSED && first && tid < D) {
        tk = A.k[s * D + tid];
        tq = A.q[s * D + tid];
        tv = A.v[s * D + tid];
        tb = A.beta[s];
        P = KDA ? A.alpha[s * D + tid] : A.alpha[s];
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
      if (FUSED && first && tid < D) {
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
// Dequantize: S_out = deQ(codes, a, s) + compensator rows (fp32).  Thread
// (half hh, column j) reads the 64 code bytes of its column segment and
// writes column j of rows 64hh .. 64hh+63.
// ---------------------------------------------------------------------------
template <bool DENSE>
__global__ __launch_bounds__(256) void dequant_kernel(const DequantArgs A) {
  const size_t s = blockIdx.x;
  const int j = threadIdx.x & (D - 1), hh = threadIdx.x >> 7;
  const int r = A.r;
  const float sj = A.col_scale[s * D + j];
  const uint4 *src = reinterpret_cast<const uint4 *>(A.codes + s * D * D + hh * 8192 + j * 64);
  for (int q = 0; q < 4; ++q) {
    const uint4 cq = src[q];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int slot = 16 * q + e;
      const int row = 64 * hh + code_slot(slot);  // the slot map is its own inverse
      const uint32_t wd = u4get(cq, e >> 2);
      float x = (float)(int8_t)(wd >> (8 * (e & 3))) * A.row_scale[s * D + row] * sj;
      if (DENSE) {
        for (int c = 0; c < r; ++c) x = fmaf(A.comp_key[(s * r + c) * D + row], A.comp_val[(s * r + c) * D + j], x);
      } else {
        for (int c = 0; c < r; ++c)
          if (A.comp_idx[s * r + c] == row) x += A.comp_val[(s * r + c) * D + j];
      }
      A.S_out[(s * D + row) * D + j] = x;
    }
  }
}

// ---------------------------------------------------------------------------
// Dense-state per-token decode: the uncompressed baselines the quantized path
// is compared with (an fp32 or bf16 state read and written every token).
// One 256-thread workgroup per state, one pass over the state: thread
// (rg = tid >> 5, cg = tid & 31) holds rows rg + 8m (m = 0..15) x columns
// 4cg .. 4cg+3 in registers (each wave load reads two full rows); partial
// column sums of S^T b and S^T (D q) meet in LDS, then u_t and o_t =
// S_{t-1}^T (D q) + (k~ . q) u_t, and the registers are updated to
// S_t = D S_{t-1} + k~ u^T and written back.  bf16 states are widened to
// fp32 on load and rounded to nearest even on store.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);  // inf / NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;  // round to nearest, ties to even
}

template <bool KDA, bool BF16>
__global__ __launch_bounds__(256) void dense_step_kernel(const DenseArgs A) {
  const size_t s = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int rg = tid >> 5, cg = tid & 31;
  __shared__ __attribute__((aligned(16))) float sh_b[D], sh_dq[D], sh_kt[D], sh_al[D];
  __shared__ __attribute__((aligned(16))) float sh_u[D];
  __shared__ __attribute__((aligned(16))) float2 sh_part[8 * D];
  __shared__ float sh_kq[2];

  // the state rows of this thread, issued first
  float x[16][4];
  if (BF16) {
    const uint16_t *S = reinterpret_cast<const uint16_t *>(A.S) + s * D * D;
    uint2 raw[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) raw[m] = ldu2(S + (rg + 8 * m) * D + 4 * cg);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      x[m][0] = bf16_to_f32(raw[m].x & 0xffffu);
      x[m][1] = bf16_to_f32(raw[m].x >> 16);
      x[m][2] = bf16_to_f32(raw[m].y & 0xffffu);
      x[m][3] = bf16_to_f32(raw[m].y >> 16);
    }
  } else {
    const float *S = reinterpret_cast<const float *>(A.S) + s * D * D;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const float4 f = ld4(S + (rg + 8 * m) * D + 4 * cg);
      x[m][0] = f.x; x[m][1] = f.y; x[m][2] = f.z; x[m][3] = f.w;
    }
  }
  float vv = 0.f;
  if (tid < D) {
    const float k = A.k[s * D + tid], q = A.q[s * D + tid];
    const float al = KDA ? A.alpha[s * D + tid] : A.alpha[s];
    const float kt = A.beta[s] * k;
    vv = A.v[s * D + tid];
    sh_b[tid] = (A.flags & 2u) ? 0.f : al * k;  // b_t = 0 without the delta correction
    sh_dq[tid] = al * q;
    sh_kt[tid] = kt;
    sh_al[tid] = al;
    const float kq = wave_sum(kt * q);  // waves 0 and 1, all lanes active
    if (lane == 0) sh_kq[w] = kq;
  }
  __syncthreads();
  // partial column sums over this thread's 16 rows
  float pb[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const float b = sh_b[rg + 8 * m], dq = sh_dq[rg + 8 * m];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      pb[c] = fmaf(x[m][c], b, pb[c]);
      pq[c] = fmaf(x[m][c], dq, pq[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) sh_part[rg * D + 4 * cg + c] = make_float2(pb[c], pq[c]);
  __syncthreads();
  if (tid < D) {
    float zb = 0.f, zq = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const float2 t = sh_part[g * D + tid];
      zb += t.x;
      zq += t.y;
    }
    const float u = vv - zb;
    __builtin_nontemporal_store(fmaf(sh_kq[0] + sh_kq[1], u, zq), A.o + s * D + tid);
    sh_u[tid] = u;
  }
  __syncthreads();
  // S_t = D S_{t-1} + k~ u^T, written back in place
  const float4 u4 = *reinterpret_cast<const float4 *>(sh_u + 4 * cg);
  const float uu[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const float al = sh_al[rg + 8 * m], kt = sh_kt[rg + 8 * m];
#pragma unroll
    for (int c = 0; c < 4; ++c) x[m][c] = fmaf(al, x[m][c], kt * uu[c]);
  }
  if (BF16) {
    uint16_t *S = reinterpret_cast<uint16_t *>(A.S) + s * D * D;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const uint32_t lo = f32_to_bf16(x[m][0]) | (f32_to_bf16(x[m][1]) << 16);
      const uint32_t hi = f32_to_bf16(x[m][2]) | (f32_to_bf16(x[m][3]) << 16);
      __builtin_nontemporal_store(vu2{lo, hi}, reinterpret_cast<vu2 *>(S + (rg + 8 * m) * D + 4 * cg));
    }
  } else {
    float *S = reinterpret_cast<float *>(A.S) + s * D * D;
#pragma unroll
    for (int m = 0; m < 16; ++m)
      st4(S + (rg + 8 * m) * D + 4 * cg, make_float4(x[m][0], x[m][1], x[m][2], x[m][3]));
  }
}

// ---------------------------------------------------------------------------
// "BF16 + per-window" ([EL] Table 2): a dense bf16 boundary state B, fixed
// for the window; the window's tokens are buffered in the fp32 records.
// Decode: one 256-thread workgroup per state.  Threads 0..127 own key row
// tid for the record dots (the newest kRecChunk records prefetched);
// thread (rg = tid >> 4, cg = tid & 15) owns rows rg + 16m (m = 0..7) x
// columns 8cg .. 8cg+7 of B (one 16-byte load per row) for the GEMV
// z = B^T (Gamma y); threads 0..127 then combine column tid.
// ---------------------------------------------------------------------------
template <bool KDA>
__global__ __launch_bounds__(256) void bf16w_decode_kernel(const Bf16WinArgs A) {
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int p = A.p, t = A.t;
  const int rg = tid >> 4, cg = tid & 15;
  __shared__ float2 sh_gy[D];           // Gamma_i * (y_b, y_q)_i
  __shared__ float2 sh_hp[2][64];       // per-wave record dots (rows 0..63, 64..127)
  __shared__ float2 sh_zp[4][D];        // per-wave GEMV partials
  __shared__ float sh_kq[2];
  const size_t so = (size_t)s * D, rec0 = (size_t)s * p;
  const uint16_t *Bs = A.B + (size_t)s * D * D;
  uint4 bw[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) bw[m] = ldu4(Bs + (rg + 16 * m) * D + 8 * cg);
  if (tid < D) {
    const int row = tid;
    const float kk = A.k[so + row], qq = A.q[so + row];
    const float al = KDA ? A.alpha[so + row] : A.alpha[s];
    const float bt = A.beta[s];
    const float yb = (A.flags & 2u) ? 0.f : al * kk, yq = al * qq;
    const float kt = bt * kk;
    A.buf_k[(rec0 + t) * D + row] = kt;
    if (KDA) A.buf_gate[(rec0 + t) * D + row] = al;
    else if (row == 0) A.buf_gate[rec0 + t] = al;
    const float kq = wave_sum(kt * qq);
    if (lane == 0) sh_kq[w] = kq;
    // record dots h_i = k~_i . (rho_i * y), newest first, chunks of kRecChunk
    float P = 1.f;
    int hi = t;
    while (hi > 0) {
      const int lo = hi > kRecChunk ? hi - kRecChunk : 0, cnt = hi - lo;
      float kr[kRecChunk], gr[kRecChunk];
#pragma unroll
      for (int j = 0; j < kRecChunk; ++j) {
        if (j < cnt) {
          kr[j] = A.buf_k[(rec0 + lo + j) * D + row];
          gr[j] = KDA ? A.buf_gate[(rec0 + lo + j) * D + row] : A.buf_gate[rec0 + lo + j];
        }
      }
#pragma unroll
      for (int j = kRecChunk - 1; j >= 0; --j) {
        if (j < cnt) {
          const float kw = kr[j] * P;
          const float hb = wave_sum(kw * yb), hq = wave_sum(kw * yq);
          if (lane == 0) sh_hp[w][lo + j] = make_float2(hb, hq);
          P *= gr[j];
        }
      }
      hi = lo;
    }
    sh_gy[row] = make_float2(P * yb, P * yq);
  }
  __syncthreads();
  // ---- z = B^T (Gamma y): 8 rows x 8 columns per thread, then the rows of
  // the wave (lanes 16 and 32 apart) and the 4 waves
  {
    float zb[8], zq[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) zb[c] = zq[c] = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float2 g = sh_gy[rg + 16 * m];
      const uint32_t wd[4] = {bw[m].x, bw[m].y, bw[m].z, bw[m].w};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float b = (c & 1) ? __uint_as_float(wd[c >> 1] & 0xffff0000u) : bf16_to_f32(wd[c >> 1] & 0xffffu);
        zb[c] = fmaf(b, g.x, zb[c]);
        zq[c] = fmaf(b, g.y, zq[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      zb[c] += __shfl_xor(zb[c], 16);
      zb[c] += __shfl_xor(zb[c], 32);
      zq[c] += __shfl_xor(zq[c], 16);
      zq[c] += __shfl_xor(zq[c], 32);
    }
    if (lane < 16) {
#pragma unroll
      for (int c = 0; c < 8; ++c) sh_zp[w][8 * cg + c] = make_float2(zb[c], zq[c]);
    }
  }
  __syncthreads();
  if (tid < D) {
    const int col = tid;
    float zb = 0.f, zq = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      zb += sh_zp[ww][col].x;
      zq += sh_zp[ww][col].y;
    }
    for (int i = 0; i < t; ++i) {
      const float u = A.buf_u[(rec0 + i) * D + col];
      const float2 h0 = sh_hp[0][i], h1 = sh_hp[1][i];
      zb = fmaf(u, h0.x + h1.x, zb);
      zq = fmaf(u, h0.y + h1.y, zq);
    }
    const float ut = A.v[so + col] - zb;
    __builtin_nontemporal_store(fmaf(sh_kq[0] + sh_kq[1], ut, zq), A.o + so + col);
    __builtin_nontemporal_store(ut, A.buf_u + (rec0 + t) * D + col);
  }
}

// Close: S = Gamma * B + K_w U in fp32, stored rounded to bf16 (nearest,
// ties to even).  Thread (rg, cg) owns rows rg + 16m x columns 8cg .. 8cg+7;
// record chunks are staged in LDS and folded with the decays (newest
// first) as in the int8 close; the contraction runs on fp32 FMAs (the
// kernel moves 64 KiB of state per workgroup and is bound by HBM).
template <bool KDA>
__global__ __launch_bounds__(256) void bf16w_close_kernel(const Bf16WinArgs A) {
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int p = A.p, len = A.t;
  const int rg = tid >> 4, cg = tid & 15;
  __shared__ __attribute__((aligned(16))) float sh_K[kRecChunk * D];
  __shared__ __attribute__((aligned(16))) float sh_U[kRecChunk * D];
  __shared__ float sh_g[KDA ? kRecChunk * D : kRecChunk];
  __shared__ float sh_gam[D];
  const size_t rec0 = (size_t)s * p;
  uint16_t *Bs = A.B + (size_t)s * D * D;
  uint4 bw[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) bw[m] = ldu4(Bs + (rg + 16 * m) * D + 8 * cg);
  float acc[8][8];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[m][c] = 0.f;
  float P = 1.f;  // running decay product of row tid (tid < D)
  for (int hi = len; hi > 0;) {
    const int lo = hi > kRecChunk ? hi - kRecChunk : 0, cnt = hi - lo;
    __syncthreads();  // the previous chunk's contraction is done
    for (int e = tid; e < cnt * (D / 4); e += 256) {
      reinterpret_cast<float4 *>(sh_K)[e] = ld4(A.buf_k + (rec0 + lo) * D + 4 * e);
      reinterpret_cast<float4 *>(sh_U)[e] = ld4(A.buf_u + (rec0 + lo) * D + 4 * e);
      if (KDA) reinterpret_cast<float4 *>(sh_g)[e] = ld4(A.buf_gate + (rec0 + lo) * D + 4 * e);
    }
    if (!KDA && tid < cnt) sh_g[tid] = A.buf_gate[rec0 + lo + tid];
    __syncthreads();
    if (tid < D) {
      for (int j = cnt - 1; j >= 0; --j) {
        sh_K[j * D + tid] *= P;
        P *= KDA ? sh_g[j * D + tid] : sh_g[j];
      }
    }
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      float kr[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) kr[m] = sh_K[j * D + rg + 16 * m];
      const float4 u0 = *reinterpret_cast<const float4 *>(sh_U + j * D + 8 * cg);
      const float4 u1 = *reinterpret_cast<const float4 *>(sh_U + j * D + 8 * cg + 4);
      const float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[m][c] = fmaf(kr[m], uu[c], acc[m][c]);
    }
    hi = lo;
  }
  if (tid < D) sh_gam[tid] = P;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const float G = sh_gam[rg + 16 * m];
    const uint32_t wd[4] = {bw[m].x, bw[m].y, bw[m].z, bw[m].w};
    uint32_t out[4];
#pragma unroll
    for (int h2 = 0; h2 < 4; ++h2) {
      const float b0 = bf16_to_f32(wd[h2] & 0xffffu), b1 = __uint_as_float(wd[h2] & 0xffff0000u);
      const uint32_t lo16 = f32_to_bf16(fmaf(G, b0, acc[m][2 * h2]));
      const uint32_t hi16 = f32_to_bf16(fmaf(G, b1, acc[m][2 * h2 + 1]));
      out[h2] = lo16 | (hi16 << 16);
    }
    __builtin_nontemporal_store(vu4{out[0], out[1], out[2], out[3]},
                                reinterpret_cast<vu4 *>(Bs + (rg + 16 * m) * D + 8 * cg));
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_dense_step(const DenseArgs &a, bool kda, bool bf16, hipStream_t stream) {
  if (kda && bf16)
    hipLaunchKernelGGL((dense_step_kernel<true, true>), dim3(a.n), dim3(256), 0, stream, a);
  else if (kda)
    hipLaunchKernelGGL((dense_step_kernel<true, false>), dim3(a.n), dim3(256), 0, stream, a);
  else if (bf16)
    hipLaunchKernelGGL((dense_step_kernel<false, true>), dim3(a.n), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((dense_step_kernel<false, false>), dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Slabs of at most this many states take the two-wave decode kernel.
constexpr int kSmallSlab = 4096;

template <bool KDA, bool DENSE>
void launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
  if (a.n <= kSmallSlab)
    hipLaunchKernelGGL((decode_step2_kernel<KDA, DENSE>), dim3(a.n), dim3(128), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_step_kernel<KDA, DENSE>), dim3(a.n), dim3(64), 0, stream, a);
}

// Dense compensator tokens are on when the caller passes their keys.
hipError_t launch_decode_step(const DecodeArgs &a, bool kda, hipStream_t stream) {
  const bool dense = a.comp_key != nullptr;
  if (kda && dense) launch_decode_t<true, true>(a, stream);
  else if (kda) launch_decode_t<true, false>(a, stream);
  else if (dense) launch_decode_t<false, true>(a, stream);
  else launch_decode_t<false, false>(a, stream);
  return hipGetLastError();
}

template <bool FUSED>
hipError_t launch_close(const CloseArgs &a, bool kda, hipStream_t stream) {
  const bool dense = a.comp_key != nullptr;
  if (kda && dense)
    hipLaunchKernelGGL((close_kernel<true, FUSED, true>), dim3(a.n), dim3(256), 0, stream, a);
  else if (kda)
    hipLaunchKernelGGL((close_kernel<true, FUSED, false>), dim3(a.n), dim3(256), 0, stream, a);
  else if (dense)
    hipLaunchKernelGGL((close_kernel<false, FUSED, true>), dim3(a.n), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((close_kernel<false, FUSED, false>), dim3(a.n), dim3(256), 0, stream, a);
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

hipError_t launch_bf16w_decode(const Bf16WinArgs &a, bool kda, hipStream_t stream) {
  if (kda)
    hipLaunchKernelGGL(bf16w_decode_kernel<true>, dim3(a.n), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bf16w_decode_kernel<false>, dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bf16w_close(const Bf16WinArgs &a, bool kda, hipStream_t stream) {
  if (kda)
    hipLaunchKernelGGL(bf16w_close_kernel<true>, dim3(a.n), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bf16w_close_kernel<false>, dim3(a.n), dim3(256), 0, stream, a);
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
