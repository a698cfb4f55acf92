// Device-side helpers shared by the LeapQuant kernels for gfx950 (CDNA4,
// wave64): the state layout, streaming loads and stores, DPP reductions.
// The kernels are in lq_decode.hip (decode step), lq_close.hip (window
// close, initial split, dequantize) and lq_baselines.hip (the dense-state
// and bf16 per-window baselines).
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
#pragma once
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
// Count-guarded loads through a raw buffer resource: a buffer over the
// first `bytes` bytes at p returns zero for loads at byte offsets at or
// beyond `bytes` without touching memory, so a loop of loads guarded by a
// run-time count becomes straight-line code.  The compiler then knows
// exactly which loads are outstanding at each use and waits for those only;
// with branches around the loads it waits for every load in flight
// (the state's whole code stream included).  Dword 3 holds the gfx9 raw
// buffer format (32-bit data, no swizzle, no stride); nontemporal like ld2.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
__device__ __forceinline__ BufRsrc buf_rsrc(const void *p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}
constexpr int kBufNt = 2;  // cache policy bits of the buffer loads: nt
__device__ __forceinline__ float2 bld2(BufRsrc r, int off) {
  const vu2 t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kBufNt);
  return make_float2(__uint_as_float(t.x), __uint_as_float(t.y));
}
__device__ __forceinline__ uint32_t bld1(BufRsrc r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kBufNt);
}
__device__ __forceinline__ void st2(float *p, float2 v) {
  __builtin_nontemporal_store(vf2{v.x, v.y}, reinterpret_cast<vf2 *>(p));
}
// The same 8 bytes as an ordinary write-back store.  The GDN decode step
// writes its three 512-byte rows per state this way: a whole window of the
// batch-256 workload (60 decode launches and 4 fused closes) ran 0.6-0.85%
// faster than with nontemporal stores, in alternating runs of the two
// builds.  Elsewhere nontemporal stores measured faster and stay: the KDA
// and two-wave steps (KDA's window 1.7%), the fused close (2.8%) and a
// plain stream of the decode's shape (4%).
__device__ __forceinline__ void st2_wb(float *p, float2 v) {
  *reinterpret_cast<vf2 *>(p) = vf2{v.x, v.y};
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

constexpr int kRecChunk = 16;    // records in flight per chunk

// slot of row i & 63 inside its column segment (see the state layout)
__device__ __forceinline__ int code_slot(int x) {
  return ((x & 0x0C) << 2) | ((x & 0x30) >> 2) | (x & 3);
}

}  // namespace lq
