// Constants, LDS layout and helpers of one wave's decode step (the int8
// boundary-state GEMV on the matrix path, the window's records, the
// compensator rows), whose body (lq_decode_body.inc) the decode kernel
// (lq_decode.hip) and the continuous-batching launch that mixes decode
// steps with fused window closes (lq_close.hip) both include.
#pragma once
#include "lq_device.h"

namespace lq {

// Slabs of at most this many states take the two-wave decode kernel
// (lq_decode.hip); larger ones the one-wave decode step below.
constexpr int kSmallSlab = 4096;

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
// known; o_t and u_t close the wave.
// ---------------------------------------------------------------------------
constexpr int kCompEarly = 4;    // compensator rows loaded with the records
constexpr int kCompBatch = 4;    // later compensator rows: loads issued together, then used
constexpr int kOldBatch = 8;     // u rows older than the newest record chunk, per batch
constexpr int kRedStride = 33;   // odd row stride of the transposed partials: no bank conflicts

typedef int v4i __attribute__((ext_vector_type(4)));

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

// LDS of one wave's decode step (one-wave decode body)
struct DecodeLds {
  float2 *gy;    // [D] Gamma_i * (y_b, y_q)_i
  float2 *h;     // [64] record weights (h_b, h_q)
  float2 *hc;    // [16] dense compensator weights (h_b, h_q)
  float2 *z;     // [D] GEMV result (z_b, z_q) per column
  uint8_t *dig;  // [8 * 2 * 64] digits [vector*4+digit][half][slot], 16-byte aligned
  float *red;    // [64 * kRedStride] transposed partials
};
// LDS bytes of one wave's decode step.  The GEMV's arrays (z: D float2,
// digits: 8 x 2 x 64 bytes) live in the record dots' transpose buffer, which
// is free by then, so that the one-wave kernel (without dense weights, under
// 10 KB) fits sixteen workgroups per CU.
constexpr int kDecodeLdsBytes = (D + 64 + 16) * 8 + 64 * kRedStride * 4;
static_assert(D * 8 + 8 * 2 * 64 <= 64 * kRedStride * 4, "z and the digits fit in the transpose buffer");

// LDS hand-off between the lanes of one wave: a wave's LDS operations
// complete in order, so only the compiler must not move them across this
// point; a workgroup of one wave takes the plain barrier.
template <bool WAVE>
__device__ __forceinline__ void lds_sync() {
  if (WAVE) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }
}

}  // namespace lq
