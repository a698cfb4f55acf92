// LeapQuant decode step for gfx950: one wave per state (large slabs) or two
// waves per state (slabs of at most 4,096 states).
#include "lq_device.h"

namespace lq {

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
  // Per-state scalars (GDN gates, compensator row indices) are read with
  // lane-indexed vector loads and broadcast with readlane where used.  As
  // scalar loads they were waited for before the codes were issued (scalar
  // loads return out of order, so any later scalar wait covers them), which
  // put a second memory round trip in front of every wave.
  float gv = 1.f;  // GDN: lane j holds the gate of record lo + j
  auto load_chunk = [&](int lo_, int cnt_) {
    if (!KDA && lane < cnt_) gv = A.buf_gate[rec0 + lo_ + lane];
#pragma unroll
    for (int j = 0; j < kRecChunk; ++j) {
      if (j < cnt_) {
        const size_t rr = (rec0 + lo_ + j) * D + 2 * lane;
        kr[j] = ld2(A.buf_k + rr);
        if (KDA) gr[j] = ld2(A.buf_gate + rr);
      }
    }
  };
  load_chunk(lo, hi - lo);
  int civ = -1;  // lane c < r: compensator row index c
  if (!DENSE && lane < r) civ = A.comp_idx[(size_t)s * r + lane];
  float2 cw[kCompEarly];
  float2 ck[DENSE ? kCompEarly : 1];  // dense keys, rows 2l and 2l+1
#pragma unroll
  for (int c = 0; c < kCompEarly; ++c) {
    if (c < r) {
      if constexpr (DENSE) ck[c] = ld2(A.comp_key + ((size_t)s * r + c) * D + 2 * lane);
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
          Pg *= __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), j));
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
    if (hi > 0) {
      // Every load of the chunk just used has returned.  Saying so lets the
      // next chunk's loads issue back to back: the compiler cannot pair the
      // guarded loads (j < cnt) with their guarded uses, and would otherwise
      // wait for each earlier load into the same registers first.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      load_chunk(lo, hi - lo);
    }
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
    // the later keys, four loads in flight before their use
    for (int c0 = kCompEarly; c0 < r; c0 += kCompBatch) {
      float2 kc[kCompBatch];
#pragma unroll
      for (int j = 0; j < kCompBatch; ++j)
        if (c0 + j < r) kc[j] = ld2(A.comp_key + ((size_t)s * r + c0 + j) * D + 2 * lane);
#pragma unroll
      for (int j = 0; j < kCompBatch; ++j) {
        if (c0 + j < r) {
          red[2 * (c0 + j)] = kc[j].x * gb.x + kc[j].y * gb.y;
          red[2 * (c0 + j) + 1] = kc[j].x * gq.x + kc[j].y * gq.y;
        }
      }
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
  // U of the newest chunk, in flight during the GEMV.  The explicit wait
  // (the codes are due for the GEMV next) lets these loads issue back to
  // back: the compiler would otherwise wait before each of them, for the
  // guarded loads that last used the same registers.
  const int ulo = t > kRecChunk ? t - kRecChunk : 0;
  float2 ur[kRecChunk];
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
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
    for (int c0 = kCompEarly; c0 < r; c0 += kCompBatch) {
      float2 wv[kCompBatch];
#pragma unroll
      for (int j = 0; j < kCompBatch; ++j)
        if (c0 + j < r) wv[j] = ld2(A.comp_val + ((size_t)s * r + c0 + j) * D + 2 * lane);
#pragma unroll
      for (int j = 0; j < kCompBatch; ++j) {
        if (c0 + j < r) {
          const float2 gg = sh_hc[c0 + j];
          zb.x = fmaf(wv[j].x, gg.x, zb.x); zb.y = fmaf(wv[j].y, gg.x, zb.y);
          zq.x = fmaf(wv[j].x, gg.y, zq.x); zq.y = fmaf(wv[j].y, gg.y, zq.y);
        }
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < kCompEarly; ++c) {
      const int idx = __builtin_amdgcn_readlane(civ, c);
      if (c < r && (unsigned)idx < (unsigned)D) {
        const float2 gg = sh_gy[idx];
        zb.x = fmaf(cw[c].x, gg.x, zb.x); zb.y = fmaf(cw[c].y, gg.x, zb.y);
        zq.x = fmaf(cw[c].x, gg.y, zq.x); zq.y = fmaf(cw[c].y, gg.y, zq.y);
      }
    }
    // the later rows, four loads in flight before their use
    for (int c0 = kCompEarly; c0 < r; c0 += kCompBatch) {
      int idx[kCompBatch];
      float2 wv[kCompBatch];
#pragma unroll
      for (int j = 0; j < kCompBatch; ++j) {
        idx[j] = c0 + j < r ? __builtin_amdgcn_readlane(civ, c0 + j) : -1;
        if ((unsigned)idx[j] < (unsigned)D) wv[j] = ld2(A.comp_val + ((size_t)s * r + c0 + j) * D + 2 * lane);
      }
#pragma unroll
      for (int j = 0; j < kCompBatch; ++j) {
        if ((unsigned)idx[j] < (unsigned)D) {
          const float2 gg = sh_gy[idx[j]];
          zb.x = fmaf(wv[j].x, gg.x, zb.x); zb.y = fmaf(wv[j].y, gg.x, zb.y);
          zq.x = fmaf(wv[j].x, gg.y, zq.x); zq.y = fmaf(wv[j].y, gg.y, zq.y);
        }
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
    // older records (p > kRecChunk): kOldBatch loads in flight before use
    for (int i0 = 0; i0 < ulo; i0 += kOldBatch) {
      float2 uo[kOldBatch];
#pragma unroll
      for (int j = 0; j < kOldBatch; ++j)
        if (i0 + j < ulo) uo[j] = ld2(A.buf_u + (rec0 + i0 + j) * D + 2 * lane);
#pragma unroll
      for (int j = 0; j < kOldBatch; ++j) {
        if (i0 + j < ulo) {
          const float2 h = sh_h[i0 + j];
          zub.x = fmaf(uo[j].x, h.x, zub.x); zub.y = fmaf(uo[j].y, h.x, zub.y);
          zuq.x = fmaf(uo[j].x, h.y, zuq.x); zuq.y = fmaf(uo[j].y, h.y, zuq.y);
        }
      }
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
  // GDN gates and compensator row indices: lane-indexed vector loads,
  // broadcast with readlane (no scalar-load wait before the codes issue)
  float gv = 1.f;  // GDN: lane j holds the gate of record lo + j
  auto load_chunk = [&](int lo_, int cnt_) {
    if (!KDA && lane < cnt_) gv = A.buf_gate[rec0 + lo_ + lane];
#pragma unroll
    for (int j = 0; j < kRecChunk; ++j) {
      if (j < cnt_) {
        kr[j] = A.buf_k[(rec0 + lo_ + j) * D + row];
        if (KDA) gr[j] = A.buf_gate[(rec0 + lo_ + j) * D + row];
      }
    }
  };
  load_chunk(lo, hi - lo);
  // u rows of this wave's columns: issued with the first loads (one round
  // trip to memory fewer per wave; the registers fit 4 waves per SIMD)
  const int ulo = t > kRecChunk ? t - kRecChunk : 0;
  float ur[kRecChunk];
#pragma unroll
  for (int j = 0; j < kRecChunk; ++j)
    if (j < t - ulo) ur[j] = A.buf_u[(rec0 + ulo + j) * D + col];
  int civ = -1;  // lane c < r: compensator row index c
  if (!DENSE && lane < r) civ = A.comp_idx[(size_t)s * r + lane];
  float cw[kCompEarly];
  float ck[DENSE ? kCompEarly : 1];  // dense keys at this lane's row
#pragma unroll
  for (int c = 0; c < kCompEarly; ++c) {
    if (c < r) {
      if constexpr (DENSE) ck[c] = A.comp_key[((size_t)s * r + c) * D + row];
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
        P *= KDA ? gr[j] : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), j));
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
    if (hi > 0) {
      // Every load of the chunk just used has returned.  Saying so lets the
      // next chunk's loads issue back to back: the compiler cannot pair the
      // guarded loads (j < cnt) with their guarded uses, and would otherwise
      // wait for each earlier load into the same registers first.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      load_chunk(lo, hi - lo);
    }
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
    for (int c0 = kCompEarly; c0 < r; c0 += kCompBatch) {  // four loads in flight
      float kc[kCompBatch];
#pragma unroll
      for (int j = 0; j < kCompBatch; ++j)
        if (c0 + j < r) kc[j] = A.comp_key[((size_t)s * r + c0 + j) * D + row];
#pragma unroll
      for (int j = 0; j < kCompBatch; ++j)
        if (c0 + j < r) put(c0 + j, kc[j]);
    }
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
    for (int c0 = kCompEarly; c0 < r; c0 += kCompBatch) {
      float wv[kCompBatch];
#pragma unroll
      for (int j = 0; j < kCompBatch; ++j)
        if (c0 + j < r) wv[j] = A.comp_val[((size_t)s * r + c0 + j) * D + col];
#pragma unroll
      for (int j = 0; j < kCompBatch; ++j) {
        if (c0 + j < r) {
          const float2 h0 = sh_hcp[0][c0 + j], h1 = sh_hcp[1][c0 + j];
          zb = fmaf(wv[j], h0.x + h1.x, zb);
          zq = fmaf(wv[j], h0.y + h1.y, zq);
        }
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < kCompEarly; ++c) {
      const int idx = __builtin_amdgcn_readlane(civ, c);
      if (c < r && (unsigned)idx < (unsigned)D) {
        const float2 gg = sh_gy[idx];
        zb = fmaf(cw[c], gg.x, zb);
        zq = fmaf(cw[c], gg.y, zq);
      }
    }
    for (int c0 = kCompEarly; c0 < r; c0 += kCompBatch) {  // four loads in flight
      int idx[kCompBatch];
      float wv[kCompBatch];
#pragma unroll
      for (int j = 0; j < kCompBatch; ++j) {
        idx[j] = c0 + j < r ? __builtin_amdgcn_readlane(civ, c0 + j) : -1;
        if ((unsigned)idx[j] < (unsigned)D) wv[j] = A.comp_val[((size_t)s * r + c0 + j) * D + col];
      }
#pragma unroll
      for (int j = 0; j < kCompBatch; ++j) {
        if ((unsigned)idx[j] < (unsigned)D) {
          const float2 gg = sh_gy[idx[j]];
          zb = fmaf(wv[j], gg.x, zb);
          zq = fmaf(wv[j], gg.y, zq);
        }
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
    // older records (p > kRecChunk): kOldBatch loads in flight before use
    for (int i0 = 0; i0 < ulo; i0 += kOldBatch) {
      float uo[kOldBatch];
#pragma unroll
      for (int j = 0; j < kOldBatch; ++j)
        if (i0 + j < ulo) uo[j] = A.buf_u[(rec0 + i0 + j) * D + col];
#pragma unroll
      for (int j = 0; j < kOldBatch; ++j) {
        if (i0 + j < ulo) {
          const float2 h0 = sh_hp[0][i0 + j], h1 = sh_hp[1][i0 + j];
          zub = fmaf(uo[j], h0.x + h1.x, zub);
          zuq = fmaf(uo[j], h0.y + h1.y, zuq);
        }
      }
    }
    zb += zub;
    zq += zuq;
  }
  const float ut = vv - zb;
  __builtin_nontemporal_store(fmaf(sh_kq[0] + sh_kq[1], ut, zq), A.o + so + col);
  __builtin_nontemporal_store(ut, A.buf_u + (rec0 + t) * D + col);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
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

}  // namespace lq
