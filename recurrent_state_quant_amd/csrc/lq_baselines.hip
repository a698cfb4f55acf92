// Baselines the quantized path is compared with, for gfx950: the dense
// fp32 / bf16 per-step state update and the bf16 per-window state.
#include "lq_device.h"

namespace lq {

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
  // u rows of the newest kRecChunk records at this thread's column (threads
  // tid < D), issued with the state loads: they are consumed after the
  // GEMV, one round trip later than these
  const int ulo = t > kRecChunk ? t - kRecChunk : 0;
  float ur[kRecChunk];
  if (tid < D) {
#pragma unroll
    for (int j = 0; j < kRecChunk; ++j)
      if (j < t - ulo) ur[j] = A.buf_u[(rec0 + ulo + j) * D + tid];
  }
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
      // GDN: lane j holds the gate of record lo + j (a vector load, so no
      // scalar-load wait lands between the record loads)
      float gv = 1.f;
      if (!KDA && lane < cnt) gv = A.buf_gate[rec0 + lo + lane];
#pragma unroll
      for (int j = 0; j < kRecChunk; ++j) {
        if (j < cnt) {
          kr[j] = A.buf_k[(rec0 + lo + j) * D + row];
          if (KDA) gr[j] = A.buf_gate[(rec0 + lo + j) * D + row];
        }
      }
#pragma unroll
      for (int j = kRecChunk - 1; j >= 0; --j) {
        if (j < cnt) {
          const float kw = kr[j] * P;
          const float hb = wave_sum(kw * yb), hq = wave_sum(kw * yq);
          if (lane == 0) sh_hp[w][lo + j] = make_float2(hb, hq);
          P *= KDA ? gr[j] : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), j));
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
    // records older than the newest chunk (p > kRecChunk), eight loads in
    // flight before their use
    for (int i0 = 0; i0 < ulo; i0 += 8) {
      float uo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (i0 + j < ulo) uo[j] = A.buf_u[(rec0 + i0 + j) * D + col];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (i0 + j < ulo) {
          const float2 h0 = sh_hp[0][i0 + j], h1 = sh_hp[1][i0 + j];
          zb = fmaf(uo[j], h0.x + h1.x, zb);
          zq = fmaf(uo[j], h0.y + h1.y, zq);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kRecChunk; ++j) {
      if (j < t - ulo) {
        const float2 h0 = sh_hp[0][ulo + j], h1 = sh_hp[1][ulo + j];
        zb = fmaf(ur[j], h0.x + h1.x, zb);
        zq = fmaf(ur[j], h0.y + h1.y, zq);
      }
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
    {
      // kRecChunk * D / 4 = 512 float4 per array: two per thread, every
      // load issued before the first LDS write
      static_assert(kRecChunk * D / 4 == 512, "staging assumes two float4 per thread");
      const int nvec = cnt * (D / 4), e0 = tid, e1 = tid + 256;
      const float *sk = A.buf_k + (rec0 + lo) * D, *su = A.buf_u + (rec0 + lo) * D;
      const float *sg = A.buf_gate + (rec0 + lo) * D;
      const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
      float4 k0 = z4, k1 = z4, u0 = z4, u1 = z4, g0 = z4, g1 = z4;
      if (e0 < nvec) {
        k0 = ld4(sk + 4 * e0);
        u0 = ld4(su + 4 * e0);
        if (KDA) g0 = ld4(sg + 4 * e0);
      }
      if (e1 < nvec) {
        k1 = ld4(sk + 4 * e1);
        u1 = ld4(su + 4 * e1);
        if (KDA) g1 = ld4(sg + 4 * e1);
      }
      float gs = 1.f;
      if (!KDA && tid < cnt) gs = A.buf_gate[rec0 + lo + tid];
      float4 *dk = reinterpret_cast<float4 *>(sh_K), *du = reinterpret_cast<float4 *>(sh_U);
      float4 *dg = reinterpret_cast<float4 *>(sh_g);
      if (e0 < nvec) {
        dk[e0] = k0;
        du[e0] = u0;
        if (KDA) dg[e0] = g0;
      }
      if (e1 < nvec) {
        dk[e1] = k1;
        du[e1] = u1;
        if (KDA) dg[e1] = g1;
      }
      if (!KDA && tid < cnt) sh_g[tid] = gs;
    }
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

hipError_t launch_bf16w_decode(const Bf16WinArgs &a, bool kda, hipStream_t stream) {
  if (kda)
    hipLaunchKernelGGL(bf16w_decode_kernel<true>, dim3(a.n), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bf16w_decode_kernel<false>, dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stream reference for the decode step's launch shape (a measurement aid,
// no arithmetic of the method): one 64-lane wave per block of per_wave
// bytes, read with 16-byte nontemporal loads in batches of 16 per lane
// (16 KiB per wave, every load of a batch issued before any is used, as
// the decode issues its code stream; loads past the block's end return
// zero without a memory access), then `idle` sleeps of 512 cycles each
// with nothing in flight (standing in for the work a decode wave does after
// its loads return), then write_bytes bytes written per wave at its end (8
// bytes per lane per 512-byte row, as the decode stores its output rows).
// Each lane also writes one checksum word.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void stream_ref_kernel(const uint8_t *src, uint32_t per_wave, float *dst,
                                                        uint32_t write_bytes, int idle, uint32_t *out) {
  const int lane = threadIdx.x;
  const BufRsrc rs = buf_rsrc(src + (size_t)blockIdx.x * per_wave, (int)per_wave);
  uint32_t acc = 0;
  for (uint32_t off = 0; off < per_wave; off += 16384) {
    vu4 x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      x[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + 1024 * j + 16 * lane), 0, kBufNt);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc += x[j].x ^ x[j].y ^ x[j].z ^ x[j].w;
  }
  for (int i = 0; i < idle; ++i) __builtin_amdgcn_s_sleep(8);  // 8 x 64 cycles
  const float f = __uint_as_float(acc);
  float *row = dst + (size_t)blockIdx.x * (write_bytes / 4) + 2 * lane;
  for (uint32_t b = 0; b < write_bytes; b += 512, row += 128) st2(row, make_float2(f, f));
  out[(size_t)blockIdx.x * 64 + lane] = acc;
}

hipError_t launch_stream_ref(const void *src, uint32_t per_wave, void *dst, uint32_t write_bytes, int idle,
                             int waves, uint32_t *out, hipStream_t stream) {
  hipLaunchKernelGGL(stream_ref_kernel, dim3(waves), dim3(64), 0, stream, static_cast<const uint8_t *>(src),
                     per_wave, static_cast<float *>(dst), write_bytes, idle, out);
  return hipGetLastError();
}

hipError_t launch_bf16w_close(const Bf16WinArgs &a, bool kda, hipStream_t stream) {
  if (kda)
    hipLaunchKernelGGL(bf16w_close_kernel<true>, dim3(a.n), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bf16w_close_kernel<false>, dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lq
