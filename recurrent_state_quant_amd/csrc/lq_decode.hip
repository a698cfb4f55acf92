// LeapQuant decode step for gfx950: one wave per state (large slabs) or two
// waves per state (slabs of at most 4,096 states).
#include "lq_decode_one.h"

namespace lq {

// The GDN step of windows up to 17 tokens fits 128 VGPRs and 9,984 bytes
// of LDS: four waves per SIMD (the others take what they need).
template <bool KDA, bool DENSE, bool LONG>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(KDA || DENSE || LONG ? 1 : 4))) void
decode_step_kernel(const DecodeArgs A) {
  const int s = blockIdx.x;
  // per-slot positions (continuous batching): out-of-range slots are idle;
  // with skip_last the window's last position is left to a fused close
  const int t = A.pos ? A.pos[s] : A.t;
  if (t < 0 || t >= (A.skip_last ? A.p - 1 : A.p)) return;
  __shared__ float2 ls_gy[D];
  __shared__ float2 ls_h[64];
  __shared__ float2 ls_hc[DENSE ? 16 : 1];
  __shared__ __attribute__((aligned(16))) float ls_red[64 * kRedStride];
  // z and the digits share the record dots' transpose buffer
  const DecodeLds Ls{ls_gy, ls_h, ls_hc, reinterpret_cast<float2 *>(ls_red),
                     reinterpret_cast<uint8_t *>(ls_red) + D * 8, ls_red};
  const int lane = threadIdx.x;
  constexpr bool WAVE = false;
#include "lq_decode_body.inc"
}

// Decode step for small slabs, two waves per state: wave w owns key rows
// 64w .. 64w+63 (code half w) for the record dots and the GEMV, and value
// columns 64w .. 64w+63 for the combine.  Each wave scales its half of the
// weights by its own power of two; the halves' GEMV results and record dots
// meet in fp32 through LDS.  A slab of n states is n workgroups of two
// waves: with n <= 4,096 this fills the chip where one wave per state would
// not (measured: +5% at 2,048 states, +18% for KDA at 4,096), while at
// 8,192 states and more the one-wave kernel is faster (1.6%).
template <bool KDA, bool DENSE, bool LONG>
__global__ __launch_bounds__(128) void decode_step2_kernel(const DecodeArgs A) {
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int p = A.p, r = A.r;
  const int t = A.pos ? A.pos[s] : A.t;
  if (t < 0 || t >= (A.skip_last ? p - 1 : p)) return;
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
  // record dots of the chunk [lo_, lo_ + cnt), newest record first
  auto chunk_dots = [&](const int lo_, const int cnt) {
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
    lds_sync<true>();
    {
      const int v = lane & 31, half = lane >> 5;
      float acc = 0.f;
      if (v < 2 * cnt) {
#pragma unroll 8
        for (int m = 0; m < 16; ++m) acc += red[(16 * half + m) * kRedStride + v];
      }
      acc += __shfl_xor(acc, 32);
      if (lane < 2 * cnt) reinterpret_cast<float *>(&sh_hp[w][lo_ + (lane >> 1)])[lane & 1] = acc;
    }
    lds_sync<true>();
  };
  // The newest chunk (loaded above) outside any loop, so that its uses wait
  // for its own loads only; older chunks (windows longer than kRecChunk + 1
  // tokens) are loaded and used one after the other.
  if (hi > 0) chunk_dots(lo, hi - lo);
  if constexpr (LONG) {
    for (hi = lo; hi > 0; hi = lo) {
      lo = hi > kRecChunk ? hi - kRecChunk : 0;
      load_chunk(lo, hi - lo);
      chunk_dots(lo, hi - lo);
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
    for (int i0 = 0; LONG && i0 < ulo; i0 += kOldBatch) {
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

template <bool KDA, bool DENSE>
void launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
  if (a.n <= kSmallSlab && a.p > kRecChunk + 1)
    hipLaunchKernelGGL((decode_step2_kernel<KDA, DENSE, true>), dim3(a.n), dim3(128), 0, stream, a);
  else if (a.n <= kSmallSlab)
    hipLaunchKernelGGL((decode_step2_kernel<KDA, DENSE, false>), dim3(a.n), dim3(128), 0, stream, a);
  else if (a.p > kRecChunk + 1)
    hipLaunchKernelGGL((decode_step_kernel<KDA, DENSE, true>), dim3(a.n), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_step_kernel<KDA, DENSE, false>), dim3(a.n), dim3(64), 0, stream, a);
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
