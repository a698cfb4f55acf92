// C ABI of the LeapQuant decode path: argument validation and launches.
// Operation semantics are documented in include/leapquant.h.
#include <stdint.h>

#include "leapquant.h"
#include "lq_kernels.h"

namespace {

constexpr int kDim = 128;
constexpr int kMaxP = 64;
constexpr int kMaxR = 16;
constexpr int kMaxIters = 8;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range span(const void *p, size_t bytes) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  return Range{b, b + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int check_params(const lq_params *prm) {
  if (!prm) return LQ_ERR_NULL;
  if (prm->dk != kDim || prm->dv != kDim) return LQ_ERR_UNSUPPORTED;
  if (prm->n < 1 || prm->p < 1 || prm->p > kMaxP || prm->r < 0 || prm->r > kMaxR) return LQ_ERR_SHAPE;
  if (prm->gate != LQ_GATE_GDN && prm->gate != LQ_GATE_KDA) return LQ_ERR_SHAPE;
  if (prm->flags & ~static_cast<uint32_t>(LQ_NO_SMOOTH | LQ_NO_DELTA | LQ_DENSE_COMP))
    return LQ_ERR_SHAPE;
  if (prm->comp_iters < 0 || prm->comp_iters > kMaxIters) return LQ_ERR_SHAPE;
  return LQ_OK;
}

bool dense_comp(const lq_params *prm) { return (prm->flags & LQ_DENSE_COMP) && prm->r > 0; }

// Byte range of the compensator keys (empty without dense compensators).
Range key_span(const lq_params *prm, const lq_state *st) {
  if (!dense_comp(prm)) return Range{0, 0};
  return span(st->comp_key, static_cast<size_t>(prm->n) * prm->r * kDim * sizeof(float));
}

// Boundary-state arrays (always needed).
int check_boundary(const lq_params *prm, const lq_state *st) {
  if (!st) return LQ_ERR_NULL;
  if (!st->codes || !st->row_scale || !st->col_scale) return LQ_ERR_NULL;
  if (prm->r > 0 && (!st->comp_idx || !st->comp_val)) return LQ_ERR_NULL;
  if (!aligned(st->codes, 16) || !aligned(st->row_scale, 16) || !aligned(st->col_scale, 16))
    return LQ_ERR_ALIGN;
  if (prm->r > 0 && (!aligned(st->comp_idx, 4) || !aligned(st->comp_val, 16))) return LQ_ERR_ALIGN;
  if (dense_comp(prm)) {
    if (!st->comp_key) return LQ_ERR_NULL;
    if (!aligned(st->comp_key, 16)) return LQ_ERR_ALIGN;
  }
  return LQ_OK;
}

int check_buffer(const lq_params *prm, const lq_state *st) {
  if (!st->buf_gate || !st->buf_k || !st->buf_u) return LQ_ERR_NULL;
  const uintptr_t ga = prm->gate == LQ_GATE_KDA ? 16 : 4;
  if (!aligned(st->buf_gate, ga) || !aligned(st->buf_k, 16) || !aligned(st->buf_u, 16))
    return LQ_ERR_ALIGN;
  return LQ_OK;
}

// Byte ranges of the state's arrays: the boundary half and / or the buffer
// half; arrays a call does not use give empty ranges.  Returns the count.
int state_ranges(const lq_params *prm, const lq_state *st, bool boundary, bool buffer, Range *rs) {
  const size_t n = static_cast<size_t>(prm->n), p = static_cast<size_t>(prm->p);
  const size_t r = static_cast<size_t>(prm->r);
  const size_t vec = n * kDim * sizeof(float);
  int m = 0;
  if (boundary) {
    rs[m++] = span(st->codes, n * kDim * kDim);
    rs[m++] = span(st->row_scale, vec);
    rs[m++] = span(st->col_scale, vec);
    if (r > 0) {
      rs[m++] = span(st->comp_idx, n * r * sizeof(int32_t));
      rs[m++] = span(st->comp_val, n * r * kDim * sizeof(float));
    }
    rs[m++] = key_span(prm, st);
  }
  if (buffer) {
    const size_t gate_elems = prm->gate == LQ_GATE_KDA ? n * p * kDim : n * p;
    rs[m++] = span(st->buf_gate, gate_elems * sizeof(float));
    rs[m++] = span(st->buf_k, n * p * kDim * sizeof(float));
    rs[m++] = span(st->buf_u, n * p * kDim * sizeof(float));
  }
  return m;
}

// The arrays of one state must not overlap one another: a launch that writes
// the state reads the same arrays (the boundary in the close, the buffer row
// of the current token in the decode).  `boundary` and `buffer` select the
// halves the call uses.
int check_state_disjoint(const lq_params *prm, const lq_state *st, bool boundary, bool buffer) {
  Range rs[9];
  const int m = state_ranges(prm, st, boundary, buffer, rs);
  for (int i = 0; i < m; ++i)
    for (int j = i + 1; j < m; ++j)
      if (overlap(rs[i], rs[j])) return LQ_ERR_ALIAS;
  return LQ_OK;
}

// A caller array `x` must not overlap any array of the state: the token
// calls write records (decode) or the whole boundary (fused close) while
// their workgroups read the inputs, so any overlap is a race.
bool overlaps_state(Range x, const lq_params *prm, const lq_state *st, bool boundary, bool buffer) {
  Range rs[9];
  const int m = state_ranges(prm, st, boundary, buffer, rs);
  for (int i = 0; i < m; ++i)
    if (overlap(x, rs[i])) return true;
  return false;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LQ_OK : LQ_ERR_HIP; }

// Kernel arguments of a call: the state's arrays (the window buffer too if
// `buffer`) and the parameters.
lq::CloseArgs close_args(const lq_params *prm, const lq_state *st, bool buffer) {
  lq::CloseArgs a{};
  a.codes = st->codes;
  a.row_scale = st->row_scale;
  a.col_scale = st->col_scale;
  a.comp_idx = st->comp_idx;
  a.comp_val = st->comp_val;
  a.comp_key = dense_comp(prm) ? st->comp_key : nullptr;
  if (buffer) {
    a.buf_gate = st->buf_gate;
    a.buf_k = st->buf_k;
    a.buf_u = st->buf_u;
  }
  a.n = prm->n;
  a.p = prm->p;
  a.r = prm->r;
  a.flags = prm->flags;
  a.iters = prm->comp_iters;
  return a;
}

// The token's inputs and output
template <class Args>
void set_token(Args &a, const float *q, const float *k, const float *v, const float *beta, const float *alpha,
               float *o) {
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.alpha = alpha;
  a.o = o;
}

lq::DecodeArgs decode_args(const lq_params *prm, const lq_state *st, const float *q, const float *k,
                           const float *v, const float *beta, const float *alpha, float *o) {
  lq::DecodeArgs a{};
  a.codes = st->codes;
  a.row_scale = st->row_scale;
  a.col_scale = st->col_scale;
  a.comp_idx = st->comp_idx;
  a.comp_val = st->comp_val;
  a.comp_key = dense_comp(prm) ? st->comp_key : nullptr;
  a.buf_gate = st->buf_gate;
  a.buf_k = st->buf_k;
  a.buf_u = st->buf_u;
  set_token(a, q, k, v, beta, alpha, o);
  a.n = prm->n;
  a.p = prm->p;
  a.r = prm->r;
  a.flags = prm->flags;
  return a;
}

}  // namespace

extern "C" {

int leapquant_abi_version(void) { return LEAPQUANT_ABI_VERSION; }

const char *leapquant_status_string(int status) {
  switch (status) {
    case LQ_OK: return "ok";
    case LQ_ERR_NULL: return "a required pointer is NULL";
    case LQ_ERR_SHAPE: return "invalid size or parameter (n, p, r, gate, flags, t or len)";
    case LQ_ERR_UNSUPPORTED: return "unsupported head size (dk and dv must be 128)";
    case LQ_ERR_ALIGN: return "pointer is not aligned as required";
    case LQ_ERR_ALIAS: return "an output overlaps an input, or two arrays of the state overlap";
    case LQ_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int leapquant_quantize_state(const lq_params *prm, const float *S, const lq_state *st,
                             hipStream_t stream) {
  int rc = check_params(prm);
  if (rc) return rc;
  if ((rc = check_boundary(prm, st))) return rc;
  if (!S) return LQ_ERR_NULL;
  if (!aligned(S, 16)) return LQ_ERR_ALIGN;
  const size_t n = static_cast<size_t>(prm->n);
  const Range src = span(S, n * kDim * kDim * sizeof(float));
  if (overlap(src, span(st->codes, n * kDim * kDim)) ||
      overlap(src, span(st->row_scale, n * kDim * sizeof(float))) ||
      overlap(src, span(st->col_scale, n * kDim * sizeof(float))) ||
      (prm->r > 0 && (overlap(src, span(st->comp_idx, n * prm->r * sizeof(int32_t))) ||
                      overlap(src, span(st->comp_val, n * prm->r * kDim * sizeof(float))))) ||
      overlap(src, key_span(prm, st)))
    return LQ_ERR_ALIAS;
  if ((rc = check_state_disjoint(prm, st, true, false))) return rc;
  lq::CloseArgs a = close_args(prm, st, false);
  a.S_in = S;
  return hip_status(lq::launch_quantize_state(a, stream));
}

}  // extern "C"

namespace {

// Checks shared by the token entry points: parameters, state, t, the token
// inputs, that o overlaps no input, and that no input or o overlaps an array
// of the state.
int check_token_call(const lq_params *prm, const lq_state *st, int32_t t, const float *q,
                     const float *k, const float *v, const float *beta, const float *alpha,
                     const float *o) {
  int rc = check_params(prm);
  if (rc) return rc;
  if ((rc = check_boundary(prm, st))) return rc;
  if ((rc = check_buffer(prm, st))) return rc;
  if ((rc = check_state_disjoint(prm, st, true, true))) return rc;
  if (t < 0 || t >= prm->p) return LQ_ERR_SHAPE;
  if (!q || !k || !v || !beta || !alpha || !o) return LQ_ERR_NULL;
  const bool kda = prm->gate == LQ_GATE_KDA;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(beta, 4) || !aligned(alpha, kda ? 16 : 4))
    return LQ_ERR_ALIGN;
  const size_t n = static_cast<size_t>(prm->n);
  const size_t vec = n * kDim * sizeof(float);
  const Range out = span(o, vec);
  const Range in[5] = {span(q, vec), span(k, vec), span(v, vec), span(beta, n * sizeof(float)),
                       span(alpha, kda ? vec : n * sizeof(float))};
  if (overlaps_state(out, prm, st, true, true)) return LQ_ERR_ALIAS;
  for (const Range &x : in)
    if (overlap(out, x) || overlaps_state(x, prm, st, true, true)) return LQ_ERR_ALIAS;
  return LQ_OK;
}

}  // namespace

extern "C" {

int leapquant_decode_step(const lq_params *prm, const lq_state *st, int32_t t, const float *q,
                          const float *k, const float *v, const float *beta, const float *alpha,
                          float *o, hipStream_t stream) {
  const int rc = check_token_call(prm, st, t, q, k, v, beta, alpha, o);
  if (rc) return rc;
  lq::DecodeArgs a = decode_args(prm, st, q, k, v, beta, alpha, o);
  a.t = t;
  return hip_status(lq::launch_decode_step(a, prm->gate == LQ_GATE_KDA, stream));
}

int leapquant_window_close(const lq_params *prm, const lq_state *st, int32_t len,
                           hipStream_t stream) {
  int rc = check_params(prm);
  if (rc) return rc;
  if ((rc = check_boundary(prm, st))) return rc;
  if ((rc = check_buffer(prm, st))) return rc;
  if ((rc = check_state_disjoint(prm, st, true, true))) return rc;
  if (len < 1 || len > prm->p) return LQ_ERR_SHAPE;
  lq::CloseArgs a = close_args(prm, st, true);
  a.len = len;
  return hip_status(lq::launch_window_close(a, prm->gate == LQ_GATE_KDA, stream));
}

int leapquant_decode_close(const lq_params *prm, const lq_state *st, int32_t t, const float *q,
                           const float *k, const float *v, const float *beta, const float *alpha,
                           float *o, hipStream_t stream) {
  const int rc = check_token_call(prm, st, t, q, k, v, beta, alpha, o);
  if (rc) return rc;
  lq::CloseArgs a = close_args(prm, st, true);
  set_token(a, q, k, v, beta, alpha, o);
  a.len = t;
  return hip_status(lq::launch_decode_close(a, prm->gate == LQ_GATE_KDA, stream));
}

// ---- continuous batching: per-slot window positions on the device
static int check_slots(const lq_params *prm, const lq_state *st, const int32_t *v, const float *o) {
  if (!v) return LQ_ERR_NULL;
  if (!aligned(v, 4)) return LQ_ERR_ALIGN;
  const size_t n = static_cast<size_t>(prm->n);
  const Range in = span(v, n * sizeof(int32_t));
  if ((o && overlap(in, span(o, n * kDim * sizeof(float)))) || overlaps_state(in, prm, st, true, true))
    return LQ_ERR_ALIAS;
  return LQ_OK;
}

int leapquant_decode_step_slots(const lq_params *prm, const lq_state *st, const int32_t *pos,
                                const float *q, const float *k, const float *v, const float *beta,
                                const float *alpha, float *o, hipStream_t stream) {
  int rc = check_token_call(prm, st, 0, q, k, v, beta, alpha, o);
  if (rc) return rc;
  if ((rc = check_slots(prm, st, pos, o))) return rc;
  lq::DecodeArgs a = decode_args(prm, st, q, k, v, beta, alpha, o);
  a.pos = pos;
  return hip_status(lq::launch_decode_step(a, prm->gate == LQ_GATE_KDA, stream));
}

int leapquant_decode_close_slots(const lq_params *prm, const lq_state *st, const int32_t *pos,
                                 const float *q, const float *k, const float *v, const float *beta,
                                 const float *alpha, float *o, hipStream_t stream) {
  int rc = check_token_call(prm, st, 0, q, k, v, beta, alpha, o);
  if (rc) return rc;
  if ((rc = check_slots(prm, st, pos, o))) return rc;
  lq::CloseArgs a = close_args(prm, st, true);
  set_token(a, q, k, v, beta, alpha, o);
  a.lens = pos;
  return hip_status(lq::launch_decode_close(a, prm->gate == LQ_GATE_KDA, stream));
}

int leapquant_window_close_slots(const lq_params *prm, const lq_state *st, const int32_t *len,
                                 hipStream_t stream) {
  int rc = check_params(prm);
  if (rc) return rc;
  if ((rc = check_boundary(prm, st))) return rc;
  if ((rc = check_buffer(prm, st))) return rc;
  if ((rc = check_state_disjoint(prm, st, true, true))) return rc;
  if ((rc = check_slots(prm, st, len, nullptr))) return rc;
  lq::CloseArgs a = close_args(prm, st, true);
  a.lens = len;
  a.len = 1;
  return hip_status(lq::launch_window_close(a, prm->gate == LQ_GATE_KDA, stream));
}

// Compacted forms: the slot list (count int32 ids on the device) must not
// overlap the state, the outputs or the per-slot array.
static int check_list(const lq_params *prm, const lq_state *st, const int32_t *v, const int32_t *list,
                      int32_t count, const float *o) {
  if (count < 0 || count > prm->n) return LQ_ERR_SHAPE;
  if (count == 0) return LQ_OK;
  if (!list) return LQ_ERR_NULL;
  if (!aligned(list, 4)) return LQ_ERR_ALIGN;
  const size_t n = static_cast<size_t>(prm->n);
  const Range in = span(list, static_cast<size_t>(count) * sizeof(int32_t));
  if ((o && overlap(in, span(o, n * kDim * sizeof(float)))) || overlap(in, span(v, n * sizeof(int32_t))) ||
      overlaps_state(in, prm, st, true, true))
    return LQ_ERR_ALIAS;
  return LQ_OK;
}

int leapquant_decode_close_list(const lq_params *prm, const lq_state *st, const int32_t *pos,
                                const int32_t *list, int32_t count, const float *q, const float *k,
                                const float *v, const float *beta, const float *alpha, float *o,
                                hipStream_t stream) {
  int rc = check_token_call(prm, st, 0, q, k, v, beta, alpha, o);
  if (rc) return rc;
  if ((rc = check_slots(prm, st, pos, o))) return rc;
  if ((rc = check_list(prm, st, pos, list, count, o))) return rc;
  if (count == 0) return LQ_OK;
  lq::CloseArgs a = close_args(prm, st, true);
  set_token(a, q, k, v, beta, alpha, o);
  a.lens = pos;
  a.slots = list;
  a.n_launch = count;
  return hip_status(lq::launch_decode_close(a, prm->gate == LQ_GATE_KDA, stream));
}

int leapquant_decode_step_close_list(const lq_params *prm, const lq_state *st, const int32_t *pos,
                                     const int32_t *list, int32_t count, const float *q, const float *k,
                                     const float *v, const float *beta, const float *alpha, float *o,
                                     hipStream_t stream) {
  int rc = check_token_call(prm, st, 0, q, k, v, beta, alpha, o);
  if (rc) return rc;
  if ((rc = check_slots(prm, st, pos, o))) return rc;
  if ((rc = check_list(prm, st, pos, list, count, o))) return rc;
  lq::MixedArgs m{};
  lq::DecodeArgs &d = m.d;
  d = decode_args(prm, st, q, k, v, beta, alpha, o);
  d.pos = pos;
  d.skip_last = true;
  lq::CloseArgs &c = m.c;
  c = close_args(prm, st, true);
  set_token(c, q, k, v, beta, alpha, o);
  c.lens = pos;
  c.slots = list;
  c.n_launch = count;
  c.only_last = true;
  const bool kda = prm->gate == LQ_GATE_KDA;
  if (lq::mixed_supported(c)) return hip_status(lq::launch_mixed(m, kda, stream));
  // other shapes: the same work as two launches, the closes first
  if (count > 0 && (rc = hip_status(lq::launch_decode_close(c, kda, stream)))) return rc;
  return hip_status(lq::launch_decode_step(d, kda, stream));
}

int leapquant_window_close_list(const lq_params *prm, const lq_state *st, const int32_t *len,
                                const int32_t *list, int32_t count, hipStream_t stream) {
  int rc = check_params(prm);
  if (rc) return rc;
  if ((rc = check_boundary(prm, st))) return rc;
  if ((rc = check_buffer(prm, st))) return rc;
  if ((rc = check_state_disjoint(prm, st, true, true))) return rc;
  if ((rc = check_slots(prm, st, len, nullptr))) return rc;
  if ((rc = check_list(prm, st, len, list, count, nullptr))) return rc;
  if (count == 0) return LQ_OK;
  lq::CloseArgs a = close_args(prm, st, true);
  a.lens = len;
  a.slots = list;
  a.n_launch = count;
  a.len = 1;
  return hip_status(lq::launch_window_close(a, prm->gate == LQ_GATE_KDA, stream));
}

int leapquant_dense_step(const lq_params *prm, void *S, int32_t dtype, const float *q,
                         const float *k, const float *v, const float *beta, const float *alpha,
                         float *o, hipStream_t stream) {
  int rc = check_params(prm);
  if (rc) return rc;
  if (dtype != LQ_DENSE_FP32 && dtype != LQ_DENSE_BF16) return LQ_ERR_SHAPE;
  if (!S || !q || !k || !v || !beta || !alpha || !o) return LQ_ERR_NULL;
  const bool kda = prm->gate == LQ_GATE_KDA, bf16 = dtype == LQ_DENSE_BF16;
  if (!aligned(S, bf16 ? 8 : 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(o, 16) || !aligned(beta, 4) || !aligned(alpha, kda ? 16 : 4))
    return LQ_ERR_ALIGN;
  const size_t n = static_cast<size_t>(prm->n);
  const size_t vec = n * kDim * sizeof(float);
  const Range state = span(S, n * kDim * kDim * (bf16 ? 2 : 4));
  const Range out = span(o, vec);
  const Range in[5] = {span(q, vec), span(k, vec), span(v, vec), span(beta, n * sizeof(float)),
                       span(alpha, kda ? vec : n * sizeof(float))};
  if (overlap(state, out)) return LQ_ERR_ALIAS;
  for (const Range &x : in)
    if (overlap(state, x) || overlap(out, x)) return LQ_ERR_ALIAS;
  lq::DenseArgs a{};
  a.S = S;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.alpha = alpha;
  a.o = o;
  a.n = prm->n;
  a.flags = prm->flags;
  return hip_status(lq::launch_dense_step(a, kda, bf16, stream));
}

// ---- stream reference (measurement aid)
int leapquant_stream_reference(const void *src, int64_t read_bytes_per_wave, void *dst,
                               int64_t write_bytes_per_wave, int32_t idle_sleeps, int32_t waves,
                               uint32_t *out, hipStream_t stream) {
  if (!src || !out || (write_bytes_per_wave > 0 && !dst)) return LQ_ERR_NULL;
  const int64_t kMax = int64_t(1) << 30;
  if (read_bytes_per_wave < 1024 || read_bytes_per_wave > kMax || read_bytes_per_wave % 1024 != 0 ||
      write_bytes_per_wave < 0 || write_bytes_per_wave > kMax || write_bytes_per_wave % 512 != 0 ||
      idle_sleeps < 0 || idle_sleeps > 4096 || waves < 1)
    return LQ_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(out, 4) || (write_bytes_per_wave > 0 && !aligned(dst, 16)))
    return LQ_ERR_ALIGN;
  const size_t w = static_cast<size_t>(waves);
  const Range rd = span(src, static_cast<size_t>(read_bytes_per_wave) * w);
  const Range ck = span(out, w * 64 * sizeof(uint32_t));
  if (overlap(rd, ck)) return LQ_ERR_ALIAS;
  if (write_bytes_per_wave > 0) {
    const Range wr = span(dst, static_cast<size_t>(write_bytes_per_wave) * w);
    if (overlap(wr, rd) || overlap(wr, ck)) return LQ_ERR_ALIAS;
  }
  return hip_status(lq::launch_stream_ref(src, static_cast<uint32_t>(read_bytes_per_wave), dst,
                                          static_cast<uint32_t>(write_bytes_per_wave), idle_sleeps, waves, out,
                                          stream));
}

// ---- "BF16 + per-window": dense bf16 boundary state, fp32 window buffer
static int check_bf16w(const lq_params *prm, const void *B, const lq_state *st) {
  int rc = check_params(prm);
  if (rc) return rc;
  if (prm->flags & ~static_cast<uint32_t>(LQ_NO_DELTA)) return LQ_ERR_SHAPE;
  if (!st || !B) return LQ_ERR_NULL;
  if ((rc = check_buffer(prm, st))) return rc;
  if (!aligned(B, 16)) return LQ_ERR_ALIGN;
  const size_t n = static_cast<size_t>(prm->n);
  const Range b = span(B, n * kDim * kDim * 2);
  const size_t gate_elems = prm->gate == LQ_GATE_KDA ? n * prm->p * kDim : n * prm->p;
  if (overlap(b, span(st->buf_gate, gate_elems * sizeof(float))) ||
      overlap(b, span(st->buf_k, n * prm->p * kDim * sizeof(float))) ||
      overlap(b, span(st->buf_u, n * prm->p * kDim * sizeof(float))))
    return LQ_ERR_ALIAS;
  return check_state_disjoint(prm, st, false, true);
}

int leapquant_bf16w_decode_step(const lq_params *prm, const void *B, const lq_state *st, int32_t t,
                                const float *q, const float *k, const float *v, const float *beta,
                                const float *alpha, float *o, hipStream_t stream) {
  int rc = check_bf16w(prm, B, st);
  if (rc) return rc;
  if (t < 0 || t >= prm->p) return LQ_ERR_SHAPE;
  if (!q || !k || !v || !beta || !alpha || !o) return LQ_ERR_NULL;
  const bool kda = prm->gate == LQ_GATE_KDA;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(beta, 4) || !aligned(alpha, kda ? 16 : 4))
    return LQ_ERR_ALIGN;
  const size_t n = static_cast<size_t>(prm->n);
  const size_t vec = n * kDim * sizeof(float);
  const Range out = span(o, vec), bs = span(B, n * kDim * kDim * 2);
  const Range in[5] = {span(q, vec), span(k, vec), span(v, vec), span(beta, n * sizeof(float)),
                       span(alpha, kda ? vec : n * sizeof(float))};
  if (overlap(out, bs) || overlaps_state(out, prm, st, false, true)) return LQ_ERR_ALIAS;
  for (const Range &x : in)
    if (overlap(out, x) || overlap(bs, x) || overlaps_state(x, prm, st, false, true)) return LQ_ERR_ALIAS;
  lq::Bf16WinArgs a{};
  a.B = static_cast<uint16_t *>(const_cast<void *>(B));
  a.buf_gate = st->buf_gate;
  a.buf_k = st->buf_k;
  a.buf_u = st->buf_u;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.alpha = alpha;
  a.o = o;
  a.n = prm->n;
  a.p = prm->p;
  a.t = t;
  a.flags = prm->flags;
  return hip_status(lq::launch_bf16w_decode(a, kda, stream));
}

int leapquant_bf16w_window_close(const lq_params *prm, void *B, const lq_state *st, int32_t len,
                                 hipStream_t stream) {
  int rc = check_bf16w(prm, B, st);
  if (rc) return rc;
  if (len < 1 || len > prm->p) return LQ_ERR_SHAPE;
  lq::Bf16WinArgs a{};
  a.B = static_cast<uint16_t *>(B);
  a.buf_gate = st->buf_gate;
  a.buf_k = st->buf_k;
  a.buf_u = st->buf_u;
  a.n = prm->n;
  a.p = prm->p;
  a.t = len;
  a.flags = prm->flags;
  return hip_status(lq::launch_bf16w_close(a, prm->gate == LQ_GATE_KDA, stream));
}

int leapquant_dequantize_state(const lq_params *prm, const lq_state *st, float *S_out,
                               hipStream_t stream) {
  int rc = check_params(prm);
  if (rc) return rc;
  if ((rc = check_boundary(prm, st))) return rc;
  if (!S_out) return LQ_ERR_NULL;
  if (!aligned(S_out, 16)) return LQ_ERR_ALIGN;
  const size_t n = static_cast<size_t>(prm->n);
  const Range out = span(S_out, n * kDim * kDim * sizeof(float));
  if (overlap(out, span(st->codes, n * kDim * kDim)) ||
      overlap(out, span(st->row_scale, n * kDim * sizeof(float))) ||
      overlap(out, span(st->col_scale, n * kDim * sizeof(float))) ||
      (prm->r > 0 && (overlap(out, span(st->comp_idx, n * prm->r * sizeof(int32_t))) ||
                      overlap(out, span(st->comp_val, n * prm->r * kDim * sizeof(float))))) ||
      overlap(out, key_span(prm, st)))
    return LQ_ERR_ALIAS;
  lq::DequantArgs a{};
  a.comp_key = dense_comp(prm) ? st->comp_key : nullptr;
  a.codes = st->codes;
  a.row_scale = st->row_scale;
  a.col_scale = st->col_scale;
  a.comp_idx = st->comp_idx;
  a.comp_val = st->comp_val;
  a.S_out = S_out;
  a.n = prm->n;
  a.r = prm->r;
  return hip_status(lq::launch_dequantize(a, stream));
}

}  // extern "C"
