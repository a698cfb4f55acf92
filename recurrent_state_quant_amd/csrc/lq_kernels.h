// Internal launch interface between the C ABI (lq_abi.cpp) and the gfx950
// kernels (lq_decode.hip, lq_close.hip, lq_baselines.hip).  Arguments are
// validated by the caller.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace lq {

struct DecodeArgs {
  const int8_t *codes;
  const float *row_scale;
  const float *col_scale;
  const int32_t *comp_idx;
  const float *comp_val;
  const float *comp_key;  // dense compensator keys [n][r][dk] (nullptr: one-hot rows)
  float *buf_gate;
  float *buf_k;
  float *buf_u;
  const float *q;
  const float *k;
  const float *v;
  const float *beta;
  const float *alpha;
  float *o;
  const int32_t *pos;  // per-state window position (nullptr: t for all)
  int n, p, r, t;
  unsigned flags;      // bit 1: b_t = 0 (no delta correction)
  bool skip_last;      // states at position p - 1 are left to a fused close
};

struct CloseArgs {
  int8_t *codes;
  float *row_scale;
  float *col_scale;
  int32_t *comp_idx;
  float *comp_val;
  float *comp_key;    // dense compensator keys [n][r][dk] (nullptr: one-hot rows)
  const float *buf_gate;
  const float *buf_k;
  const float *buf_u;
  const float *S_in;  // quantize_state source; nullptr for a window close
  // decode_close only: the last token's inputs and output
  const float *q, *k, *v, *beta, *alpha;
  float *o;
  // per-state record counts (nullptr: len for all); for decode_close the
  // last token's window position
  const int32_t *lens;
  // compacted launch: workgroup i closes state slots[i] (ids outside
  // [0, n) skipped); nullptr: workgroup i closes state i
  const int32_t *slots;
  int n_launch;      // workgroups when slots != nullptr
  int n, p, r, len;  // len: buffered records the rebuild replays
  int iters;         // dense compensators: subspace iterations of the split
  unsigned flags;
  bool only_last;    // decode_close over a slot list: listed slots not at position p - 1 are skipped
};

// One launch for a continuous-batching token: the fused decode_close of the
// listed slots at their window's last position (workgroups spread through
// the first half of the grid), and the decode step of every slot at
// positions 0 .. p-2 (four slots per workgroup).  mixed_supported() names
// the shapes it covers (windows of 4 to 16 tokens, at most 8 compensator
// rows, slabs above 4,096 slots); others take two launches.
struct MixedArgs {
  DecodeArgs d;   // pos = the per-slot positions, skip_last = true
  CloseArgs c;    // lens = the same positions, slots = the list, only_last = true
};
bool mixed_supported(const CloseArgs &c);

struct DequantArgs {
  const int8_t *codes;
  const float *row_scale;
  const float *col_scale;
  const int32_t *comp_idx;
  const float *comp_val;
  const float *comp_key;  // dense compensator keys (nullptr: one-hot rows)
  float *S_out;
  int n, r;
};

// Dense-state per-token decode (the uncompressed baselines): S is fp32 or
// bf16 [n][dk][dv], updated in place.
struct DenseArgs {
  void *S;
  const float *q, *k, *v, *beta, *alpha;
  float *o;
  int n;
  unsigned flags;  // bit 1: b_t = 0 (no delta correction)
};

// "BF16 + per-window": a dense bf16 boundary state B [n][dk][dv] and the
// fp32 window buffer.  t: the token's window position (decode) or the
// number of records to replay (close).
struct Bf16WinArgs {
  uint16_t *B;
  float *buf_gate;
  float *buf_k;
  float *buf_u;
  const float *q, *k, *v, *beta, *alpha;
  float *o;
  int n, p, t;
  unsigned flags;  // bit 1: b_t = 0 (no delta correction)
};

hipError_t launch_decode_step(const DecodeArgs &a, bool kda, hipStream_t stream);
hipError_t launch_bf16w_decode(const Bf16WinArgs &a, bool kda, hipStream_t stream);
hipError_t launch_bf16w_close(const Bf16WinArgs &a, bool kda, hipStream_t stream);
hipError_t launch_dense_step(const DenseArgs &a, bool kda, bool bf16, hipStream_t stream);
hipError_t launch_stream_ref(const void *src, uint32_t per_wave, void *dst, uint32_t write_bytes, int idle,
                             int waves, uint32_t *out, hipStream_t stream);
hipError_t launch_window_close(const CloseArgs &a, bool kda, hipStream_t stream);
hipError_t launch_decode_close(const CloseArgs &a, bool kda, hipStream_t stream);
hipError_t launch_quantize_state(const CloseArgs &a, hipStream_t stream);
hipError_t launch_dequantize(const DequantArgs &a, hipStream_t stream);
hipError_t launch_mixed(const MixedArgs &a, bool kda, hipStream_t stream);

}  // namespace lq
