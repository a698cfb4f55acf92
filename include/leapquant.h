/*
 * leapquant.h -- C ABI of the LeapQuant decode hot path for AMD Instinct
 * MI355X (gfx950).
 *
 * The operations follow the pages about LeapQuant:
 *   [EL] "LeapQuant: Efficient Linear Attention with Accurate Recurrent State
 *        Quantization" (paper listing page): Abstract, Figure 2 (per-token
 *        vs per-window quantization), Figure 4 (state = quantized residual +
 *        compensator tokens + buffered updates), Appendix Table 4 (the
 *        delta-rule instances and the buffered record (d_i, k~_i, u_i)).
 *   [TM] "LeapQuant trims the memory burden of linear-attention models"
 *        (news write-up), section "Quantize less often, protect the
 *        outliers" (window, compensators, smoothing across channels).
 *
 * Model.  Each of n independent states S (dk x dv, one per sequence, head and
 * layer) evolves by the delta rule of [EL] Table 4:
 *     u_t = v_t - S_{t-1}^T b_t,   S_t = D_t S_{t-1} + k~_t u_t^T,   o_t = S_t^T q_t
 *   LQ_GATE_GDN (Gated DeltaNet row): D_t = alpha_t I, k~_t = beta_t k_t,
 *                b_t = alpha_t k_t (alpha_t one scalar per state).
 *   LQ_GATE_KDA (Kimi Delta Attention): D_t = Diag(alpha_t), k~_t = beta_t k_t,
 *                b_t = alpha_t * k_t (alpha_t one value per key channel).
 *   With the LQ_NO_DELTA flag, b_t = 0 (the other rows of Table 4).
 * Between window boundaries the state is kept as ([EL] Figure 2, Figure 4)
 *   B  = deQ(codes, a, s) + sum_c e_{idx_c} w_c^T      (fixed, low-bit)
 *   records (d_i, k~_i, u_i), i < t                    (fp32 buffer)
 * and S_{t-1} is exactly the recurrence started from B and replayed through
 * the records.  deQ(c, a, s)_ij = c_ij * a_i * s_j.  At the end of a window
 * the state is rebuilt and split again: the r rows of largest L2 norm become
 * compensator rows w_c (fp32, descending norm, ties to the lower row), the
 * remaining residual R is smoothed per value column by s_j = max_i |R_ij|
 * (1 for a zero column, or 1 everywhere with LQ_NO_SMOOTH) and quantized
 * per row: m_i = max_j |R_ij * (1/s_j)|, a_i = m_i / 127,
 * c_ij = clamp(rne(R_ij * (1/s_j) * (127/m_i)), -127, 127), all in fp32.
 *
 * Conventions for every entry point.
 *   - All array pointers are DEVICE memory owned by the caller; the library
 *     allocates, frees and synchronizes nothing and keeps no global state,
 *     so calls are reentrant.  lq_params and lq_state are host structs read
 *     only during the call.
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call
 *     returns without waiting.  Device faults surface at the caller's next
 *     synchronization.  Every pointer is memory of the device the launch
 *     runs on; call with that device current (hipSetDevice), since the
 *     default stream belongs to the current device.  The library keeps no
 *     state of its own and allocates no memory (the kernels use only the
 *     caller's arrays, registers and LDS), so every call may be captured in
 *     a graph; calls on different streams or host threads do not interfere
 *     unless their arrays overlap.
 *   - Arrays are dense, row-major, in the shapes given below; n is the
 *     leading dimension of every per-state array.  The codes of one state
 *     are a 16 KiB block stored column-major in two 64-row halves: code
 *     (i, j) is byte (i >> 6) * 8192 + j * 64 + slot(i & 63), where
 *     slot(x) = (x & 0x0C) << 2 | (x & 0x30) >> 2 | (x & 3) swaps the two
 *     2-bit fields above the lowest two bits.  Both kernels then move codes
 *     as 16-byte column segments (the int8 MFMA operand of the decode GEMV
 *     and the accumulator rows of one lane in the window close).
 *   - Alignment: codes and every float array whose per-state extent is a
 *     multiple of 128 floats must be 16-byte aligned; beta, a scalar alpha,
 *     comp_idx and a scalar buf_gate need 4-byte alignment.
 *   - Argument errors are returned synchronously and nothing is launched:
 *       LQ_ERR_NULL        a required pointer is NULL
 *       LQ_ERR_SHAPE       n < 1, p outside [1, 64], r outside [0, 16],
 *                          unknown gate or flag, t or len out of range
 *       LQ_ERR_UNSUPPORTED dk != 128 or dv != 128
 *       LQ_ERR_ALIGN       a pointer violates the alignment above
 *       LQ_ERR_ALIAS       an output range overlaps an input range, or two
 *                          arrays of the lq_state overlap (checked by every
 *                          call that writes the state)
 *     A failed launch returns LQ_ERR_HIP.
 *   - Values are not checked: NaN or Inf inputs give unspecified (but
 *     in-bounds) results.  comp_idx entries outside [0, dk) are ignored when
 *     the state is read; the r entries of a state are distinct rows (the
 *     split always writes them so), and duplicates give unspecified results.
 */
#ifndef LEAPQUANT_H
#define LEAPQUANT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LEAPQUANT_ABI_VERSION 6

typedef enum lq_status {
  LQ_OK = 0,
  LQ_ERR_NULL = -1,
  LQ_ERR_SHAPE = -2,
  LQ_ERR_UNSUPPORTED = -3,
  LQ_ERR_ALIGN = -4,
  LQ_ERR_ALIAS = -5,
  LQ_ERR_HIP = -6
} lq_status;

typedef enum lq_gate {
  LQ_GATE_GDN = 0, /* scalar decay per state and token (Gated DeltaNet)  */
  LQ_GATE_KDA = 1  /* per-key-channel decay (Kimi Delta Attention)       */
} lq_gate;

enum {
  LQ_NO_SMOOTH = 1u, /* ablation: s_j = 1 for every column                     */
  LQ_NO_DELTA = 2u,  /* b_t = 0, so u_t = v_t: the rows of [EL] Appendix Table 4
                        without the delta correction.  With LQ_GATE_GDN: linear
                        attention (alpha = 1, beta = 1), RetNet (alpha = gamma,
                        beta = 1), Mamba2 (beta = 1); with LQ_GATE_KDA: GLA /
                        RWKV6 / HGRN2 (beta = 1).  DeltaNet is LQ_GATE_GDN with
                        alpha = 1 and the flag clear.                          */
  LQ_DENSE_COMP = 4u /* compensator tokens with dense keys (below)             */
};

/* Dense compensator tokens (LQ_DENSE_COMP).  The compensators are r tokens
 * (k_c, w_c) with dense fp32 keys k_c (comp_key) and values w_c (comp_val):
 * the boundary state is B = deQ + sum_c k_c w_c^T, and a compensator enters
 * the window like a buffered record written before the window's first token
 * (decay Gamma, weight k_c . (Gamma * y), update w_c): it is updated
 * exactly like a real token ([EL] Abstract; in Figure 4 the compensators
 * hold the state's largest components).  The window
 * close joins them to the fp32 rebuild as r more records of the same MFMA
 * contraction (K = len + r).  The split finds the keys by comp_iters rounds
 * of subspace iteration on S S^T started from the one-hot keys of the r
 * largest-norm rows: K <- MGS(S S^T K), modified Gram-Schmidt in compensator
 * order, a key whose projected norm is zero or at most 2e-2 of its norm
 * before projection becoming the zero key.  Then w_c = S^T k_c and the
 * residual S - sum_c k_c w_c^T is smoothed and quantized as usual; comp_idx
 * receives the starting rows.  With comp_iters = 0 the keys are the one-hot
 * rows and every result equals the row extraction's.  Without the flag,
 * comp_key is neither read nor written and comp_iters is ignored. */

typedef struct lq_params {
  int32_t n;      /* number of independent states in the slab (>= 1)     */
  int32_t dk;     /* key dimension, rows of S; must be 128                */
  int32_t dv;     /* value dimension, columns of S; must be 128           */
  int32_t p;      /* window length in tokens, 1..64                       */
  int32_t r;      /* compensator rows per state, 0..16                    */
  int32_t gate;   /* lq_gate                                              */
  uint32_t flags; /* LQ_NO_SMOOTH | LQ_NO_DELTA | LQ_DENSE_COMP, or 0      */
  int32_t comp_iters; /* LQ_DENSE_COMP: subspace iterations, 0..8         */
} lq_params;

/* One slab of n states.  codes .. comp_val and comp_key are the boundary
 * state (the prefix-cache snapshot); buf_gate, buf_k and buf_u are the
 * window buffer.  For r == 0, comp_idx, comp_val and comp_key may be NULL;
 * comp_key may be NULL without LQ_DENSE_COMP.  The arrays a call uses must
 * not overlap one another, since a launch that writes some of them reads the
 * others: the calls that write the state return LQ_ERR_ALIAS otherwise. */
typedef struct lq_state {
  int8_t *codes;     /* [n][dk*dv]  int8 residual codes c_ij (layout above) */
  float *row_scale;  /* [n][dk]     a_i                                     */
  float *col_scale;  /* [n][dv]     s_j                                     */
  int32_t *comp_idx; /* [n][r]      row index of each compensator row       */
  float *comp_val;   /* [n][r][dv]  compensator rows w_c                    */
  float *buf_gate;   /* GDN: [n][p]; KDA: [n][p][dk]   d_i (alpha_i)        */
  float *buf_k;      /* [n][p][dk]  k~_i = beta_i k_i                       */
  float *buf_u;      /* [n][p][dv]  u_i                                     */
  float *comp_key;   /* [n][r][dk]  LQ_DENSE_COMP: compensator keys k_c     */
} lq_state;

/* Split fp32 states S [n][dk][dv] into the boundary state of `st` (codes,
 * row_scale, col_scale, comp_idx, comp_val); the window buffer is neither
 * read nor written.  This is the window-boundary split of [EL] Figure 4
 * applied to a state that has no buffered updates, i.e. the quantized
 * boundary state that precedes the first window of [EL] Figure 2.  S must
 * not overlap the boundary-state arrays. */
int leapquant_quantize_state(const lq_params *prm, const float *S,
                             const lq_state *st, hipStream_t stream);

/* Decode token t (0-based position inside the current window, 0 <= t < p)
 * for all n states ([EL] Figure 2, per-window quantization; [EL] Abstract,
 * compensators are updated like real tokens).  Reads the boundary
 * state and the records 0..t-1 of the buffer, writes
 *   o[n][dv] = S_t^T q_t, with S_t the exact recurrence from the boundary
 *              state through the buffered records and this token,
 * and appends record t: buf_gate[.][t] = alpha_t, buf_k[.][t] = beta_t k_t,
 * buf_u[.][t] = v_t - S_{t-1}^T b_t.
 * Inputs: q, k [n][dk]; v [n][dv]; beta [n]; alpha [n] (GDN) or [n][dk]
 * (KDA); all read-only.  o must not overlap any input or state array.
 * The caller closes the window (leapquant_window_close with len = p)
 * after t = p - 1 and before the next t = 0. */
int leapquant_decode_step(const lq_params *prm, const lq_state *st, int32_t t,
                          const float *q, const float *k, const float *v,
                          const float *beta, const float *alpha, float *o,
                          hipStream_t stream);

/* Close a window of len buffered records (1 <= len <= p; len < p only for
 * a final partial window): rebuild S_len = D_len..D_1 B + sum_i
 * (D_len..D_{i+1}) k~_i u_i^T in fp32, then split it into compensator rows,
 * smoothing scales, row scales and int8 codes, overwriting the boundary
 * state in place ([EL] Figure 2: quantize once per window; [EL] Figure 4).
 * The buffer is read, not cleared. */
int leapquant_window_close(const lq_params *prm, const lq_state *st,
                           int32_t len, hipStream_t stream);

/* Decode token t and close the window in one pass (the fused form of
 * leapquant_decode_step(t) followed by leapquant_window_close(len = t + 1);
 * [EL] Figure 2: the state is quantized once per window, at its last
 * token).  Reads the boundary state and the records 0..t-1, rebuilds
 * D_t S_{t-1} in fp32, writes o[n][dv] = S_t^T q_t with
 *   u_t = v_t - S_{t-1}^T b_t,  S_t = D_t S_{t-1} + k~_t u_t^T,
 * then splits S_t into the new boundary state, overwriting it in place.
 * Record t is not written to the buffer (the window is closed).  Arguments,
 * layouts, alignment and aliasing rules are those of leapquant_decode_step;
 * t is normally p - 1 (t < p - 1 closes a final partial window).  Results
 * agree with the two-call form to fp32 rounding, not bit for bit: the
 * fused form reads S_{t-1} from the rebuilt state instead of the windowed
 * sums. */
int leapquant_decode_close(const lq_params *prm, const lq_state *st, int32_t t,
                           const float *q, const float *k, const float *v,
                           const float *beta, const float *alpha, float *o,
                           hipStream_t stream);

/* Write the boundary state B = deQ(codes, a, s) + compensator rows as fp32
 * S_out [n][dk][dv]: the quantized residual plus the compensators that
 * [EL] Figure 4 splits the state into, i.e. the state the next window
 * starts from ([EL] Figure 2); used for state error tracking (the MSE of
 * [EL] Figure 3) and prefix-cache reads.  Row-major, 16-byte aligned;
 * S_out must not overlap `st` (LQ_ERR_ALIAS); other errors as for
 * leapquant_quantize_state. */
int leapquant_dequantize_state(const lq_params *prm, const lq_state *st,
                               float *S_out, hipStream_t stream);

/* ---- Continuous batching.  The slots of a slab hold sequences at
 * different positions of their own windows (requests join and finish
 * independently).  pos[n] and len[n] are int32 arrays in DEVICE memory,
 * read by the kernels (4-byte aligned, read-only, overlapping no state
 * array or output); the host keeps them up to date, typically with one
 * small device operation per token.
 *
 * leapquant_decode_step_slots: slot s decodes its token at window position
 * pos[s] exactly as leapquant_decode_step would with t = pos[s]; a slot with
 * pos[s] outside [0, p) is idle (its o row and state are left as they are).
 * leapquant_decode_close_slots: the same for the fused last-token decode
 * and close of leapquant_decode_close (slot s closes with pos[s] + 1
 * records); idle slots as above.
 * leapquant_window_close_slots: slot s is closed with len[s] records when
 * 1 <= len[s] <= p (len[s] < p closes a partial window at the end of a
 * sequence); other slots are left as they are.
 * The other arguments and the error codes are those of the uniform calls;
 * values in pos and len cannot be checked on the host. */
int leapquant_decode_step_slots(const lq_params *prm, const lq_state *st, const int32_t *pos,
                                const float *q, const float *k, const float *v,
                                const float *beta, const float *alpha, float *o,
                                hipStream_t stream);
int leapquant_decode_close_slots(const lq_params *prm, const lq_state *st, const int32_t *pos,
                                 const float *q, const float *k, const float *v,
                                 const float *beta, const float *alpha, float *o,
                                 hipStream_t stream);
int leapquant_window_close_slots(const lq_params *prm, const lq_state *st, const int32_t *len,
                                 hipStream_t stream);

/* Compacted closes.  At a given token only the slots whose windows end
 * close, about one slot in p; the _slots calls above still start one
 * workgroup per slot, and the idle ones cost launch time.  These calls take
 * list[count], int32 slot ids in DEVICE memory (4-byte aligned, read-only,
 * overlapping no state array, output or the per-slot array), and start
 * one workgroup per entry: listed slot s is processed exactly as the
 * matching _slots call processes it with pos[s] / len[s] (a listed slot
 * whose pos or len is out of range is idle); ids outside [0, n) are
 * skipped; unlisted slots are not touched.  0 <= count <= n (LQ_ERR_SHAPE
 * otherwise); count == 0 launches nothing and returns LQ_OK.  A slot listed
 * twice is closed twice concurrently, which races: the caller lists each
 * slot at most once (device values cannot be checked on the host).  The
 * other arguments and error codes are those of the _slots calls. */
int leapquant_decode_close_list(const lq_params *prm, const lq_state *st, const int32_t *pos,
                                const int32_t *list, int32_t count, const float *q,
                                const float *k, const float *v, const float *beta,
                                const float *alpha, float *o, hipStream_t stream);
int leapquant_window_close_list(const lq_params *prm, const lq_state *st, const int32_t *len,
                                const int32_t *list, int32_t count, hipStream_t stream);

/* One continuous-batching token in one launch ([EL] Figure 2: each slot
 * decodes against its fixed boundary state and closes its own window after
 * its p-th token).  Slot s with 0 <= pos[s] < p - 1 decodes its token
 * exactly as leapquant_decode_step_slots does; listed slot s with
 * pos[s] == p - 1 decodes its token and closes its window exactly as
 * leapquant_decode_close_list does.  Slots at position p - 1 that are not
 * listed, listed slots at any other position, ids outside [0, n) and slots
 * outside [0, p) are left as they are.  The result equals
 * leapquant_decode_step_slots over the positions with p - 1 replaced by -1
 * followed by leapquant_decode_close_list over the listed slots at p - 1,
 * bit for bit.  For slabs of more than 4,096 slots with 4 <= p <= 16 and
 * at most 8 compensator rows (no dense compensator tokens) it is a single
 * launch: the closing slots' workgroups run among the decode steps, which
 * keep memory busy around them, so the closes no longer cost a launch of
 * their own; other shapes run the two launches.  Arguments, list rules
 * and error codes are those of leapquant_decode_close_list. */
int leapquant_decode_step_close_list(const lq_params *prm, const lq_state *st, const int32_t *pos,
                                     const int32_t *list, int32_t count, const float *q,
                                     const float *k, const float *v, const float *beta,
                                     const float *alpha, float *o, hipStream_t stream);

/* ---- Uncompressed baselines ([EL] Table 2, rows "FP32 per-step" and
 * "BF16 per-step"): the same token update on a dense state that is read
 * and written in full every token.  Provided to measure the quantized path
 * against in the same harness; not part of the quantized decode. */
typedef enum lq_dense_dtype {
  LQ_DENSE_FP32 = 0, /* S is float [n][dk][dv]                            */
  LQ_DENSE_BF16 = 1  /* S is bfloat16 (uint16 bit patterns) [n][dk][dv];
                        computed in fp32, stored rounded to nearest even   */
} lq_dense_dtype;

/* One token for n dense states, in place: u_t = v_t - S^T b_t,
 * S <- D_t S + k~_t u_t^T, o[n][dv] = S^T q_t (the recurrence of [EL]
 * Table 4 with no quantization).  prm supplies n, dk, dv and gate (p, r
 * and flags must be valid but are not used).  S is row-major (row = key
 * channel), 16-byte aligned (fp32) or 8-byte aligned (bf16); the token
 * inputs follow leapquant_decode_step.  S and o must not overlap each other
 * or any input. */
int leapquant_dense_step(const lq_params *prm, void *S, int32_t dtype,
                         const float *q, const float *k, const float *v,
                         const float *beta, const float *alpha, float *o,
                         hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *leapquant_status_string(int status);

/* ---- "BF16 + per-window" ([EL] Table 2, the row between BF16 per-step and
 * INT8 per-step): the boundary state is a dense bf16 state B [n][dk][dv]
 * (row-major, bfloat16 bit patterns), fixed for the window.  Within the
 * window the tokens are buffered in the fp32 records of `st` exactly as in
 * the int8 path (only buf_gate, buf_k and buf_u of `st` are used; r,
 * LQ_NO_SMOOTH and LQ_DENSE_COMP do not apply: flags may hold only
 * LQ_NO_DELTA).  The decode step reads B and the records.  The window close
 * rebuilds S = Gamma * B + K_w U in fp32 (rows scaled by the decay product
 * Gamma of the window) and writes it back into B rounded to bf16, nearest
 * with ties to even.  There is no fused last-token close for this row. */

/* Decode token t (0 <= t < p) of the window for all n states: reads B and
 * records 0 .. t-1, writes o and record t.  Errors as for
 * leapquant_decode_step; B must be 16-byte aligned and overlap neither the
 * buffer nor o. */
int leapquant_bf16w_decode_step(const lq_params *prm, const void *B, const lq_state *st, int32_t t,
                                const float *q, const float *k, const float *v, const float *beta,
                                const float *alpha, float *o, hipStream_t stream);

/* Close the window after len tokens (1 <= len <= p): B <- bf16(Gamma * B +
 * K_w U).  The buffer is read, not written. */
int leapquant_bf16w_window_close(const lq_params *prm, void *B, const lq_state *st, int32_t len,
                                 hipStream_t stream);

/* ---- Measurement reference, no part of the method: a plain stream in
 * the decode step's launch shape.  One 64-lane wave per block of
 * read_bytes_per_wave bytes at src reads its block with 16-byte nontemporal
 * loads, 16 KiB per wave issued at a time, then sleeps idle_sleeps times
 * 512 cycles with nothing in flight (a stand-in for the work a decode wave
 * does after its loads return), then writes write_bytes_per_wave bytes at
 * dst + wave * write_bytes_per_wave (8 bytes per lane per 512-byte row, as
 * the decode step stores its output rows).  Timed beside the decode step
 * with idle_sleeps = 0, it gives the rate the device reaches for the same
 * bytes per wave, read/write mix and waves per launch with no arithmetic
 * between.  Also
 * writes waves * 64 checksum words to out (each the sum over the lane's
 * 16-byte loads of the XOR of their four 32-bit words).
 * read_bytes_per_wave a positive multiple of 1024, write_bytes_per_wave a
 * multiple of 512 (0 allowed, then dst may be NULL), both at most 2^30;
 * 0 <= idle_sleeps <= 4096; waves >= 1 (LQ_ERR_SHAPE otherwise); src and
 * dst 16-byte aligned, out
 * 4-byte aligned (LQ_ERR_ALIGN); dst and out must not overlap each other
 * or the bytes read (LQ_ERR_ALIAS). */
int leapquant_stream_reference(const void *src, int64_t read_bytes_per_wave, void *dst,
                               int64_t write_bytes_per_wave, int32_t idle_sleeps, int32_t waves,
                               uint32_t *out, hipStream_t stream);

/* LEAPQUANT_ABI_VERSION of the loaded library. */
int leapquant_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LEAPQUANT_H */
