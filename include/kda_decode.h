/*
 * kda_decode.h -- C ABI of the fused single-token KDA decode step on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the one described on the page "PR #50654 完整报告 --
 * [ROCm][Perf] Kimi-K3 Fused kernel for KDA decode" (prhub.com.cn report of
 * vLLM PR #50654):
 *   - section "Feature and motivation": for every sequence and every value
 *     head of a decode batch, advance the causal conv1d state, run the gated
 *     delta-rule recurrence, apply a gated RMSNorm -- in one launch instead
 *     of three;
 *   - section "Implementation breakdown", item 1: a [128, 128] fp32
 *     recurrent state per head, read and written once per token; output norm
 *     on or off; the fixed head counts; rows of the null padding slot 0
 *     produce zeros and skip the state;
 *   - section "Implementation breakdown", item 3 and the kda_decode.py
 *     excerpt in "Key source excerpts": head counts 12/24/48/96, head dim
 *     128, conv width 4, bf16 input and conv state, a width-major fp32 conv
 *     weight [3, width, channels] and an fp32 norm weight;
 *   - the kda.py excerpt in "Key source excerpts": the argument list of the
 *     fused op (input, conv weight, conv state, gate terms, state indices,
 *     recurrent state, output, output gate, norm weight, norm eps).
 *
 * Per row n (one token) and head h, with D = 128, C = H*D, W = 4:
 *   conv (each channel c of the head's q, k and v parts):
 *       a = sum_{t<W} conv_w[p][t][h*D+i] * window[t],
 *       window = (conv_state[s][c][0..W-2], qkv[n][c]), oldest first;
 *       x = a * sigmoid(a);  conv_state[s][c] <- window[1..W-1] (bit copy)
 *   recurrence on S = rec_state[s][h] (S[i][j]: i key, j value):
 *       Sd[i][j] = exp(g[n][h][i]) * S[i][j]
 *       delta[j] = beta[n][h] * (v[j] - sum_i k[i] Sd[i][j])
 *       S'[i][j] = Sd[i][j] + k[i] * delta[j]    (written back to slot s)
 *       o[j]     = sum_i q[i] S'[i][j]
 *   output (KDA_OUTPUT_NORM set):
 *       y[j] = o[j] / sqrt(mean_j o^2 + norm_eps) * norm_w[j]
 *              * sigmoid(gate[n][h*D+j])
 *     (flag clear: y = o);  out[n][h*D+j] = bf16_rne(y[j]).
 *   A row whose slot s = state_idx[n] is <= 0 (null padding slot) or
 *   >= num_slots writes +0.0 to its output and reads or writes no state.
 *
 * kda_decode takes g and beta already activated (log-decay <= 0, beta in
 * (0, 1)) and no conv bias; kda_decode_raw_gates takes the raw gate inputs
 * and the bias of the page's op.  By default q and k are used as produced
 * by the conv (no normalisation, no scale); the flags below select the
 * variants.
 */
#ifndef KDA_DECODE_H
#define KDA_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1, /* null/negative sizes, null pointer, bad eps/flags */
  KDA_ERR_UNSUPPORTED = 2, /* head count not in {12,24,48,96}, D != 128, W != 4 */
  KDA_ERR_MISALIGNED = 3,  /* a buffer pointer not 16-byte aligned           */
  KDA_ERR_DEVICE = 4,      /* no HIP device, or the current one is not gfx950 */
  KDA_ERR_LAUNCH = 5,      /* the kernel launch reported an error            */
  KDA_ERR_TOO_LARGE = 6    /* request exceeds the library's static scratch  */
} kda_status;

/* flags (kda_dims.flags).  The page's kernel has template switches for
 * the output norm, for updating the conv state and for a "safe" gate
 * ("Implementation breakdown", item 1); the others guard readings of the
 * page that it leaves open. */
#define KDA_OUTPUT_NORM 0x01u    /* apply the gated RMSNorm epilogue         */
#define KDA_NO_CONV_UPDATE 0x02u /* read the conv state, do not write it     */
#define KDA_CONV_TAP_MAJOR 0x04u /* conv_state stored [num_slots, W-1, 3C]:
                                    the page's physical layout, of which the
                                    default [num_slots, 3C, W-1] is the
                                    transposed view (kda.py excerpt)        */
#define KDA_QK_L2NORM 0x08u      /* after the conv: q <- q / sqrt(|q|^2 +
                                    1e-6) * D^-1/2, k <- k / sqrt(|k|^2 +
                                    1e-6) (not on the page)                  */
#define KDA_GATE_SILU 0x10u      /* output gate activation x*sigmoid(x)
                                    instead of sigmoid(x)                    */
#define KDA_BOUNDED_GATE 0x20u   /* raw-gate entry points only: bounded gate */

typedef struct kda_dims {
  int32_t batch;      /* B >= 0 rows, one decode token each                 */
  int32_t num_heads;  /* H in {12, 24, 48, 96} value heads on this device  */
  int32_t head_dim;   /* D = 128 (key dim = value dim)                     */
  int32_t conv_width; /* W = 4                                             */
  int32_t num_slots;  /* state pool size >= 1; slot 0 is the null slot     */
  uint32_t flags;     /* KDA_* flags above                                 */
  float norm_eps;     /* > 0 and finite when KDA_OUTPUT_NORM is set        */
} kda_dims;

/*
 * One fused decode step over B rows and H heads, queued on `hip_stream`
 * (a hipStream_t; NULL = the null stream).  Every pointer is a device
 * pointer to a contiguous row-major buffer, 16-byte aligned:
 *
 *   qkv        in      bf16 [B, 3C]           q | k | v parts, head-major
 *   conv_w     in      fp32 [3, W, C]         tap W-1 multiplies the token
 *   conv_state in/out  bf16 [num_slots, 3C, W-1]   oldest tap first
 *                      ([num_slots, W-1, 3C] with KDA_CONV_TAP_MAJOR)
 *   rec_state  in/out  fp32 [num_slots, H, D, D]   [slot][head][key][value]
 *   g          in      fp32 [B, H, D]         log-decay per key channel
 *   beta       in      fp32 [B, H]
 *   gate       in      bf16 [B, C]            not read when the norm is off
 *   norm_w     in      fp32 [D]               not read when the norm is off
 *   state_idx  in      int32 [B]              slot per row
 *   out        out     bf16 [B, C]            every element written
 *
 * Ownership: the caller owns every buffer; the library allocates nothing,
 * keeps no per-call state and does not synchronise, so the call can be
 * captured into a HIP graph.  conv_state and rec_state change only in the
 * slots named by non-null rows; all other bytes, slot 0 included, are left
 * untouched.  Non-null slots must be distinct within one call (two rows on
 * one slot race; the result is then unspecified).  `out` must not overlap
 * an input.  The state_idx values are read on the device only.
 *
 * Errors: checked on the host before anything is queued, in this order:
 * INVALID_ARG (dims, eps, unknown flags -- KDA_BOUNDED_GATE is unknown
 * here), UNSUPPORTED, (B = 0 returns KDA_OK with nothing queued),
 * INVALID_ARG / MISALIGNED for null or misaligned pointers, DEVICE; LAUNCH
 * if the launch itself fails.  A non-OK status means nothing was queued
 * (except LAUNCH).  Thread-safe.
 */
kda_status kda_decode(const kda_dims* dims, const void* qkv,
                      const float* conv_w, void* conv_state, float* rec_state,
                      const float* g, const float* beta, const void* gate,
                      const float* norm_w, const int32_t* state_idx, void* out,
                      void* hip_stream);

/*
 * The page's op with its raw gate inputs and conv bias (kda.py excerpt in
 * "Key source excerpts": raw_g, raw_beta, A_log, dt_bias, lower_bound,
 * bias).  The page does not give the gate formula; this entry point reads
 * the names plainly (softplus with a linear branch above 20):
 *   z = raw_g[n][h][i] + dt_bias[h*D+i],  a = exp(A_log[h])
 *   g = -a * softplus(z)                       (default)
 *   g = lower_bound * sigmoid(a * z)           (KDA_BOUNDED_GATE; g in
 *                                               (lower_bound, 0))
 *   beta = sigmoid(raw_beta[n][h])
 *   conv: a_c = conv_bias[c] + sum_t conv_w[..] * window[t]
 * then the same step as kda_decode.  Extra buffers (device, 16-byte aligned):
 *   conv_bias  in  fp32 [3C]     may be NULL (no bias)
 *   raw_g      in  bf16 [B, H, D]
 *   raw_beta   in  bf16 [B, H]
 *   A_log      in  fp32 [H]
 *   dt_bias    in  fp32 [C]
 * lower_bound must be finite and < 0 when KDA_BOUNDED_GATE is set (else
 * KDA_ERR_INVALID_ARG); it is ignored otherwise.  Other rules, checks and
 * status codes as kda_decode.
 */
kda_status kda_decode_raw_gates(const kda_dims* dims, const void* qkv,
                                const float* conv_w, const float* conv_bias,
                                void* conv_state, float* rec_state,
                                const void* raw_g, const void* raw_beta,
                                const float* A_log, const float* dt_bias,
                                float lower_bound, const void* gate,
                                const float* norm_w, const int32_t* state_idx,
                                void* out, void* hip_stream);

/*
 * Multi-token decode: `tokens` (T, 1..1024) successive tokens per row in
 * one call, equal to T successive kda_decode calls on the same slots (the
 * page's fused op covers one token per sequence and excludes speculative
 * decoding -- the gate's num_spec == 0 -- so this extends it).  The state
 * tile is read once and written once per (row, head); the conv window
 * advances once per token.  Token-major buffers:
 *   qkv   bf16 [B, T, 3C];  g fp32 [B, T, H, D];  beta fp32 [B, T, H];
 *   gate  bf16 [B, T, C];   out bf16 [B, T, C]
 * Other buffers, flags (KDA_BOUNDED_GATE excluded), rules and status codes
 * as kda_decode; T outside 1..1024 is KDA_ERR_INVALID_ARG.  With
 * KDA_NO_CONV_UPDATE every token sees the stored conv window, as T
 * successive calls with that flag would.  From T = 5 on, the call runs
 * the chunk form of kda_prefill_chunked (the rows' tokens in chunks of 8,
 * one workgroup per row and head, up to 16 tokens per row or up to 64 with
 * at least 4 rows x heads per compute unit; else the chunked prefill
 * kernel itself, each row one sequence of T tokens): equal up to rounding,
 * and faster there.  The contract on g does not change with T: any g <= 0
 * down to -inf is accepted by every form (-inf forgets the key row, as
 * exp(-inf) = 0).
 */
kda_status kda_decode_tokens(const kda_dims* dims, int32_t tokens,
                             const void* qkv, const float* conv_w,
                             void* conv_state, float* rec_state, const float* g,
                             const float* beta, const void* gate,
                             const float* norm_w, const int32_t* state_idx,
                             void* out, void* hip_stream);

/*
 * Variable-length prefill: dims->batch = N sequences; sequence n covers
 * tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 (device int32 [N+1],
 * non-decreasing; a decreasing pair counts as empty) of token-major
 * buffers qkv bf16 [tokens, 3C], g fp32 [tokens, H, D], beta fp32
 * [tokens, H], gate bf16 [tokens, C], out bf16 [tokens, C], and slot
 * state_idx[n].  The result is the single-token step applied to each
 * sequence's tokens in order, from the state held in its slot (the state
 * tile stays on chip across the sequence).  Empty sequences and rows of the
 * null slot leave every state untouched (null rows write +0.0 outputs).
 * The prefill is the workload of the page "PR #51862 完整报告 -- Remove
 * prefill pipeline stall in chunk KDA" (chunked there; its chunk
 * algorithm is not on the page).  Flags as kda_decode_tokens; status codes
 * as kda_decode (cu_seqlens NULL: INVALID_ARG).
 */
kda_status kda_prefill(const kda_dims* dims, const int32_t* cu_seqlens,
                       const void* qkv, const float* conv_w, void* conv_state,
                       float* rec_state, const float* g, const float* beta,
                       const void* gate, const float* norm_w,
                       const int32_t* state_idx, void* out, void* hip_stream);

/*
 * The same prefill computed in chunks of 16 tokens on the matrix cores
 * (the fp32 products as three bf16 pieces per operand, accumulated in
 * fp32): per chunk the deltas solve a 16 x 16 unit lower-triangular
 * system (I + diag(beta) A) Delta = diag(beta) (V - K~ S), with A the
 * decayed key Gram matrix of the chunk, K~ the keys scaled by their
 * cumulative decay and S the state before the chunk; outputs and the next
 * state follow from Delta by matrix products.  In exact arithmetic this is
 * the token-by-token recurrence; in fp32 it differs only by rounding.  One
 * workgroup per (sequence, head) carries the state across the sequence's
 * chunks.  Chunks whose cumulative decay exceeds 80 in magnitude in any
 * channel take an exact per-entry path; a token's decay below -200 log2
 * units (e^g = 0 in fp32), -inf included, is taken as -200 log2 units,
 * which leaves every decay factor of the chunk exactly as it would be
 * (zero) for g <= 0.  Arguments, flags, rules and status codes as
 * kda_prefill.
 */
kda_status kda_prefill_chunked(const kda_dims* dims, const int32_t* cu_seqlens,
                               const void* qkv, const float* conv_w,
                               void* conv_state, float* rec_state,
                               const float* g, const float* beta,
                               const void* gate, const float* norm_w,
                               const int32_t* state_idx, void* out,
                               void* hip_stream);

/*
 * The same prefill in two passes over the device-side chunk table (the
 * structure of the page "PR #51862 完整报告 -- Remove prefill pipeline
 * stall in chunk KDA": chunk kernels driven by chunk_indices/chunk_offsets
 * built on the device).  Pass 1 computes, for every (chunk, head) of every
 * sequence in parallel, everything that does not depend on the state (conv,
 * q/k normalisation, decay tables, the A / B products and the 16 x 16
 * inverse) into `workspace`; pass 2 carries each (sequence, head) state
 * through its chunks.  Same result as kda_prefill_chunked up to rounding.
 *   chunk_indices  device int32 [total, 2], chunk_offsets device int64
 *                  [N + 1]: from kda_chunk_metadata(cu_seqlens, N, 16, ...)
 *                  (chunk size 16).
 *   max_chunks     >= the total chunk count (kda_chunk_count on a host copy
 *                  of cu_seqlens, or a bound such as tokens/16 + N); sizes
 *                  the first pass's grid.
 *   workspace      device, 16-byte aligned, caller-owned, at least
 *                  kda_prefill_chunks_workspace_bytes(dims, max_chunks).
 * A chunk table that does not match cu_seqlens, or holds more than
 * max_chunks chunks, cannot be detected without a synchronisation: the
 * kernels then skip what lies outside the workspace (outputs of those
 * sequences are left as they were) and never access memory out of range.
 * Other arguments, flags and status codes as kda_prefill; a workspace too
 * small or max_chunks < 0 is KDA_ERR_INVALID_ARG.
 */
uint64_t kda_prefill_chunks_workspace_bytes(const kda_dims* dims,
                                            int64_t max_chunks);
kda_status kda_prefill_chunks(const kda_dims* dims, const int32_t* cu_seqlens,
                              const int32_t* chunk_indices,
                              const int64_t* chunk_offsets, int64_t max_chunks,
                              const void* qkv, const float* conv_w,
                              void* conv_state, float* rec_state,
                              const float* g, const float* beta,
                              const void* gate, const float* norm_w,
                              const int32_t* state_idx, void* out,
                              void* workspace, uint64_t workspace_bytes,
                              void* hip_stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc:
 * kda_prefill_chunks with its per-(chunk, head) records kept in a scratch
 * array inside the library instead of a caller workspace.  The array is a
 * file-scope device array of KDA_STATIC_SCRATCH_BYTES bytes, one per GPU,
 * created when the library is loaded on that GPU and held until the process
 * ends; the call allocates nothing and frees nothing.
 *   max_chunks * H * kda_prefill_chunks_workspace_bytes(dims, 1) must be
 *   at most KDA_STATIC_SCRATCH_BYTES (else KDA_ERR_TOO_LARGE, nothing
 *   queued): e.g. 123 chunks of 16 tokens at 48 heads, 495 at 12.
 * Every call on one GPU uses that GPU's array, which keeps the last call's
 * records (the kernels read only what the same call wrote): calls that
 * overlap on one GPU -- on two streams, from two threads, or a graph
 * replay beside an eager call -- race on it and give undefined results.
 * Arguments other than the workspace, flags, rules and status codes as
 * kda_prefill_chunks; KDA_ERR_DEVICE also if the array cannot be located
 * on the current device.
 */
#define KDA_STATIC_SCRATCH_BYTES (256ull << 20)
kda_status kda_prefill_chunks_static(
    const kda_dims* dims, const int32_t* cu_seqlens,
    const int32_t* chunk_indices, const int64_t* chunk_offsets,
    int64_t max_chunks, const void* qkv, const float* conv_w, void* conv_state,
    float* rec_state, const float* g, const float* beta, const void* gate,
    const float* norm_w, const int32_t* state_idx, void* out,
    void* hip_stream);

/*
 * Raw gate inputs of a prefill call, token-major (the chunk op of the page
 * "PR #51862 完整报告" is chunk_kda_with_fused_gate: the gate activation
 * runs inside the chunk kernels).  Per token n (a row of the varlen batch)
 * and head h the gates are those of kda_decode_raw_gates:
 *   z = raw_g[n][h][i] + dt_bias[h*D+i],  a = exp(A_log[h])
 *   g = -a * softplus(z), or lower_bound * sigmoid(a * z) with
 *       KDA_BOUNDED_GATE
 *   beta = sigmoid(raw_beta[n][h]); conv: a_c = conv_bias[c] + sum_t ...
 * All device pointers, 16-byte aligned; the struct itself is host memory,
 * read during the call only.
 */
typedef struct {
  const float* conv_bias; /* fp32 [3C], or NULL for no bias                */
  const void* raw_g;      /* bf16 [tokens, H, D]                            */
  const void* raw_beta;   /* bf16 [tokens, H]                               */
  const float* A_log;     /* fp32 [H]                                       */
  const float* dt_bias;   /* fp32 [C]                                       */
  float lower_bound;      /* KDA_BOUNDED_GATE: finite and < 0               */
} kda_gate_inputs;

/*
 * kda_prefill_chunked and kda_prefill_chunks with the gate activation fused
 * (raw gates in place of g and beta).  Flags as kda_prefill plus
 * KDA_BOUNDED_GATE.  gates NULL, or any of raw_g, raw_beta, A_log, dt_bias
 * NULL, or a bad lower_bound with KDA_BOUNDED_GATE: KDA_ERR_INVALID_ARG;
 * misaligned: KDA_ERR_MISALIGNED.  Other arguments, rules and status codes
 * as the entry points they extend.
 */
kda_status kda_prefill_chunked_raw_gates(const kda_dims* dims,
                                         const int32_t* cu_seqlens,
                                         const void* qkv, const float* conv_w,
                                         void* conv_state, float* rec_state,
                                         const kda_gate_inputs* gates,
                                         const void* gate, const float* norm_w,
                                         const int32_t* state_idx, void* out,
                                         void* hip_stream);
kda_status kda_prefill_chunks_raw_gates(
    const kda_dims* dims, const int32_t* cu_seqlens,
    const int32_t* chunk_indices, const int64_t* chunk_offsets,
    int64_t max_chunks, const void* qkv, const float* conv_w, void* conv_state,
    float* rec_state, const kda_gate_inputs* gates, const void* gate,
    const float* norm_w, const int32_t* state_idx, void* out, void* workspace,
    uint64_t workspace_bytes, void* hip_stream);

/*
 * Device-side chunk bookkeeping of a variable-length batch (page "PR
 * #51862 完整报告", implementation item 2 and the kda_metadata.py excerpt):
 * sequence i of cu_seqlens (device int32 [num_seqs + 1]) gets
 * nt_i = ceil(len_i / chunk_size) chunks (a negative length counts as
 * empty); chunk_offsets (int64 [num_seqs + 1]) receives the first chunk row
 * of every sequence and the total; chunk_indices (int32 [total, 2])
 * receives (i, c) for c < nt_i in sequence order.  No host synchronisation:
 * size chunk_indices with kda_chunk_count on a host copy of cu_seqlens.
 * Errors: num_seqs < 0, chunk_size < 1 or a null pointer: INVALID_ARG;
 * MISALIGNED (16 bytes), DEVICE, LAUNCH as kda_decode.
 */
kda_status kda_chunk_metadata(const int32_t* cu_seqlens, int32_t num_seqs,
                              int32_t chunk_size, int32_t* chunk_indices,
                              int64_t* chunk_offsets, void* hip_stream);

/* Host helper: total chunk count of a host cu_seqlens (-1 on bad input). */
int64_t kda_chunk_count(const int32_t* cu_seqlens_host, int32_t num_seqs,
                        int32_t chunk_size);

/* Static, NUL-terminated description of a status code. */
const char* kda_status_string(kda_status status);

/* Algorithmic HBM bytes one kda_decode call moves, for bandwidth reports:
 * per non-null (row, head) 2*D*D*4 state bytes, 2*3*D*(W-1)*2 conv-state
 * bytes (read only with KDA_NO_CONV_UPDATE: half), 3*D*2 input, D*4 + 4
 * gate-term bytes, plus the D*2 output (and D*2 gate when the norm is on);
 * per null (row, head) the D*2 output; plus state_idx, conv_w and norm_w
 * once.  `live_rows` = rows with a valid slot.  Returns 0 for invalid dims. */
uint64_t kda_decode_bytes(const kda_dims* dims, int32_t live_rows);

/* The same for kda_decode_raw_gates: gate terms are D*2 + 2 bytes per
 * (row, head), plus A_log and dt_bias once, plus conv_bias once when
 * has_conv_bias is nonzero. */
uint64_t kda_decode_raw_gates_bytes(const kda_dims* dims, int32_t live_rows,
                                    int32_t has_conv_bias);

/* The same for kda_decode_tokens: state and conv-state bytes once per
 * (row, head), inputs and outputs once per token. */
uint64_t kda_decode_tokens_bytes(const kda_dims* dims, int32_t tokens,
                                 int32_t live_rows);

#ifdef __cplusplus
}
#endif

#endif /* KDA_DECODE_H */
