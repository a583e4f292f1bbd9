// Internal interface between the C ABI (kda_decode.hip) and the chunked
// prefill kernel (kda_chunked.hip).  Not part of the public headers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda_gate_args.h"

struct KdaChunkedArgs {
  const uint16_t* qkv;        // bf16 [tokens, 3C]
  const float* conv_w;        // fp32 [3, 4, C]
  uint16_t* conv_state;       // bf16 [slots, 3C, 3] (or [slots, 3, 3C])
  float* rec_state;           // fp32 [slots, H, 128, 128]
  const float* g;             // fp32 [tokens, H, 128]
  const float* beta;          // fp32 [tokens, H]
  const uint16_t* gate;       // bf16 [tokens, C] (output norm only)
  const float* norm_w;        // fp32 [128] (output norm only)
  const int32_t* state_idx;   // int32 [N]
  const int32_t* cu_seqlens;  // int32 [N + 1], or null: tokens_per_row
  int32_t tokens_per_row;     // with cu_seqlens null: row n owns tokens
                              // n*T .. n*T + T-1
  uint16_t* out;              // bf16 [tokens, C]
  KdaRawGateArgs rg;          // raw gates (rg.raw_g null: g and beta)
  uint32_t flags;
  int32_t heads;
  int32_t num_slots;
  float eps;
};

// Queues the chunked prefill of `num_seqs` sequences (cu_seqlens) or rows
// (tokens_per_row) on `stream`: one workgroup per (sequence, head).
hipError_t kda_chunked_prefill_launch(const KdaChunkedArgs& args,
                                      int32_t num_seqs, hipStream_t stream);

// Rows of tokens_per_row tokens (cu_seqlens null, rg.raw_g null) through
// the short-row kernel: one workgroup per (row, head), the row's tokens in
// chunks of 8 with the state held in registers between them, several
// workgroups per compute unit.
hipError_t kda_short_rows_launch(const KdaChunkedArgs& args, int32_t num_rows,
                                 hipStream_t stream);
