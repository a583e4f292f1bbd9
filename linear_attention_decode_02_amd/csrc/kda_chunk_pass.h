// Internal interface between the C ABI (kda_decode.hip) and the two-pass
// chunked prefill (kda_chunk_pass.hip).  Not part of the public headers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda_gate_args.h"

struct KdaPassArgs {
  const uint16_t* qkv;           // bf16 [tokens, 3C]
  const float* conv_w;           // fp32 [3, 4, C]
  uint16_t* conv_state;          // bf16 [slots, 3C, 3] (or [slots, 3, 3C])
  float* rec_state;              // fp32 [slots, H, 128, 128]
  const float* g;                // fp32 [tokens, H, 128]
  const float* beta;             // fp32 [tokens, H]
  const uint16_t* gate;          // bf16 [tokens, C] (output norm only)
  const float* norm_w;           // fp32 [128] (output norm only)
  const int32_t* state_idx;      // int32 [N]
  const int32_t* cu_seqlens;     // int32 [N + 1]
  const int32_t* chunk_indices;  // int32 [chunks, 2]: (sequence, chunk)
  const int64_t* chunk_offsets;  // int64 [N + 1]: first chunk of each
  float* workspace;              // max_chunks * H records
  uint16_t* out;                 // bf16 [tokens, C]
  KdaRawGateArgs rg;             // raw gates (rg.raw_g null: g and beta)
  int64_t max_chunks;            // chunk rows the workspace holds
  int32_t num_seqs;
  uint32_t flags;
  int32_t heads;
  int32_t num_slots;
  float eps;
};

// Bytes of one (chunk, head) record.
uint64_t kda_pass_record_bytes();

// Device address of the library's static record array on device `dev`
// (KDA_STATIC_SCRATCH_BYTES bytes), looked up once per device with that
// device current; null if the lookup failed.
void* kda_pass_static_scratch(int dev);

// Queues both passes on `stream`.
hipError_t kda_chunk_pass_launch(const KdaPassArgs& args, hipStream_t stream);
