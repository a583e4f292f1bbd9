// Raw gate operands of the chunked prefill kernels (internal).  With raw_g
// null the kernels read the activated g and beta instead.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

struct KdaRawGateArgs {
  const float* conv_bias;    // fp32 [3C] or null
  const uint16_t* raw_g;     // bf16 [tokens, H, 128], or null
  const uint16_t* raw_beta;  // bf16 [tokens, H]
  const float* A_log;        // fp32 [H]
  const float* dt_bias;      // fp32 [C]
  float lower_bound;         // KDA_BOUNDED_GATE
};

// Log decay of one key channel in log2 units from its raw gate input
// z = raw_g + dt_bias, with a = e^{A_log}:
//   default  -a softplus(z) log2(e) = -a log2(1 + 2^{z log2 e})
//            (z log2 e itself above z = 20, where the two agree in fp32)
//   bounded  lb2 sigmoid(a z), lb2 = lower_bound log2(e)
// on the transcendental unit (v_exp_f32 / v_log_f32 are base 2).  The form
// is a template argument: a per-element runtime choice costs the kernels
// their instruction scheduling.
template <bool kBounded>
__device__ __forceinline__ float kda_gate2_from_raw(float z, float a_rate,
                                                    float lb2) {
  constexpr float kLog2e = 1.44269504088896341f;
  const float z2 = z * kLog2e;
  if (kBounded)
    return lb2 * __builtin_amdgcn_rcpf(
                     1.0f + __builtin_amdgcn_exp2f(-(a_rate * z2)));
  const float sp2 =
      z > 20.0f ? z2 : __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(z2));
  return -(a_rate * sp2);
}

// Floor of a per-token log2 decay.  2^x is exactly 0 in fp32 for every
// x <= -200, so clamping there leaves every decay factor of the chunk form
// unchanged for non-positive decays: a factor e^{G_t - G_s} whose span
// holds a clamped token has exponent <= -200 either way.  It keeps the
// cumulative sums finite, so that g = -inf (full forgetting) gives zeros
// instead of -inf - -inf = NaN.  NaN passes through: the IEEE 754-2019
// maximum propagates it (one v_maximum3_f32 per element on gfx950).
typedef float kda_f2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ kda_f2 kda_decay_floor2(kda_f2 g2) {
  return __builtin_elementwise_maximum(g2, kda_f2{-200.0f, -200.0f});
}
