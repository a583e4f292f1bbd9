// State-stream bandwidth probe: the decode kernel's memory access pattern
// without its arithmetic (see include/kda_probe.h).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "kda_probe.h"

namespace {

constexpr int kD = 128;
typedef float f4 __attribute__((ext_vector_type(4)));

// mode 0: read every float4 and write it back times `scale`; mode 1: read
// only; mode 2: write only.
template <int kWaves, int kMode>
__global__ __launch_bounds__(64 * kWaves) void state_stream_kernel(
    float* tiles, float scale) {
  constexpr int kThreads = 64 * kWaves;
  constexpr int kRows = kD * kD / (kThreads * 4);
  constexpr int kStride = kThreads / 32;
  const int tid = threadIdx.x;
  const int col4 = tid & 31;
  const int rgrp = tid >> 5;
  f4* st = reinterpret_cast<f4*>(tiles + static_cast<int64_t>(blockIdx.x) *
                                             (kD * kD));
  if (kMode == 2) {
    const f4 v = {scale, scale, scale, scale};
#pragma unroll
    for (int m = 0; m < kRows; ++m)
      __builtin_nontemporal_store(v, st + (rgrp + kStride * m) * (kD / 4) +
                                         col4);
    return;
  }
  f4 s[kRows];
#pragma unroll
  for (int m = 0; m < kRows; ++m)
    s[m] = __builtin_nontemporal_load(st + (rgrp + kStride * m) * (kD / 4) +
                                      col4);
  if (kMode == 1) {
    f4 acc = s[0];
#pragma unroll
    for (int m = 1; m < kRows; ++m) acc += s[m];
    // keeps the loads: on the rare tile whose sum equals scale, the first
    // float4 is written back unchanged
    if (acc.x + acc.y + acc.z + acc.w == scale)
      st[rgrp * (kD / 4) + col4] = s[0];
    return;
  }
#pragma unroll
  for (int m = 0; m < kRows; ++m)
    __builtin_nontemporal_store(s[m] * scale,
                                st + (rgrp + kStride * m) * (kD / 4) + col4);
}

template <int kWaves>
void launch_probe(int mode, dim3 grid, hipStream_t s, float* tiles,
                  float scale) {
  if (mode == 0)
    hipLaunchKernelGGL((state_stream_kernel<kWaves, 0>), grid,
                       dim3(64 * kWaves), 0, s, tiles, scale);
  else if (mode == 1)
    hipLaunchKernelGGL((state_stream_kernel<kWaves, 1>), grid,
                       dim3(64 * kWaves), 0, s, tiles, scale);
  else
    hipLaunchKernelGGL((state_stream_kernel<kWaves, 2>), grid,
                       dim3(64 * kWaves), 0, s, tiles, scale);
}

bool is_gfx950(int dev) {
  hipDeviceProp_t prop;
  return hipGetDeviceProperties(&prop, dev) == hipSuccess &&
         std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
}

}  // namespace

extern "C" kda_status kda_state_stream_probe(float* tiles, int64_t n_tiles,
                                             int32_t waves, int32_t mode,
                                             float scale, void* hip_stream) {
  if (!tiles || n_tiles < 0 || n_tiles > INT32_MAX ||
      (waves != 4 && waves != 8 && waves != 16) || mode < 0 || mode > 2 ||
      !std::isfinite(scale))
    return KDA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(tiles) & 15u) return KDA_ERR_MISALIGNED;
  if (n_tiles == 0) return KDA_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !is_gfx950(dev))
    return KDA_ERR_DEVICE;
  const dim3 grid(static_cast<unsigned>(n_tiles));
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (waves == 4)
    launch_probe<4>(mode, grid, s, tiles, scale);
  else if (waves == 8)
    launch_probe<8>(mode, grid, s, tiles, scale);
  else
    launch_probe<16>(mode, grid, s, tiles, scale);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}
