// Fused single-token KDA decode step for gfx950 (MI355X), and its C ABI.
//
// Operation: the decode step of the page "PR #50654 完整报告 -- [ROCm][Perf]
// Kimi-K3 Fused kernel for KDA decode" (vLLM PR #50654 report): conv1d state
// advance, gated delta-rule recurrence on a [128, 128] fp32 state, gated
// RMSNorm, per (sequence, value head), in one launch (sections "Feature and
// motivation" and "Implementation breakdown", item 1).  The equations and the
// buffer layouts are stated in include/kda_decode.h.
//
// Design (gfx950, wave64).  The step moves 128 KiB of recurrent state per
// (row, head) -- the page names that traffic as the bottleneck -- against
// about 120 kflop, i.e. ~0.9 flop/byte, twenty times below the fp32 ridge:
// this is HBM-streaming work, so there is no MFMA here.  One 1024-thread
// workgroup (16 waves) owns one (row, head) unit, and at most 64 VGPRs per
// lane let two such workgroups share a CU (measured on MI355X: 16 waves with
// two workgroups per CU beat 4 or 8 waves per workgroup, and beat three or
// four resident workgroups; spreading consecutive units over the XCDs, the
// hardware's round-robin, beats giving each XCD a contiguous range):
//   * thread t holds a 4-row x 4-column slice of the state in VGPRs:
//     columns 4*(t%32) .. +3, key rows (t/32) + 32*m, m = 0..3.  Each load
//     instruction of a wave covers two adjacent 512-byte rows (1 KiB
//     contiguous, dwordx4, nontemporal -- worth ~15% over cached loads and
//     stores); the whole 64 KiB tile is in flight at once, issued right after
//     the small conv/gate loads so the conv math runs under the state
//     latency.
//   * conv (waves 0-2, one q/k/v part each, two channels per lane) and the
//     decay factors exp(g) (wave 3) go to LDS as {alpha, k, q} per key row.
//   * column sums u = Sd^T k and p = Sd^T q (and the scalar q.k) are formed
//     in registers, folded across the two half-waves with one lane swap,
//     then across waves through LDS: 256 threads each finish one column
//     (delta_j = beta (v_j - u_j), or p_j) and broadcast it.  The readout
//     uses o = Sd^T q + (q.k) delta, which equals S'^T q exactly in real
//     arithmetic, so the updated state is never re-read.
//   * the RMSNorm sum of squares needs no further barrier: the first
//     half-wave holds all 128 columns.
//   * rows of the null slot (or an out-of-range slot) take a block-uniform
//     early exit before any barrier and only write zeros.
//   * HBM traffic per launch, from calibrated FETCH_SIZE / WRITE_SIZE
//     counters, equals the algorithmic bytes to within 0.1%.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <cstdint>
#include <mutex>

#include "kda_decode.h"

namespace {

constexpr int kD = 128;          // head dim (key = value)
constexpr int kW = 4;            // conv width
constexpr int kWaves = 16;                                // per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerThread = kD * kD / (kThreads * 4);  // float4 per thread
constexpr int kRowStride = kThreads / 32;                 // key rows apart
static_assert(kWaves >= 4 && kD * kD % (kThreads * 4) == 0, "tile shape");

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

struct Params {
  const uint16_t* qkv;
  const float* conv_w;
  uint16_t* conv_state;
  float* rec_state;
  const float* g;
  const float* beta;
  const uint16_t* gate;
  const float* norm_w;
  const int32_t* state_idx;
  uint16_t* out;
  // raw gate inputs (kda_decode_raw_gates) and the optional conv bias
  const float* conv_bias;   // [3C] or null
  const uint16_t* raw_g;    // bf16 [B, H, D]
  const uint16_t* raw_beta; // bf16 [B, H]
  const float* A_log;       // [H]
  const float* dt_bias;     // [C]
  float lower_bound;
  uint32_t flags;
  int32_t heads;
  int32_t num_slots;
  float eps;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const unsigned short a = __builtin_bit_cast(unsigned short, (__bf16)lo);
  const unsigned short b = __builtin_bit_cast(unsigned short, (__bf16)hi);
  return static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float sigmoidf_(float x) {
  return 1.0f / (1.0f + __expf(-x));
}

// softplus with the usual linear branch above 20
__device__ __forceinline__ float softplusf_(float z) {
  return z > 20.0f ? z : log1pf(__expf(z));
}

// kNorm: gated RMSNorm epilogue; kRawGates: g and beta from raw inputs.
// Other variants (conv-state layout and update, q/k L2 norm, SiLU gate,
// bounded gate, conv bias) are block-uniform runtime flags.
template <bool kNorm, bool kRawGates>
// At most 64 VGPRs, so that two 16-wave workgroups share a CU.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8)))
void kda_decode_kernel(Params p) {
  __shared__ f4 s_akq[kD];          // {exp(g_i), k_i, q_i, 0} per key row i
  __shared__ float s_v[kD];
  __shared__ float s_red[kWaves][2][kD];  // per-wave partial u, p columns
  __shared__ float s_qk[kWaves];
  __shared__ float s_delta[kD];
  __shared__ float s_p[kD];
  __shared__ float s_qk_total;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int unit = blockIdx.x;
  const int H = p.heads;
  const int n = unit / H;
  const int h = unit - n * H;
  const int64_t C = static_cast<int64_t>(H) * kD;

  const int32_t slot = p.state_idx[n];
  if (slot <= 0 || slot >= p.num_slots) {
    // Null padding row: zero output, no state traffic.  Block-uniform.
    if (tid < kD / 8) {
      uint4* o = reinterpret_cast<uint4*>(p.out + n * C + h * kD);
      o[tid] = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }

  // ---- small loads first (they retire before the state loads) ----------
  // Waves 0..2 run the conv of part `wave` (q, k, v) on channels i0, i0+1;
  // wave 3 computes exp(g) for key rows i0, i0+1.  The loads are issued by
  // every wave without branching (waves 3+ re-read part 2's conv inputs, an
  // L2 hit) so that no wave has to drain them before its state loads.
  const uint32_t flags = p.flags;
  const bool tap_major = (flags & KDA_CONV_TAP_MAJOR) != 0;
  const int i0 = 2 * lane;
  const int part = wave < 3 ? wave : 2;
  const int64_t c = part * C + h * kD + i0;
  const uint32_t x2 = *reinterpret_cast<const uint32_t*>(p.qkv + n * 3 * C + c);
  // Conv state words of channels c, c+1.  [slot][channel][tap]: three
  // consecutive words hold (c t0, c t1 | c t2, c+1 t0 | c+1 t1, c+1 t2);
  // [slot][tap][channel]: word t holds (c tap t, c+1 tap t), 3C apart.
  uint32_t* cs_base = reinterpret_cast<uint32_t*>(
      p.conv_state + static_cast<int64_t>(slot) * 3 * C * (kW - 1) +
      (tap_major ? c : c * (kW - 1)));
  const int64_t cs_step = tap_major ? (3 * C) / 2 : 1;  // in words
  const uint32_t cw0 = cs_base[0];
  const uint32_t cw1 = cs_base[cs_step];
  const uint32_t cw2 = cs_base[2 * cs_step];
  f2 w_t[kW];
#pragma unroll
  for (int t = 0; t < kW; ++t)
    w_t[t] = *reinterpret_cast<const f2*>(p.conv_w + (part * kW + t) * C +
                                          h * kD + i0);
  const f2 bias2 = *reinterpret_cast<const f2*>(
      (p.conv_bias ? p.conv_bias : p.conv_w) + c);
  f2 g2;
  float beta;
  if (kRawGates) {
    const uint32_t rg = *reinterpret_cast<const uint32_t*>(
        p.raw_g + (static_cast<int64_t>(n) * H + h) * kD + i0);
    const f2 db = *reinterpret_cast<const f2*>(p.dt_bias + h * kD + i0);
    const float a_rate = __expf(p.A_log[h]);
    const float z0 = bf16_lo(rg) + db.x, z1 = bf16_hi(rg) + db.y;
    if (flags & KDA_BOUNDED_GATE) {
      g2.x = p.lower_bound * sigmoidf_(a_rate * z0);
      g2.y = p.lower_bound * sigmoidf_(a_rate * z1);
    } else {
      g2.x = -(a_rate * softplusf_(z0));
      g2.y = -(a_rate * softplusf_(z1));
    }
    const uint32_t rb = p.raw_beta[static_cast<int64_t>(n) * H + h];
    beta = sigmoidf_(bf16_lo(rb));
  } else {
    g2 = *reinterpret_cast<const f2*>(
        p.g + (static_cast<int64_t>(n) * H + h) * kD + i0);
    beta = p.beta[static_cast<int64_t>(n) * H + h];
  }

  // ---- issue the whole state tile ----------------------------------------
  // Keep the small loads above ahead of the 16 state loads: the conv math
  // then waits only for them (vmcnt retires in issue order).
  __builtin_amdgcn_sched_barrier(0);
  const int col4 = tid & 31;
  const int rgrp = tid >> 5;
  f4* st = reinterpret_cast<f4*>(
      p.rec_state + (static_cast<int64_t>(slot) * H + h) * (kD * kD));
  f4 s[kRowsPerThread];
#pragma unroll
  for (int m = 0; m < kRowsPerThread; ++m)
    s[m] = __builtin_nontemporal_load(st + (rgrp + kRowStride * m) * (kD / 4) +
                                      col4);
  __builtin_amdgcn_sched_barrier(0);

  // ---- conv update + SiLU, decay factors ---------------------------------
  // Computed by every wave without branching on the wave (loads used
  // unconditionally stay where they are issued); only the stores depend on
  // the wave.  Window of channel c: (c0, c1, c2, token lo); of c+1:
  // (d0, d1, d2, token hi), oldest first.
  float c0, c1, c2, d0, d1, d2;
  if (tap_major) {
    c0 = bf16_lo(cw0); c1 = bf16_lo(cw1); c2 = bf16_lo(cw2);
    d0 = bf16_hi(cw0); d1 = bf16_hi(cw1); d2 = bf16_hi(cw2);
  } else {
    c0 = bf16_lo(cw0); c1 = bf16_hi(cw0); c2 = bf16_lo(cw1);
    d0 = bf16_hi(cw1); d1 = bf16_lo(cw2); d2 = bf16_hi(cw2);
  }
  const bool has_bias = p.conv_bias != nullptr;
  float a0 = has_bias ? bias2.x : 0.0f;
  a0 += w_t[0].x * c0;
  a0 += w_t[1].x * c1;
  a0 += w_t[2].x * c2;
  a0 += w_t[3].x * bf16_lo(x2);
  float a1 = has_bias ? bias2.y : 0.0f;
  a1 += w_t[0].y * d0;
  a1 += w_t[1].y * d1;
  a1 += w_t[2].y * d2;
  a1 += w_t[3].y * bf16_hi(x2);
  float y0 = wave < 3 ? a0 * sigmoidf_(a0) : __expf(g2.x);
  float y1 = wave < 3 ? a1 * sigmoidf_(a1) : __expf(g2.y);
  if ((flags & KDA_QK_L2NORM) && wave < 2) {
    // wave 0 holds all of q, wave 1 all of k: x / sqrt(sum x^2 + 1e-6),
    // q also scaled by D^-1/2
    float ss = y0 * y0 + y1 * y1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float r = rsqrtf(ss + 1e-6f) * (wave == 0 ? 0.08838834764831845f
                                                     : 1.0f);
    y0 *= r;
    y1 *= r;
  }
  if (wave < 3 && !(flags & KDA_NO_CONV_UPDATE)) {
    // shifted windows, exact bit copies
    if (tap_major) {
      cs_base[0] = cw1;
      cs_base[cs_step] = cw2;
      cs_base[2 * cs_step] = x2;
    } else {
      // (cw0.hi, cw1.lo, x.lo) and (cw2.lo, cw2.hi, x.hi)
      cs_base[0] = (cw0 >> 16) | (cw1 << 16);
      cs_base[1] = (x2 & 0xffffu) | (cw2 << 16);
      cs_base[2] = (cw2 >> 16) | (x2 & 0xffff0000u);
    }
  }
  if (wave == 2) {
    *reinterpret_cast<f2*>(&s_v[i0]) = f2{y0, y1};
  } else if (wave < 4) {
    // q -> .z, k -> .y, exp(g) -> .x
    const int comp = wave == 0 ? 2 : (wave == 1 ? 1 : 0);
    float* base = reinterpret_cast<float*>(s_akq);
    base[i0 * 4 + comp] = y0;
    base[(i0 + 1) * 4 + comp] = y1;
  }
  __syncthreads();

  // ---- decay and column sums ---------------------------------------------
  f4 u = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
  float qk = 0.f;
#pragma unroll
  for (int m = 0; m < kRowsPerThread; ++m) {
    const f4 akq = s_akq[rgrp + kRowStride * m];
    const f4 sd = s[m] * akq.x;
    s[m] = sd;
    u += akq.y * sd;
    pq += akq.z * sd;
    qk += akq.y * akq.z;
  }
  // fold the two half-waves (key rows rgrp and rgrp+1 of this wave)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    u[e] += __shfl_xor(u[e], 32);
    pq[e] += __shfl_xor(pq[e], 32);
  }
  qk += __shfl_xor(qk, 32);
  if (lane < 32) {
    *reinterpret_cast<f4*>(&s_red[wave][0][4 * col4]) = u;
    *reinterpret_cast<f4*>(&s_red[wave][1][4 * col4]) = pq;
  }
  if (lane == 0) s_qk[wave] = qk;
  __syncthreads();
  // Reduce, then broadcast: threads 0..255 each finish one column of u
  // (delta_j = beta (v_j - u_j)) or of p, instead of every thread summing
  // all partials of its four columns.
  if (tid < 2 * kD) {
    const int which = tid / kD;
    const int j = tid % kD;
    float acc = s_red[0][which][j];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) acc += s_red[w][which][j];
    if (which == 0)
      s_delta[j] = beta * (s_v[j] - acc);
    else
      s_p[j] = acc;
    if (tid == 0) {
      float t = s_qk[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) t += s_qk[w];
      s_qk_total = t;
    }
  }
  __syncthreads();

  // ---- delta rule update, streamed back ------------------------------------
  const f4 delta = *reinterpret_cast<const f4*>(&s_delta[4 * col4]);
#pragma unroll
  for (int m = 0; m < kRowsPerThread; ++m) {
    const float ki = s_akq[rgrp + kRowStride * m].y;
    __builtin_nontemporal_store(s[m] + ki * delta,
                                st + (rgrp + kRowStride * m) * (kD / 4) + col4);
  }

  // ---- readout and gated RMSNorm (wave 0, lanes 0..31 own the output) -----
  if (tid >= 32) return;
  const f4 o = *reinterpret_cast<const f4*>(&s_p[4 * col4]) + s_qk_total * delta;
  f4 y = o;
  if (kNorm) {
    float ss = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 32);
    const float r = rsqrtf(ss * (1.0f / kD) + p.eps);
    const f4 w = *reinterpret_cast<const f4*>(p.norm_w + 4 * col4);
    const uint2 gb = *reinterpret_cast<const uint2*>(
        p.gate + static_cast<int64_t>(n) * C + h * kD + 4 * col4);
    f4 gv = {bf16_lo(gb.x), bf16_hi(gb.x), bf16_lo(gb.y), bf16_hi(gb.y)};
    f4 ga = {sigmoidf_(gv.x), sigmoidf_(gv.y), sigmoidf_(gv.z), sigmoidf_(gv.w)};
    if (flags & KDA_GATE_SILU) ga *= gv;
    y = o * r * w * ga;
  }
  uint2 ob;
  ob.x = pack_bf16x2(y.x, y.y);
  ob.y = pack_bf16x2(y.z, y.w);
  *reinterpret_cast<uint2*>(p.out + static_cast<int64_t>(n) * C + h * kD +
                            4 * col4) = ob;
}

// ---- host side -----------------------------------------------------------

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
bool g_dev_ok[kMaxDevices];

bool device_is_gfx950(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return false;
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t prop;
    g_dev_ok[dev] = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                    std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  });
  return g_dev_ok[dev];
}

bool aligned16(const void* ptr) {
  return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0;
}

bool supported_heads(int h) { return h == 12 || h == 24 || h == 48 || h == 96; }

constexpr uint32_t kPlainFlags = KDA_OUTPUT_NORM | KDA_NO_CONV_UPDATE |
                                 KDA_CONV_TAP_MAJOR | KDA_QK_L2NORM |
                                 KDA_GATE_SILU;

kda_status check_dims(const kda_dims* d, uint32_t allowed_flags) {
  if (!d) return KDA_ERR_INVALID_ARG;
  if (d->batch < 0 || d->num_heads < 1 || d->head_dim < 1 ||
      d->conv_width < 2 || d->num_slots < 1 || (d->flags & ~allowed_flags))
    return KDA_ERR_INVALID_ARG;
  if ((d->flags & KDA_OUTPUT_NORM) &&
      !(std::isfinite(d->norm_eps) && d->norm_eps > 0.0f))
    return KDA_ERR_INVALID_ARG;
  if (!supported_heads(d->num_heads) || d->head_dim != kD ||
      d->conv_width != kW)
    return KDA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(d->batch) * d->num_heads > INT32_MAX)
    return KDA_ERR_INVALID_ARG;
  return KDA_OK;
}

// Pointer checks shared by both entry points (after the dims checks).
kda_status check_common(const kda_dims* d, const void* qkv, const void* conv_w,
                        const void* conv_state, const void* rec_state,
                        const void* gate, const void* norm_w,
                        const void* state_idx, const void* out) {
  const bool norm = (d->flags & KDA_OUTPUT_NORM) != 0;
  if (!qkv || !conv_w || !conv_state || !rec_state || !state_idx || !out ||
      (norm && (!gate || !norm_w)))
    return KDA_ERR_INVALID_ARG;
  if (!aligned16(qkv) || !aligned16(conv_w) || !aligned16(conv_state) ||
      !aligned16(rec_state) || !aligned16(state_idx) || !aligned16(out) ||
      (norm && (!aligned16(gate) || !aligned16(norm_w))))
    return KDA_ERR_MISALIGNED;
  return KDA_OK;
}

Params base_params(const kda_dims* d, const void* qkv, const float* conv_w,
                   void* conv_state, float* rec_state, const void* gate,
                   const float* norm_w, const int32_t* state_idx, void* out) {
  Params p{};
  p.qkv = static_cast<const uint16_t*>(qkv);
  p.conv_w = conv_w;
  p.conv_state = static_cast<uint16_t*>(conv_state);
  p.rec_state = rec_state;
  p.gate = static_cast<const uint16_t*>(gate);
  p.norm_w = norm_w;
  p.state_idx = state_idx;
  p.out = static_cast<uint16_t*>(out);
  p.flags = d->flags;
  p.heads = d->num_heads;
  p.num_slots = d->num_slots;
  p.eps = d->norm_eps;
  return p;
}

template <bool kRaw>
kda_status launch(const kda_dims* d, const Params& p, void* hip_stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev))
    return KDA_ERR_DEVICE;
  const dim3 grid(static_cast<unsigned>(d->batch * d->num_heads));
  const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (d->flags & KDA_OUTPUT_NORM)
    hipLaunchKernelGGL((kda_decode_kernel<true, kRaw>), grid, dim3(kThreads),
                       0, stream, p);
  else
    hipLaunchKernelGGL((kda_decode_kernel<false, kRaw>), grid, dim3(kThreads),
                       0, stream, p);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

uint64_t bytes_model(const kda_dims* d, int32_t live_rows, bool raw_gates,
                     bool conv_bias) {
  if (!d || d->batch < 0 || d->num_heads < 1 || d->head_dim < 1 ||
      d->conv_width < 2 || live_rows < 0 || live_rows > d->batch)
    return 0;
  const uint64_t H = d->num_heads, D = d->head_dim, W = d->conv_width;
  const bool norm = (d->flags & KDA_OUTPUT_NORM) != 0;
  const bool conv_write = (d->flags & KDA_NO_CONV_UPDATE) == 0;
  const uint64_t conv_state = 3 * D * (W - 1) * 2;
  const uint64_t gates = raw_gates ? D * 2 + 2 : D * 4 + 4;
  const uint64_t per_unit = 2 * D * D * 4 + conv_state * (conv_write ? 2 : 1) +
                            3 * D * 2 + gates + D * 2 + (norm ? D * 2 : 0);
  const uint64_t live = static_cast<uint64_t>(live_rows) * H;
  const uint64_t null_units =
      static_cast<uint64_t>(d->batch - live_rows) * H;
  return live * per_unit + null_units * D * 2 +
         static_cast<uint64_t>(d->batch) * 4 + 3 * W * H * D * 4 +
         (norm ? D * 4 : 0) + (raw_gates ? H * 4 + H * D * 4 : 0) +
         (conv_bias ? 3 * H * D * 4 : 0);
}

}  // namespace

extern "C" {

kda_status kda_decode(const kda_dims* d, const void* qkv, const float* conv_w,
                      void* conv_state, float* rec_state, const float* g,
                      const float* beta, const void* gate, const float* norm_w,
                      const int32_t* state_idx, void* out, void* hip_stream) {
  kda_status st = check_dims(d, kPlainFlags);
  if (st != KDA_OK) return st;
  if (d->batch == 0) return KDA_OK;
  st = check_common(d, qkv, conv_w, conv_state, rec_state, gate, norm_w,
                    state_idx, out);
  if (st != KDA_OK) return st;
  if (!g || !beta) return KDA_ERR_INVALID_ARG;
  if (!aligned16(g) || !aligned16(beta)) return KDA_ERR_MISALIGNED;
  Params p = base_params(d, qkv, conv_w, conv_state, rec_state, gate, norm_w,
                         state_idx, out);
  p.g = g;
  p.beta = beta;
  return launch<false>(d, p, hip_stream);
}

kda_status kda_decode_raw_gates(const kda_dims* d, const void* qkv,
                                const float* conv_w, const float* conv_bias,
                                void* conv_state, float* rec_state,
                                const void* raw_g, const void* raw_beta,
                                const float* A_log, const float* dt_bias,
                                float lower_bound, const void* gate,
                                const float* norm_w, const int32_t* state_idx,
                                void* out, void* hip_stream) {
  kda_status st = check_dims(d, kPlainFlags | KDA_BOUNDED_GATE);
  if (st != KDA_OK) return st;
  if ((d->flags & KDA_BOUNDED_GATE) &&
      !(std::isfinite(lower_bound) && lower_bound < 0.0f))
    return KDA_ERR_INVALID_ARG;
  if (d->batch == 0) return KDA_OK;
  st = check_common(d, qkv, conv_w, conv_state, rec_state, gate, norm_w,
                    state_idx, out);
  if (st != KDA_OK) return st;
  if (!raw_g || !raw_beta || !A_log || !dt_bias) return KDA_ERR_INVALID_ARG;
  if (!aligned16(raw_g) || !aligned16(raw_beta) || !aligned16(A_log) ||
      !aligned16(dt_bias) || (conv_bias && !aligned16(conv_bias)))
    return KDA_ERR_MISALIGNED;
  Params p = base_params(d, qkv, conv_w, conv_state, rec_state, gate, norm_w,
                         state_idx, out);
  p.conv_bias = conv_bias;
  p.raw_g = static_cast<const uint16_t*>(raw_g);
  p.raw_beta = static_cast<const uint16_t*>(raw_beta);
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.lower_bound = lower_bound;
  return launch<true>(d, p, hip_stream);
}

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported shape (H in {12,24,48,96}, D=128, W=4)";
    case KDA_ERR_MISALIGNED: return "buffer not 16-byte aligned";
    case KDA_ERR_DEVICE: return "no gfx950 HIP device current";
    case KDA_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

uint64_t kda_decode_bytes(const kda_dims* d, int32_t live_rows) {
  return bytes_model(d, live_rows, false, false);
}

uint64_t kda_decode_raw_gates_bytes(const kda_dims* d, int32_t live_rows,
                                    int32_t has_conv_bias) {
  return bytes_model(d, live_rows, true, has_conv_bias != 0);
}

}  // extern "C"
