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
//     in registers and published
//     per half-wave (32 partial rows) in LDS: 256 threads each finish one
//     column (delta_j = beta (v_j - u_j), or p_j) and broadcast it.  The readout
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
#include <type_traits>

#include "kda_chunk_pass.h"
#include "kda_chunked.h"
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
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

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
  const int32_t* cu_seqlens;  // prefill: token range of each row (or null)
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
// 1 / (1 + e^-x) with the hardware reciprocal (v_rcp_f32, ~1 ulp) instead
// of the IEEE division sequence
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// Global-memory pointers (address space 1).
template <typename T>
using gptr = __attribute__((address_space(1))) T*;

// A wave-uniform global pointer made opaque to the compiler (readfirstlane
// of both halves): it stays in SGPRs and is not merged with per-lane
// offsets into 64-bit VGPR addresses kept live across loops.
template <typename T>
__device__ __forceinline__ gptr<T> uniform_gptr(T* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<gptr<T>>((static_cast<uint64_t>(hi) << 32) | lo);
}

// base + a 32-bit byte offset, viewed as U: the access becomes a scalar
// 64-bit base plus one 32-bit VGPR offset.
template <typename U, typename T>
__device__ __forceinline__ gptr<U> at_bytes(gptr<T> base, uint32_t byte_off) {
  using C = typename std::conditional<std::is_const<T>::value, const char,
                                      char>::type;
  return reinterpret_cast<gptr<U>>(
      reinterpret_cast<__attribute__((address_space(1))) C*>(base) + byte_off);
}

// Cross-lane sums on the VALU (DPP) plus scalar lane reads: no lane-address
// registers (ds_bpermute needs one per pattern, which the compiler keeps
// live across loops) and no LDS round trips.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                         0xF, 0xF, false));
}
// Sum over each row of 16 lanes, in every lane of the row: quad_perm
// [1,0,3,2] and [2,3,0,1] (quads), row_half_mirror (8), row_mirror (16).
__device__ __forceinline__ float sum16(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}
// v of lane l (a wave-uniform value)
__device__ __forceinline__ float lane_value(float v, int l) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// softplus with the usual linear branch above 20 (for z < -17 the result
// rounds to 0 instead of e^z; the decay exp(-a e^z) is then 1 either way)
__device__ __forceinline__ float softplusf_(float z) {
  return z > 20.0f ? z : __logf(1.0f + __expf(z));
}

// The thread's m-th float4 of a [128, 128] fp32 tile: key row rgrp + 32 m,
// columns 4 col4 .. 4 col4 + 3, as a uniform row-block base plus the lane's
// byte offset lane_off = rgrp * 512 + col4 * 16.
__device__ __forceinline__ gptr<f4> tile_at(f4* st, uint32_t lane_off, int m) {
  return at_bytes<f4>(uniform_gptr(st + m * kRowStride * (kD / 4)), lane_off);
}
__device__ __forceinline__ uint32_t tile_lane_off(int rgrp, int col4) {
  return static_cast<uint32_t>(rgrp * (kD * 4) + col4 * 16);
}

// Workgroup-shared buffers of one unit.
struct Lds {
  f4 akq[kD];                // {exp(g_i), k_i, q_i, -} per key row i
  float v[kD];
  // per-half-wave partial sums of u and p; rows padded by 4 floats (a row
  // pair 264 words apart, 8 banks of 32) so the quad of threads finishing
  // one column, which read rows q, q + 4, ..., hit four different banks
  float red[2 * kWaves][2][kD + 4];
  float qk[2 * kWaves];          // per-half-wave partial q.k
  float delta[kD];
  float p[kD];
  float qk_total;
  f4 gate_act[kD / 4];  // output gate after its activation (norm only)
  f4 norm_w[kD / 4];    // norm weight (norm only)
};

// Conv window of channels c, c+1 from the three state words: element t of
// the window of c is c[t], of c+1 is d[t] (oldest first).  [slot][channel]
// [tap]: the words hold (c0, c1 | c2, d0 | d1, d2); [slot][tap][channel]:
// word t holds (c_t, d_t).
__device__ __forceinline__ void unpack_window(bool tap_major, uint32_t w0,
                                              uint32_t w1, uint32_t w2,
                                              float c[3], float d[3]) {
  if (tap_major) {
    c[0] = bf16_lo(w0); c[1] = bf16_lo(w1); c[2] = bf16_lo(w2);
    d[0] = bf16_hi(w0); d[1] = bf16_hi(w1); d[2] = bf16_hi(w2);
  } else {
    c[0] = bf16_lo(w0); c[1] = bf16_hi(w0); c[2] = bf16_lo(w1);
    d[0] = bf16_hi(w1); d[1] = bf16_lo(w2); d[2] = bf16_hi(w2);
  }
}

// The three state words after appending token pair x2 (exact bit moves).
__device__ __forceinline__ void shift_window(bool tap_major, uint32_t& w0,
                                             uint32_t& w1, uint32_t& w2,
                                             uint32_t x2) {
  if (tap_major) {
    w0 = w1;
    w1 = w2;
    w2 = x2;
  } else {
    // (c1, c2, x.lo) and (d1, d2, x.hi)
    const uint32_t n0 = (w0 >> 16) | (w1 << 16);
    const uint32_t n1 = (x2 & 0xffffu) | (w2 << 16);
    const uint32_t n2 = (w2 >> 16) | (x2 & 0xffff0000u);
    w0 = n0;
    w1 = n1;
    w2 = n2;
  }
}

// Per-lane inputs of one token: waves 0..2 produce q, k or v of channels
// i0, i0+1 (4-tap conv + SiLU, then optional L2 normalisation of q and k
// across the wave); wave 3 produces exp(g) of key rows i0, i0+1.  Every
// wave computes without branching on the wave; the caller stores.
__device__ __forceinline__ void token_inputs(
    uint32_t flags, int wave, uint32_t w0, uint32_t w1, uint32_t w2,
    uint32_t x2, const f2 (&w_t)[kW], f2 bias2, bool has_bias, f2 g2,
    float& y0, float& y1) {
  float c[3], d[3];
  unpack_window((flags & KDA_CONV_TAP_MAJOR) != 0, w0, w1, w2, c, d);
  float a0 = has_bias ? bias2.x : 0.0f;
  a0 += w_t[0].x * c[0];
  a0 += w_t[1].x * c[1];
  a0 += w_t[2].x * c[2];
  a0 += w_t[3].x * bf16_lo(x2);
  float a1 = has_bias ? bias2.y : 0.0f;
  a1 += w_t[0].y * d[0];
  a1 += w_t[1].y * d[1];
  a1 += w_t[2].y * d[2];
  a1 += w_t[3].y * bf16_hi(x2);
  y0 = wave < 3 ? a0 * sigmoidf_(a0) : __expf(g2.x);
  y1 = wave < 3 ? a1 * sigmoidf_(a1) : __expf(g2.y);
  if ((flags & KDA_QK_L2NORM) && wave < 2) {
    // wave 0 holds all of q, wave 1 all of k: x / sqrt(sum x^2 + 1e-6),
    // q also scaled by D^-1/2
    const float rows = sum16(y0 * y0 + y1 * y1);
    const float ss = (lane_value(rows, 0) + lane_value(rows, 16)) +
                     (lane_value(rows, 32) + lane_value(rows, 48));
    const float r =
        rsqrtf(ss + 1e-6f) * (wave == 0 ? 0.08838834764831845f : 1.0f);
    y0 *= r;
    y1 *= r;
  }
}

__device__ __forceinline__ void store_token_inputs(Lds& L, int wave, int i0,
                                                   float y0, float y1,
                                                   f4* akq_rows = nullptr) {
  if (wave == 2) {
    *reinterpret_cast<f2*>(&L.v[i0]) = f2{y0, y1};
  } else if (wave < 4) {
    // q -> .z, k -> .y, exp(g) -> .x
    const int comp = wave == 0 ? 2 : (wave == 1 ? 1 : 0);
    float* base = reinterpret_cast<float*>(akq_rows ? akq_rows : L.akq);
    base[i0 * 4 + comp] = y0;
    base[(i0 + 1) * 4 + comp] = y1;
  }
}

// Decay the thread's state rows in place and publish the half-wave's
// partial column sums u = Sd^T k, p = Sd^T q and q.k (each half-wave covers
// all 128 columns for its key rows).  k_rows receives k_i of the rows.
// kLean: at most two rows' LDS reads in flight (fewer live VGPRs).
// akq: the {exp(g), k, q} rows to use (L.akq by default).
template <bool kLean = false>
__device__ __forceinline__ void decay_and_partials(
    Lds& L, f4 (&s)[kRowsPerThread], float (&k_rows)[kRowsPerThread],
    int rgrp, int wave, int lane, int col4, const f4* akq_rows = nullptr) {
  const f4* rows = akq_rows ? akq_rows : L.akq;
  f4 u = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
  float qk = 0.f;
#pragma unroll
  for (int m = 0; m < kRowsPerThread; ++m) {
    const f4 akq = rows[rgrp + kRowStride * m];
    const f4 sd = s[m] * akq.x;
    s[m] = sd;
    u += akq.y * sd;
    pq += akq.z * sd;
    qk += akq.y * akq.z;
    k_rows[m] = akq.y;
    if (kLean && (m & 1)) __builtin_amdgcn_sched_barrier(0);
  }
  const int half = 2 * wave + (lane >> 5);  // == rgrp
  *reinterpret_cast<f4*>(&L.red[half][0][4 * col4]) = u;
  *reinterpret_cast<f4*>(&L.red[half][1][4 * col4]) = pq;
  if ((lane & 31) == 0) L.qk[half] = qk;
}

// Reduce, then broadcast: each column of u (delta_j = beta (v_j - u_j)) and
// of p is finished by a quad of threads, each summing 8 of the 32 half-wave
// partials (partials q, q + 4, ... for quad lane q), folded across the quad
// by DPP; threads 0..3 finish q.k the same way.  All 1024 threads take
// part, so the dependent chain is 8 adds deep instead of 32.
__device__ __forceinline__ void finish_columns(Lds& L, int tid, float beta) {
  static_assert(2 * kWaves == 32 && kThreads == 8 * kD, "quad finish shape");
  const int q = tid & 3;
  const int col = tid >> 2;
  const int which = col / kD;
  const int j = col % kD;
  float a = L.red[q][which][j], b = L.red[q + 4][which][j];
#pragma unroll
  for (int i = 2; i < 8; i += 2) {
    a += L.red[q + 4 * i][which][j];
    b += L.red[q + 4 * i + 4][which][j];
  }
  float acc = a + b;
  acc += dpp_mov<0xB1>(acc);  // quad_perm [1,0,3,2]
  acc += dpp_mov<0x4E>(acc);  // quad_perm [2,3,0,1]
  if (q == 0) {
    if (which == 0)
      L.delta[j] = beta * (L.v[j] - acc);
    else
      L.p[j] = acc;
  }
  if (tid < 4) {
    float ta = L.qk[q], tb = L.qk[q + 4];
#pragma unroll
    for (int i = 2; i < 8; i += 2) {
      ta += L.qk[q + 4 * i];
      tb += L.qk[q + 4 * i + 4];
    }
    float t = ta + tb;
    t += dpp_mov<0xB1>(t);
    t += dpp_mov<0x4E>(t);
    if (tid == 0) L.qk_total = t;
  }
}

// The output gate of columns 4 col4 .. +3 after its activation (sigmoid,
// or SiLU with KDA_GATE_SILU), from its four bf16 values.
__device__ __forceinline__ f4 gate_activation(uint32_t flags, u2 gb) {
  const f4 gv = {bf16_lo(gb.x), bf16_hi(gb.x), bf16_lo(gb.y), bf16_hi(gb.y)};
  f4 ga = {sigmoidf_(gv.x), sigmoidf_(gv.y), sigmoidf_(gv.z), sigmoidf_(gv.w)};
  if (flags & KDA_GATE_SILU) ga *= gv;
  return ga;
}

// Readout o = Sd^T q + (q.k) delta and the gated RMSNorm of one token, by
// lanes 0..31 of wave 0 (four columns each, the activated gate and the norm
// weight already in LDS); writes 4 bf16 at out4.
template <bool kNorm>
__device__ __forceinline__ void emit_output(const Lds& L, float eps, int col4,
                                            f4 delta, gptr<uint16_t> out4) {
  const f4 o = *reinterpret_cast<const f4*>(&L.p[4 * col4]) +
               L.qk_total * delta;
  f4 y = o;
  if (kNorm) {
    const float rows = sum16(o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w);
    const float ss = lane_value(rows, 0) + lane_value(rows, 16);
    const float r = rsqrtf(ss * (1.0f / kD) + eps);
    y = o * r * L.norm_w[col4] * L.gate_act[col4];
  }
  u2 ob;
  ob.x = pack_bf16x2(y.x, y.y);
  ob.y = pack_bf16x2(y.z, y.w);
  *reinterpret_cast<gptr<u2>>(out4) = ob;
}

// Request order of the single-token kernel, chosen by the launcher from the
// units per compute unit (see load_mode):
//   kLoadLean      the small inputs, then the state tile; only the waves
//                  that use a small input load it (calls up to one unit per
//                  compute unit, and large ones up to 32 per compute unit);
//   kLoadTileFirst the state tile, then the small inputs (some compute units
//                  hold two units);
//   kLoadAllWaves  the small inputs, then the tile, every wave loading the
//                  conv and decay inputs (larger calls, where that stream
//                  order keeps HBM busier).
enum LoadMode { kLoadLean = 0, kLoadTileFirst = 1, kLoadAllWaves = 2 };

// kNorm: gated RMSNorm epilogue; kRawGates: g and beta from raw inputs;
// kMode: a LoadMode.  Other variants (conv-state layout and update, q/k L2
// norm, SiLU gate, bounded gate, conv bias) are block-uniform runtime flags.
// state_idx and heads (equal to p.state_idx, p.heads) come first as
// arguments of their own: the library is built to preload the first
// argument dwords into scalar registers, so the slot index, on which every
// state and conv access waits, is requested without first reading the
// argument block from memory.
template <bool kNorm, bool kRawGates, int kMode>
// At most 64 VGPRs, so that two 16-wave workgroups share a CU.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8)))
void kda_decode_kernel(const int32_t* state_idx, int32_t heads, Params p) {
  __shared__ Lds L;
  constexpr bool kTileFirst = kMode == kLoadTileFirst;
  constexpr bool kAllWaves = kMode == kLoadAllWaves;

  const int tid = threadIdx.x;
  // scalar: the branches on the wave below are uniform and cost no masks
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int unit = blockIdx.x;
  const int H = heads;
  // unit / H on the scalar unit: every supported head count (12, 24, 48,
  // 96; others are rejected before launch) is 3 * 2^k, and for any 32-bit
  // x, x / 3 = (x * 0xAAAAAAAB) >> 33
  const uint32_t x3 = static_cast<uint32_t>(unit) >> __builtin_ctz(H);
  const int n = static_cast<int>(__builtin_amdgcn_readfirstlane(
                    static_cast<uint32_t>(
                        (static_cast<uint64_t>(x3) * 0xAAAAAAABull) >> 33)));
  const int h = unit - n * H;
  const int64_t C = static_cast<int64_t>(H) * kD;

  const int32_t slot = state_idx[n];
  if (slot <= 0 || slot >= p.num_slots) {
    // Null padding row: zero output, no state traffic.  Block-uniform.
    if (tid < kD / 8) {
      uint4* o = reinterpret_cast<uint4*>(p.out + n * C + h * kD);
      o[tid] = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }

  const int col4 = tid & 31;
  const int rgrp = tid >> 5;
  f4* st = reinterpret_cast<f4*>(
      p.rec_state + (static_cast<int64_t>(slot) * H + h) * (kD * kD));
  const uint32_t lane_off = tile_lane_off(rgrp, col4);
  f4 s[kRowsPerThread];
  auto issue_tile = [&]() {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < kRowsPerThread; ++m)
      s[m] = __builtin_nontemporal_load(tile_at(st, lane_off, m));
    __builtin_amdgcn_sched_barrier(0);
  };
  if (kTileFirst) issue_tile();

  // ---- small loads (they retire before the state loads unless kTileFirst)
  // Waves 0..2 run the conv of part `wave` (q, k, v) on channels i0, i0+1;
  // wave 3 computes exp(g) for key rows i0, i0+1.  Unless kAllWaves, only
  // those waves issue these loads (wave-uniform branches), so the other
  // waves' state loads queue behind no redundant requests in the compute
  // unit's address path; with kAllWaves waves 3+ re-read part 2's conv
  // inputs (cache hits) and every wave reads its decays.
  const uint32_t flags = p.flags;
  const bool tap_major = (flags & KDA_CONV_TAP_MAJOR) != 0;
  const int i0 = 2 * lane;
  const int64_t cs_step = tap_major ? (3 * C) / 2 : 1;  // in words
  uint32_t* cs_base = nullptr;
  uint32_t x2 = 0u, cw0 = 0u, cw1 = 0u, cw2 = 0u;
  f2 w_t[kW] = {};
  f2 bias2 = {0.f, 0.f};
  if (kAllWaves || wave < 3) {
    const int part = wave < 3 ? wave : 2;
    const int64_t c = part * C + h * kD + i0;
    // conv state words of channels c, c+1 (see unpack_window)
    cs_base = reinterpret_cast<uint32_t*>(
        p.conv_state + static_cast<int64_t>(slot) * 3 * C * (kW - 1) +
        (tap_major ? c : c * (kW - 1)));
    x2 = *reinterpret_cast<const uint32_t*>(p.qkv + n * 3 * C + c);
    cw0 = cs_base[0];
    cw1 = cs_base[cs_step];
    cw2 = cs_base[2 * cs_step];
#pragma unroll
    for (int t = 0; t < kW; ++t)
      w_t[t] = *reinterpret_cast<const f2*>(p.conv_w + (part * kW + t) * C +
                                            h * kD + i0);
    if (p.conv_bias) bias2 = *reinterpret_cast<const f2*>(p.conv_bias + c);
  }
  f2 g2 = {0.f, 0.f};
  float beta;
  if (kRawGates) {
    if (kAllWaves || wave == 3) {
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
    }
    const uint32_t rb = p.raw_beta[static_cast<int64_t>(n) * H + h];
    beta = sigmoidf_(bf16_lo(rb));
  } else {
    if (kAllWaves || wave == 3)
      g2 = *reinterpret_cast<const f2*>(
          p.g + (static_cast<int64_t>(n) * H + h) * kD + i0);
    beta = p.beta[static_cast<int64_t>(n) * H + h];
  }
  // Output gate and norm weight of columns 4 lane .. +3, by lanes 0..31 of
  // wave 4 (idle in the conv): activated and put in LDS before the first
  // barrier, so the readout at the end depends on no memory access.
  const bool gate_lanes = kNorm && wave == 4 && lane < 32;
  u2 gb = {0u, 0u};
  f4 nw = {0.f, 0.f, 0.f, 0.f};
  if (gate_lanes) {
    gb = *reinterpret_cast<const u2*>(p.gate + static_cast<int64_t>(n) * C +
                                      h * kD + 4 * lane);
    nw = *reinterpret_cast<const f4*>(p.norm_w + 4 * lane);
  }

  // ---- the whole state tile, after (or, kTileFirst, before) the small
  // loads: the conv math then waits only for what precedes it (vmcnt
  // retires in issue order)
  if (!kTileFirst) issue_tile();

  // ---- conv update + SiLU, decay factors (waves 0..3) ---------------------
  // In kLoadLean waves 4..15 skip this (16 % of the vector instructions,
  // 0.3 us at one row); in the other modes they run a discarded copy, which
  // measured faster there (288 units, 12 heads: 9.0 against 9.5 us).
  if (kMode != kLoadLean || wave < 4) {
    float y0, y1;
    token_inputs(flags, wave, cw0, cw1, cw2, x2, w_t, bias2,
                 p.conv_bias != nullptr, g2, y0, y1);
    if (wave < 3 && !(flags & KDA_NO_CONV_UPDATE)) {
      shift_window(tap_major, cw0, cw1, cw2, x2);
      cs_base[0] = cw0;
      cs_base[cs_step] = cw1;
      cs_base[2 * cs_step] = cw2;
    }
    store_token_inputs(L, wave, i0, y0, y1);
  }
  if (gate_lanes) {
    L.gate_act[lane] = gate_activation(flags, gb);
    L.norm_w[lane] = nw;
  }
  __syncthreads();

  // ---- decay, column sums, delta --------------------------------------------
  float k_rows[kRowsPerThread];
  decay_and_partials(L, s, k_rows, rgrp, wave, lane, col4);
  __syncthreads();
  finish_columns(L, tid, beta);
  __syncthreads();

  // ---- delta rule update, streamed back ------------------------------------
  const f4 delta = *reinterpret_cast<const f4*>(&L.delta[4 * col4]);
#pragma unroll
  for (int m = 0; m < kRowsPerThread; ++m)
    __builtin_nontemporal_store(s[m] + k_rows[m] * delta,
                                tile_at(st, lane_off, m));

  // ---- readout and gated RMSNorm (wave 0, lanes 0..31 own the output) -----
  if (tid >= 32) return;
  emit_output<kNorm>(L, p.eps, col4, delta,
                     at_bytes<uint16_t>(uniform_gptr(p.out + n * C + h * kD),
                                        8 * col4));
}

// Several tokens per row in one launch, equal to successive single-token
// steps on the same slots: the state tile is read once, kept in VGPRs
// across the tokens and written once, the conv window advances in LDS.
// Token-major buffers (qkv [tokens, 3C], g [tokens, H, D], beta
// [tokens, H], gate and out [tokens, C]); row n covers tokens
// n*T_fixed .. +T_fixed-1, or cu_seqlens[n] .. cu_seqlens[n+1]-1 when
// p.cu_seqlens is set (variable-length prefill).
//
// Two barriers per token, software-pipelined one token deep: waves 4..7
// compute token t+1's inputs (conv + SiLU of q, k, v; exp(g)) while waves
// 0..3 finish token t's column sums, wave 9 its q.k, and wave 8 emits token
// t-1's output (readout + gated RMSNorm), so the token chain holds only
//   decay + partial sums | barrier | column sums (next inputs, previous
//   output) | barrier | rank-1 update.
// Each input wave fetches its next token's small inputs one token ahead.

// finish_columns with the token's v row taken from `v` and delta and p
// written to dp[0] and dp[1] (double-buffered by token parity: the next
// token's are written while this one's are read).  Two interleaved
// accumulators halve the dependent-add chain.
__device__ __forceinline__ void finish_columns_v(const Lds& L, int tid,
                                                 float beta, const float* v,
                                                 float (*dp)[kD]) {
  const int which = tid / kD;
  const int j = tid % kD;
  float a0 = L.red[0][which][j], a1 = L.red[1][which][j];
#pragma unroll
  for (int r = 2; r < 2 * kWaves; r += 2) {
    a0 += L.red[r][which][j];
    a1 += L.red[r + 1][which][j];
  }
  const float acc = a0 + a1;
  dp[which][j] = which == 0 ? beta * (v[j] - acc) : acc;
}

// q.k of one token from the 32 half-wave partials, by one whole wave
// (lanes 0..31 read one partial each; DPP row sums, then two lane reads).
__device__ __forceinline__ void finish_qk(const Lds& L, int lane, float* qk) {
  const float rows = sum16(lane < 2 * kWaves ? L.qk[lane] : 0.0f);
  const float t = lane_value(rows, 0) + lane_value(rows, 16);
  if (lane == 0) *qk = t;
}

// Readout and gated RMSNorm of one finished token from its delta, p and q.k
// rows, by 32 lanes of one wave (four columns each; lanes 32..63 idle).
template <bool kNorm>
__device__ __forceinline__ void emit_token_output(
    const float (*dp)[kD], float qk_total, const float* norm_w,
    uint32_t flags, float eps, int col4, u2 gb, gptr<uint16_t> out4) {
  const f4 delta = *reinterpret_cast<const f4*>(&dp[0][4 * col4]);
  const f4 o = *reinterpret_cast<const f4*>(&dp[1][4 * col4]) +
               qk_total * delta;
  f4 y = o;
  if (kNorm) {
    const float rows = sum16(o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w);
    const float ss = lane_value(rows, 0) + lane_value(rows, 16);
    const float r = rsqrtf(ss * (1.0f / kD) + eps);
    const f4 w = *reinterpret_cast<const f4*>(norm_w + 4 * col4);
    const f4 gv = {bf16_lo(gb.x), bf16_hi(gb.x), bf16_lo(gb.y), bf16_hi(gb.y)};
    f4 ga = {sigmoidf_(gv.x), sigmoidf_(gv.y), sigmoidf_(gv.z),
             sigmoidf_(gv.w)};
    if (flags & KDA_GATE_SILU) ga *= gv;
    y = o * r * w * ga;
  }
  u2 ob;
  ob.x = pack_bf16x2(y.x, y.y);
  ob.y = pack_bf16x2(y.z, y.w);
  *reinterpret_cast<gptr<u2>>(out4) = ob;
}

template <bool kNorm>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8)))
void kda_decode_tokens_kernel(Params p, int T_fixed) {
  __shared__ Lds L;
  __shared__ f2 s_w[3][kW][kD / 2];   // conv taps, per part and lane
  __shared__ float s_norm_w[kD];
  // {exp(g), k, q} rows and v by token parity: token t+1's rows are
  // written while token t's are read
  __shared__ f4 s_akq[2][kD];
  __shared__ float s_v[2][kD];
  // finished delta and p rows and q.k by token parity: token t-1's are
  // read by the output wave while token t's are written
  __shared__ float s_dp[2][2][kD];
  __shared__ float s_qk[2];
  // conv window words of input waves 4..6, kept in LDS across the tokens
  __shared__ uint32_t s_win[3][3][kD / 2];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar
  const int lane = tid & 63;
  const int unit = blockIdx.x;
  const int H = p.heads;
  const int n = unit / H;
  const int h = unit - n * H;
  const int C = H * kD;
  int64_t row_tok;  // first token of the row
  int T;            // tokens of the row
  if (p.cu_seqlens) {
    const int32_t bos = p.cu_seqlens[n], eos = p.cu_seqlens[n + 1];
    row_tok = bos;
    T = eos > bos ? eos - bos : 0;
    if (T == 0) return;  // empty sequence: no output, state untouched
  } else {
    row_tok = static_cast<int64_t>(n) * T_fixed;
    T = T_fixed;
  }

  const int32_t slot = p.state_idx[n];
  if (slot <= 0 || slot >= p.num_slots) {
    for (int i = tid; i < T * (kD / 8); i += kThreads) {
      uint4* o = reinterpret_cast<uint4*>(
          p.out + (row_tok + i / (kD / 8)) * C + h * kD);
      o[i % (kD / 8)] = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }

  const uint32_t flags = p.flags;
  const bool tap_major = (flags & KDA_CONV_TAP_MAJOR) != 0;
  // input waves 4..7: role 0 q, 1 k, 2 v (conv + SiLU), 3 exp(g)
  const bool input_wave = wave >= 4 && wave < 8;
  const int role = wave - 4;
  const int i0 = 2 * lane;
  const int part = input_wave && role < 3 ? role : 2;
  // per-lane 32-bit offsets from per-token uniform bases
  const uint32_t c = part * C + h * kD + i0;         // into a qkv token row
  const uint32_t gi = h * kD + i0;                   // into a g token row
  const uint32_t oc = h * kD + 4 * (tid & 31);       // into gate/out rows
  const uint16_t* qkv_row = p.qkv + row_tok * 3 * C;
  const float* g_row = p.g + row_tok * H * kD;
  const float* beta_row = p.beta + row_tok * H;
  // small inputs of the token an input wave computes next
  uint32_t x2 = 0u;
  f2 g2 = {0.f, 0.f};
  if (input_wave) {
    x2 = *at_bytes<const uint32_t>(uniform_gptr(qkv_row), 2 * c);
    g2 = *at_bytes<const f2>(uniform_gptr(g_row), 4 * gi);
  }
  float beta = beta_row[h];  // of the token waves 0..3 finish next
  // output gate words of lanes 0..31 of the output wave (wave 8, which
  // emits token t-1 while token t's column sums are finished)
  constexpr int kOutWave = 8;
  u2 gate_w = {0u, 0u};
  if (kNorm && wave == kOutWave)
    gate_w = *at_bytes<const u2>(uniform_gptr(p.gate + row_tok * C), 2 * oc);
  uint32_t* cs_slot = reinterpret_cast<uint32_t*>(
      p.conv_state + static_cast<int64_t>(slot) * 3 * C * (kW - 1));
  const uint32_t cs_off = (tap_major ? c : c * (kW - 1)) / 2;  // in words
  const uint32_t cs_step = tap_major ? (3 * C) / 2 : 1;
  const gptr<uint32_t> cs_g = uniform_gptr(cs_slot);
  const bool conv_wave = input_wave && role < 3;
  if (conv_wave) {
    s_win[0][role][lane] = *at_bytes<uint32_t>(cs_g, 4 * cs_off);
    s_win[1][role][lane] = *at_bytes<uint32_t>(cs_g, 4 * (cs_off + cs_step));
    s_win[2][role][lane] =
        *at_bytes<uint32_t>(cs_g, 4 * (cs_off + 2 * cs_step));
    // conv taps to LDS once (read per token: fewer live VGPRs)
#pragma unroll
    for (int t = 0; t < kW; ++t)
      s_w[role][t][lane] = *reinterpret_cast<const f2*>(
          p.conv_w + (role * kW + t) * C + h * kD + i0);
  } else if (wave == 3 && kNorm) {
    *reinterpret_cast<f2*>(&s_norm_w[i0]) =
        *reinterpret_cast<const f2*>(p.norm_w + i0);
  }

  __builtin_amdgcn_sched_barrier(0);
  const int col4 = tid & 31;
  const int rgrp = tid >> 5;
  f4* st = reinterpret_cast<f4*>(
      p.rec_state + (static_cast<int64_t>(slot) * H + h) * (kD * kD));
  const uint32_t lane_off = tile_lane_off(rgrp, col4);
  f4 s[kRowsPerThread];
#pragma unroll
  for (int m = 0; m < kRowsPerThread; ++m)
    s[m] = __builtin_nontemporal_load(tile_at(st, lane_off, m));
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();   // s_w, s_win, s_norm_w visible

  // Input waves: token tt's q/k/v/exp(g) into the buffers of its parity,
  // the conv window advanced in LDS, then the small inputs of token tn
  // fetched for the next call.
  auto inputs = [&](int tt, int tn) {
    int tid_t = tid;
    asm volatile("" : "+v"(tid_t));
    const int lane_t = tid_t & 63;
    const int role_t = (tid_t >> 6) - 4;
    const int part_t = role_t < 3 ? role_t : 2;
    const int i0_t = 2 * lane_t;
    f2 w_t[kW];
#pragma unroll
    for (int tap = 0; tap < kW; ++tap) w_t[tap] = s_w[part_t][tap][lane_t];
    uint32_t cw0 = 0, cw1 = 0, cw2 = 0;
    if (role_t < 3) {
      cw0 = s_win[0][role_t][lane_t];
      cw1 = s_win[1][role_t][lane_t];
      cw2 = s_win[2][role_t][lane_t];
    }
    float y0, y1;
    token_inputs(flags, role_t, cw0, cw1, cw2, x2, w_t, f2{0.f, 0.f}, false,
                 g2, y0, y1);
    // successive calls with the update off all see the stored window
    if (role_t < 3 && !(flags & KDA_NO_CONV_UPDATE)) {
      shift_window(tap_major, cw0, cw1, cw2, x2);
      s_win[0][role_t][lane_t] = cw0;
      s_win[1][role_t][lane_t] = cw1;
      s_win[2][role_t][lane_t] = cw2;
    }
    if (role_t == 2) {
      *reinterpret_cast<f2*>(&s_v[tt & 1][i0_t]) = f2{y0, y1};
    } else {
      // q -> .z, k -> .y, exp(g) -> .x
      const int comp = role_t == 0 ? 2 : (role_t == 1 ? 1 : 0);
      float* base = reinterpret_cast<float*>(s_akq[tt & 1]);
      base[i0_t * 4 + comp] = y0;
      base[(i0_t + 1) * 4 + comp] = y1;
    }
    const uint32_t c_t = part_t * C + h * kD + i0_t;
    const uint32_t gi_t = h * kD + i0_t;
    x2 = *at_bytes<const uint32_t>(
        uniform_gptr(qkv_row + static_cast<int64_t>(tn) * 3 * C), 2 * c_t);
    g2 = *at_bytes<const f2>(
        uniform_gptr(g_row + static_cast<int64_t>(tn) * H * kD), 4 * gi_t);
  };

  if (input_wave) inputs(0, T > 1 ? 1 : 0);
  __syncthreads();   // token 0's inputs

  for (int t = 0; t < T; ++t) {
    // Lane-derived offsets are recomputed every token from an opaque copy
    // of the thread id (a dozen of them kept live across the loop would
    // not fit the 64-VGPR budget); the state rows' key-row group and column
    // block stay live (rgrp, col4: measured ~1 % faster than recomputing).
    int tid_t = tid;
    asm volatile("" : "+v"(tid_t));
    const int wave_t = tid_t >> 6;
    const int lane_t = tid_t & 63;
    const int col4_t = tid_t & 31;
    const uint32_t oc_t = h * kD + 4 * col4_t;

    const f4* akq_t = s_akq[t & 1];
    float k_unused[kRowsPerThread];
    decay_and_partials<true>(L, s, k_unused, rgrp, wave, lane, col4, akq_t);
    __syncthreads();
    if (wave_t < 4) {
      finish_columns_v(L, tid_t, beta, s_v[t & 1], s_dp[t & 1]);
      const int tn = t + 1 < T ? t + 1 : t;
      beta = beta_row[static_cast<int64_t>(tn) * H + h];
    } else if (wave_t < 8) {
      if (t + 1 < T) inputs(t + 1, t + 2 < T ? t + 2 : t + 1);
    } else if (wave_t == kOutWave + 1) {
      finish_qk(L, lane_t, &s_qk[t & 1]);
    } else if (wave_t == kOutWave && t > 0) {
      // output of the previous token, off the token chain
      if (lane_t < 32)
        emit_token_output<kNorm>(
            s_dp[(t - 1) & 1], s_qk[(t - 1) & 1], s_norm_w, flags, p.eps,
            col4_t, gate_w,
            at_bytes<uint16_t>(uniform_gptr(p.out + (row_tok + t - 1) * C),
                               2 * oc_t));
      if (kNorm)
        gate_w = *at_bytes<const u2>(
            uniform_gptr(p.gate + (row_tok + t) * C), 2 * oc_t);
    }
    __syncthreads();
    const f4 delta = *reinterpret_cast<const f4*>(&s_dp[t & 1][0][4 * col4]);
#pragma unroll
    for (int m = 0; m < kRowsPerThread; ++m)
      s[m] += akq_t[rgrp + kRowStride * m].y * delta;
  }
  // output of the last token (its rows are final after the last barrier)
  if (wave == kOutWave && lane < 32)
    emit_token_output<kNorm>(
        s_dp[(T - 1) & 1], s_qk[(T - 1) & 1], s_norm_w, flags, p.eps,
        lane, gate_w,
        at_bytes<uint16_t>(uniform_gptr(p.out + (row_tok + T - 1) * C),
                           2 * (h * kD + 4 * lane)));

  // ---- write back: state tile once, conv window once ----------------------
#pragma unroll
  for (int m = 0; m < kRowsPerThread; ++m)
    __builtin_nontemporal_store(s[m], tile_at(st, lane_off, m));
  if (conv_wave && !(flags & KDA_NO_CONV_UPDATE)) {
    *at_bytes<uint32_t>(cs_g, 4 * cs_off) = s_win[0][role][lane];
    *at_bytes<uint32_t>(cs_g, 4 * (cs_off + cs_step)) = s_win[1][role][lane];
    *at_bytes<uint32_t>(cs_g, 4 * (cs_off + 2 * cs_step)) =
        s_win[2][role][lane];
  }
}

// Chunk bookkeeping of a variable-length batch: one workgroup per sequence
// i computes its chunk count nt_i = ceil(len_i / BT) (a negative length
// counts as empty), its first chunk row base_i = sum_{j<i} nt_j (a
// workgroup reduction over the earlier sequences), writes
// chunk_offsets[i] = base_i (workgroup 0 also the total at [N]) and the
// rows (i, c) for c < nt_i at chunk_indices[base_i + c].
constexpr int kMetaThreads = 256;

__device__ __forceinline__ int64_t chunks_of(const int32_t* cu, int j,
                                             int bt) {
  const int64_t len = static_cast<int64_t>(cu[j + 1]) - cu[j];
  return len > 0 ? (len + bt - 1) / bt : 0;
}

__global__ __launch_bounds__(kMetaThreads) void chunk_metadata_kernel(
    const int32_t* cu, int n_seqs, int bt, int32_t* chunk_indices,
    int64_t* chunk_offsets) {
  __shared__ int64_t s_part[kMetaThreads];
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  // block 0 sums all sequences (for the total), block i those before i
  const int upto = i == 0 ? n_seqs : i;
  int64_t acc = 0, before = 0;
  for (int j = tid; j < upto; j += kMetaThreads) {
    const int64_t nt = chunks_of(cu, j, bt);
    acc += nt;
    if (j < i) before += nt;
  }
  // reduce `before` (and for block 0 the total) over the workgroup
  s_part[tid] = i == 0 ? acc : before;
  __syncthreads();
  for (int w = kMetaThreads / 2; w > 0; w >>= 1) {
    if (tid < w) s_part[tid] += s_part[tid + w];
    __syncthreads();
  }
  const int64_t base = i == 0 ? 0 : s_part[0];
  if (tid == 0) {
    chunk_offsets[i] = base;
    if (i == 0) chunk_offsets[n_seqs] = s_part[0];
  }
  const int64_t nt_i = i < n_seqs ? chunks_of(cu, i, bt) : 0;
  for (int64_t c = tid; c < nt_i; c += kMetaThreads) {
    chunk_indices[(base + c) * 2] = i;
    chunk_indices[(base + c) * 2 + 1] = static_cast<int32_t>(c);
  }
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

// Compute units of device `dev` (read once per device; 256 if unknown).
std::once_flag g_cu_once[kMaxDevices];
int g_cus[kMaxDevices];
int cu_count(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_cu_once[dev], [dev] {
    int cus = 0;
    g_cus[dev] = hipDeviceGetAttribute(&cus,
                                       hipDeviceAttributeMultiprocessorCount,
                                       dev) == hipSuccess && cus > 0
                     ? cus
                     : 256;
  });
  return g_cus[dev];
}

bool aligned16(const void* ptr) {
  return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0;
}

bool supported_heads(int h) { return h == 12 || h == 24 || h == 48 || h == 96; }

constexpr int32_t kMaxTokens = 1024;

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

// Which form kda_decode_tokens runs for rows of T tokens, from timings on
// MI355X (us per call):
//   * T = 2 .. 4: token by token (224 live rows x 48 heads, token by token
//     / short rows: 296 / 320 at T = 4);
//   * T = 5 .. 16: the short-row kernel (341 / 314 at T = 5, 432 / 320 at
//     T = 8; against the chunked kernel 494 / 528 at T = 12);
//   * T = 17 .. 64 with at least 4 (row, head) units per compute unit: the
//     short-row kernel (224 x 48: 619 / 889 at T = 24, 1360 / 1429 at 64;
//     64 x 24: 117 / 132 at 32);  with fewer units, and from T = 65: the
//     chunked kernel, whose prep overlaps the state chain of each
//     (row, head) (1 x 12: 30 / 32 at T = 32, 33 / 57 at 64; 224 x 48:
//     2199 / 2307 at 128).
constexpr int32_t kShortMinTokens = 5;
constexpr int32_t kShortAnyUnitsMaxTokens = 16;
constexpr int32_t kShortMaxTokens = 64;
constexpr int64_t kShortMinUnitsPerCU = 4;

// Whether kda_decode_tokens runs the short-row kernel for these rows.
bool use_short_rows(const kda_dims* d, int32_t tokens, int dev) {
  if (tokens < kShortMinTokens || tokens > kShortMaxTokens) return false;
  if (tokens <= kShortAnyUnitsMaxTokens) return true;
  return static_cast<int64_t>(d->batch) * d->num_heads >=
         kShortMinUnitsPerCU * cu_count(dev);
}

KdaChunkedArgs chunked_args(const kda_dims* d, const int32_t* cu_seqlens,
                            int32_t tokens_per_row, const void* qkv,
                            const float* conv_w, void* conv_state,
                            float* rec_state, const float* g,
                            const float* beta, const void* gate,
                            const float* norm_w, const int32_t* state_idx,
                            void* out) {
  KdaChunkedArgs a{};
  a.qkv = static_cast<const uint16_t*>(qkv);
  a.conv_w = conv_w;
  a.conv_state = static_cast<uint16_t*>(conv_state);
  a.rec_state = rec_state;
  a.g = g;
  a.beta = beta;
  a.gate = static_cast<const uint16_t*>(gate);
  a.norm_w = norm_w;
  a.state_idx = state_idx;
  a.cu_seqlens = cu_seqlens;
  a.tokens_per_row = tokens_per_row;
  a.out = static_cast<uint16_t*>(out);
  a.flags = d->flags;
  a.heads = d->num_heads;
  a.num_slots = d->num_slots;
  a.eps = d->norm_eps;
  return a;
}

// Load mode of the single-token kernel from the units per compute unit.
// Measured on MI355X (us per call; graph replay for small calls):
//   * tile first when some compute units hold a second unit (CUs < units
//     <= 2 CUs): 288 units 8.9 against 9.7 (lean), 384 units 10.8-11.3
//     against 11.4-11.9; but 12 units 4.0 against 3.95, 192 units 6.3
//     against 6.0, 768 units 21.3 against 20.8;
//   * every wave loading the small inputs from 32 units per compute unit:
//     49,152 units (96 heads, norm off) 1027 against 1072 (lean), 12,288
//     units (48 heads) 265 against 270; lean is faster up to ~24 units per
//     compute unit (3,072 units 72.3 against 73.3, 6,144 units 140.6
//     against 141.6).
constexpr int64_t kAllWavesMinUnitsPerCU = 32;
int load_mode(int64_t units, int dev) {
  const int64_t cus = cu_count(dev);
  if (units > cus && units <= 2 * cus) return kLoadTileFirst;
  if (units >= kAllWavesMinUnitsPerCU * cus) return kLoadAllWaves;
  return kLoadLean;
}

template <bool kNorm, bool kRaw>
void launch_decode(int mode, dim3 grid, hipStream_t stream, const Params& p) {
  if (mode == kLoadTileFirst)
    hipLaunchKernelGGL((kda_decode_kernel<kNorm, kRaw, kLoadTileFirst>), grid,
                       dim3(kThreads), 0, stream, p.state_idx, p.heads, p);
  else if (mode == kLoadAllWaves)
    hipLaunchKernelGGL((kda_decode_kernel<kNorm, kRaw, kLoadAllWaves>), grid,
                       dim3(kThreads), 0, stream, p.state_idx, p.heads, p);
  else
    hipLaunchKernelGGL((kda_decode_kernel<kNorm, kRaw, kLoadLean>), grid,
                       dim3(kThreads), 0, stream, p.state_idx, p.heads, p);
}

template <bool kRaw>
kda_status launch(const kda_dims* d, const Params& p, void* hip_stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev))
    return KDA_ERR_DEVICE;
  const int64_t units = static_cast<int64_t>(d->batch) * d->num_heads;
  const dim3 grid(static_cast<unsigned>(units));
  const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int mode = load_mode(units, dev);
  if (d->flags & KDA_OUTPUT_NORM)
    launch_decode<true, kRaw>(mode, grid, stream, p);
  else
    launch_decode<false, kRaw>(mode, grid, stream, p);
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

kda_status kda_decode_tokens(const kda_dims* d, int32_t tokens,
                             const void* qkv, const float* conv_w,
                             void* conv_state, float* rec_state, const float* g,
                             const float* beta, const void* gate,
                             const float* norm_w, const int32_t* state_idx,
                             void* out, void* hip_stream) {
  kda_status st = check_dims(d, kPlainFlags);
  if (st != KDA_OK) return st;
  if (tokens < 1 || tokens > kMaxTokens) return KDA_ERR_INVALID_ARG;
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
  // one token: the buffers are the single-token layout
  if (tokens == 1) return launch<false>(d, p, hip_stream);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev))
    return KDA_ERR_DEVICE;
  const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (use_short_rows(d, tokens, dev)) {
    const KdaChunkedArgs a =
        chunked_args(d, nullptr, tokens, qkv, conv_w, conv_state, rec_state,
                     g, beta, gate, norm_w, state_idx, out);
    return kda_short_rows_launch(a, d->batch, stream) == hipSuccess
               ? KDA_OK
               : KDA_ERR_LAUNCH;
  }
  if (tokens > kShortAnyUnitsMaxTokens) {
    // [B, T, ...] token-major buffers are the prefill layout with row n
    // owning tokens n*T .. n*T + T-1
    if (static_cast<int64_t>(d->batch) * tokens > INT32_MAX)
      return KDA_ERR_INVALID_ARG;
    const KdaChunkedArgs a =
        chunked_args(d, nullptr, tokens, qkv, conv_w, conv_state, rec_state,
                     g, beta, gate, norm_w, state_idx, out);
    return kda_chunked_prefill_launch(a, d->batch, stream) == hipSuccess
               ? KDA_OK
               : KDA_ERR_LAUNCH;
  }
  const dim3 grid(static_cast<unsigned>(d->batch * d->num_heads));
  if (d->flags & KDA_OUTPUT_NORM)
    hipLaunchKernelGGL(kda_decode_tokens_kernel<true>, grid, dim3(kThreads), 0,
                       stream, p, tokens);
  else
    hipLaunchKernelGGL(kda_decode_tokens_kernel<false>, grid, dim3(kThreads),
                       0, stream, p, tokens);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

uint64_t kda_decode_tokens_bytes(const kda_dims* d, int32_t tokens,
                                 int32_t live_rows) {
  if (tokens < 1) return 0;
  const uint64_t one = bytes_model(d, live_rows, false, false);
  if (one == 0) return 0;
  // per (row, head): the state and conv-state traffic once, the per-token
  // inputs and outputs T times; per call: the weights once
  const uint64_t H = d->num_heads, D = d->head_dim;
  const bool norm = (d->flags & KDA_OUTPUT_NORM) != 0;
  const uint64_t per_token_unit = 3 * D * 2 + D * 4 + 4 + D * 2 +
                                  (norm ? D * 2 : 0);
  const uint64_t live = static_cast<uint64_t>(live_rows) * H;
  const uint64_t null_units = static_cast<uint64_t>(d->batch - live_rows) * H;
  const uint64_t extra = static_cast<uint64_t>(tokens - 1) *
                         (live * per_token_unit + null_units * D * 2);
  return one + extra;
}

kda_status kda_prefill(const kda_dims* d, const int32_t* cu_seqlens,
                       const void* qkv, const float* conv_w, void* conv_state,
                       float* rec_state, const float* g, const float* beta,
                       const void* gate, const float* norm_w,
                       const int32_t* state_idx, void* out, void* hip_stream) {
  kda_status st = check_dims(d, kPlainFlags);
  if (st != KDA_OK) return st;
  if (d->batch == 0) return KDA_OK;
  if (!cu_seqlens) return KDA_ERR_INVALID_ARG;
  if (!aligned16(cu_seqlens)) return KDA_ERR_MISALIGNED;
  st = check_common(d, qkv, conv_w, conv_state, rec_state, gate, norm_w,
                    state_idx, out);
  if (st != KDA_OK) return st;
  if (!g || !beta) return KDA_ERR_INVALID_ARG;
  if (!aligned16(g) || !aligned16(beta)) return KDA_ERR_MISALIGNED;
  Params p = base_params(d, qkv, conv_w, conv_state, rec_state, gate, norm_w,
                         state_idx, out);
  p.g = g;
  p.beta = beta;
  p.cu_seqlens = cu_seqlens;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev))
    return KDA_ERR_DEVICE;
  const dim3 grid(static_cast<unsigned>(d->batch * d->num_heads));
  const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (d->flags & KDA_OUTPUT_NORM)
    hipLaunchKernelGGL(kda_decode_tokens_kernel<true>, grid, dim3(kThreads), 0,
                       stream, p, 0);
  else
    hipLaunchKernelGGL(kda_decode_tokens_kernel<false>, grid, dim3(kThreads),
                       0, stream, p, 0);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

namespace {

// Flags of a prefill call with g and beta (gi null) or the raw gate
// inputs gi, and the bound of the bounded gate.
kda_status check_prefill_gates(const kda_dims* d, const kda_gate_inputs* gi) {
  kda_status st = check_dims(d, gi ? kPlainFlags | KDA_BOUNDED_GATE
                                   : kPlainFlags);
  if (st != KDA_OK) return st;
  if (!gi) return KDA_OK;
  if ((d->flags & KDA_BOUNDED_GATE) &&
      !(std::isfinite(gi->lower_bound) && gi->lower_bound < 0.0f))
    return KDA_ERR_INVALID_ARG;
  return KDA_OK;
}

// Pointer checks of the gate operands (after the batch-0 early return).
kda_status check_gate_ptrs(const float* g, const float* beta,
                           const kda_gate_inputs* gi) {
  if (!gi) {
    if (!g || !beta) return KDA_ERR_INVALID_ARG;
    if (!aligned16(g) || !aligned16(beta)) return KDA_ERR_MISALIGNED;
    return KDA_OK;
  }
  if (!gi->raw_g || !gi->raw_beta || !gi->A_log || !gi->dt_bias)
    return KDA_ERR_INVALID_ARG;
  if (!aligned16(gi->raw_g) || !aligned16(gi->raw_beta) ||
      !aligned16(gi->A_log) || !aligned16(gi->dt_bias) ||
      (gi->conv_bias && !aligned16(gi->conv_bias)))
    return KDA_ERR_MISALIGNED;
  return KDA_OK;
}

KdaRawGateArgs raw_gate_args(const kda_gate_inputs* gi) {
  KdaRawGateArgs r{};
  if (gi) {
    r.conv_bias = gi->conv_bias;
    r.raw_g = static_cast<const uint16_t*>(gi->raw_g);
    r.raw_beta = static_cast<const uint16_t*>(gi->raw_beta);
    r.A_log = gi->A_log;
    r.dt_bias = gi->dt_bias;
    r.lower_bound = gi->lower_bound;
  }
  return r;
}

kda_status prefill_chunked_impl(const kda_dims* d, const int32_t* cu_seqlens,
                                const void* qkv, const float* conv_w,
                                void* conv_state, float* rec_state,
                                const float* g, const float* beta,
                                const kda_gate_inputs* gi, const void* gate,
                                const float* norm_w, const int32_t* state_idx,
                                void* out, void* hip_stream) {
  kda_status st = check_prefill_gates(d, gi);
  if (st != KDA_OK) return st;
  if (d->batch == 0) return KDA_OK;
  if (!cu_seqlens) return KDA_ERR_INVALID_ARG;
  if (!aligned16(cu_seqlens)) return KDA_ERR_MISALIGNED;
  st = check_common(d, qkv, conv_w, conv_state, rec_state, gate, norm_w,
                    state_idx, out);
  if (st != KDA_OK) return st;
  st = check_gate_ptrs(g, beta, gi);
  if (st != KDA_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev))
    return KDA_ERR_DEVICE;
  KdaChunkedArgs a =
      chunked_args(d, cu_seqlens, 0, qkv, conv_w, conv_state, rec_state, g,
                   beta, gate, norm_w, state_idx, out);
  a.rg = raw_gate_args(gi);
  return kda_chunked_prefill_launch(a, d->batch,
                                    static_cast<hipStream_t>(hip_stream)) ==
                 hipSuccess
             ? KDA_OK
             : KDA_ERR_LAUNCH;
}

}  // namespace

kda_status kda_prefill_chunked(const kda_dims* d, const int32_t* cu_seqlens,
                               const void* qkv, const float* conv_w,
                               void* conv_state, float* rec_state,
                               const float* g, const float* beta,
                               const void* gate, const float* norm_w,
                               const int32_t* state_idx, void* out,
                               void* hip_stream) {
  return prefill_chunked_impl(d, cu_seqlens, qkv, conv_w, conv_state,
                              rec_state, g, beta, nullptr, gate, norm_w,
                              state_idx, out, hip_stream);
}

kda_status kda_prefill_chunked_raw_gates(
    const kda_dims* d, const int32_t* cu_seqlens, const void* qkv,
    const float* conv_w, void* conv_state, float* rec_state,
    const kda_gate_inputs* gates, const void* gate, const float* norm_w,
    const int32_t* state_idx, void* out, void* hip_stream) {
  if (!gates) return KDA_ERR_INVALID_ARG;
  return prefill_chunked_impl(d, cu_seqlens, qkv, conv_w, conv_state,
                              rec_state, nullptr, nullptr, gates, gate, norm_w,
                              state_idx, out, hip_stream);
}

uint64_t kda_prefill_chunks_workspace_bytes(const kda_dims* d,
                                            int64_t max_chunks) {
  if (!d || d->num_heads < 1 || max_chunks < 0) return 0;
  return static_cast<uint64_t>(max_chunks) *
         static_cast<uint64_t>(d->num_heads) * kda_pass_record_bytes();
}

namespace {

// With static_scratch the records go to the library's per-device array
// (workspace and workspace_bytes are ignored); a request larger than the
// array is KDA_ERR_TOO_LARGE.
kda_status prefill_chunks_impl(
    const kda_dims* d, const int32_t* cu_seqlens, const int32_t* chunk_indices,
    const int64_t* chunk_offsets, int64_t max_chunks, const void* qkv,
    const float* conv_w, void* conv_state, float* rec_state, const float* g,
    const float* beta, const kda_gate_inputs* gi, const void* gate,
    const float* norm_w, const int32_t* state_idx, void* out, void* workspace,
    uint64_t workspace_bytes, void* hip_stream, bool static_scratch = false) {
  kda_status st = check_prefill_gates(d, gi);
  if (st != KDA_OK) return st;
  if (max_chunks < 0 ||
      max_chunks * static_cast<int64_t>(d->num_heads) > INT32_MAX ||
      static_cast<int64_t>(d->batch) * d->num_heads * 8 > INT32_MAX)
    return KDA_ERR_INVALID_ARG;
  if (static_scratch &&
      kda_prefill_chunks_workspace_bytes(d, max_chunks) >
          KDA_STATIC_SCRATCH_BYTES)
    return KDA_ERR_TOO_LARGE;
  if (d->batch == 0) return KDA_OK;
  if (!cu_seqlens || !chunk_offsets ||
      (max_chunks > 0 && (!chunk_indices || (!static_scratch && !workspace))))
    return KDA_ERR_INVALID_ARG;
  if (!static_scratch &&
      workspace_bytes < kda_prefill_chunks_workspace_bytes(d, max_chunks))
    return KDA_ERR_INVALID_ARG;
  if (!aligned16(cu_seqlens) || !aligned16(chunk_offsets) ||
      (chunk_indices && !aligned16(chunk_indices)) ||
      (!static_scratch && workspace && !aligned16(workspace)))
    return KDA_ERR_MISALIGNED;
  st = check_gate_ptrs(g, beta, gi);
  if (st != KDA_OK) return st;
  st = check_common(d, qkv, conv_w, conv_state, rec_state, gate, norm_w,
                    state_idx, out);
  if (st != KDA_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev))
    return KDA_ERR_DEVICE;
  if (static_scratch) {
    workspace = kda_pass_static_scratch(dev);
    if (!workspace) return KDA_ERR_DEVICE;
  }
  KdaPassArgs a{};
  a.qkv = static_cast<const uint16_t*>(qkv);
  a.conv_w = conv_w;
  a.conv_state = static_cast<uint16_t*>(conv_state);
  a.rec_state = rec_state;
  a.g = g;
  a.beta = beta;
  a.gate = static_cast<const uint16_t*>(gate);
  a.norm_w = norm_w;
  a.state_idx = state_idx;
  a.cu_seqlens = cu_seqlens;
  a.chunk_indices = chunk_indices;
  a.chunk_offsets = chunk_offsets;
  a.workspace = static_cast<float*>(workspace);
  a.out = static_cast<uint16_t*>(out);
  a.max_chunks = max_chunks;
  a.num_seqs = d->batch;
  a.flags = d->flags;
  a.heads = d->num_heads;
  a.num_slots = d->num_slots;
  a.eps = d->norm_eps;
  a.rg = raw_gate_args(gi);
  return kda_chunk_pass_launch(a, static_cast<hipStream_t>(hip_stream)) ==
                 hipSuccess
             ? KDA_OK
             : KDA_ERR_LAUNCH;
}

}  // namespace

kda_status kda_prefill_chunks(const kda_dims* d, const int32_t* cu_seqlens,
                              const int32_t* chunk_indices,
                              const int64_t* chunk_offsets, int64_t max_chunks,
                              const void* qkv, const float* conv_w,
                              void* conv_state, float* rec_state,
                              const float* g, const float* beta,
                              const void* gate, const float* norm_w,
                              const int32_t* state_idx, void* out,
                              void* workspace, uint64_t workspace_bytes,
                              void* hip_stream) {
  return prefill_chunks_impl(d, cu_seqlens, chunk_indices, chunk_offsets,
                             max_chunks, qkv, conv_w, conv_state, rec_state, g,
                             beta, nullptr, gate, norm_w, state_idx, out,
                             workspace, workspace_bytes, hip_stream);
}

kda_status kda_prefill_chunks_static(
    const kda_dims* d, const int32_t* cu_seqlens, const int32_t* chunk_indices,
    const int64_t* chunk_offsets, int64_t max_chunks, const void* qkv,
    const float* conv_w, void* conv_state, float* rec_state, const float* g,
    const float* beta, const void* gate, const float* norm_w,
    const int32_t* state_idx, void* out, void* hip_stream) {
  return prefill_chunks_impl(d, cu_seqlens, chunk_indices, chunk_offsets,
                             max_chunks, qkv, conv_w, conv_state, rec_state, g,
                             beta, nullptr, gate, norm_w, state_idx, out,
                             nullptr, 0, hip_stream, /*static_scratch=*/true);
}

kda_status kda_prefill_chunks_raw_gates(
    const kda_dims* d, const int32_t* cu_seqlens, const int32_t* chunk_indices,
    const int64_t* chunk_offsets, int64_t max_chunks, const void* qkv,
    const float* conv_w, void* conv_state, float* rec_state,
    const kda_gate_inputs* gates, const void* gate, const float* norm_w,
    const int32_t* state_idx, void* out, void* workspace,
    uint64_t workspace_bytes, void* hip_stream) {
  if (!gates) return KDA_ERR_INVALID_ARG;
  return prefill_chunks_impl(d, cu_seqlens, chunk_indices, chunk_offsets,
                             max_chunks, qkv, conv_w, conv_state, rec_state,
                             nullptr, nullptr, gates, gate, norm_w, state_idx,
                             out, workspace, workspace_bytes, hip_stream);
}

kda_status kda_chunk_metadata(const int32_t* cu_seqlens, int32_t num_seqs,
                              int32_t chunk_size, int32_t* chunk_indices,
                              int64_t* chunk_offsets, void* hip_stream) {
  if (num_seqs < 0 || chunk_size < 1) return KDA_ERR_INVALID_ARG;
  if (!cu_seqlens || !chunk_offsets) return KDA_ERR_INVALID_ARG;
  if (num_seqs > 0 && !chunk_indices) return KDA_ERR_INVALID_ARG;
  if (!aligned16(cu_seqlens) || !aligned16(chunk_offsets) ||
      (chunk_indices && !aligned16(chunk_indices)))
    return KDA_ERR_MISALIGNED;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev))
    return KDA_ERR_DEVICE;
  const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (num_seqs == 0) {
    // chunk_offsets = [0]: a one-workgroup launch with nothing else to do
    hipLaunchKernelGGL(chunk_metadata_kernel, dim3(1), dim3(kMetaThreads), 0,
                       stream, cu_seqlens, 0, chunk_size, chunk_indices,
                       chunk_offsets);
  } else {
    hipLaunchKernelGGL(chunk_metadata_kernel,
                       dim3(static_cast<unsigned>(num_seqs)),
                       dim3(kMetaThreads), 0, stream, cu_seqlens, num_seqs,
                       chunk_size, chunk_indices, chunk_offsets);
  }
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int64_t kda_chunk_count(const int32_t* cu_seqlens_host, int32_t num_seqs,
                        int32_t chunk_size) {
  if (!cu_seqlens_host || num_seqs < 0 || chunk_size < 1) return -1;
  int64_t total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int64_t len =
        static_cast<int64_t>(cu_seqlens_host[i + 1]) - cu_seqlens_host[i];
    if (len > 0) total += (len + chunk_size - 1) / chunk_size;
  }
  return total;
}

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported shape (H in {12,24,48,96}, D=128, W=4)";
    case KDA_ERR_MISALIGNED: return "buffer not 16-byte aligned";
    case KDA_ERR_DEVICE: return "no gfx950 HIP device current";
    case KDA_ERR_LAUNCH: return "kernel launch failed";
    case KDA_ERR_TOO_LARGE:
      return "request exceeds the library's static scratch "
             "(KDA_STATIC_SCRATCH_BYTES)";
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
