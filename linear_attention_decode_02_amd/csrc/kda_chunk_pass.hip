// Variable-length KDA prefill in two passes over the chunk metadata.
//
// Operation: the prefill of the page "PR #51862 完整报告 -- Remove prefill
// pipeline stall in chunk KDA" -- each sequence of a variable-length batch
// runs the gated delta-rule step of the page "PR #50654 完整报告 --
// [ROCm][Perf] Kimi-K3 Fused kernel for KDA decode" over its tokens from
// the state in its slot.  As on that page, the chunk kernels are driven by
// the device-side chunk table (chunk_indices: (sequence, chunk) pairs;
// chunk_offsets: each sequence's first chunk), built without a host
// synchronisation.  The arithmetic is the 16-token chunk form of
// kda_chunked.hip (include/kda_decode.h states it).
//
// Pass 1, kda_chunk_prep_kernel: one 256-thread workgroup per (chunk, head),
// all chunks of all sequences in parallel.  It needs only the chunk's inputs
// (and the three inputs before it), not the state: causal conv + SiLU,
// q/k L2 normalisation, the cumulative decay G, the decayed operands
// K~ = K e^G, Q~ = Q e^G, K^ = K e^{G_last - G}, the Gram products A and B on
// the matrix cores (per entry with its own exponential when |G| > 80), and
// T = (I + diag(beta) A)^{-1}.  It writes them as one fixed-size record per
// (chunk, head) into the caller's workspace, laid out as the second pass
// reads them (rows padded against LDS bank conflicts).
//
// Pass 2, kda_chunk_state_kernel: one wave per 16-column block of the
// state (the value columns evolve independently: the delta rule couples
// keys, not values), kStateWaves waves per workgroup and kSplits = 8 /
// kStateWaves workgroups per (sequence, head).  A wave holds its 128 x 16
// block in MFMA accumulator registers through the sequence's chunks: K~S and
// Q~S, the deltas T beta (V - K~S), the outputs Q~S + B Delta (into the
// record's output rows, before the norm) and the state update
// e^{G_last} S + K^^T Delta.  The next chunks' records stream into LDS
// (global_load_lds, kBufs records in flight) while the current one is
// processed.  Eight waves in one
// workgroup (two per SIMD) measured fastest: one wave per SIMD issues at
// most one fp32 MFMA per 32 cycles, two waves share a SIMD at one per 24, so
// splitting a (sequence, head) over more compute units with fewer waves each
// gained nothing.  The workgroups of one (sequence, head) share
// blockIdx % 8, i.e. one XCD and its L2, when kSplits > 1.
//
// Pass 3, kda_chunk_out_kernel: one workgroup per (chunk, head) applies the
// gated RMSNorm, which needs all 128 columns of a token, and writes bf16.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "kda_chunk_pass.h"
#include "kda_decode.h"

namespace {

// Records of kda_prefill_chunks_static, for callers that cannot allocate:
// one array per GPU, created when the library's code object is loaded on
// that GPU and held until the process ends.  Host code never passes this
// name to a kernel (on the host it is only a stand-in for the symbol): it
// uses the device address that kda_pass_static_scratch looks up once per
// device.
constexpr uint64_t kStaticScratchBytes = KDA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kD = 128;
constexpr int kW = 4;
constexpr int kC = 16;
constexpr int kThreads = 256;
constexpr int kLd = kD + 4;   // padded [kC][kD] rows (floats)
constexpr int kTd = kC + 4;   // padded [kD][kC] and [kC][kC] rows
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kSafeExp2 = 80.0f * kLog2e;  // |G| <= 80 in natural units

// Record of one (chunk, head), in floats.
constexpr int kRecKt = 0;                     // K~   [kC][kLd]
constexpr int kRecQt = kRecKt + kC * kLd;     // Q~   [kC][kLd]
constexpr int kRecV = kRecQt + kC * kLd;      // V    [kC][kLd]
constexpr int kRecKh = kRecV + kC * kLd;      // K^   [kC][kLd]
constexpr int kRecGam = kRecKh + kC * kLd;    // e^{G_last} [kD]
constexpr int kRecBeta = kRecGam + kD;        // beta [kC]
constexpr int kRecT = kRecBeta + kC;          // T    [kC][kTd]
constexpr int kRecB = kRecT + kC * kTd;       // B    [kC][kTd]
constexpr int kRecO = kRecB + kC * kTd;       // O (pass 2) [kC][kD]
constexpr int kRecStaged = kRecO;             // what pass 2 copies to LDS
constexpr int kRecFloats = kRecO + kC * kD;
static_assert(kRecFloats % 4 == 0 && kRecStaged % 4 == 0, "16-byte records");
constexpr int kStateWaves = 8;                // 16 value columns per wave
constexpr int kSplits = kD / (16 * kStateWaves);
constexpr int kBufs = 3;                      // records in flight in LDS
// LDS-direct copy instructions per wave per record (the fewest any wave of
// the workgroup issues: the last wave's count)
constexpr int kStageBytes = kRecStaged * 4;
constexpr int kDmaMin =
    (kStageBytes - (kStateWaves - 1) * 1024 + kStateWaves * 1024 - 1) /
    (kStateWaves * 1024);
static_assert(kDmaMin >= 1 && kDmaMin < 64, "vmcnt range");

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {  // RNE
  return static_cast<uint32_t>(__builtin_bit_cast(unsigned short, (__bf16)lo)) |
         (static_cast<uint32_t>(__builtin_bit_cast(unsigned short, (__bf16)hi))
          << 16);
}
__device__ __forceinline__ float exp2_(float x) {
  return __builtin_amdgcn_exp2f(x);
}
__device__ __forceinline__ float sigmoid_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
template <int kCtrl>
__device__ __forceinline__ float dpp_(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                         0xF, 0xF, false));
}
// Sum over each row of 16 lanes (quad_perm [1,0,3,2], [2,3,0,1],
// row_half_mirror, row_mirror), in every lane of the row.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_<0xB1>(v);
  v += dpp_<0x4E>(v);
  v += dpp_<0x141>(v);
  v += dpp_<0x140>(v);
  return v;
}
// Eight wave sums side by side, each result in every lane.
__device__ __forceinline__ void wave_sum8(float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = row_sum16(v[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int b = __builtin_bit_cast(int, v[i]);
    v[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  }
}
__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 ld4(const float* p) {
  return *reinterpret_cast<const f4*>(p);
}
// Sixteen bytes per lane from global memory straight into LDS: lane l's
// bytes land at dst + 16 l (dst wave-uniform).  Counted by vmcnt.
__device__ __forceinline__ void load_lds16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}
// s_waitcnt (gfx9 fields): vmcnt 0, the other counters at their maximum
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// vmcnt N (bits 3:0 and 15:14), expcnt and lgkmcnt at their maximum
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}

// Sequence n's token range; false for an empty sequence.
__device__ __forceinline__ bool seq_range(const KdaPassArgs& p, int n,
                                          int32_t& tb, int& len) {
  tb = p.cu_seqlens[n];
  const int32_t te = p.cu_seqlens[n + 1];
  len = te > tb ? te - tb : 0;
  return len > 0;
}

// ---- pass 1 -----------------------------------------------------------------

struct PrepSmem {
  // Gram inputs: K~ and Q~ on the factored path, or raw q and the
  // cumulative log2 decay on the exact path (one or the other per chunk)
  union {
    struct {
      float kt[kC][kLd];
      float qt[kC][kLd];
    } f;
    struct {
      float qraw[kC][kLd];
      float graw[kC][kLd];
    } x;
  } g;
  float ki[kC][kLd];   // k e^{-G}; raw k on the exact path
  float part[4][kC][kC];
  float LT[kC][kTd];   // LT[s][t] = beta_t A_ts (s < t)
  float beta[kC];
  int unsafe;
};

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void kda_chunk_prep_kernel(
    KdaPassArgs p) {
  __shared__ alignas(16) PrepSmem sm;
  const int tid = threadIdx.x;
  // this wave's tokens: 4pw .. 4pw+3 (scalar: wave-uniform offsets stay on
  // the scalar unit)
  const int pw = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c = lane & 15;
  const int gq = lane >> 4;
  const int H = p.heads;
  const int C = H * kD;
  const int C3 = 3 * C;
  const int64_t q = blockIdx.x / H;
  const int h = static_cast<int>(blockIdx.x % H);
  const int64_t total = p.chunk_offsets[p.num_seqs];
  if (q >= total || q >= p.max_chunks) return;
  const int n = p.chunk_indices[2 * q];
  const int ci = p.chunk_indices[2 * q + 1];
  if (n < 0 || n >= p.num_seqs || ci < 0) return;
  int32_t tb;
  int len;
  if (!seq_range(p, n, tb, len) || ci * kC >= len) return;
  const int32_t slot = p.state_idx[n];
  if (slot <= 0 || slot >= p.num_slots) return;  // null rows need no record
  const uint32_t flags = p.flags;
  const bool tap_major = (flags & KDA_CONV_TAP_MAJOR) != 0;
  const bool conv_update = (flags & KDA_NO_CONV_UPDATE) == 0;
  const bool l2 = (flags & KDA_QK_L2NORM) != 0;
  const int nv = len - ci * kC < kC ? len - ci * kC : kC;
  const int64_t tok0 = tb + static_cast<int64_t>(ci) * kC;
  const int64_t col0 = static_cast<int64_t>(h) * kD;
  float* rec = p.workspace + (q * H + h) * kRecFloats;

  // stored conv window element e of channels ch, ch + 1 (a bf16 pair)
  auto window = [&](int64_t ch, int e) -> uint32_t {
    if (tap_major)
      return *reinterpret_cast<const uint32_t*>(
          p.conv_state + (static_cast<int64_t>(slot) * (kW - 1) + e) * C3 +
          ch);
    const uint16_t* cs =
        p.conv_state + (static_cast<int64_t>(slot) * C3 + ch) * (kW - 1) + e;
    return static_cast<uint32_t>(cs[0]) |
           (static_cast<uint32_t>(cs[kW - 1]) << 16);
  };
  // conv inputs, channels 2 lane, 2 lane + 1 of each part: raw[pp][u] is
  // token 4pw - 3 + u (rows past the end re-read the last row, masked
  // below); taps before the sequence, or every tap but the current one
  // without the conv-state update, come from the stored window
  uint32_t raw[3][7];
#pragma unroll
  for (int pp = 0; pp < 3; ++pp) {
    const int64_t ch = static_cast<int64_t>(pp) * C + col0 + 2 * lane;
#pragma unroll
    for (int u = 0; u < 7; ++u) {
      const int rel = 4 * pw - 3 + u;
      if (u >= 3 || (conv_update && (rel >= 0 || ci > 0))) {
        const int rr = rel < nv - 1 ? rel : nv - 1;
        raw[pp][u] = *reinterpret_cast<const uint32_t*>(
            p.qkv + (tok0 + rr) * C3 + ch);
      } else {
        raw[pp][u] = window(ch, conv_update ? 3 + rel : u);
      }
    }
  }
  const bool raw_gates = p.rg.raw_g != nullptr;
  f2 cw[3][kW];
  f2 cb[3] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
  for (int pp = 0; pp < 3; ++pp) {
#pragma unroll
    for (int t = 0; t < kW; ++t)
      cw[pp][t] = *reinterpret_cast<const f2*>(
          p.conv_w + (static_cast<int64_t>(pp) * kW + t) * C + col0 + 2 * lane);
    if (p.rg.conv_bias)
      cb[pp] = *reinterpret_cast<const f2*>(
          p.rg.conv_bias + static_cast<int64_t>(pp) * C + col0 + 2 * lane);
  }
  // per-token decays (log2 units) of keys 2 lane, 2 lane + 1
  f2 gl[kC];
  if (raw_gates) {
    const f2 db =
        *reinterpret_cast<const f2*>(p.rg.dt_bias + col0 + 2 * lane);
    const float a_rate = __expf(p.rg.A_log[h]);
    const float lb2 = p.rg.lower_bound * kLog2e;
    uint32_t w[kC];
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      const int rr = t < nv - 1 ? t : nv - 1;
      w[t] = *reinterpret_cast<const uint32_t*>(
          p.rg.raw_g + ((tok0 + rr) * H + h) * kD + 2 * lane);
    }
    // one branch for the whole chunk, straight-line code inside
    if (p.flags & KDA_BOUNDED_GATE) {
#pragma unroll
      for (int t = 0; t < kC; ++t)
        gl[t] = f2{kda_gate2_from_raw<true>(bf16_lo(w[t]) + db.x, a_rate, lb2),
                   kda_gate2_from_raw<true>(bf16_hi(w[t]) + db.y, a_rate, lb2)};
    } else {
#pragma unroll
      for (int t = 0; t < kC; ++t)
        gl[t] =
            f2{kda_gate2_from_raw<false>(bf16_lo(w[t]) + db.x, a_rate, lb2),
               kda_gate2_from_raw<false>(bf16_hi(w[t]) + db.y, a_rate, lb2)};
    }
  } else {
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      const int rr = t < nv - 1 ? t : nv - 1;
      gl[t] = *reinterpret_cast<const f2*>(p.g + ((tok0 + rr) * H + h) * kD +
                                           2 * lane) *
              kLog2e;
    }
  }
#pragma unroll
  for (int t = 0; t < kC; ++t) gl[t] = kda_decay_floor2(gl[t]);
  f2 Gu[4] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
  f2 G = {0.f, 0.f};
  float gmax = 0.0f;
  // in groups of the 4 tokens a wave owns: the wave keeps its own group's
  // prefixes under a wave-uniform branch (no per-token select)
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    f2 Gt[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = 4 * grp + u;
      if (t < nv) G += gl[t];
      gmax = fmaxf(gmax, fmaxf(fabsf(G.x), fabsf(G.y)));
      Gt[u] = G;
    }
    if (grp == pw) {
#pragma unroll
      for (int u = 0; u < 4; ++u) Gu[u] = Gt[u];
    }
  }
  // NaN counts as unsafe; every wave reaches the same verdict
  const bool unsafe = __any(!(gmax <= kSafeExp2));
  if (lane < 4) {
    const int t = 4 * pw + lane;
    float b = 0.0f;
    if (t < nv)
      b = raw_gates ? sigmoid_(bf16_lo(p.rg.raw_beta[(tok0 + t) * H + h]))
                    : p.beta[(tok0 + t) * H + h];
    sm.beta[t] = b;
    rec[kRecBeta + t] = b;
  }

  // conv + SiLU of the wave's 4 tokens, then the L2 norms side by side
  float y[4][3][2];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const bool valid = 4 * pw + u < nv;
#pragma unroll
    for (int pp = 0; pp < 3; ++pp)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float a = cb[pp][e];
#pragma unroll
        for (int tap = 0; tap < kW; ++tap) {
          const uint32_t w2 = conv_update || tap == kW - 1 ? raw[pp][u + tap]
                                                           : raw[pp][tap];
          a += cw[pp][tap][e] * (e ? bf16_hi(w2) : bf16_lo(w2));
        }
        y[u][pp][e] = valid ? a * sigmoid_(a) : 0.0f;
      }
  }
  if (l2) {
    const float qscale = 0.08838834764831845f;  // D^-1/2
    float ss[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ss[2 * u] = y[u][0][0] * y[u][0][0] + y[u][0][1] * y[u][0][1];
      ss[2 * u + 1] = y[u][1][0] * y[u][1][0] + y[u][1][1] * y[u][1][1];
    }
    wave_sum8(ss);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float rq = rsqrtf(ss[2 * u] + 1e-6f);
      const float rk = rsqrtf(ss[2 * u + 1] + 1e-6f);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        y[u][0][e] = (y[u][0][e] * rq) * qscale;
        y[u][1][e] = y[u][1][e] * rk;
      }
    }
  }
  // decayed tables: to the record, and to LDS for the Gram products
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = 4 * pw + u;
    const f2 ee = {exp2_(Gu[u].x), exp2_(Gu[u].y)};
    const f2 qv = {y[u][0][0] * ee.x, y[u][0][1] * ee.y};
    const f2 kv = {y[u][1][0] * ee.x, y[u][1][1] * ee.y};
    *reinterpret_cast<f2*>(&rec[kRecQt + t * kLd + 2 * lane]) = qv;
    *reinterpret_cast<f2*>(&rec[kRecKt + t * kLd + 2 * lane]) = kv;
    *reinterpret_cast<f2*>(&rec[kRecV + t * kLd + 2 * lane]) =
        f2{y[u][2][0], y[u][2][1]};
    *reinterpret_cast<f2*>(&rec[kRecKh + t * kLd + 2 * lane]) =
        f2{y[u][1][0] * exp2_(G.x - Gu[u].x), y[u][1][1] * exp2_(G.y - Gu[u].y)};
    if (!unsafe) {
      *reinterpret_cast<f2*>(&sm.g.f.qt[t][2 * lane]) = qv;
      *reinterpret_cast<f2*>(&sm.g.f.kt[t][2 * lane]) = kv;
      *reinterpret_cast<f2*>(&sm.ki[t][2 * lane]) =
          f2{y[u][1][0] * exp2_(-Gu[u].x), y[u][1][1] * exp2_(-Gu[u].y)};
    } else {
      *reinterpret_cast<f2*>(&sm.ki[t][2 * lane]) = f2{y[u][1][0], y[u][1][1]};
      *reinterpret_cast<f2*>(&sm.g.x.qraw[t][2 * lane]) =
          f2{y[u][0][0], y[u][0][1]};
      *reinterpret_cast<f2*>(&sm.g.x.graw[t][2 * lane]) = Gu[u];
    }
  }
  if (pw == 0)
    *reinterpret_cast<f2*>(&rec[kRecGam + 2 * lane]) =
        f2{exp2_(G.x), exp2_(G.y)};
  __syncthreads();

  // A = K~ (K e^{-G})^T and B = Q~ (K e^{-G})^T: wave 0 / 1 A over keys
  // 0-63 / 64-127, wave 2 / 3 B likewise; or the exact per-entry sums
  const int t16 = tid >> 4;  // (t, s) of threads 0..255
  const int s16 = tid & 15;
  if (!unsafe) {
    const float(*src)[kLd] = pw < 2 ? sm.g.f.kt : sm.g.f.qt;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = 64 * (pw & 1) + 16 * kb + 4 * gq;
      const f4 a = ld4(&src[c][key]);
      const f4 b = ld4(&sm.ki[c][key]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma(a[j], b[j], acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.part[pw][4 * gq + r][c] = acc[r];
    __syncthreads();
    const float a = sm.part[0][t16][s16] + sm.part[1][t16][s16];
    const float b = sm.part[2][t16][s16] + sm.part[3][t16][s16];
    sm.LT[s16][t16] = s16 < t16 ? sm.beta[t16] * a : 0.0f;
    rec[kRecB + t16 * kTd + s16] = s16 <= t16 ? b : 0.0f;
  } else {
    float a = 0.0f, b = 0.0f;
    if (s16 <= t16) {
      for (int i = 0; i < kD; ++i) {
        const float ks =
            sm.ki[s16][i] * exp2_(sm.g.x.graw[t16][i] - sm.g.x.graw[s16][i]);
        a += sm.ki[t16][i] * ks;
        b += sm.g.x.qraw[t16][i] * ks;
      }
    }
    sm.LT[s16][t16] = s16 < t16 ? sm.beta[t16] * a : 0.0f;
    rec[kRecB + t16 * kTd + s16] = b;
  }
  __syncthreads();
  // T = (I + L)^{-1}: lane c of wave 0 solves column c by forward
  // substitution, T[t][c] = [t == c] - sum_{s<t} L[t][s] T[s][c]
  if (pw == 0 && lane < kC) {
    float tc[kC];
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      float v = t == lane ? 1.0f : 0.0f;
#pragma unroll
      for (int s = 0; s < t; ++s) v -= sm.LT[s][t] * tc[s];
      tc[t] = v;
    }
#pragma unroll
    for (int t = 0; t < kC; ++t) rec[kRecT + t * kTd + lane] = tc[t];
  }
}

// ---- pass 2 -----------------------------------------------------------------

__global__ __launch_bounds__(64 * kStateWaves) void kda_chunk_state_kernel(
    KdaPassArgs p) {
  __shared__ alignas(16) float rec[kBufs][kRecStaged];  // records in flight
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar
  const int lane = tid & 63;
  const int c = lane & 15;
  const int gq = lane >> 4;
  const int H = p.heads;
  const int C = H * kD;
  const int C3 = 3 * C;
  // blockIdx = ((unit / 8) * kSplits + split) * 8 + unit % 8
  const int64_t b = blockIdx.x;
  const int split = static_cast<int>((b >> 3) % kSplits);
  const int64_t unit = ((b >> 3) / kSplits) * 8 + (b & 7);
  if (unit >= static_cast<int64_t>(p.num_seqs) * H) return;
  const int n = static_cast<int>(unit / H);
  const int h = static_cast<int>(unit % H);
  int32_t tb;
  int len;
  if (!seq_range(p, n, tb, len)) return;
  const int32_t slot = p.state_idx[n];
  if (slot <= 0 || slot >= p.num_slots) return;  // pass 3 writes the zeros
  const int nchunks = (len + kC - 1) / kC;
  const int64_t q0 = p.chunk_offsets[n];
  // records beyond the workspace: a table inconsistent with max_chunks
  if (q0 < 0 || q0 + nchunks > p.max_chunks) return;
  const int col = 16 * (split * kStateWaves + wave) + c;  // this lane's column
  const int64_t col0 = static_cast<int64_t>(h) * kD;

  float* st =
      p.rec_state + (static_cast<int64_t>(slot) * H + h) * (kD * kD) + col;
  f4 S[8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[kb][r] = st[(16 * kb + 4 * gq + r) * kD];

  // chunk ci's record into buffer ci % kBufs: 16 bytes per lane, spread
  // over the waves (wave w issues kDmaMin or more copy instructions)
  auto stage = [&](int ci) {
    const char* src = reinterpret_cast<const char*>(
        p.workspace + ((q0 + ci) * H + h) * kRecFloats);
    char* dst = reinterpret_cast<char*>(&rec[ci % kBufs][0]);
    for (int off = wave * 1024; off < kStageBytes;
         off += kStateWaves * 1024) {
      if (off + 16 * lane < kStageBytes)
        load_lds16(src + off + 16 * lane, dst + off);
    }
  };
  for (int i = 0; i < kBufs - 1 && i < nchunks; ++i) stage(i);
  wait_vmem();
  __syncthreads();

  for (int ci = 0; ci < nchunks; ++ci) {
    // the buffer of chunk ci + kBufs - 1 was last read in chunk ci - 1,
    // before the barrier that ended it
    if (ci + kBufs - 1 < nchunks) stage(ci + kBufs - 1);
    const float* R = rec[ci % kBufs];
    const int nv = len - ci * kC < kC ? len - ci * kC : kC;
    // K~ S and Q~ S for this wave's 16 columns
    f4 ks = {0.f, 0.f, 0.f, 0.f};
    f4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const f4 ak = ld4(&R[kRecKt + c * kLd + 16 * kb + 4 * gq]);
      const f4 aq = ld4(&R[kRecQt + c * kLd + 16 * kb + 4 * gq]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ks = mfma(ak[j], S[kb][j], ks);
        o = mfma(aq[j], S[kb][j], o);
      }
    }
    // Delta = T beta (V - K~ S);  O += B Delta
    const f4 at = ld4(&R[kRecT + c * kTd + 4 * gq]);
    const f4 ab = ld4(&R[kRecB + c * kTd + 4 * gq]);
    f4 br;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * gq + r;
      br[r] = R[kRecBeta + t] * (R[kRecV + t * kLd + col] - ks[r]);
    }
    f4 dl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) dl = mfma(at[j], br[j], dl);
#pragma unroll
    for (int j = 0; j < 4; ++j) o = mfma(ab[j], dl[j], o);
    // S <- e^{G_last} S + K^^T Delta; A operand K^[token 4gq + j][key
    // 16kb + c] (rows of K^, one dword per token)
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const f4 gm = ld4(&R[kRecGam + 16 * kb + 4 * gq]);
      f4 ah;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ah[j] = R[kRecKh + (4 * gq + j) * kLd + 16 * kb + c];
      S[kb] *= gm;
#pragma unroll
      for (int j = 0; j < 4; ++j) S[kb] = mfma(ah[j], dl[j], S[kb]);
    }
    // the next record is in LDS (this wave's part): with a younger record
    // in flight, vector memory loads return in order, so at most kDmaMin
    // outstanding operations means the older copies have all landed
    if (kBufs > 2 && ci + kBufs - 1 < nchunks)
      wait_vmcnt<kDmaMin>();
    else
      wait_vmem();
    __syncthreads();  // ... and every other wave's; this buffer is free
    // outputs before the norm into the record's O rows (valid tokens),
    // issued after the wait: vmcnt counts stores too, so stores issued
    // before it would hold every chunk until they are acknowledged
    float* O = p.workspace + ((q0 + ci) * H + h) * kRecFloats + kRecO + col;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * gq + r < nv) O[(4 * gq + r) * kD] = o[r];
  }

#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) st[(16 * kb + 4 * gq + r) * kD] = S[kb][r];
  // conv window: the last W-1 inputs of (stored window ++ tokens)
  if (split == 0 && (p.flags & KDA_NO_CONV_UPDATE) == 0) {
    const bool tap_major = (p.flags & KDA_CONV_TAP_MAJOR) != 0;
    for (int i = tid; i < 3 * kD; i += 64 * kStateWaves) {
      const int64_t ch = (i >> 7) * static_cast<int64_t>(C) + col0 + (i & 127);
      auto at = [&](int e) -> int64_t {
        return tap_major
                   ? (static_cast<int64_t>(slot) * (kW - 1) + e) * C3 + ch
                   : (static_cast<int64_t>(slot) * C3 + ch) * (kW - 1) + e;
      };
      uint16_t nwin[kW - 1];
#pragma unroll
      for (int e = 0; e < kW - 1; ++e) {
        const int idx = len - (kW - 1) + e;
        nwin[e] = idx >= 0
                      ? p.qkv[(static_cast<int64_t>(tb) + idx) * C3 + ch]
                      : p.conv_state[at(e + len)];
      }
#pragma unroll
      for (int e = 0; e < kW - 1; ++e) p.conv_state[at(e)] = nwin[e];
    }
  }
}

// ---- pass 3 -----------------------------------------------------------------

template <bool kNorm>
__global__ __launch_bounds__(kThreads) void kda_chunk_out_kernel(
    KdaPassArgs p) {
  const int tid = threadIdx.x;
  const int H = p.heads;
  const int C = H * kD;
  const int64_t q = blockIdx.x / H;
  const int h = static_cast<int>(blockIdx.x % H);
  const int64_t total = p.chunk_offsets[p.num_seqs];
  if (q >= total || q >= p.max_chunks) return;
  const int n = p.chunk_indices[2 * q];
  const int ci = p.chunk_indices[2 * q + 1];
  if (n < 0 || n >= p.num_seqs || ci < 0) return;
  int32_t tb;
  int len;
  if (!seq_range(p, n, tb, len) || ci * kC >= len) return;
  // the state pass skipped this sequence: leave its outputs alone
  const int64_t q0 = p.chunk_offsets[n];
  if (q0 < 0 || q0 + (len + kC - 1) / kC > p.max_chunks) return;
  const int nv = len - ci * kC < kC ? len - ci * kC : kC;
  const int ot = tid >> 4;        // token of the chunk
  const int oc = 8 * (tid & 15);  // and 8 of its columns
  const int64_t col0 = static_cast<int64_t>(h) * kD;
  u4* dst = reinterpret_cast<u4*>(
      p.out + (tb + static_cast<int64_t>(ci) * kC + ot) * C + col0 + oc);
  const int32_t slot = p.state_idx[n];
  if (slot <= 0 || slot >= p.num_slots) {  // null row: +0.0
    if (ot < nv) *dst = u4{0u, 0u, 0u, 0u};
    return;
  }
  const float* O =
      p.workspace + (q * H + h) * kRecFloats + kRecO + ot * kD + oc;
  // rows past the end of the sequence read the last valid row (not stored)
  const int rr = ot < nv ? 0 : (nv - 1 - ot) * kD;
  const f4 v0 = ld4(O + rr);
  const f4 v1 = ld4(O + rr + 4);
  float yv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  if (kNorm) {
    const bool gate_silu = (p.flags & KDA_GATE_SILU) != 0;
    const int tr = ot < nv ? ot : nv - 1;
    const u4 gate_raw = *reinterpret_cast<const u4*>(
        p.gate + (tb + static_cast<int64_t>(ci) * kC + tr) * C + col0 + oc);
    const f4 w0 = ld4(p.norm_w + oc);
    const f4 w1 = ld4(p.norm_w + oc + 4);
    const float nw[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += yv[j] * yv[j];
    ss = row_sum16(ss);
    const float rs = rsqrtf(ss * (1.0f / kD) + p.eps);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w2 = gate_raw[j >> 1];
      const float gv = (j & 1) ? bf16_hi(w2) : bf16_lo(w2);
      const float ga = gate_silu ? gv * sigmoid_(gv) : sigmoid_(gv);
      yv[j] = ((yv[j] * rs) * nw[j]) * ga;
    }
  }
  if (ot < nv)
    *dst = u4{pack_bf16(yv[0], yv[1]), pack_bf16(yv[2], yv[3]),
              pack_bf16(yv[4], yv[5]), pack_bf16(yv[6], yv[7])};
}

}  // namespace

uint64_t kda_pass_record_bytes() {
  return static_cast<uint64_t>(kRecFloats) * sizeof(float);
}

namespace {
constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
void* g_scratch_ptr[kScratchDevices];
}  // namespace

void* kda_pass_static_scratch(int dev) {
  if (dev < 0 || dev >= kScratchDevices) return nullptr;
  // once per device, with that device current (the caller's)
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess)
      g_scratch_ptr[dev] = ptr;
  });
  return g_scratch_ptr[dev];
}

hipError_t kda_chunk_pass_launch(const KdaPassArgs& args, hipStream_t stream) {
  const unsigned chunk_blocks =
      static_cast<unsigned>(args.max_chunks * args.heads);
  if (chunk_blocks > 0)
    hipLaunchKernelGGL(kda_chunk_prep_kernel, dim3(chunk_blocks),
                       dim3(kThreads), 0, stream, args);
  const int64_t units = static_cast<int64_t>(args.num_seqs) * args.heads;
  const dim3 grid(static_cast<unsigned>((units + 7) / 8 * 8 * kSplits));
  hipLaunchKernelGGL(kda_chunk_state_kernel, grid, dim3(64 * kStateWaves), 0,
                     stream, args);
  if (chunk_blocks > 0) {
    if (args.flags & KDA_OUTPUT_NORM)
      hipLaunchKernelGGL(kda_chunk_out_kernel<true>, dim3(chunk_blocks),
                         dim3(kThreads), 0, stream, args);
    else
      hipLaunchKernelGGL(kda_chunk_out_kernel<false>, dim3(chunk_blocks),
                         dim3(kThreads), 0, stream, args);
  }
  return hipGetLastError();
}
