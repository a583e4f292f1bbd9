// Chunked variable-length KDA prefill on gfx950 matrix cores (MFMA).
//
// Operation: the prefill of the page "PR #51862 完整报告 -- Remove prefill
// pipeline stall in chunk KDA" -- every sequence of a variable-length batch
// runs the gated delta-rule step of the page "PR #50654 完整报告 --
// [ROCm][Perf] Kimi-K3 Fused kernel for KDA decode" over its tokens in
// order, from the state in its slot.  The result equals the token-by-token
// recurrence up to rounding (include/kda_decode.h states it); only the
// order of the arithmetic changes.
//
// Chunk form (16 tokens; derived from the recurrence, the page gives only
// the chunk bookkeeping).  Per key channel i let G_t = g_1 + ... + g_t
// inside the chunk and S the state before it.  Then
//   u_t  = S^T (k_t e^{G_t}) + sum_{s<t} A_ts delta_s,
//   A_ts = sum_i k_t[i] k_s[i] e^{G_t[i] - G_s[i]},
// so the deltas solve (I + diag(beta) A) Delta = diag(beta) (V - K~ S)
// with K~ = K e^{G}; the outputs are O = Q~ S + B Delta with
//   B_ts = sum_i q_t[i] k_s[i] e^{G_t[i] - G_s[i]}  (s <= t),
// and the state after the chunk is e^{G_last} S + K^^T Delta with
// K^_s = k_s e^{G_last - G_s}.  Every factor applied to S, K~, Q~, K^ is
// at most 1 for non-positive g.  A and B are formed as K~ (K e^{-G})^T and
// Q~ (K e^{-G})^T on the matrix cores when every |G| in the chunk is at
// most 80 (e^{+-80} stays a normal fp32 number); otherwise each entry is
// summed with its own exponential, which is exact for any decay.
//
// Mapping: one 512-thread workgroup (8 waves) per (sequence, head), in two
// roles that share each SIMD (waves w and w + 4 run on SIMD w):
//   * state waves 0-3 own value columns 32w .. 32w+31 of the [128 key,
//     128 value] fp32 state, held for the whole sequence in registers in
//     the accumulator layout of v_mfma_f32_16x16x4_f32 (lane l: column
//     l%16, key rows 4(l/16) .. +3 of each 16-row block).  That layout is
//     also the B operand of the next product once the summation index is
//     permuted (key 16kb + 4(l/16) + j in step j), so the state never
//     leaves the registers.  Per chunk and wave: 64 MFMAs for K~ S, 64 for
//     Q~ S, 16 for the triangular solve and B Delta, 64 for the state
//     update; every lane also solves for the row of the 16 x 16 inverse
//     T = (I + diag(beta) A)^{-1} its operand needs, by backward
//     substitution, in the shadow of its matrix products.
//   * prep waves 4-7 build the next chunk's operands meanwhile (4 tokens
//     each): causal conv + SiLU from the raw bf16 inputs, q/k L2
//     normalisation (wave-local: a wave holds all channels of its tokens),
//     the cumulative decay, the decayed tables K~, Q~, K^, K e^{-G}, and
//     then the A / B products on the matrix cores.
// The tables are double-buffered in LDS; three barriers per chunk hand
// them over.  The state waves also write the gated-RMSNorm outputs, one
// 16-byte store per lane.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kda_chunked.h"
#include "kda_decode.h"

namespace {

constexpr int kD = 128;      // head dim (key = value)
constexpr int kW = 4;        // conv width
constexpr int kC = 16;       // tokens per chunk (one MFMA row block)
constexpr int kThreads = 512;
constexpr int kLd = kD + 4;  // padded row of [kC][kD] tables (floats)
constexpr int kTd = kC + 4;  // padded row of [kD][kC] and [kC][kC] tables
constexpr float kLog2e = 1.44269504088896341f;
// |G| <= 80 (natural log units): e^{+-80} is a normal fp32 number
constexpr float kSafeExp2 = 80.0f * kLog2e;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Operands of one chunk for the state waves (double-buffered).
struct ChunkTables {
  float qt[kC][kLd];    // q_t e^{G_t}
  float kt[kC][kLd];    // k_t e^{G_t}
  float v[kC][kLd];     // v_t
  float khT[kD][kTd];   // k_t e^{G_last - G_t}, as [key][token]
  float gam[kD];        // e^{G_last}
  float beta[kC];
};

struct alignas(16) Smem {
  ChunkTables tab[2];
  float ki[kC][kLd];    // k_t e^{-G_t}; raw k on the exact path
  float qraw[kC][kLd];  // exact path: q_t
  float graw[kC][kLd];  // exact path: cumulative log2 decay
  float part[4][kC][kC];  // A (keys 0-63, 64-127), B (same)
  float LT[kC][kTd];    // LT[s][t] = beta_t A_ts for s < t, else 0
  float B[kC][kTd];     // B_ts for s <= t, else 0
  float o[kC][kLd];     // this chunk's outputs before the norm
  float cw[3][kW][kD];  // this head's conv weights
  float cb[3][kD];      // raw gates: conv bias (zeros without one)
  float dtb[kD];        // raw gates: this head's dt_bias
  float nw[kD];         // norm weight
  uint32_t win[3][kW - 1][kD / 2];  // stored conv window, channel pairs
  // raw inputs of the next chunk, copied in by the prep waves' LDS-direct
  // loads: per prep wave its 7 input rows (3 parts, channel pairs), the
  // chunk's 16 rows of g and its 16 betas
  // (g and beta are read by every prep wave: two buffers by chunk parity;
  // raw gates fill the first half of each g row with bf16 pairs)
  uint32_t stage[4][7][3][kD / 2];
  float gst[2][kC][kD];
  float bst[2][64];
  int unsafe;           // exact path for the chunk being prepared
};

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
// 2^x on the transcendental unit (v_exp_f32)
__device__ __forceinline__ float exp2_(float x) {
  return __builtin_amdgcn_exp2f(x);
}
__device__ __forceinline__ float sigmoid_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
// Sum over each row of 16 lanes (quad_perm [1,0,3,2], [2,3,0,1],
// row_half_mirror, row_mirror), in every lane of the row.
template <int kCtrl>
__device__ __forceinline__ float dpp_(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                         0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_<0xB1>(v);
  v += dpp_<0x4E>(v);
  v += dpp_<0x141>(v);
  v += dpp_<0x140>(v);
  return v;
}
// Global-memory pointers (address space 1).
template <typename T>
using gptr = __attribute__((address_space(1))) T*;
// A wave-uniform global pointer made opaque to the compiler (readfirstlane
// of both halves): loads become a scalar base plus a 32-bit lane offset
// instead of a 64-bit address per lane.
template <typename T>
__device__ __forceinline__ gptr<const T> uniform_gptr(const T* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<gptr<const T>>((static_cast<uint64_t>(hi) << 32) |
                                         lo);
}
// *(U*)(base + byte_off)
template <typename U, typename T>
__device__ __forceinline__ U load_at(gptr<const T> base, uint32_t byte_off) {
  return *reinterpret_cast<gptr<const U>>(
      reinterpret_cast<__attribute__((address_space(1))) const char*>(base) +
      byte_off);
}

// One dword per lane from global memory straight into LDS: lane l's value
// lands at dst[l] (dst wave-uniform).  Counted by vmcnt.
__device__ __forceinline__ void load_lds(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}
// s_waitcnt fields (gfx9 encoding): vmcnt 0 with the others at maximum,
// and lgkmcnt 0 with the others at maximum
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Eight wave sums side by side (independent DPP chains), each result in
// every lane.
__device__ __forceinline__ void wave_sum8(float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] += dpp_<0xB1>(v[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] += dpp_<0x4E>(v[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] += dpp_<0x141>(v[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] += dpp_<0x140>(v[i]);
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

// Gate operands of a launch: activated g and beta, or the raw inputs with
// the default (softplus) or the bounded gate.
enum GateForm { kGateInput = 0, kGateSoftplus = 1, kGateBounded = 2 };

template <bool kNorm, int kGate>
__global__ __launch_bounds__(kThreads) void kda_chunked_prefill_kernel(
    KdaChunkedArgs p) {
  constexpr bool kRaw = kGate != kGateInput;
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  // wave index in a scalar register: role tests and role-derived offsets
  // stay on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c = lane & 15;   // MFMA column / A-operand row
  const int gq = lane >> 4;  // MFMA row group
  const int H = p.heads;
  const int C = H * kD;
  const int C3 = 3 * C;
  const int n = static_cast<int>(blockIdx.x) / H;
  const int h = static_cast<int>(blockIdx.x) % H;
  // token offsets in 64 bits: tb * 3C passes 2^31 from 58,255 tokens at
  // 96 heads
  const int64_t tb = p.cu_seqlens ? p.cu_seqlens[n] : n * p.tokens_per_row;
  const int64_t te =
      p.cu_seqlens ? p.cu_seqlens[n + 1] : (n + 1) * p.tokens_per_row;
  const int len = te > tb ? static_cast<int>(te - tb) : 0;
  if (len == 0) return;
  const int32_t slot = p.state_idx[n];
  const int64_t col0 = static_cast<int64_t>(h) * kD;
  if (slot <= 0 || slot >= p.num_slots) {
    // null slot: +0.0 outputs, no state traffic
    uint32_t* o32 = reinterpret_cast<uint32_t*>(p.out);
    for (int64_t idx = tid; idx < static_cast<int64_t>(len) * (kD / 2);
         idx += kThreads) {
      const int64_t t = idx / (kD / 2);
      o32[((tb + t) * C + col0) / 2 + idx % (kD / 2)] = 0u;
    }
    return;
  }
  const uint32_t flags = p.flags;
  const bool tap_major = (flags & KDA_CONV_TAP_MAJOR) != 0;
  const bool conv_update = (flags & KDA_NO_CONV_UPDATE) == 0;
  const bool l2 = (flags & KDA_QK_L2NORM) != 0;
  const bool gate_silu = (flags & KDA_GATE_SILU) != 0;
  const int nchunks = (len + kC - 1) / kC;
  const bool state_wave = wave < 4;
  const int pw = wave & 3;  // index within the role

  // ---- per-sequence set-up ----------------------------------------------
  // state waves: the wave's 32 columns of the state, 2 blocks of 16
  float* st = p.rec_state + (static_cast<int64_t>(slot) * H + h) * (kD * kD) +
              32 * pw + c;
  f4 S[2][8];
  // output lanes: token tid/16 (of the 16), columns 8 (tid%16) .. +7
  const int ot = (tid & 255) >> 4;
  const int oc = 8 * (tid & 15);
  if (state_wave) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[cb][kb][r] = st[(16 * kb + 4 * gq + r) * kD + 16 * cb];
  } else {
    // conv weights and the norm weight of this head into LDS
    const int i = tid - 256;  // 0..255
    for (int e = i; e < 3 * kW * kD; e += 256) {
      const int pp = e / (kW * kD), t = (e / kD) % kW, k = e % kD;
      sm.cw[pp][t][k] =
          p.conv_w[(static_cast<int64_t>(pp) * kW + t) * C + col0 + k];
    }
    if (i < kD) sm.nw[i] = kNorm ? p.norm_w[i] : 0.0f;
    if (kRaw) {
      for (int e = i; e < 3 * kD; e += 256)
        sm.cb[e / kD][e % kD] =
            p.rg.conv_bias
                ? p.rg.conv_bias[(e / kD) * static_cast<int64_t>(C) + col0 +
                                 e % kD]
                : 0.0f;
      if (i < kD) sm.dtb[i] = p.rg.dt_bias[col0 + i];
    }
    // the stored window of channels 2 lane, 2 lane + 1 of each part
    if (i < kD / 2) {
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
#pragma unroll
        for (int e = 0; e < kW - 1; ++e) {
          const int64_t ch = static_cast<int64_t>(pp) * C + col0 + 2 * i;
          uint32_t wv;
          if (tap_major) {
            wv = *reinterpret_cast<const uint32_t*>(
                p.conv_state +
                (static_cast<int64_t>(slot) * (kW - 1) + e) * C3 + ch);
          } else {
            const uint16_t* cs = p.conv_state +
                                 (static_cast<int64_t>(slot) * C3 + ch) *
                                     (kW - 1) + e;
            wv = static_cast<uint32_t>(cs[0]) |
                 (static_cast<uint32_t>(cs[kW - 1]) << 16);
          }
          sm.win[pp][e][i] = wv;
        }
    }
  }

  // ---- prep stage 1 of chunk ci: conv, norms, decay, tables (wave-local)
  // Requests chunk ci's raw inputs into the staging buffers (prep waves):
  // wave pw the input rows of tokens 4pw-3 .. 4pw+3 (chunk-relative; rows
  // before the sequence or past its end are clamped to valid rows and
  // replaced or masked where used), rows 4pw .. 4pw+3 of g, and (wave 0)
  // the betas.  The loads land while the wave works on the current chunk.
  uint32_t rbeta = 0;  // raw gates: bf16 beta of token 4pw + lane (lane < 4)
  auto stage_chunk = [&](int ci) {
    const int c0 = ci * kC;
    const int nv = len - c0 < kC ? len - c0 : kC;
    const int64_t tok0 = tb + c0;
#pragma unroll
    for (int u = 0; u < 7; ++u) {
      const int rel = 4 * pw - 3 + u;
      const int rr =
          rel < 0 ? (ci > 0 ? rel : 0) : (rel < nv - 1 ? rel : nv - 1);
      const uint16_t* row = p.qkv + (tok0 + rr) * C3 + col0 + 2 * lane;
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
        load_lds(row + pp * C, &sm.stage[pw][u][pp][0]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = 4 * pw + u;
      const int rr = t < nv - 1 ? t : nv - 1;
      if (kRaw) {
        load_lds(p.rg.raw_g + ((tok0 + rr) * H + h) * kD + 2 * lane,
                 &sm.gst[ci & 1][t][0]);
      } else {
        const float* row = p.g + ((tok0 + rr) * H + h) * kD + lane;
        load_lds(row, &sm.gst[ci & 1][t][0]);
        load_lds(row + 64, &sm.gst[ci & 1][t][64]);
      }
    }
    if (kRaw) {
      if (lane < 4) {
        const int t = 4 * pw + lane;
        const int rr = t < nv - 1 ? t : nv - 1;
        rbeta = p.rg.raw_beta[(tok0 + rr) * H + h];
      }
    } else if (pw == 0) {
      const int rr = lane < nv - 1 ? lane : nv - 1;
      load_lds(p.beta + (tok0 + rr) * H + h, &sm.bst[ci & 1][0]);
    }
  };

  // Raw gates: once its own requests for chunk cj have landed, prep wave pw
  // turns its 4 staged g rows (bf16 pairs of raw_g, keys 2 lane, 2 lane + 1
  // in dword lane) into log2-unit decays in place, and its 4 betas into
  // bst.  Each wave activates a quarter of the chunk; the barrier that
  // follows publishes the rows to the other prep waves.
  auto activate = [&](int cj) {
    if (!kRaw || cj >= nchunks) return;
    const f2 db = *reinterpret_cast<const f2*>(&sm.dtb[2 * lane]);
    const float a_rate = __expf(p.rg.A_log[h]);
    const float lb2 = p.rg.lower_bound * kLog2e;
    float(*rows)[kD] = sm.gst[cj & 1];
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      w[u] = reinterpret_cast<const uint32_t*>(&rows[4 * pw + u][0])[lane];
    // every lane's read is done before any lane's write lands over it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    constexpr bool kB = kGate == kGateBounded;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<f2*>(&rows[4 * pw + u][2 * lane]) =
          f2{kda_gate2_from_raw<kB>(bf16_lo(w[u]) + db.x, a_rate, lb2),
             kda_gate2_from_raw<kB>(bf16_hi(w[u]) + db.y, a_rate, lb2)};
    if (lane < 4) sm.bst[cj & 1][4 * pw + lane] = sigmoid_(bf16_lo(rbeta));
  };

  auto prep_tables = [&](int ci) {
    ChunkTables& T = sm.tab[ci & 1];
    const int c0 = ci * kC;
    const int nv = len - c0 < kC ? len - c0 : kC;
    // raw[pp][u]: input of token 4pw - 3 + u (chunk-relative) for channels
    // 2 lane, 2 lane + 1 of part pp (staged during the previous chunk)
    uint32_t raw[3][7];
#pragma unroll
    for (int u = 0; u < 7; ++u)
#pragma unroll
      for (int pp = 0; pp < 3; ++pp) raw[pp][u] = sm.stage[pw][u][pp][lane];
    // per-token decays of keys 2 lane, 2 lane + 1 in log2 units (raw
    // gates: activated in place by activate())
    f2 gl[kC];
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      gl[t] = *reinterpret_cast<const f2*>(&sm.gst[ci & 1][t][2 * lane]);
      if (!kRaw) gl[t] *= kLog2e;
      gl[t] = kda_decay_floor2(gl[t]);
    }
    const float bt = lane < 4 ? sm.bst[ci & 1][4 * pw + lane] : 0.0f;
    // the staging buffers are free again: request the next chunk
    wait_lds();
    if (ci + 1 < nchunks) stage_chunk(ci + 1);
    uint32_t wv[3][kW - 1];
#pragma unroll
    for (int pp = 0; pp < 3; ++pp)
#pragma unroll
      for (int e = 0; e < kW - 1; ++e) wv[pp][e] = sm.win[pp][e][lane];
    // cumulative decay of keys 2 lane, 2 lane + 1 (log2 units) over the
    // whole chunk; the values at this wave's 4 tokens and at the end
    f2 Gu[4] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
    f2 G = {0.f, 0.f};
    float gmax = 0.0f;
    {
      // in groups of the 4 tokens a wave owns: the wave keeps its own
      // group's prefixes under a wave-uniform branch (no per-token select)
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
    }
    // NaN counts as unsafe; the same verdict in every prep wave
    const bool unsafe = __any(!(gmax <= kSafeExp2));
    const float qscale = 0.08838834764831845f;  // D^-1/2
    // conv + SiLU of the 4 tokens (weights read once), then the 8 norm
    // reductions side by side, then the tables
    f2 cwv[3][kW];
    f2 cbv[3] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
    for (int pp = 0; pp < 3; ++pp) {
#pragma unroll
      for (int tap = 0; tap < kW; ++tap)
        cwv[pp][tap] = *reinterpret_cast<const f2*>(&sm.cw[pp][tap][2 * lane]);
      if (kRaw) cbv[pp] = *reinterpret_cast<const f2*>(&sm.cb[pp][2 * lane]);
    }
    float y[4][3][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool valid = 4 * pw + u < nv;
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float a = cbv[pp][e];
#pragma unroll
          for (int tap = 0; tap < kW; ++tap) {
            // with the update a token sees the inputs before it (the stored
            // window before the sequence); without it, the stored window
            const int rin = 4 * pw + u - (kW - 1) + tap;
            const uint32_t w2 =
                tap == kW - 1 ? raw[pp][u + tap]
                : conv_update ? (rin < 0 && ci == 0 ? wv[pp][(kW - 1) + rin]
                                                    : raw[pp][u + tap])
                              : wv[pp][tap];
            a += cwv[pp][tap][e] * (e ? bf16_hi(w2) : bf16_lo(w2));
          }
          y[u][pp][e] = valid ? a * sigmoid_(a) : 0.0f;
        }
    }
    if (l2) {
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
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = 4 * pw + u;
      const f2 ee = {exp2_(Gu[u].x), exp2_(Gu[u].y)};
      *reinterpret_cast<f2*>(&T.qt[t][2 * lane]) =
          f2{y[u][0][0] * ee.x, y[u][0][1] * ee.y};
      *reinterpret_cast<f2*>(&T.kt[t][2 * lane]) =
          f2{y[u][1][0] * ee.x, y[u][1][1] * ee.y};
      *reinterpret_cast<f2*>(&T.v[t][2 * lane]) = f2{y[u][2][0], y[u][2][1]};
      T.khT[2 * lane][t] = y[u][1][0] * exp2_(G.x - Gu[u].x);
      T.khT[2 * lane + 1][t] = y[u][1][1] * exp2_(G.y - Gu[u].y);
      if (!unsafe) {
        *reinterpret_cast<f2*>(&sm.ki[t][2 * lane]) =
            f2{y[u][1][0] * exp2_(-Gu[u].x), y[u][1][1] * exp2_(-Gu[u].y)};
      } else {
        *reinterpret_cast<f2*>(&sm.ki[t][2 * lane]) =
            f2{y[u][1][0], y[u][1][1]};
        *reinterpret_cast<f2*>(&sm.qraw[t][2 * lane]) =
            f2{y[u][0][0], y[u][0][1]};
        *reinterpret_cast<f2*>(&sm.graw[t][2 * lane]) = Gu[u];
      }
    }
    if (pw == 0) {
      *reinterpret_cast<f2*>(&T.gam[2 * lane]) = f2{exp2_(G.x), exp2_(G.y)};
      if (lane == 0) sm.unsafe = unsafe ? 1 : 0;
    }
    if (lane < 4) {
      const int t = 4 * pw + lane;
      T.beta[t] = t < nv ? bt : 0.0f;
    }
  };

  // ---- prep stage 2: A / B products (or the exact per-entry sums) -------
  auto prep_gram = [&](int ci) {
    const ChunkTables& T = sm.tab[ci & 1];
    if (!sm.unsafe) {
      // wave 4: A over keys 0-63, 5: A over 64-127, 6 / 7: B likewise
      const float(*src)[kLd] = pw < 2 ? T.kt : T.qt;
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
    } else {
      // large decay: one exponential per (t, s, key)
      const int t = (tid & 255) >> 4;
      const int s = tid & 15;
      float a = 0.0f, b = 0.0f;
      if (s <= t) {
        for (int i = 0; i < kD; ++i) {
          const float ks = sm.ki[s][i] * exp2_(sm.graw[t][i] - sm.graw[s][i]);
          a += sm.ki[t][i] * ks;
          b += sm.qraw[t][i] * ks;
        }
      }
      sm.LT[s][t] = s < t ? T.beta[t] * a : 0.0f;
      sm.B[t][s] = b;
    }
  };

  // ---- prep stage 3: sum the partial products, mask, scale by beta ------
  auto prep_reduce = [&](int ci) {
    if (sm.unsafe) return;
    const ChunkTables& T = sm.tab[ci & 1];
    const int t = (tid & 255) >> 4;
    const int s = tid & 15;
    const float a = sm.part[0][t][s] + sm.part[1][t][s];
    const float b = sm.part[2][t][s] + sm.part[3][t][s];
    sm.LT[s][t] = s < t ? T.beta[t] * a : 0.0f;
    sm.B[t][s] = s <= t ? b : 0.0f;
  };

  // ---- state stage: one chunk through the recurrence ---------------------
  auto state_chunk = [&](int ci) {
    const ChunkTables& T = sm.tab[ci & 1];
    f4 ks[2], o[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      ks[cb] = f4{0.f, 0.f, 0.f, 0.f};
      o[cb] = f4{0.f, 0.f, 0.f, 0.f};
    }
    // operands one key block ahead; the scheduling fence keeps the
    // compiler from hoisting all of them (register pressure)
    f4 ak = ld4(&T.kt[c][4 * gq]);
    f4 aq = ld4(&T.qt[c][4 * gq]);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      f4 akn = ak, aqn = aq;
      if (kb < 7) {
        akn = ld4(&T.kt[c][16 * kb + 16 + 4 * gq]);
        aqn = ld4(&T.qt[c][16 * kb + 16 + 4 * gq]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          ks[cb] = mfma(ak[j], S[cb][kb][j], ks[cb]);
          o[cb] = mfma(aq[j], S[cb][kb][j], o[cb]);
        }
      ak = akn;
      aq = aqn;
      __builtin_amdgcn_sched_barrier(0);
    }
    // row c of T: (I + L)^T y = e_c, backward
    float y[kC];
#pragma unroll
    for (int t = kC - 1; t >= 0; --t) {
      float v = t == c ? 1.0f : 0.0f;
#pragma unroll
      for (int s4 = 0; s4 < kC; s4 += 4) {
        if (s4 + 3 <= t) continue;  // all of s4 .. s4+3 <= t
        const f4 lt = ld4(&sm.LT[t][s4]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (s4 + u > t) v -= lt[u] * y[s4 + u];
      }
      y[t] = v;
    }
    f4 at;  // T[c][4gq + j]
#pragma unroll
    for (int j = 0; j < 4; ++j)
      at[j] = gq == 0 ? y[j] : gq == 1 ? y[4 + j] : gq == 2 ? y[8 + j]
                                                           : y[12 + j];
    const f4 ab = ld4(&sm.B[c][4 * gq]);
    f4 dl[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int col = 32 * pw + 16 * cb + c;
      f4 br;  // beta (V - K~ S) in the accumulator layout
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * gq + r;
        br[r] = T.beta[t] * (T.v[t][col] - ks[cb][r]);
      }
      dl[cb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) dl[cb] = mfma(at[j], br[j], dl[cb]);
#pragma unroll
      for (int j = 0; j < 4; ++j) o[cb] = mfma(ab[j], dl[cb][j], o[cb]);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.o[4 * gq + r][col] = o[cb][r];
    }
    f4 gm = ld4(&T.gam[4 * gq]);
    f4 ah = ld4(&T.khT[c][4 * gq]);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      f4 gmn = gm, ahn = ah;
      if (kb < 7) {
        gmn = ld4(&T.gam[16 * kb + 16 + 4 * gq]);
        ahn = ld4(&T.khT[16 * kb + 16 + c][4 * gq]);
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        S[cb][kb] *= gm;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          S[cb][kb] = mfma(ah[j], dl[cb][j], S[cb][kb]);
      }
      gm = gmn;
      ah = ahn;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- state stage: gated RMSNorm and bf16 outputs of a chunk ------------
  auto emit = [&](int ci, u4 gate_raw) {
    const int c0 = ci * kC;
    const int nv = len - c0 < kC ? len - c0 : kC;
    const f4 v0 = ld4(&sm.o[ot][oc]);
    const f4 v1 = ld4(&sm.o[ot][oc + 4]);
    float yv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    if (kNorm) {
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += yv[j] * yv[j];
      ss = row_sum16(ss);  // the 16 lanes of token ot
      const float rs = rsqrtf(ss * (1.0f / kD) + p.eps);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w2 = gate_raw[j >> 1];
        const float gv = (j & 1) ? bf16_hi(w2) : bf16_lo(w2);
        const float ga = gate_silu ? gv * sigmoid_(gv) : sigmoid_(gv);
        yv[j] = ((yv[j] * rs) * sm.nw[oc + j]) * ga;
      }
    }
    if (ot < nv) {
      const u4 pk = {pack_bf16(yv[0], yv[1]), pack_bf16(yv[2], yv[3]),
                     pack_bf16(yv[4], yv[5]), pack_bf16(yv[6], yv[7])};
      *reinterpret_cast<u4*>(p.out + (tb + c0 + ot) * C + col0 + oc) = pk;
    }
  };

  // ---- the pipeline --------------------------------------------------------
  if (!state_wave) {
    stage_chunk(0);
    wait_vmem();
  }
  __syncthreads();  // conv and norm weights, the first chunk's inputs
  if (kRaw) {       // (activate reads the dt_bias row written above)
    if (!state_wave) activate(0);
    __syncthreads();
  }
  if (!state_wave) prep_tables(0);
  __syncthreads();
  if (!state_wave) prep_gram(0);
  __syncthreads();
  if (!state_wave) {
    prep_reduce(0);
    wait_vmem();
    activate(1);
  }
  __syncthreads();
  for (int ci = 0; ci < nchunks; ++ci) {
    const bool more = ci + 1 < nchunks;
    u4 gate_raw = {0u, 0u, 0u, 0u};
    if (state_wave) {
      if (kNorm) {
        const int nv = len - ci * kC < kC ? len - ci * kC : kC;
        const int rr = ot < nv - 1 ? ot : nv - 1;
        gate_raw = *reinterpret_cast<const u4*>(
            p.gate + (tb + ci * kC + rr) * C + col0 + oc);
      }
      state_chunk(ci);
    } else if (more) {
      prep_tables(ci + 1);
    }
    __syncthreads();
    if (state_wave)
      emit(ci, gate_raw);
    else if (more)
      prep_gram(ci + 1);
    __syncthreads();
    if (!state_wave && more) prep_reduce(ci + 1);
    if (!state_wave) {
      wait_vmem();  // the staged inputs of the chunk after the next
      activate(ci + 2);
    }
    __syncthreads();
  }

  // ---- write back the state and the conv window ---------------------------
  if (state_wave) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          st[(16 * kb + 4 * gq + r) * kD + 16 * cb] = S[cb][kb][r];
  }
  if (conv_update && tid < 3 * kD) {
    // new window = the last W-1 inputs of (stored window ++ tokens)
    const int64_t ch =
        (tid >> 7) * static_cast<int64_t>(C) + col0 + (tid & 127);
    auto at = [&](int e) -> int64_t {
      return tap_major ? (static_cast<int64_t>(slot) * (kW - 1) + e) * C3 + ch
                       : (static_cast<int64_t>(slot) * C3 + ch) * (kW - 1) + e;
    };
    uint16_t nwin[kW - 1];
#pragma unroll
    for (int e = 0; e < kW - 1; ++e) {
      const int idx = len - (kW - 1) + e;  // token index in the sequence
      nwin[e] = idx >= 0 ? p.qkv[(tb + idx) * C3 + ch]
                         : p.conv_state[at(e + len)];
    }
#pragma unroll
    for (int e = 0; e < kW - 1; ++e) p.conv_state[at(e)] = nwin[e];
  }
}

template <int kGate>
void launch_gate(const KdaChunkedArgs& args, dim3 grid, hipStream_t stream) {
  if (args.flags & KDA_OUTPUT_NORM)
    hipLaunchKernelGGL((kda_chunked_prefill_kernel<true, kGate>), grid,
                       dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((kda_chunked_prefill_kernel<false, kGate>), grid,
                       dim3(kThreads), 0, stream, args);
}

}  // namespace

hipError_t kda_chunked_prefill_launch(const KdaChunkedArgs& args,
                                      int32_t num_seqs, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(num_seqs * args.heads));
  if (!args.rg.raw_g)
    launch_gate<kGateInput>(args, grid, stream);
  else if (args.flags & KDA_BOUNDED_GATE)
    launch_gate<kGateBounded>(args, grid, stream);
  else
    launch_gate<kGateSoftplus>(args, grid, stream);
  return hipGetLastError();
}
