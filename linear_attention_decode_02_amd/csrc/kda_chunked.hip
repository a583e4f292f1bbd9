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
// Mapping.  One 512-thread workgroup (8 waves) per (sequence, head).  Wave
// w owns value columns 16w .. 16w+15 of the [128 key, 128 value] fp32 state,
// held for the whole sequence in registers in the accumulator layout of
// v_mfma_f32_16x16x4_f32 (lane l: column l%16, key rows 4(l/16) .. +3 of
// each 16-row block).  That layout is also the B operand of the next
// product once the summation index is permuted (key 16kb + 4(l/16) + j in
// step j), so the state never leaves the registers between chunks.  The
// other operands (K~, Q~, K^, T, B) are staged in LDS.  Per chunk and
// wave: 32 MFMAs for K~ S, 32 for Q~ S, 32 for the state update, 8 for the
// partial A or B products, 8 for the triangular solve and B Delta.  The
// unit lower-triangular inverse T = (I + diag(beta) A)^{-1} (16 x 16) is one
// column per lane of wave 0 by forward substitution.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kda_chunked.h"
#include "kda_decode.h"

namespace {

constexpr int kD = 128;      // head dim (key = value)
constexpr int kW = 4;        // conv width
constexpr int kC = 16;       // tokens per chunk (one MFMA row block)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLd = kD + 4;  // padded row of [kC][kD] tables (floats)
constexpr int kTd = kC + 4;  // padded row of [kD][kC] and [kC][kC] tables
constexpr float kLog2e = 1.44269504088896341f;
// |G| <= 80 (natural log units): e^{+-80} is a normal fp32 number
constexpr float kSafeExp2 = 80.0f * kLog2e;
static_assert(kWaves * 16 == kD, "one 16-column block per wave");
static_assert(3 * kD + kD == kThreads, "conv and gate threads");

typedef float f4 __attribute__((ext_vector_type(4)));

struct alignas(16) Smem {
  float x[3][kC][kLd];        // conv outputs q, k, v (q, k normalised)
  float G[kC][kLd];           // cumulative log2 decay inside the chunk
  float qt[kC][kLd];          // q_t e^{G_t}
  float kt[kC][kLd];          // k_t e^{G_t}
  float ki[kC][kLd];          // k_t e^{-G_t}
  float khT[kD][kTd];         // k_t e^{G_last - G_t}, as [key][token]
  float part[kWaves][kC][kC]; // partial A (waves 0-3) and B (4-7) products
  float L[kC][kTd];           // beta_t A_ts for s < t, else 0
  float B[kC][kTd];           // B_ts for s <= t, else 0
  float T[kC][kTd];           // (I + L)^{-1}
  float gam[kD];              // e^{G_last}
  float beta[kC];
  float red[kWaves][kC];      // per-wave output sums of squares
  int unsafe[2];              // |G| > kSafeExp seen by gate wave 6 / 7
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  return __builtin_bit_cast(unsigned short, (__bf16)v);  // RNE
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
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  const int b = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
}
__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 ld4(const float* p) {
  return *reinterpret_cast<const f4*>(p);
}

template <bool kNorm>
__global__ __launch_bounds__(kThreads) void kda_chunked_prefill_kernel(
    KdaChunkedArgs p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 15;   // MFMA column / A-operand row
  const int gq = lane >> 4;  // MFMA row group
  const int H = p.heads;
  const int C = H * kD;
  const int C3 = 3 * C;
  const int n = static_cast<int>(blockIdx.x) / H;
  const int h = static_cast<int>(blockIdx.x) % H;
  const int32_t tb = p.cu_seqlens[n];
  const int32_t te = p.cu_seqlens[n + 1];
  const int len = te > tb ? te - tb : 0;
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

  // ---- per-sequence set-up ----------------------------------------------
  // conv threads 0..383: channel part*C + h*D + i; gate threads 384..511
  const bool conv_thread = tid < 3 * kD;
  const int part = tid >> 7;
  const int ci = tid & (kD - 1);
  const int64_t gc = static_cast<int64_t>(part) * C + col0 + ci;
  float cw[kW] = {0.f, 0.f, 0.f, 0.f};
  uint16_t win[kW - 1] = {0, 0, 0};
  // element t of the channel's stored window
  auto cs_at = [&](int t) -> int64_t {
    return tap_major ? (static_cast<int64_t>(slot) * (kW - 1) + t) * C3 + gc
                     : (static_cast<int64_t>(slot) * C3 + gc) * (kW - 1) + t;
  };
  if (conv_thread) {
    for (int t = 0; t < kW; ++t)
      cw[t] = p.conv_w[(static_cast<int64_t>(part) * kW + t) * C + col0 + ci];
    for (int t = 0; t < kW - 1; ++t) win[t] = p.conv_state[cs_at(t)];
  }
  // the wave's 16 state columns, all 128 key rows: 8 row blocks of 16
  float* st = p.rec_state +
              (static_cast<int64_t>(slot) * H + h) * (kD * kD) + 16 * wave + c;
  f4 S[8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[kb][r] = st[(16 * kb + 4 * gq + r) * kD];
  const float nw = kNorm ? p.norm_w[16 * wave + c] : 0.0f;

  // raw inputs of one chunk, held in registers until the chunk runs: conv
  // threads the bf16 qkv of their channel, gate threads the g of their key,
  // every thread the 4 gate values of its output rows
  uint32_t pf[kC];
  float pgate[4];
  float pbeta;
  // Rows past the end of a short last chunk re-read the last valid row
  // (branch-free loads; the values are masked where they are used).
  auto prefetch = [&](int c0) {
    const int last = (len - c0 < kC ? len - c0 : kC) - 1;
    const int64_t tk = tb + c0;
    if (conv_thread) {
      const uint16_t* base = p.qkv + tk * C3 + gc;
#pragma unroll
      for (int t = 0; t < kC; ++t) pf[t] = base[(t < last ? t : last) * C3];
    } else {
      const float* base = p.g + (tk * H + h) * kD + (tid - 3 * kD);
#pragma unroll
      for (int t = 0; t < kC; ++t)
        pf[t] = __float_as_uint(base[(t < last ? t : last) * (H * kD)]);
    }
    pbeta = p.beta[tk * H + h + (ci < last ? ci : last) * H];
    const uint16_t* gbase = p.gate + tk * C + col0 + 16 * wave + c;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * gq + r;
      pgate[r] = kNorm ? bf16_to_f32(gbase[(t < last ? t : last) * C]) : 0.0f;
    }
  };
  prefetch(0);

  for (int t0 = 0; t0 < len; t0 += kC) {
    const int nv = len - t0 < kC ? len - t0 : kC;
    const int64_t tok0 = tb + t0;

    // ---- phase 1: conv + SiLU (q, k, v), cumulative decay, beta ---------
    // this chunk's raw inputs arrived during the previous chunk; the next
    // chunk's are requested now
    const uint32_t* xr = pf;
    const float gatev[4] = {pgate[0], pgate[1], pgate[2], pgate[3]};
    if (conv_thread) {
#pragma unroll
      for (int t = 0; t < kC; ++t) {
        const bool valid = t < nv;
        const uint16_t xb = static_cast<uint16_t>(xr[t]);
        const float xv = bf16_to_f32(xb);
        float a = cw[0] * bf16_to_f32(win[0]);
        a += cw[1] * bf16_to_f32(win[1]);
        a += cw[2] * bf16_to_f32(win[2]);
        a += cw[3] * xv;
        sm.x[part][t][ci] = valid ? a * sigmoid_(a) : 0.0f;
        if (conv_update) {  // else every token sees the stored window
          win[0] = valid ? win[1] : win[0];
          win[1] = valid ? win[2] : win[1];
          win[2] = valid ? xb : win[2];
        }
      }
    } else {
      // cumulative decay in log2 units (exp2 on the hardware unit)
      const int i = tid - 3 * kD;
      float G = 0.0f, gmax = 0.0f;
#pragma unroll
      for (int t = 0; t < kC; ++t) {
        G += t < nv ? __uint_as_float(xr[t]) * kLog2e : 0.0f;
        sm.G[t][i] = G;
        gmax = fmaxf(gmax, fabsf(G));
      }
      if (i < kC) sm.beta[i] = i < nv ? pbeta : 0.0f;
      const bool bad = __any(!(gmax <= kSafeExp2));  // NaN counts as unsafe
      if (lane == 0) sm.unsafe[wave - 6] = bad ? 1 : 0;
    }
    __syncthreads();
    if (t0 + kC < len) prefetch(t0 + kC);  // lands during this chunk

    // ---- phase 2: q/k L2 normalisation (optional) -----------------------
    if (l2) {
      const float qscale = 1.0f / sqrtf(static_cast<float>(kD));
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = 2 * wave + tt;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const float v0 = sm.x[pp][t][lane];
          const float v1 = sm.x[pp][t][lane + 64];
          const float ss = wave_sum(v0 * v0 + v1 * v1);
          const float r = 1.0f / sqrtf(ss + 1e-6f);
          const float sc = pp == 0 ? qscale : 1.0f;
          sm.x[pp][t][lane] = (v0 * r) * sc;
          sm.x[pp][t][lane + 64] = (v1 * r) * sc;
        }
      }
      __syncthreads();
    }
    const bool unsafe = (sm.unsafe[0] | sm.unsafe[1]) != 0;

    // ---- phase 3: decayed operand tables --------------------------------
    {
      const int i = tid & (kD - 1);
      const int tq = tid >> 7;
      const float Gl = sm.G[kC - 1][i];
#pragma unroll
      for (int m = 0; m < kC / 4; ++m) {
        const int t = tq + 4 * m;
        const float G = sm.G[t][i];
        const float e = exp2_(G);
        const float q = sm.x[0][t][i];
        const float k = sm.x[1][t][i];
        sm.qt[t][i] = q * e;
        sm.kt[t][i] = k * e;
        sm.khT[i][t] = k * exp2_(Gl - G);
        if (!unsafe) sm.ki[t][i] = k * exp2_(-G);
      }
      if (tq == 0) sm.gam[i] = exp2_(Gl);
    }
    __syncthreads();

    // ---- phase 4: A = K~ (K e^{-G})^T, B = Q~ (K e^{-G})^T ---------------
    if (!unsafe) {
      // waves 0-3: A over keys 32(w%4) .. +31; waves 4-7: B likewise
      const float(*src)[kLd] = wave < 4 ? sm.kt : sm.qt;
      const int kbase = 32 * (wave & 3) + 8 * gq;
      const f4 a0 = ld4(&src[c][kbase]);
      const f4 a1 = ld4(&src[c][kbase + 4]);
      const f4 b0 = ld4(&sm.ki[c][kbase]);
      const f4 b1 = ld4(&sm.ki[c][kbase + 4]);
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma(a0[j], b0[j], acc);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma(a1[j], b1[j], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.part[wave][4 * gq + r][c] = acc[r];
      __syncthreads();
      const int idx = tid & 255;
      const int t = idx >> 4;
      const int s = idx & 15;
      if (tid < 256) {
        const float a = sm.part[0][t][s] + sm.part[1][t][s] +
                        sm.part[2][t][s] + sm.part[3][t][s];
        sm.L[t][s] = s < t ? sm.beta[t] * a : 0.0f;
      } else {
        const float b = sm.part[4][t][s] + sm.part[5][t][s] +
                        sm.part[6][t][s] + sm.part[7][t][s];
        sm.B[t][s] = s <= t ? b : 0.0f;
      }
    } else if (tid < 256) {
      // large decay: one exponential per (t, s, key)
      const int t = tid >> 4;
      const int s = tid & 15;
      float a = 0.0f, b = 0.0f;
      if (s <= t) {
        for (int i = 0; i < kD; ++i) {
          const float ks = sm.x[1][s][i] * exp2_(sm.G[t][i] - sm.G[s][i]);
          a += sm.x[1][t][i] * ks;
          b += sm.x[0][t][i] * ks;
        }
      }
      sm.L[t][s] = s < t ? sm.beta[t] * a : 0.0f;
      sm.B[t][s] = b;
    }
    __syncthreads();

    // ---- phase 5: T = (I + L)^{-1} (wave 0), K~ S and Q~ S (all) --------
    if (wave == 0 && lane < kC) {
      float tc[kC];
#pragma unroll
      for (int t = 0; t < kC; ++t) {
        float v = t == lane ? 1.0f : 0.0f;
#pragma unroll
        for (int s = 0; s < t; ++s) v -= sm.L[t][s] * tc[s];
        tc[t] = v;
      }
#pragma unroll
      for (int t = 0; t < kC; ++t) sm.T[t][lane] = tc[t];
    }
    f4 ks = {0.f, 0.f, 0.f, 0.f};  // (K~ S)[token 4gq + r][col c]
    f4 o = {0.f, 0.f, 0.f, 0.f};   // (Q~ S)[token 4gq + r][col c]
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const f4 ak = ld4(&sm.kt[c][16 * kb + 4 * gq]);
      const f4 aq = ld4(&sm.qt[c][16 * kb + 4 * gq]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ks = mfma(ak[j], S[kb][j], ks);
        o = mfma(aq[j], S[kb][j], o);
      }
    }
    // beta (V - K~ S) in the accumulator layout
    f4 br;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * gq + r;
      br[r] = sm.beta[t] * (sm.x[2][t][16 * wave + c] - ks[r]);
    }
    __syncthreads();

    // ---- phase 6: Delta = T br, O += B Delta, S <- e^{G_last} S + K^^T Delta
    f4 dl = {0.f, 0.f, 0.f, 0.f};
    {
      const f4 at = ld4(&sm.T[c][4 * gq]);
#pragma unroll
      for (int j = 0; j < 4; ++j) dl = mfma(at[j], br[j], dl);
      const f4 ab = ld4(&sm.B[c][4 * gq]);
#pragma unroll
      for (int j = 0; j < 4; ++j) o = mfma(ab[j], dl[j], o);
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const f4 gm = ld4(&sm.gam[16 * kb + 4 * gq]);
      S[kb] *= gm;
      const f4 ah = ld4(&sm.khT[16 * kb + c][4 * gq]);
#pragma unroll
      for (int j = 0; j < 4; ++j) S[kb] = mfma(ah[j], dl[j], S[kb]);
    }
    if (kNorm) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ss = row_sum16(o[r] * o[r]);
        if (c == 0) sm.red[wave][4 * gq + r] = ss;
      }
    }
    __syncthreads();

    // ---- phase 7: gated RMSNorm and bf16 outputs -------------------------
    uint16_t* obase = p.out + tok0 * C + col0 + 16 * wave + c;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * gq + r;
      if (t >= nv) continue;
      float y = o[r];
      if (kNorm) {
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tot += sm.red[w][t];
        const float rs = 1.0f / sqrtf(tot * (1.0f / kD) + p.eps);
        const float gv = gatev[r];
        const float ga = gate_silu ? gv * sigmoid_(gv) : sigmoid_(gv);
        y = ((y * rs) * nw) * ga;
      }
      obase[t * C] = f32_to_bf16(y);
    }
  }

  // ---- write back the state and the conv window ---------------------------
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) st[(16 * kb + 4 * gq + r) * kD] = S[kb][r];
  if (conv_thread && conv_update)
    for (int t = 0; t < kW - 1; ++t) p.conv_state[cs_at(t)] = win[t];
}

}  // namespace

hipError_t kda_chunked_prefill_launch(const KdaChunkedArgs& args,
                                      int32_t num_seqs, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(num_seqs * args.heads));
  if (args.flags & KDA_OUTPUT_NORM)
    hipLaunchKernelGGL(kda_chunked_prefill_kernel<true>, grid,
                       dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(kda_chunked_prefill_kernel<false>, grid,
                       dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}
