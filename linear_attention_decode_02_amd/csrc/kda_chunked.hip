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
// roles that share each SIMD (waves w and w + 4 run on SIMD w), each role
// in a loop of its own; three barriers per chunk hand the double-buffered
// LDS tables over.  Rows of tokens_per_row tokens (no cu_seqlens: the
// multi-token decode of long rows) are sequences of equal length.
//   * state waves 0-3 own value columns 32w .. 32w+31 of the [128 key,
//     128 value] fp32 state, held for the whole sequence in registers in
//     the accumulator layout of the 16x16 MFMAs (lane l: column l%16, key
//     rows 4(l/16) .. +3 of each 16-row block).  The products with the
//     state run on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16) with
//     every fp32 operand split into three bf16 pieces hi + mid + lo (about
//     24 significant bits) and the six products of pieces down to 2^-18 of
//     the leading one accumulated in fp32: the result matches fp32
//     products.  The state's accumulator layout is the B operand once the
//     summation index is permuted (lane l holds keys 32P + 4(l/16) .. +3
//     and 32P + 16 + 4(l/16) .. +3 of block P; the prep waves store the
//     A-operand tables in that key order), so the state never leaves the
//     registers.  Per chunk and wave: 48 MFMAs for K~ S and 48 for Q~ S,
//     16 fp32 MFMAs for the triangular solve and B Delta, 48 for the
//     state update (its k runs over 2 pieces x 4 tokens per lane group);
//     every lane also solves for the row of T = (I + diag(beta) A)^{-1}
//     its operand needs, by backward substitution.
//   * prep waves 4-7 build the next chunk's operands meanwhile (4 tokens
//     each): causal conv + SiLU from the raw bf16 inputs, q/k L2
//     normalisation (wave-local: a wave holds all channels of its tokens),
//     the cumulative decay, the decayed tables K~, Q~, K^, K e^{-G} (split
//     in three), and then the A / B products on the matrix cores.  Their
//     inputs are loaded straight into registers a chunk ahead.  At a
//     segment's last chunk the prep wave holding its last three input rows
//     writes them as the new stored conv window.
// Why bf16 pieces and not fp32 MFMAs (v_mfma_f32_16x16x4_f32): while one
// wave of a SIMD streams fp32 MFMAs, LDS reads and global loads of the
// other wave on that SIMD return about 20 times later (measured on gfx950:
// LDS 77 -> 2125 cycles, global 224 -> 4318); bf16 MFMA streams leave them
// untouched, and 3-piece products take fewer matrix cycles besides (6 x 17
// cycles per 32 keys against 8 x 32).  The state waves also write the
// gated-RMSNorm outputs, one 16-byte store per lane.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

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
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

// Split rows: a [16 token][128 key] table as three bf16 pieces hi + mid +
// lo of every fp32 value (each the rounded remainder of the ones before:
// together about 24 significant bits), in the operand order of
// v_mfma_f32_16x16x32_bf16: per 32-key block P and lane group g, 12 dwords
// -- hi of keys 32P+4g .. +3 and 32P+16+4g .. +3, then mid, then lo of
// the same keys -- so each piece of one lane's operand is one aligned
// 16-byte read.
constexpr int kRowU = 4 * 4 * 12 + 4;  // dwords per split row (+ pad)
// Split K^ rows: per key and group g of 4 tokens, 8 dwords: the pieces
// [hi | mid] and [hi | lo] of the 4 tokens (two A operands of the state
// update, k = 8 slots = 2 pieces x 4 tokens)
constexpr int kKhU = 4 * 8 + 4;        // dwords per split K^ row (+ pad)

// Operands of one chunk for the state waves (double-buffered).
struct ChunkTables {
  uint32_t qt[kC][kRowU];  // q_t e^{G_t}, split
  uint32_t kt[kC][kRowU];  // k_t e^{G_t}, split
  float v[kC][kLd];        // v_t
  uint32_t kh[kD][kKhU];   // k_t e^{G_last - G_t} per key, split
  float gam[kD];           // e^{G_last}
  float beta[kC];
};

struct alignas(16) Smem {
  ChunkTables tab[2];
  uint32_t kis[kC][kRowU];  // k_t e^{-G_t}, split (matrix-core path)
  float ki[kC][kLd];    // exact path: raw k
  float qraw[kC][kLd];  // exact path: q_t
  float graw[kC][kLd];  // exact path: cumulative log2 decay
  union {
    float part[4][kC][kC];  // stages 2-3: A (keys 0-63, 64-127), B (same)
    f2 gtok[kC][kD / 2];    // stage 1: token t's log2 decays of keys
                            // 2 lane, 2 lane + 1, from the wave that owns t
  };
  float LT[kC][kTd];    // LT[s][t] = beta_t A_ts for s < t, else 0
  float B[kC][kTd];     // B_ts for s <= t, else 0
  float o[kC][kLd];     // this chunk's outputs before the norm
  float nw[kD];         // norm weight
  int unsafe;           // exact path for the chunk being prepared
  int gseq[4];  // per prep wave: the chunk whose decays it last put in gtok
                // (-1: none yet)
};

// Spins of a prep wave waiting for the others' decays before it gives up
// (then with whatever is in gtok): every wave finishes.
constexpr int kGseqSpinMax = 1 << 20;

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
// (a, b) in three bf16 pieces, each a pair (a in the low half): hi =
// RNE(a, b), mid = RNE of the remainders, lo = RNE of what is left; the
// sum of the pieces is within 2^-26 of each value (relative)
struct Split3 {
  uint32_t h, m, l;
};
__device__ __forceinline__ uint32_t bf2_(f2 v) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2v));
}
__device__ __forceinline__ f2 bf2_val(uint32_t w) {
  return f2{__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
}
__device__ __forceinline__ Split3 split3(float a, float b) {
  const f2 v = {a, b};
  const uint32_t h = bf2_(v);
  const f2 r1 = v - bf2_val(h);
  const uint32_t m = bf2_(r1);
  const f2 r2 = r1 - bf2_val(m);
  return Split3{h, m, bf2_(r2)};
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
// 4x4 transpose across the 4 lanes of each quad: lane b's element r goes
// to lane r's element b (two butterfly stages: lane bit 0 with element
// bit 0, then bit 1 with bit 1).  odd1 / odd2: bit 0 / bit 1 of the lane.
__device__ __forceinline__ f4 quad_transpose(f4 x, bool odd1, bool odd2) {
  const float p0 = dpp_<0xB1>(x[0]), p1 = dpp_<0xB1>(x[1]);
  const float p2 = dpp_<0xB1>(x[2]), p3 = dpp_<0xB1>(x[3]);
  const f4 y = {odd1 ? p1 : x[0], odd1 ? x[1] : p0, odd1 ? p3 : x[2],
                odd1 ? x[3] : p2};
  const float q0 = dpp_<0x4E>(y[0]), q1 = dpp_<0x4E>(y[1]);
  const float q2 = dpp_<0x4E>(y[2]), q3 = dpp_<0x4E>(y[3]);
  return f4{odd2 ? q2 : y[0], odd2 ? q3 : y[1], odd2 ? y[2] : q0,
            odd2 ? y[3] : q1};
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
// A wave-uniform address made opaque to the compiler (readfirstlane of both
// halves): loads from it become a scalar base plus a 32-bit lane offset
// instead of a 64-bit address per lane.
__device__ __forceinline__ gptr<const char> uniform_gptr(const void* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<gptr<const char>>((static_cast<uint64_t>(hi) << 32) |
                                            lo);
}
// *(U*)(base + byte_off); the offset is made opaque where the load is, so
// the 32-bit lane offset is not widened ahead of the loop and the load
// keeps the scalar-base form
template <typename U>
__device__ __forceinline__ U load_at(gptr<const char> base, uint32_t byte_off) {
  asm volatile("" : "+v"(byte_off));
  return *reinterpret_cast<gptr<const U>>(base + byte_off);
}

// DPP with a row mask: rows outside it keep 0
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_rows_(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                         kRowMask, 0xF, false));
}
// N wave sums side by side (independent DPP chains), each result in every
// lane: the row sums (xor butterfly), then row_bcast:15 into rows 1 and 3
// and row_bcast:31 into rows 2 and 3, so lane 63 holds the total.
template <int N>
__device__ __forceinline__ void wave_sum(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_<0xB1>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_<0x4E>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_<0x141>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_<0x140>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_rows_<0x142, 0xA>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_rows_<0x143, 0xC>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[i]), 63));
}

__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// D += A B with 8 bf16 per lane of each operand (16x16x32)
__device__ __forceinline__ f4 mfma_bf(u4 a, u4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf8v, a), __builtin_bit_cast(bf8v, b), c, 0, 0, 0);
}
__device__ __forceinline__ u4 ld_u4(const uint32_t* p) {
  return *reinterpret_cast<const u4*>(p);
}
// D += A B over 32 keys from split operands (hi, mid, lo at dwords 0, 4, 8
// of each): the six products of pieces down to 2^-18 of the leading term
__device__ __forceinline__ f4 mfma6_(u4 ah, u4 am, u4 al, u4 bh, u4 bm, u4 bl,
                                    f4 acc) {
  acc = mfma_bf(al, bh, acc);
  acc = mfma_bf(ah, bl, acc);
  acc = mfma_bf(am, bm, acc);
  acc = mfma_bf(am, bh, acc);
  acc = mfma_bf(ah, bm, acc);
  return mfma_bf(ah, bh, acc);
}
__device__ __forceinline__ f4 mfma6(const uint32_t* a, const uint32_t* b,
                                   f4 acc) {
  return mfma6_(ld_u4(a), ld_u4(a + 4), ld_u4(a + 8), ld_u4(b), ld_u4(b + 4),
                ld_u4(b + 8), acc);
}
__device__ __forceinline__ f4 ld4(const float* p) {
  return *reinterpret_cast<const f4*>(p);
}

// Gate operands of a launch: activated g and beta, or the raw inputs with
// the default (softplus) or the bounded gate.
enum GateForm { kGateInput = 0, kGateSoftplus = 1, kGateBounded = 2 };

// The tokens of one (sequence or row, head): the workgroup's work.
struct Seg {
  int64_t tb;  // first token
  int len;     // tokens
  int slot;
  int h;
  int nch;     // 16-token chunks
};

template <bool kNorm, int kGate>
__global__ __launch_bounds__(kThreads) void kda_chunked_prefill_kernel(
    KdaChunkedArgs p) {
  constexpr bool kRaw = kGate != kGateInput;
  // Raw gates cost a softplus (or sigmoid) per channel and token: each prep
  // wave then converts only its own 4 tokens and the waves exchange them
  // through LDS (raw-gate prefill 629 -> 573 us at 16 sequences x 48
  // heads).  Plain decays are cheaper to convert than to exchange (555 ->
  // 562 us), so there every prep wave converts all 16 itself.
  constexpr bool kShareDecays = kRaw;
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
  const uint32_t flags = p.flags;
  const bool tap_major = (flags & KDA_CONV_TAP_MAJOR) != 0;
  const bool conv_update = (flags & KDA_NO_CONV_UPDATE) == 0;
  const bool l2 = (flags & KDA_QK_L2NORM) != 0;
  const bool gate_silu = (flags & KDA_GATE_SILU) != 0;
  const bool state_wave = wave < 4;
  const int pw = wave & 3;  // index within the role
  // output lanes: token tid/16 (of the 16), columns 8 (tid%16) .. +7
  const int ot = (tid & 255) >> 4;
  const int oc = 8 * (tid & 15);

  // One (sequence, head) per workgroup, s = n H + h.
  auto seg_at = [&](int sg) -> Seg {
    Seg g;
    const int n = sg / H;
    g.h = sg - n * H;
    // token offsets in 64 bits: tb * 3C passes 2^31 from 58,255 tokens at
    // 96 heads
    const int64_t tb =
        p.cu_seqlens ? p.cu_seqlens[n] : static_cast<int64_t>(n) * p.tokens_per_row;
    const int64_t te = p.cu_seqlens ? p.cu_seqlens[n + 1]
                                    : tb + p.tokens_per_row;
    g.tb = tb;
    g.len = te > tb ? static_cast<int>(te - tb) : 0;
    g.slot = p.state_idx[n];
    g.nch = (g.len + kC - 1) / kC;
    return g;
  };
  auto live = [&](const Seg& g) {
    return g.len > 0 && g.slot > 0 && g.slot < p.num_slots;
  };
  // +0.0 outputs of a segment with tokens and a null slot (no state
  // traffic), by `nthr` threads from thread index `t0`
  auto zero_outputs = [&](const Seg& g, int t0, int nthr) {
    uint32_t* o32 = reinterpret_cast<uint32_t*>(p.out);
    const int64_t col0 = static_cast<int64_t>(g.h) * kD;
    for (int64_t idx = t0; idx < static_cast<int64_t>(g.len) * (kD / 2);
         idx += nthr) {
      const int64_t t = idx / (kD / 2);
      o32[((g.tb + t) * C + col0) / 2 + idx % (kD / 2)] = 0u;
    }
  };
  // Longest sequences first.  A workgroup takes a whole compute unit (LDS),
  // so the workgroups of a large batch run in rounds, in index order, and a
  // long sequence late in the batch would start its chunk chain only after
  // others end.  With cu_seqlens and at most kThreads sequences, workgroup
  // b takes head b % H of the (b / H)-th sequence by descending length
  // (ties by index): the rank of each sequence is counted over the lengths
  // staged in sm.o, which no wave uses before the second barrier below.
  int sg = static_cast<int>(blockIdx.x);
  const int nseq = static_cast<int>(gridDim.x) / H;
  if (p.cu_seqlens != nullptr && nseq > 1 && nseq <= kThreads) {
    __shared__ int picked;
    int* lens = reinterpret_cast<int*>(&sm.o[0][0]);
    const int want = sg / H;
    if (tid < nseq) {
      // in 64 bits, as seg_at: any two int32 offsets, a decreasing pair 0
      const int64_t d = static_cast<int64_t>(p.cu_seqlens[tid + 1]) -
                        p.cu_seqlens[tid];
      lens[tid] = d > 0 ? static_cast<int>(d < INT32_MAX ? d : INT32_MAX) : 0;
    }
    if (tid == 0) picked = want;
    __syncthreads();
    if (tid < nseq) {
      const int mine = lens[tid];
      int rank = 0;
      for (int j = 0; j < nseq; ++j) {
        const int other = lens[j];
        rank += (other > mine || (other == mine && j < tid)) ? 1 : 0;
      }
      if (rank == want) picked = tid;
    }
    __syncthreads();
    sg = picked * H + (sg - want * H);
  }
  const Seg seg = seg_at(sg);
  if (seg.len == 0) return;
  if (!live(seg)) {
    zero_outputs(seg, tid, kThreads);
    return;
  }
  if (!state_wave && tid - 256 < kD)  // norm weight, read by the state waves
    sm.nw[tid - 256] = kNorm ? p.norm_w[tid - 256] : 0.0f;
  if (kShareDecays) {
    if (tid < 4) sm.gseq[tid] = -1;
    __syncthreads();  // no prep wave reads a decay flag before this
  }

  // ---- prep stage 1 of chunk ci: conv, norms, decay, tables (wave-local)
  // Prep wave pw reads what it needs straight into registers, one chunk
  // ahead (the loads are in flight while the wave works on the current
  // chunk; the first use waits for them): for channels 2 lane, 2 lane + 1
  // the input rows of tokens 4pw-3 .. 4pw+3 (chunk-relative; rows before
  // the sequence or past its end are clamped to valid rows and replaced or
  // masked where used), the gates of all 16 tokens (raw gates: of tokens
  // 4pw .. 4pw+3, see kShareDecays) and (lanes 0-3) the beta of token
  // 4pw + lane.  No LDS on this path: while the state waves
  // run their matrix products, LDS reads of the other wave on the SIMD
  // wait far longer than register loads that were issued early.
  uint32_t in_raw[3][7];
  // fp32 pair, or (raw gates) a bf16 pair in [0]
  uint32_t in_g[kShareDecays ? 4 : kC][2];
  uint32_t in_b = 0;     // fp32 or (raw gates) bf16 bits
  // this lane's byte offsets in an input row (parts q, k, v) and a gate row
  const uint32_t off_raw = 4 * lane;
  const uint32_t off_part = 2 * static_cast<uint32_t>(C);
  const uint32_t off_g = (kRaw ? 4 : 8) * lane;
  // the stored conv window of channels 2 lane, 2 lane + 1 of each part,
  // as loaded (tap-major: the channel pair in [0]; channel-major: one
  // channel in each of [0], [1], combined where used, so no load waits at
  // its issue)
  auto load_window = [&](int slot, int64_t col0,
                         uint32_t (&wv)[2][3][kW - 1]) {
#pragma unroll
    for (int pp = 0; pp < 3; ++pp)
#pragma unroll
      for (int e = 0; e < kW - 1; ++e) {
        const int64_t ch = static_cast<int64_t>(pp) * C + col0 + 2 * lane;
        if (tap_major) {
          wv[0][pp][e] = *reinterpret_cast<const uint32_t*>(
              p.conv_state +
              (static_cast<int64_t>(slot) * (kW - 1) + e) * C3 + ch);
          wv[1][pp][e] = 0u;
        } else {
          const uint16_t* cs =
              p.conv_state + (static_cast<int64_t>(slot) * C3 + ch) * (kW - 1) +
              e;
          wv[0][pp][e] = cs[0];
          wv[1][pp][e] = cs[kW - 1];
        }
      }
  };
  auto load_chunk = [&](const Seg& sg, int cj) {
    const int c0 = cj * kC;
    const int nv = sg.len - c0 < kC ? sg.len - c0 : kC;
    const int64_t tok0 = sg.tb + c0;
    const int h = sg.h;
    const int64_t col0 = static_cast<int64_t>(h) * kD;
    // row addresses are wave-uniform (scalar); lanes add 32-bit offsets
    const char* q0 = reinterpret_cast<const char*>(p.qkv + tok0 * C3 + col0);
    const int qrow = 2 * C3;  // bytes per token row (rows differ by < 16)
#pragma unroll
    for (int u = 0; u < 7; ++u) {
      const int rel = 4 * pw - 3 + u;
      const int rr =
          rel < 0 ? (cj > 0 ? rel : 0) : (rel < nv - 1 ? rel : nv - 1);
      const gptr<const char> row = uniform_gptr(q0 + rr * qrow);  // 32-bit
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
        in_raw[pp][u] = load_at<uint32_t>(row, off_raw + pp * off_part);
    }
    const int64_t g0 = (tok0 * H + h) * kD;
    const char* gb = kRaw ? reinterpret_cast<const char*>(p.rg.raw_g + g0)
                          : reinterpret_cast<const char*>(p.g + g0);
    const int grow = H * kD * (kRaw ? 2 : 4);
#pragma unroll
    for (int u = 0; u < (kShareDecays ? 4 : kC); ++u) {
      const int t = kShareDecays ? 4 * pw + u : u;
      const int rr = t < nv - 1 ? t : nv - 1;
      const gptr<const char> row = uniform_gptr(gb + rr * grow);
      if (kRaw) {
        in_g[u][0] = load_at<uint32_t>(row, off_g);
      } else {
        const u2 v = load_at<u2>(row, off_g);
        in_g[u][0] = v.x;
        in_g[u][1] = v.y;
      }
    }
    if (lane < 4) {
      const int t = 4 * pw + lane;
      const int rr = t < nv - 1 ? t : nv - 1;
      const int64_t e = (tok0 + rr) * H + h;
      in_b = kRaw ? static_cast<uint32_t>(p.rg.raw_beta[e])
                  : __float_as_uint(p.beta[e]);
    }
  };
  // per-head constants of the prep waves, for channels 2 lane, 2 lane + 1:
  // conv weights, conv bias and dt_bias (raw gates), and the sequence's
  // stored conv window
  f2 cwv[3][kW];
  f2 cbv[3] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
  f2 dtb = {0.f, 0.f};
  uint32_t wv[2][3][kW - 1];
  auto load_constants = [&](const Seg& sg) {
    const int64_t col0 = static_cast<int64_t>(sg.h) * kD;
#pragma unroll
    for (int pp = 0; pp < 3; ++pp) {
#pragma unroll
      for (int tap = 0; tap < kW; ++tap)
        cwv[pp][tap] = *reinterpret_cast<const f2*>(
            p.conv_w + (static_cast<int64_t>(pp) * kW + tap) * C + col0 +
            2 * lane);
      if (kRaw && p.rg.conv_bias)
        cbv[pp] = *reinterpret_cast<const f2*>(
            p.rg.conv_bias + static_cast<int64_t>(pp) * C + col0 + 2 * lane);
    }
    if (kRaw)
      dtb = *reinterpret_cast<const f2*>(p.rg.dt_bias + col0 + 2 * lane);
    load_window(sg.slot, col0, wv);
  };

  // a segment's new conv window, held from its last chunk's stage 1 to the
  // barrier after it
  bool win_pending = false;
  int win_slot = 0, win_h = 0;
  uint32_t win_new[3][kW - 1];
  auto flush_window = [&]() {
    if (!win_pending) return;
    const int64_t col0 = static_cast<int64_t>(win_h) * kD;
#pragma unroll
    for (int e = 0; e < kW - 1; ++e)
#pragma unroll
      for (int pp = 0; pp < 3; ++pp) {
        const uint32_t w = win_new[pp][e];
        const int64_t ch = static_cast<int64_t>(pp) * C + col0 + 2 * lane;
        if (tap_major) {
          *reinterpret_cast<uint32_t*>(
              p.conv_state +
              (static_cast<int64_t>(win_slot) * (kW - 1) + e) * C3 + ch) = w;
        } else {
          uint16_t* cs = p.conv_state +
                         (static_cast<int64_t>(win_slot) * C3 + ch) * (kW - 1) +
                         e;
          cs[0] = static_cast<uint16_t>(w);
          cs[kW - 1] = static_cast<uint16_t>(w >> 16);
        }
      }
    win_pending = false;
  };
  // Stage 1 of chunk ci of segment g, stream position j (its table
  // buffer); (gs, cs) is the chunk after it, whose inputs it requests.
  // `plain` (a compile-time tag) is the common case -- a full chunk that is
  // not the segment's first, with the conv update -- where no token is
  // masked and no input comes from the stored window.
  auto prep_tables = [&](auto plain, const Seg& g, int ci, int j,
                         const Seg& gs, int cs) {
    constexpr bool kPlain = decltype(plain)::value;
    ChunkTables& T = sm.tab[j & 1];
    const int c0 = ci * kC;
    const int nv = g.len - c0 < kC ? g.len - c0 : kC;
    const int h = g.h;
    // this chunk's inputs (loaded a chunk ago)
    uint32_t raw[3][7];
#pragma unroll
    for (int u = 0; u < 7; ++u)
#pragma unroll
      for (int pp = 0; pp < 3; ++pp) raw[pp][u] = in_raw[pp][u];
    uint32_t wc[3][kW - 1];
#pragma unroll
    for (int pp = 0; pp < 3; ++pp)
#pragma unroll
      for (int e = 0; e < kW - 1; ++e)
        wc[pp][e] = wv[0][pp][e] | (wv[1][pp][e] << 16);
    // per-token decays of keys 2 lane, 2 lane + 1 in log2 units: all 16
    // tokens' from this wave's loads, or (kShareDecays) this wave's 4
    // tokens', published for the other prep waves
    constexpr int kNG = kShareDecays ? 4 : kC;
    f2 gl[kC];
    if (kRaw) {
      const float a_rate = __expf(p.rg.A_log[h]);
      const float lb2 = p.rg.lower_bound * kLog2e;
      constexpr bool kB = kGate == kGateBounded;
#pragma unroll
      for (int u = 0; u < kNG; ++u)
        gl[u] = f2{kda_gate2_from_raw<kB>(bf16_lo(in_g[u][0]) + dtb.x, a_rate,
                                          lb2),
                   kda_gate2_from_raw<kB>(bf16_hi(in_g[u][0]) + dtb.y, a_rate,
                                          lb2)};
    } else {
#pragma unroll
      for (int u = 0; u < kNG; ++u)
        gl[u] = f2{__uint_as_float(in_g[u][0]), __uint_as_float(in_g[u][1])} *
                kLog2e;
    }
#pragma unroll
    for (int u = 0; u < kNG; ++u) gl[u] = kda_decay_floor2(gl[u]);
    if (kShareDecays) {
#pragma unroll
      for (int u = 0; u < 4; ++u) sm.gtok[4 * pw + u][lane] = gl[u];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0)
        __hip_atomic_store(&sm.gseq[pw], ci, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    const float bt =
        lane < 4 ? (kRaw ? sigmoid_(bf16_lo(in_b)) : __uint_as_float(in_b))
                 : 0.0f;
    const float qscale = 0.08838834764831845f;  // D^-1/2
    // conv + SiLU of the 4 tokens (weights read once), then the 8 norm
    // reductions side by side, then the tables
    float y[4][3][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool valid = kPlain || 4 * pw + u < nv;
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float a = cbv[pp][e];
#pragma unroll
          for (int tap = 0; tap < kW; ++tap) {
            // with the update a token sees the inputs before it (the stored
            // window before the sequence); without it, the stored window
            // (only wave 0 reaches before the chunk: index rin0 = rin there,
            // a constant, so the window stays in registers)
            const int rin0 = u - (kW - 1) + tap;
            const bool before = !kPlain && rin0 < 0 && pw == 0 && ci == 0;
            const uint32_t w2 =
                tap == kW - 1 ? raw[pp][u + tap]
                : (kPlain || conv_update)
                    ? (before ? wc[pp][(kW - 1) + (rin0 < 0 ? rin0 : 0)]
                              : raw[pp][u + tap])
                    : wc[pp][tap];
            a += cwv[pp][tap][e] * (e ? bf16_hi(w2) : bf16_lo(w2));
          }
          y[u][pp][e] = valid ? a * sigmoid_(a) : 0.0f;
        }
    }
    // At the segment's last chunk the prep wave whose 7 input rows hold
    // the segment's last W-1 inputs keeps them as the new stored window
    // (for a segment shorter than that, the old window's newest entries
    // come first); it writes them after the next barrier, once every prep
    // wave's reads of the old window are done (see flush_window)
    win_pending = conv_update && ci + 1 == g.nch && pw == (g.len - 1 - c0) / 4;
    if (win_pending) {
      win_slot = g.slot;
      win_h = h;
#pragma unroll
      for (int e = 0; e < kW - 1; ++e) {
        const int idx = g.len - (kW - 1) + e;  // token in the segment
        const int u = idx - c0 - (4 * pw - 3);  // its input row, 0..6
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) {
          uint32_t w = raw[pp][0];
#pragma unroll
          for (int q = 1; q < 7; ++q)
            if (u == q) w = raw[pp][q];
          if (idx < 0) {  // from the old window: entry idx + W-1
            w = wc[pp][0];
#pragma unroll
            for (int q = 1; q < kW - 1; ++q)
              if (idx + (kW - 1) == q) w = wc[pp][q];
          }
          win_new[pp][e] = w;
        }
      }
    }
    // the inputs are consumed: the next chunk's loads reuse their registers
    // (unconditional -- after the last chunk its own inputs again -- so no
    // copy has to wait for them)
    load_chunk(gs, cs);
    if (l2) {
      float ss[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ss[2 * u] = y[u][0][0] * y[u][0][0] + y[u][0][1] * y[u][0][1];
        ss[2 * u + 1] = y[u][1][0] * y[u][1][0] + y[u][1][1] * y[u][1][1];
      }
      wave_sum<8>(ss);
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
    // (kShareDecays) the other waves' decays, published before their conv,
    // so normally there by now; then the cumulative decay G over the chunk,
    // in token order: its values at this wave's tokens and at the end
    if (kShareDecays) {
      for (int it = 0; it < kGseqSpinMax; ++it) {
        bool ready = true;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          ready = ready &&
                  __hip_atomic_load(&sm.gseq[w], __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_WORKGROUP) == ci;
        if (ready) break;
        __builtin_amdgcn_s_sleep(1);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
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
          if (kPlain || t < nv) {
            if constexpr (kShareDecays)
              G += sm.gtok[t][lane];
            else
              G += gl[t];
          }
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
    // dword of keys 2 lane, 2 lane + 1 in a split row (hi; mid at + 4, lo
    // at + 8)
    const int m = lane & 15;
    const int pos = (4 * (lane >> 4) + ((m & 7) >> 1)) * 12 +
                    (m >= 8 ? 2 : 0) + (m & 1);
    auto put3 = [&](uint32_t* row, float a, float b) {
      const Split3 x = split3(a, b);
      row[pos] = x.h;
      row[pos + 4] = x.m;
      row[pos + 8] = x.l;
    };
    f2 khv[4];
    // e^{G_last}; on the matrix-core path e^{G_last - G_t} is taken as
    // e^{G_last} e^{-G_t} (every |G| <= 80 there, so both factors are
    // normal numbers), which saves an exponential per channel and token
    const f2 eG = {exp2_(G.x), exp2_(G.y)};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = 4 * pw + u;
      const f2 ee = {exp2_(Gu[u].x), exp2_(Gu[u].y)};
      put3(T.qt[t], y[u][0][0] * ee.x, y[u][0][1] * ee.y);
      put3(T.kt[t], y[u][1][0] * ee.x, y[u][1][1] * ee.y);
      *reinterpret_cast<f2*>(&T.v[t][2 * lane]) = f2{y[u][2][0], y[u][2][1]};
      if (!unsafe) {
        const f2 ei = {exp2_(-Gu[u].x), exp2_(-Gu[u].y)};
        khv[u] = f2{(y[u][1][0] * eG.x) * ei.x, (y[u][1][1] * eG.y) * ei.y};
        put3(sm.kis[t], y[u][1][0] * ei.x, y[u][1][1] * ei.y);
      } else {
        khv[u] = f2{y[u][1][0] * exp2_(G.x - Gu[u].x),
                    y[u][1][1] * exp2_(G.y - Gu[u].y)};
        *reinterpret_cast<f2*>(&sm.ki[t][2 * lane]) =
            f2{y[u][1][0], y[u][1][1]};
        *reinterpret_cast<f2*>(&sm.qraw[t][2 * lane]) =
            f2{y[u][0][0], y[u][0][1]};
        *reinterpret_cast<f2*>(&sm.graw[t][2 * lane]) = Gu[u];
      }
    }
    // K^ of keys 2 lane, 2 lane + 1 for this wave's 4 tokens: two 16-byte
    // stores per key
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const Split3 a = split3(khv[0][e], khv[1][e]);
      const Split3 b = split3(khv[2][e], khv[3][e]);
      u4* dst = reinterpret_cast<u4*>(&T.kh[2 * lane + e][8 * pw]);
      dst[0] = u4{a.h, b.h, a.m, b.m};
      dst[1] = u4{a.h, b.h, a.l, b.l};
    }
    if (pw == 0) {
      *reinterpret_cast<f2*>(&T.gam[2 * lane]) = eG;
      if (lane == 0) sm.unsafe = unsafe ? 1 : 0;
    }
    if (lane < 4) {
      const int t = 4 * pw + lane;
      T.beta[t] = t < nv ? bt : 0.0f;
    }
  };

  // ---- prep stage 2: A / B products (or the exact per-entry sums) -------
  auto prep_gram = [&](int j) {
    flush_window();  // behind the barrier: every old-window read is done
    const ChunkTables& T = sm.tab[j & 1];
    if (!sm.unsafe) {
      // wave 4: A over keys 0-63, 5: A over 64-127, 6 / 7: B likewise
      const uint32_t(*src)[kRowU] = pw < 2 ? T.kt : T.qt;
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int off = (4 * (2 * (pw & 1) + q) + gq) * 12;
        acc = mfma6(&src[c][off], &sm.kis[c][off], acc);
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
  auto prep_reduce = [&](int j) {
    if (sm.unsafe) return;
    const ChunkTables& T = sm.tab[j & 1];
    const int t = (tid & 255) >> 4;
    const int s = tid & 15;
    const float a = sm.part[0][t][s] + sm.part[1][t][s];
    const float b = sm.part[2][t][s] + sm.part[3][t][s];
    sm.LT[s][t] = s < t ? T.beta[t] * a : 0.0f;
    sm.B[t][s] = s <= t ? b : 0.0f;
  };

  // The wave's 32 columns of a segment's state, 2 blocks of 16, in the
  // accumulator layout: element (cb, kb, r) of lane l is row 16 kb +
  // 4 (l/16) + r, column 32 pw + 16 cb + l%16.  It moves as 16-byte rows:
  // a quad transpose gives lane l row 16 kb + 4 (l/16) + l%4, columns
  // 32 pw + 16 cb + 4 ((l%16)/4) .. +3.  Addressed as a wave-uniform base
  // per 16-row block, one 32-bit lane offset and immediate offsets (no
  // per-element 64-bit addresses to keep live).
  const uint32_t st_lane = ((4 * gq + (c & 3)) * kD + 4 * (c >> 2)) * 4;
  const bool q_odd1 = (c & 1) != 0;
  const bool q_odd2 = (c & 2) != 0;
  auto state_block = [&](const Seg& sg, int kb) {
    return uniform_gptr(p.rec_state +
                        (static_cast<int64_t>(sg.slot) * H + sg.h) *
                            (kD * kD) +
                        32 * pw + 16 * kb * kD);
  };
  auto load_block = [&](const Seg& sg, int kb, f4 (&S)[2][8]) {
    const gptr<const char> b = state_block(sg, kb);
    uint32_t lo = st_lane;
    asm volatile("" : "+v"(lo));
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      S[cb][kb] = *reinterpret_cast<gptr<const f4>>(b + lo + 64 * cb);
  };
  auto unpack_block = [&](int kb, f4 (&S)[2][8]) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      S[cb][kb] = quad_transpose(S[cb][kb], q_odd1, q_odd2);
  };
  auto store_block = [&](const Seg& sg, int kb, const f4 (&S)[2][8]) {
    gptr<char> b = const_cast<gptr<char>>(state_block(sg, kb));
    uint32_t lo = st_lane;
    asm volatile("" : "+v"(lo));
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      *reinterpret_cast<gptr<f4>>(b + lo + 64 * cb) =
          quad_transpose(S[cb][kb], q_odd1, q_odd2);
  };
  // ---- state stage: one chunk through the recurrence ---------------------
  auto state_chunk = [&](int j, f4 (&S)[2][8]) {
    const ChunkTables& T = sm.tab[j & 1];
    f4 ks[2], o[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      ks[cb] = f4{0.f, 0.f, 0.f, 0.f};
      o[cb] = f4{0.f, 0.f, 0.f, 0.f};
    }
    // per 32-key block P: the split K~ and Q~ rows (A operands) and the
    // state split in place (B operand: lane l holds S rows 32P + 4(l/16)
    // .. +3 and 32P + 16 + 4(l/16) .. +3 of its column, the order the split
    // rows use)
#pragma unroll
    for (int P = 0; P < 4; ++P) {
      const int off = (4 * P + gq) * 12;
      const u4 kh_ = ld_u4(&T.kt[c][off]), km_ = ld_u4(&T.kt[c][off + 4]),
               kl_ = ld_u4(&T.kt[c][off + 8]);
      const u4 qh_ = ld_u4(&T.qt[c][off]), qm_ = ld_u4(&T.qt[c][off + 4]),
               ql_ = ld_u4(&T.qt[c][off + 8]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const Split3 s0 = split3(S[cb][2 * P][0], S[cb][2 * P][1]);
        const Split3 s1 = split3(S[cb][2 * P][2], S[cb][2 * P][3]);
        const Split3 s2 = split3(S[cb][2 * P + 1][0], S[cb][2 * P + 1][1]);
        const Split3 s3 = split3(S[cb][2 * P + 1][2], S[cb][2 * P + 1][3]);
        const u4 sh = {s0.h, s1.h, s2.h, s3.h};
        const u4 sm_ = {s0.m, s1.m, s2.m, s3.m};
        const u4 sl = {s0.l, s1.l, s2.l, s3.l};
        ks[cb] = mfma6_(kh_, km_, kl_, sh, sm_, sl, ks[cb]);
        o[cb] = mfma6_(qh_, qm_, ql_, sh, sm_, sl, o[cb]);
      }
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
    // state update over the 16 tokens (k = 2 pieces x 4 tokens per lane
    // group): [K^hi | K^mid] against [Dhi; Dhi] and [Dmid; Dmid], and
    // [K^hi | K^lo] against [Dlo; Dhi] -- the six products of pieces down
    // to 2^-18 of the leading term
    u4 dh[2], dm[2], dx[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const Split3 d01 = split3(dl[cb][0], dl[cb][1]);
      const Split3 d23 = split3(dl[cb][2], dl[cb][3]);
      dh[cb] = u4{d01.h, d23.h, d01.h, d23.h};
      dm[cb] = u4{d01.m, d23.m, d01.m, d23.m};
      dx[cb] = u4{d01.l, d23.l, d01.h, d23.h};
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const f4 gm = ld4(&T.gam[16 * kb + 4 * gq]);
      const u4 ahm = ld_u4(&T.kh[16 * kb + c][8 * gq]);
      const u4 ahl = ld_u4(&T.kh[16 * kb + c][8 * gq + 4]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        S[cb][kb] *= gm;
        S[cb][kb] = mfma_bf(ahl, dx[cb], S[cb][kb]);
        S[cb][kb] = mfma_bf(ahm, dm[cb], S[cb][kb]);
        S[cb][kb] = mfma_bf(ahm, dh[cb], S[cb][kb]);
      }
    }
  };

  // ---- state stage: gated RMSNorm and bf16 outputs of a chunk ------------
  auto emit = [&](const Seg& g, int ci, u4 gate_raw) {
    const int c0 = ci * kC;
    const int nv = g.len - c0 < kC ? g.len - c0 : kC;
    const int64_t tb = g.tb;
    const int64_t col0 = static_cast<int64_t>(g.h) * kD;
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
  // Each role runs a loop of its own (the state lives only in the state
  // waves' loop, so the prep code does not carry its registers); both walk
  // the sequence's chunks in order and meet at the same barriers: 3 before
  // the first chunk, then 3 per chunk.
  if (state_wave) {
    auto gate_row = [&](const Seg& sg, int ci) -> u4 {
      u4 gate_raw = {0u, 0u, 0u, 0u};
      if (kNorm) {
        const int nv = sg.len - ci * kC < kC ? sg.len - ci * kC : kC;
        const int rr = ot < nv - 1 ? ot : nv - 1;
        gate_raw = *reinterpret_cast<const u4*>(
            p.gate + (sg.tb + ci * kC + rr) * C +
            static_cast<int64_t>(sg.h) * kD + oc);
      }
      return gate_raw;
    };
    f4 S[2][8];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) load_block(seg, kb, S);
    __syncthreads();  // first chunk's tables (and the norm weight)
    __syncthreads();  // its partial products
    __syncthreads();  // its A and B
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) unpack_block(kb, S);
    for (int ci = 0; ci < seg.nch; ++ci) {
      const u4 gate_raw = gate_row(seg, ci);
      state_chunk(ci, S);
      __syncthreads();  // outputs in sm.o; next chunk's tables ready
      emit(seg, ci, gate_raw);
      __syncthreads();  // next chunk's partial products
      __syncthreads();  // next chunk's A and B
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) store_block(seg, kb, S);
  } else {
    // chunk ci is prepared while chunk ci - 1 runs; the inputs of the chunk
    // after it (or its own again, after the last) are requested meanwhile
    load_constants(seg);
    load_chunk(seg, 0);
    prep_tables(std::false_type{}, seg, 0, 0, seg, seg.nch > 1 ? 1 : 0);
    __syncthreads();
    prep_gram(0);
    __syncthreads();
    prep_reduce(0);
    __syncthreads();
    for (int ci = 1; ci < seg.nch; ++ci) {
      const int cn = ci + 1 < seg.nch ? ci + 1 : ci;
      if (seg.len - ci * kC >= kC && conv_update)
        prep_tables(std::true_type{}, seg, ci, ci, seg, cn);
      else
        prep_tables(std::false_type{}, seg, ci, ci, seg, cn);
      __syncthreads();
      prep_gram(ci);
      __syncthreads();
      prep_reduce(ci);
      __syncthreads();
    }
    // the last chunk: nothing left to prepare
    __syncthreads();
    __syncthreads();
    __syncthreads();
  }
}

// ===========================================================================
// Short rows: the multi-token decode of rows of tokens_per_row tokens in
// chunks of kS = 8, one 256-thread workgroup per (row, head) and several
// workgroups per compute unit (four for rows of one chunk, three for longer
// rows, whose state stays in registers from chunk to chunk), so that the
// state of some units moves while others compute (the hardware dispatcher
// interleaves them; there is no pipeline inside a workgroup).  The algebra
// is the chunk form above with at most 8 tokens per chunk, which lets K~
// (rows 0-7) and Q~ (rows 8-15) share one 16-row A operand: K~ S and Q~ S
// are one product.
//   * wave w owns value columns 32w .. 32w+31 of the state, held in the
//     accumulator layout with the columns taken in pairs: lane l holds
//     columns 32w + 2(l%16) and 32w + 2(l%16) + 1 (the two 16-column
//     blocks cb = 0, 1 of the MFMAs -- any column order serves, as long as
//     v, Delta and the outputs use the same) and key rows 4(l/16) .. +3 of
//     each 16-row block, so the state moves as one 8-byte access per lane
//     and key row, a full 128-byte line per row and wave.
//   * wave w prepares tokens 2w, 2w+1 for every channel (conv + SiLU, L2
//     norms, decays, split tables), then one 16x8 Gram block over its 32
//     keys: [K~; Q~] (K e^{-G})^T; with a large decay each wave sums the
//     rows of its own tokens exactly instead.  The partial blocks are
//     summed after a barrier.
//   * the state loads issue after the tables, right before the first
//     barrier: issued earlier they hold the small input loads of the next
//     workgroups on the compute unit behind 64 KiB each (measured on
//     MI355X at 256 rows x 48 heads x 8 tokens: 375 against 327 us), and
//     the prep registers would not leave room for four workgroups.
//   * the solve uses the duplicated inverse [T 0; T 0] (16x16), so lane
//     groups 0-1 and 2-3 of the accumulator both hold Delta of tokens
//     0 .. 7; the state update packs four piece products per MFMA (groups
//     0-1: K^hi Dhi + K^mid Dhi, then K^mid Dmid + K^lo Dhi; groups 2-3:
//     K^hi Dmid + K^hi Dlo, then K^mid Dlo + K^lo Dmid).
constexpr int kS = 8;            // tokens per chunk
constexpr int kSThreads = 256;   // 4 waves
constexpr int kKhS = 16 + 4;     // dwords per split K^ key row (+ pad)

struct alignas(16) ShortSmem {
  uint32_t kq[2 * kS][kRowU];  // rows t: k_t e^{G_t}; 8 + t: q_t e^{G_t}
  float v[kS][kLd];            // v_t
  // K^ of each key, as the update's A operands: dwords 0-7 [hi | mid] of
  // tokens 0-3 then 4-7, dwords 8-15 [mid | lo] likewise (bf16 pairs)
  uint32_t kh[kD][kKhS];
  float gam[kD];               // e^{G_last}
  float beta[kS];
  union {
    uint32_t kis[kS][kRowU];   // k_t e^{-G_t}, split (matrix-core Gram)
    struct {
      float ki[kS][kLd];       // exact Gram: k_t
      float graw[kS][kLd];     // cumulative log2 decay
    } ex;
    float o[kS][kLd];          // outputs before the norm (after the Gram)
  } u;
  float part[4][2 * kS][kS];   // Gram partials (per key block or wave)
  float LT[kS][kS + 4];  // LT[s][t] = beta_t A_ts for s < t, else 0
  float Bm[kS][kS + 4];  // B_ts for s <= t, else 0
  float nw[kD];
  int unsafe;
};
// four workgroups per compute unit: 160 KiB of LDS, 128 VGPRs per lane
static_assert(4 * sizeof(ShortSmem) <= 160 * 1024, "short-row LDS");
// Rows of several chunks keep the outputs in a buffer of their own, so that
// the next chunk's tables can be written while they are emitted.
struct ShortOut {
  float o[kS][kLd];
};
struct ShortNoOut {};

template <bool kNorm, bool kMulti>
__global__ __launch_bounds__(kSThreads)
__attribute__((amdgpu_waves_per_eu(kMulti ? 3 : 4)))
void kda_short_rows_kernel(KdaChunkedArgs p) {
  __shared__ ShortSmem sm;
  __shared__ typename std::conditional<kMulti, ShortOut, ShortNoOut>::type so;
  float(*obuf)[kLd];
  if constexpr (kMulti)
    obuf = so.o;
  else
    obuf = sm.u.o;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.heads;
  const int C = H * kD;
  const int C3 = 3 * C;
  const int T = p.tokens_per_row;  // tokens of the row
  const int unit = static_cast<int>(blockIdx.x);
  const int n = unit / H;
  const int h = unit - n * H;
  const int64_t tb = static_cast<int64_t>(n) * T;  // first token of the row
  const int64_t col0 = static_cast<int64_t>(h) * kD;
  const int slot = p.state_idx[n];
  if (slot <= 0 || slot >= p.num_slots) {
    // null row: +0.0 outputs, no state traffic
    for (int i = tid; i < T * (kD / 8); i += kSThreads)
      *reinterpret_cast<u4*>(p.out + (tb + i / (kD / 8)) * C + col0 +
                             8 * (i % (kD / 8))) = u4{0u, 0u, 0u, 0u};
    return;
  }
  const uint32_t flags = p.flags;
  const bool tap_major = (flags & KDA_CONV_TAP_MAJOR) != 0;
  const bool conv_update = (flags & KDA_NO_CONV_UPDATE) == 0;
  const bool l2 = (flags & KDA_QK_L2NORM) != 0;
  const bool gate_silu = (flags & KDA_GATE_SILU) != 0;

  // the state: element (cb, kb, r) of lane l is key row 16 kb + 4 (l/16) +
  // r, column 32 w + 2 (l%16) + cb
  f4 S[2][8];
  const float* st_base =
      p.rec_state + (static_cast<int64_t>(slot) * H + h) * (kD * kD) + 32 * wave;
  // the row's tokens in chunks of kS
  const int nch = kMulti ? (T + kS - 1) / kS : 1;
  for (int ch = 0; ch < nch; ++ch) {
    const int c0 = ch * kS;
    const int nv = T - c0 < kS ? T - c0 : kS;  // tokens of this chunk
    const bool last = ch + 1 == nch;
    // lane-derived values from an opaque copy of the thread id, so that no
    // per-lane address stays live across the chunks
    int tid_l = tid;
    asm volatile("" : "+v"(tid_l));
    const int lane = tid_l & 63;
    const int c = lane & 15;
    const int gq = lane >> 4;
    const uint32_t st_lane = (4 * gq * kD + 2 * c) * 4;
    // ---- inputs of tokens 2w, 2w+1, channels 2 lane, 2 lane + 1 --------
    // input rows 2w-3 .. 2w+1 of the chunk (clamped into the row; rows
    // before the row come from the stored window)
    uint32_t raw[3][5];
    {
      const char* q0 = reinterpret_cast<const char*>(p.qkv + tb * C3 + col0);
#pragma unroll
      for (int u = 0; u < 5; ++u) {
        const int rel = 2 * wave - 3 + u;
        const int ra = c0 + rel;  // row-relative
        const int rr = ra < 0 ? 0 : (ra < T - 1 ? ra : T - 1);
        const gptr<const char> row = uniform_gptr(q0 + rr * (2 * C3));
#pragma unroll
        for (int pp = 0; pp < 3; ++pp)
          raw[pp][u] = load_at<uint32_t>(row, 4 * lane + pp * (2 * C));
      }
    }
    // the stored conv window (tap-major: the channel pair in [0];
    // channel-major: one channel in each of [0], [1])
    uint32_t wv[2][3][kW - 1] = {};
    if (ch == 0 || !conv_update) {
      // the slot's window as a uniform base (this head's first channel)
      // plus 32-bit lane offsets
      const gptr<const char> wb = uniform_gptr(
          p.conv_state + static_cast<int64_t>(slot) * (kW - 1) * C3 +
          (tap_major ? col0 : col0 * (kW - 1)));
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
#pragma unroll
        for (int e = 0; e < kW - 1; ++e) {
          // the channel relative to the head's first
          const uint32_t chr = pp * C + 2 * lane;
          if (tap_major) {
            wv[0][pp][e] = load_at<uint32_t>(wb, 2 * (e * C3 + chr));
            wv[1][pp][e] = 0u;
          } else {
            wv[0][pp][e] = load_at<uint16_t>(wb, 2 * (chr * (kW - 1) + e));
            wv[1][pp][e] =
                load_at<uint16_t>(wb, 2 * ((chr + 1) * (kW - 1) + e));
          }
        }
    }
    // decays of keys 2 lane, 2 lane + 1 for every token of the chunk
    u2 in_g[kS];
    {
      const char* gb = reinterpret_cast<const char*>(p.g + (tb * H + h) * kD);
#pragma unroll
      for (int t = 0; t < kS; ++t) {
        const int rr = c0 + t < T - 1 ? c0 + t : T - 1;
        in_g[t] = load_at<u2>(uniform_gptr(gb + rr * (H * kD * 4)), 8 * lane);
      }
    }
    float bt = 0.0f;  // beta of token 2w + lane (lanes 0, 1)
    if (lane < 2) {
      const int t = 2 * wave + lane;
      bt = p.beta[(tb + (c0 + t < T ? c0 + t : T - 1)) * H + h];
    }
    // (reloaded per chunk from the cache rather than held across chunks:
    // load_at keeps the loads in the loop)
    const gptr<const char> cwb = uniform_gptr(p.conv_w + col0);
    f2 cwv[3][kW];
#pragma unroll
    for (int pp = 0; pp < 3; ++pp)
#pragma unroll
      for (int tap = 0; tap < kW; ++tap)
        cwv[pp][tap] =
            load_at<f2>(cwb, 4 * ((pp * kW + tap) * C + 2 * lane));
    if (ch == 0 && tid_l >= 128 && tid_l < 128 + kD)
      sm.nw[tid_l - 128] = kNorm ? p.norm_w[tid_l - 128] : 0.0f;

    // ---- prep -----------------------------------------------------------
    // cumulative decay (log2 units) over the chunk, its value at this
    // wave's tokens and at the chunk's last one
    f2 G = {0.f, 0.f};
    f2 Gu[2] = {{0.f, 0.f}, {0.f, 0.f}};
    float gmax = 0.0f;
    // one copy per wave, so that picking the wave's own tokens costs no
    // selects
    auto prefix = [&](auto W) {
      constexpr int w = decltype(W)::value;
#pragma unroll
      for (int t = 0; t < kS; ++t) {
        f2 gl =
            f2{__uint_as_float(in_g[t].x), __uint_as_float(in_g[t].y)} * kLog2e;
        gl = kda_decay_floor2(gl);
        if (t < nv) G += gl;
        gmax = fmaxf(gmax, fmaxf(fabsf(G.x), fabsf(G.y)));
        if (t == 2 * w) Gu[0] = G;
        if (t == 2 * w + 1) Gu[1] = G;
      }
    };
    switch (wave) {
      case 0: prefix(std::integral_constant<int, 0>{}); break;
      case 1: prefix(std::integral_constant<int, 1>{}); break;
      case 2: prefix(std::integral_constant<int, 2>{}); break;
      default: prefix(std::integral_constant<int, 3>{}); break;
    }
    // NaN counts as unsafe; the same verdict in every wave
    const bool unsafe = __any(!(gmax <= kSafeExp2));
    // conv + SiLU
    uint32_t wc[3][kW - 1];
#pragma unroll
    for (int pp = 0; pp < 3; ++pp)
#pragma unroll
      for (int e = 0; e < kW - 1; ++e)
        wc[pp][e] = wv[0][pp][e] | (wv[1][pp][e] << 16);
    float y[2][3][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bool valid = 2 * wave + u < nv;
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float a = 0.0f;
#pragma unroll
          for (int tap = 0; tap < kW; ++tap) {
            // input row of this tap relative to the chunk start: 2w + u -
            // 3 + tap; only waves 0 and 1 of the first chunk reach before
            // the row (compile-time indices)
            const int r0 = u - (kW - 1) + tap;  // for wave 0
            uint32_t w2 = raw[pp][u + tap];
            if (tap < kW - 1) {
              if (conv_update) {
                if (ch == 0 && r0 < 0 && wave == 0)
                  w2 = wc[pp][r0 < 0 ? (kW - 1) + r0 : 0];
                if (ch == 0 && r0 + 2 < 0 && wave == 1)
                  w2 = wc[pp][r0 + 2 < 0 ? (kW - 1) + r0 + 2 : 0];
              } else {
                w2 = wc[pp][tap];
              }
            }
            a += cwv[pp][tap][e] * (e ? bf16_hi(w2) : bf16_lo(w2));
          }
          y[u][pp][e] = valid ? a * sigmoid_(a) : 0.0f;
        }
    }
    // the new conv window: the row's last W-1 inputs (older ones from the
    // stored window for rows shorter than that), held in the last chunk by
    // wave (nv-1)/2 and written after its first barrier, once every wave has
    // read the old one
    const bool win_wave = conv_update && last && wave == (nv - 1) / 2;
    uint32_t win_new[3][kW - 1];
    if (win_wave) {
#pragma unroll
      for (int e = 0; e < kW - 1; ++e) {
        const int idx = T - (kW - 1) + e;          // token in the row
        const int u = idx - c0 - (2 * wave - 3);   // its input row, 0..4
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) {
          uint32_t w = raw[pp][0];
#pragma unroll
          for (int q = 1; q < 5; ++q)
            if (u == q) w = raw[pp][q];
          if (idx < 0) {
            w = wc[pp][0];
#pragma unroll
            for (int q = 1; q < kW - 1; ++q)
              if (idx + (kW - 1) == q) w = wc[pp][q];
          }
          win_new[pp][e] = w;
        }
      }
    }
    if (l2) {
      float ss[4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        ss[2 * u] = y[u][0][0] * y[u][0][0] + y[u][0][1] * y[u][0][1];
        ss[2 * u + 1] = y[u][1][0] * y[u][1][0] + y[u][1][1] * y[u][1][1];
      }
      wave_sum<4>(ss);
      const float qscale = 0.08838834764831845f;  // D^-1/2
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float rq = rsqrtf(ss[2 * u] + 1e-6f);
        const float rk = rsqrtf(ss[2 * u + 1] + 1e-6f);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          y[u][0][e] = (y[u][0][e] * rq) * qscale;
          y[u][1][e] = y[u][1][e] * rk;
        }
      }
    }
    // split tables
    {
      const int m = lane & 15;
      const int pos = (4 * (lane >> 4) + ((m & 7) >> 1)) * 12 +
                      (m >= 8 ? 2 : 0) + (m & 1);
      auto put3 = [&](uint32_t* row, float a, float b) {
        const Split3 x = split3(a, b);
        row[pos] = x.h;
        row[pos + 4] = x.m;
        row[pos + 8] = x.l;
      };
      const f2 eG = {exp2_(G.x), exp2_(G.y)};
      f2 khv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = 2 * wave + u;
        const f2 ee = {exp2_(Gu[u].x), exp2_(Gu[u].y)};
        put3(sm.kq[t], y[u][1][0] * ee.x, y[u][1][1] * ee.y);
        put3(sm.kq[kS + t], y[u][0][0] * ee.x, y[u][0][1] * ee.y);
        *reinterpret_cast<f2*>(&sm.v[t][2 * lane]) = f2{y[u][2][0], y[u][2][1]};
        if (!unsafe) {
          const f2 ei = {exp2_(-Gu[u].x), exp2_(-Gu[u].y)};
          khv[u] = f2{(y[u][1][0] * eG.x) * ei.x, (y[u][1][1] * eG.y) * ei.y};
          put3(sm.u.kis[t], y[u][1][0] * ei.x, y[u][1][1] * ei.y);
        } else {
          khv[u] = f2{y[u][1][0] * exp2_(G.x - Gu[u].x),
                      y[u][1][1] * exp2_(G.y - Gu[u].y)};
          *reinterpret_cast<f2*>(&sm.u.ex.ki[t][2 * lane]) =
              f2{y[u][1][0], y[u][1][1]};
          *reinterpret_cast<f2*>(&sm.u.ex.graw[t][2 * lane]) = Gu[u];
        }
      }
      // K^ pieces of tokens 2w, 2w+1 (one bf16 pair per piece) into the
      // operand slots of both update products
      const int q4 = 4 * (wave >> 1) + (wave & 1);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const Split3 a = split3(khv[0][e], khv[1][e]);
        uint32_t* row = sm.kh[2 * lane + e];
        row[q4] = a.h;
        row[q4 + 2] = a.m;
        row[8 + q4] = a.m;
        row[8 + q4 + 2] = a.l;
      }
      if (wave == 0) {
        *reinterpret_cast<f2*>(&sm.gam[2 * lane]) = eG;
        if (lane == 0) sm.unsafe = unsafe ? 1 : 0;
      }
      if (lane < 2) {
        const int t = 2 * wave + lane;
        sm.beta[t] = t < nv ? bt : 0.0f;
      }
    }

    // ---- the state (first chunk; it stays in registers across the chunks)
    if (ch == 0) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const gptr<const char> b = uniform_gptr(st_base + 16 * kb * kD);
        uint32_t lo = st_lane;
        asm volatile("" : "+v"(lo));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f2 v2 = __builtin_nontemporal_load(
              reinterpret_cast<gptr<const f2>>(b + lo + r * kD * 4));
          S[0][kb][r] = v2.x;
          S[1][kb][r] = v2.y;
        }
      }
    }
    __syncthreads();  // tables
    // every wave's reads of the old window are done: the new one goes out
    if (win_wave) {
#pragma unroll
      for (int e = 0; e < kW - 1; ++e)
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) {
          const uint32_t w = win_new[pp][e];
          const int64_t chn = static_cast<int64_t>(pp) * C + col0 + 2 * lane;
          if (tap_major) {
            *reinterpret_cast<uint32_t*>(
                p.conv_state +
                (static_cast<int64_t>(slot) * (kW - 1) + e) * C3 + chn) = w;
          } else {
            uint16_t* cs =
                p.conv_state +
                (static_cast<int64_t>(slot) * C3 + chn) * (kW - 1) + e;
            cs[0] = static_cast<uint16_t>(w);
            cs[kW - 1] = static_cast<uint16_t>(w >> 16);
          }
        }
    }

    // ---- Gram block of keys 32w .. 32w+31 -----------------------------
    if (!sm.unsafe) {
      const int off = (4 * wave + gq) * 12;
      const u4 z = {0u, 0u, 0u, 0u};
      const bool bc = c < kS;
      const u4 bh = bc ? ld_u4(&sm.u.kis[c & 7][off]) : z;
      const u4 bm = bc ? ld_u4(&sm.u.kis[c & 7][off + 4]) : z;
      const u4 bl = bc ? ld_u4(&sm.u.kis[c & 7][off + 8]) : z;
      const f4 acc =
          mfma6_(ld_u4(&sm.kq[c][off]), ld_u4(&sm.kq[c][off + 4]),
                 ld_u4(&sm.kq[c][off + 8]), bh, bm, bl, f4{0.f, 0.f, 0.f, 0.f});
      if (c < kS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.part[wave][4 * gq + r][c] = acc[r];
      }
    } else {
      // large decay: each wave sums the rows of its own tokens exactly (one
      // exponential per (t, s, key), k_s and G_s from LDS)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = 2 * wave + u;
        float ab[2 * kS];  // [A, B][s]
#pragma unroll
        for (int i = 0; i < 2 * kS; ++i) ab[i] = 0.0f;
        const f2 kt2 = *reinterpret_cast<const f2*>(&sm.u.ex.ki[t][2 * lane]);
        const f2 gt2 = *reinterpret_cast<const f2*>(&sm.u.ex.graw[t][2 * lane]);
#pragma unroll
        for (int s_ = 0; s_ < kS; ++s_) {
          if (s_ > t) continue;
          const f2 ks2 =
              *reinterpret_cast<const f2*>(&sm.u.ex.ki[s_][2 * lane]);
          const f2 gs2 =
              *reinterpret_cast<const f2*>(&sm.u.ex.graw[s_][2 * lane]);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float ks = ks2[e] * exp2_(gt2[e] - gs2[e]);
            ab[s_] += kt2[e] * ks;
            ab[kS + s_] += y[u][0][e] * ks;
          }
        }
        wave_sum<2 * kS>(ab);
        // lane i < 16 writes entry i of row t of A (i < 8) or B (part 0 holds
        // the sum, parts 1-3 zero)
        float val = 0.0f;
#pragma unroll
        for (int i = 0; i < 2 * kS; ++i)
          if (lane == i) val = ab[i];
        if (lane < 2 * kS) {
          const int row = (lane >= kS ? kS : 0) + t;
          const int s_ = lane & 7;
          sm.part[0][row][s_] = val;
          sm.part[1][row][s_] = 0.0f;
          sm.part[2][row][s_] = 0.0f;
          sm.part[3][row][s_] = 0.0f;
        }
      }
    }
    __syncthreads();  // Gram partials
    if (tid_l < kS * kS) {
      const int t = tid_l >> 3;
      const int s_ = tid_l & 7;
      const float a = (sm.part[0][t][s_] + sm.part[1][t][s_]) +
                      (sm.part[2][t][s_] + sm.part[3][t][s_]);
      const float b = (sm.part[0][kS + t][s_] + sm.part[1][kS + t][s_]) +
                      (sm.part[2][kS + t][s_] + sm.part[3][kS + t][s_]);
      sm.LT[s_][t] = s_ < t ? sm.beta[t] * a : 0.0f;
      sm.Bm[t][s_] = s_ <= t ? b : 0.0f;
    }
    __syncthreads();  // A and B
    // output lanes: token tid/32 (half a wave), columns 4 (tid%32) .. +3
    const int ot = tid_l >> 5;
    const int oc = 4 * (tid_l & 31);
    u2 gate_raw = {0u, 0u};
    if (kNorm) {
      const int rr = c0 + ot < T - 1 ? c0 + ot : T - 1;
      gate_raw =
          *reinterpret_cast<const u2*>(p.gate + (tb + rr) * C + col0 + oc);
    }

    // ---- the chunk through the recurrence -----------------------------
    // X = [K~; Q~] S: accumulator rows 0-7 are K~ S, rows 8-15 Q~ S
    f4 X[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int P = 0; P < 4; ++P) {
      const int off = (4 * P + gq) * 12;
      const u4 ah = ld_u4(&sm.kq[c][off]), am = ld_u4(&sm.kq[c][off + 4]),
               al = ld_u4(&sm.kq[c][off + 8]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const Split3 s0 = split3(S[cb][2 * P][0], S[cb][2 * P][1]);
        const Split3 s1 = split3(S[cb][2 * P][2], S[cb][2 * P][3]);
        const Split3 s2 = split3(S[cb][2 * P + 1][0], S[cb][2 * P + 1][1]);
        const Split3 s3 = split3(S[cb][2 * P + 1][2], S[cb][2 * P + 1][3]);
        X[cb] = mfma6_(ah, am, al, u4{s0.h, s1.h, s2.h, s3.h},
                       u4{s0.m, s1.m, s2.m, s3.m}, u4{s0.l, s1.l, s2.l, s3.l},
                       X[cb]);
      }
    }
    // row (c mod 8) of T = (I + L)^{-1}: (I + L)^T y = e_row, backward
    const int rc = c & 7;
    float yv[kS];
#pragma unroll
    for (int t = kS - 1; t >= 0; --t) {
      float v = t == rc ? 1.0f : 0.0f;
#pragma unroll
      for (int s4 = 0; s4 < kS; s4 += 4) {
        if (s4 + 3 <= t) continue;
        const f4 lt = ld4(&sm.LT[t][s4]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (s4 + q > t) v -= lt[q] * yv[s4 + q];
      }
      yv[t] = v;
    }
    // A operands of the two small fp32 products, per k = 4 gq + j: the
    // inverse [T 0; T 0] and [0 0; B 0]
    f4 at, ab;
    {
      const f4 bl = ld4(&sm.Bm[rc][4 * (gq & 1)]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        at[j] = gq == 0 ? yv[j] : gq == 1 ? yv[4 + j] : 0.0f;
        ab[j] = (c >= kS && gq < 2) ? bl[j] : 0.0f;
      }
    }
    f4 dl[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int col = 32 * wave + 2 * c + cb;
      f4 br;  // beta (V - K~ S) of tokens 4 gq + r (groups 0-1; else 0)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * (gq & 1) + r;
        br[r] = gq < 2 ? sm.beta[t] * (sm.v[t][col] - X[cb][r]) : 0.0f;
      }
      dl[cb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) dl[cb] = mfma(at[j], br[j], dl[cb]);
#pragma unroll
      for (int j = 0; j < 4; ++j) X[cb] = mfma(ab[j], dl[cb][j], X[cb]);
      if (gq >= 2) {
#pragma unroll
        for (int r = 0; r < 4; ++r) obuf[4 * (gq - 2) + r][col] = X[cb][r];
      }
    }
    // state update: e^{G_last} S + K^T Delta
    u4 b1[2], b2[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const Split3 d01 = split3(dl[cb][0], dl[cb][1]);
      const Split3 d23 = split3(dl[cb][2], dl[cb][3]);
      b1[cb] = gq < 2 ? u4{d01.h, d23.h, d01.h, d23.h}
                      : u4{d01.m, d23.m, d01.l, d23.l};
      b2[cb] = gq < 2 ? u4{d01.m, d23.m, d01.h, d23.h}
                      : u4{d01.l, d23.l, d01.m, d23.m};
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const f4 gm = ld4(&sm.gam[16 * kb + 4 * gq]);
      u4 a1 = ld_u4(&sm.kh[16 * kb + c][4 * (gq & 1)]);
      if (gq >= 2) a1 = u4{a1.x, a1.y, a1.x, a1.y};
      const u4 a2 = ld_u4(&sm.kh[16 * kb + c][8 + 4 * (gq & 1)]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        S[cb][kb] *= gm;
        S[cb][kb] = mfma_bf(a1, b1[cb], S[cb][kb]);
        S[cb][kb] = mfma_bf(a2, b2[cb], S[cb][kb]);
      }
    }
    // the state back after the last chunk, in the layout it came in
    if (last) {
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        gptr<char> b =
            const_cast<gptr<char>>(uniform_gptr(st_base + 16 * kb * kD));
        uint32_t lo = st_lane;
        asm volatile("" : "+v"(lo));
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __builtin_nontemporal_store(
              f2{S[0][kb][r], S[1][kb][r]},
              reinterpret_cast<gptr<f2>>(b + lo + r * kD * 4));
      }
    }
    __syncthreads();  // outputs in obuf

    // ---- gated RMSNorm and bf16 outputs: 32 lanes per token -----------
    // (a row of several chunks goes on to the next chunk's tables without
    // waiting: nothing reads them after the barrier above, and its outputs
    // have a buffer of their own)
    {
      const f4 ov = ld4(&obuf[ot][oc]);
      float yo[4] = {ov.x, ov.y, ov.z, ov.w};
      if (kNorm) {
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) ss += yo[j] * yo[j];
        // the two tokens' sums: rows 0 + 1 in row 1, rows 2 + 3 in row 3
        ss = row_sum16(ss);
        ss += dpp_rows_<0x142, 0xA>(ss);
        const float s_lo = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ss), 31));
        const float s_hi = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ss), 63));
        const float rs =
            rsqrtf((lane < 32 ? s_lo : s_hi) * (1.0f / kD) + p.eps);
        const f4 nw = ld4(&sm.nw[oc]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w2 = gate_raw[j >> 1];
          const float gv = (j & 1) ? bf16_hi(w2) : bf16_lo(w2);
          const float ga = gate_silu ? gv * sigmoid_(gv) : sigmoid_(gv);
          yo[j] = ((yo[j] * rs) * nw[j]) * ga;
        }
      }
      if (ot < nv) {
        const u2 pk = {pack_bf16(yo[0], yo[1]), pack_bf16(yo[2], yo[3])};
        *reinterpret_cast<u2*>(p.out + (tb + c0 + ot) * C + col0 + oc) = pk;
      }
    }
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
  // one (sequence, head) per workgroup
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(num_seqs) *
                                        args.heads));
  if (!args.rg.raw_g)
    launch_gate<kGateInput>(args, grid, stream);
  else if (args.flags & KDA_BOUNDED_GATE)
    launch_gate<kGateBounded>(args, grid, stream);
  else
    launch_gate<kGateSoftplus>(args, grid, stream);
  return hipGetLastError();
}

hipError_t kda_short_rows_launch(const KdaChunkedArgs& args, int32_t num_rows,
                                 hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(num_rows) *
                                        args.heads));
  const bool norm = (args.flags & KDA_OUTPUT_NORM) != 0;
  if (args.tokens_per_row > kS) {
    if (norm)
      hipLaunchKernelGGL((kda_short_rows_kernel<true, true>), grid,
                         dim3(kSThreads), 0, stream, args);
    else
      hipLaunchKernelGGL((kda_short_rows_kernel<false, true>), grid,
                         dim3(kSThreads), 0, stream, args);
  } else if (norm) {
    hipLaunchKernelGGL((kda_short_rows_kernel<true, false>), grid,
                       dim3(kSThreads), 0, stream, args);
  } else {
    hipLaunchKernelGGL((kda_short_rows_kernel<false, false>), grid,
                       dim3(kSThreads), 0, stream, args);
  }
  return hipGetLastError();
}
