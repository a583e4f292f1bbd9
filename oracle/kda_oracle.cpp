// CPU oracle of the fused single-token KDA decode step.
//
// TEST INFRASTRUCTURE ONLY.  This library is the correctness reference for
// the HIP path.  Only the test suite, the smoke check and the benchmark's
// CPU-baseline leg may load it; the product path never calls it and shares
// no source with it (its own bf16 conversion, its own indexing, its own
// status codes).
//
// What it computes.  The page "PR #50654 完整报告 -- [ROCm][Perf] Kimi-K3
// Fused kernel for KDA decode" (sections "Feature and motivation" and
// "Implementation breakdown", item 1) describes one decode token per
// sequence and, for each (sequence, value head), three steps in order:
// advance the causal conv1d state, run the gated delta-rule recurrence on a
// [128, 128] fp32 state, apply a gated RMSNorm.  The page gives neither the
// equations nor eps; the plainest readings used here are:
//
//   conv (per channel c, width W, causal cross-correlation):
//       window = (cs[c][0], ..., cs[c][W-2], x[c])      oldest first
//       a      = sum_t w[t][c] * window[t]              tap W-1 = current
//       y[c]   = a * sigmoid(a)                          SiLU, on q, k and v
//       cs[c]  = window[1..W-1]                          exact bf16 copy
//     The weight is the width-major fp32 mirror [3, W, C] of a depthwise
//     Conv1d weight, as the page's conv weight loader builds it ("Key
//     source excerpts", kda_decode.py).
//   recurrence (per unit; S[i][j], i = key index, j = value index):
//       Sd[i][j] = exp(g[i]) * S[i][j]                  per-key-channel decay
//       u[j]     = sum_i k[i] * Sd[i][j]
//       delta[j] = beta * (v[j] - u[j])
//       S'[i][j] = Sd[i][j] + k[i] * delta[j]            written back
//       o[j]     = sum_i q[i] * S'[i][j]                 readout from S'
//   gated RMSNorm (norm on; over the D outputs of one head):
//       r    = 1 / sqrt(sum_j o[j]^2 / D + eps)
//       y[j] = o[j] * r * norm_w[j] * sigmoid(gate[j])
//     norm off: y[j] = o[j].  Output is bf16, round-to-nearest-even.
//   null rows ("Key source excerpts", the kernel's padding-row branch): a
//     row whose slot is <= 0 writes +0.0 to its outputs and reads or writes
//     no state.  A slot >= num_slots is treated the same way (memory safety;
//     not on the page).
//
// Variants selected by flag bits (the page's kernel has template switches
// for the output norm, for updating the conv state and for a "safe" gate,
// and its op takes raw gate inputs and a conv bias; "Implementation
// breakdown", item 1, and the kda.py excerpt):
//   0x01 output norm on;  0x02 conv state read but not written;
//   0x04 conv state stored [slot][tap][channel] instead of
//        [slot][channel][tap] (the page's physical layout, which it hands
//        to the kernel as a transposed view);
//   0x08 q and k L2-normalised after the conv, q also scaled by D^-1/2:
//        x <- x / sqrt(sum x^2 + 1e-6)  (not on the page);
//   0x10 output gate activation x * sigmoid(x) instead of sigmoid(x);
//   0x20 with raw gates: the bounded gate below.
// Raw gates (the page passes raw_g, A_log, dt_bias, lower_bound and
// raw_beta; their formula is not on the page, so this is a reading):
//   z = raw_g[i] + dt_bias[h*D+i];  a = exp(A_log[h])
//   g = -a * softplus(z)                      (default)
//   g = lower_bound * sigmoid(a * z)          (flag 0x20; lower_bound < 0)
//   beta = sigmoid(raw_beta);  softplus(z) = z for z > 20, else log1p(e^z).
// Conv bias (optional): a = bias[c] + sum_t w[t][c] * window[t].
//
// Every step is written out literally and unfused, sums run in index order
// with a separate multiply and add (built with -ffp-contract=off), and the
// whole step exists in fp32 (the page's state precision) and in fp64 (for
// the oracle's own self-checks).
//
// Parity status of each function: see the test suite's pins; all stage
// functions are pinned (closed forms, special cases reducing to torch
// library routines, brute force on tiny shapes).

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

enum : int {
  ORC_OK = 0,
  ORC_ERR_INVALID_ARG = 1,
};

// ---- bf16 from its definition: the top 16 bits of an IEEE binary32 ----

float bf16_to_f32(uint16_t h) {
  uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

// Round-to-nearest-even to 8 significand bits.  NaN stays a quiet NaN.
uint16_t f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u)
    return static_cast<uint16_t>((u >> 16) | 0x0040u);
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> T sigmoid(T x) { return T(1) / (T(1) + std::exp(-x)); }

template <typename T> T softplus(T x) {
  return x > T(20) ? x : std::log1p(std::exp(x));
}

// Raw gate of one key channel (see the header): default or bounded form.
template <typename T>
T gate_from_raw(T raw, T a_log, T bias, int bounded, T lower_bound) {
  const T z = raw + bias;
  const T a = std::exp(a_log);
  if (bounded) return lower_bound * sigmoid(a * z);
  return -(a * softplus(z));
}

// x <- x / sqrt(sum x^2 + 1e-6) * scale
template <typename T> void l2_normalize(int D, T* x, T scale) {
  T ss = T(0);
  for (int i = 0; i < D; ++i) {
    const T sq = x[i] * x[i];
    ss = ss + sq;
  }
  const T r = T(1) / std::sqrt(ss + T(1e-6));
  for (int i = 0; i < D; ++i) x[i] = (x[i] * r) * scale;
}

// ---- stage 1: causal conv update of one channel -------------------------
// cs: the channel's W-1 stored inputs (bf16 bits, oldest first, tap t at
// cs[t * cs_stride]), shifted in place when `update`; x: the current input;
// w: tap t at w[t * wstride]; bias added first.
template <typename T>
T conv_channel(int W, uint16_t* cs, std::ptrdiff_t cs_stride, uint16_t x,
               const float* w, std::ptrdiff_t wstride, T bias, bool update) {
  T acc = bias;
  for (int t = 0; t < W; ++t) {
    const uint16_t xt = (t < W - 1) ? cs[t * cs_stride] : x;
    const T prod = T(w[t * wstride]) * T(bf16_to_f32(xt));
    acc = acc + prod;
  }
  if (update) {
    for (int t = 0; t + 1 < W - 1; ++t) cs[t * cs_stride] = cs[(t + 1) * cs_stride];
    cs[(W - 2) * cs_stride] = x;
  }
  return acc * sigmoid(acc);
}

// ---- stage 2: gated delta-rule recurrence of one unit --------------------
template <typename T>
void recurrence(int D, T* S, const T* q, const T* k, const T* v, const T* g,
                T beta, T* o) {
  std::vector<T> delta(D);
  // decay: row i (key channel) scaled by exp(g[i])
  for (int i = 0; i < D; ++i) {
    const T a = std::exp(g[i]);
    for (int j = 0; j < D; ++j) S[i * D + j] = a * S[i * D + j];
  }
  // u = Sd^T k, delta = beta * (v - u)
  for (int j = 0; j < D; ++j) {
    T u = T(0);
    for (int i = 0; i < D; ++i) {
      const T prod = k[i] * S[i * D + j];
      u = u + prod;
    }
    delta[j] = beta * (v[j] - u);
  }
  // S' = Sd + k delta^T
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j) {
      const T prod = k[i] * delta[j];
      S[i * D + j] = S[i * D + j] + prod;
    }
  // o = S'^T q
  for (int j = 0; j < D; ++j) {
    T acc = T(0);
    for (int i = 0; i < D; ++i) {
      const T prod = q[i] * S[i * D + j];
      acc = acc + prod;
    }
    o[j] = acc;
  }
}

// ---- stage 3: gated RMSNorm of one unit's D outputs ----------------------
template <typename T>
void gated_norm(int D, const T* o, const uint16_t* gate, const float* norm_w,
                T eps, int norm_on, int gate_silu, T* y) {
  if (!norm_on) {
    for (int j = 0; j < D; ++j) y[j] = o[j];
    return;
  }
  T ss = T(0);
  for (int j = 0; j < D; ++j) {
    const T sq = o[j] * o[j];
    ss = ss + sq;
  }
  const T r = T(1) / std::sqrt(ss / T(D) + eps);
  for (int j = 0; j < D; ++j) {
    const T gv = T(bf16_to_f32(gate[j]));
    const T gj = gate_silu ? gv * sigmoid(gv) : sigmoid(gv);
    y[j] = ((o[j] * r) * T(norm_w[j])) * gj;
  }
}

struct Dims {
  int32_t batch, num_heads, head_dim, conv_width, num_slots;
  uint32_t flags;  // see the header
  float norm_eps;
};

enum : uint32_t {
  F_NORM = 0x01u, F_NO_CONV_UPDATE = 0x02u, F_CONV_TAP_MAJOR = 0x04u,
  F_QK_L2NORM = 0x08u, F_GATE_SILU = 0x10u, F_BOUNDED_GATE = 0x20u,
  F_ALL = 0x3fu
};

// Raw gate inputs and conv bias (any pointer may be null: see decode()).
struct Extras {
  const float* conv_bias;   // [3C]
  const uint16_t* raw_g;    // bf16 [B, H, D]
  const uint16_t* raw_beta; // bf16 [B, H]
  const float* A_log;       // [H]
  const float* dt_bias;     // [H*D]
  float lower_bound;
};

// ---- the whole step --------------------------------------------------------
// With raw gates (ex->raw_g set) g and beta are computed from raw_g,
// raw_beta, A_log and dt_bias and the `g`/`beta` arguments are not read.
template <typename T>
int decode(const Dims* d, const uint16_t* qkv, const float* conv_w,
           uint16_t* conv_state, T* rec_state, const float* g,
           const float* beta, const uint16_t* gate, const float* norm_w,
           const int32_t* state_idx, uint16_t* out, T* y_out, int nthreads,
           const Extras* ex) {
  if (!d) return ORC_ERR_INVALID_ARG;
  const int64_t B = d->batch, H = d->num_heads, D = d->head_dim,
                W = d->conv_width, S = d->num_slots;
  const uint32_t fl = d->flags;
  const int norm_on = (fl & F_NORM) ? 1 : 0;
  const bool raw_gates = ex && ex->raw_g;
  if (B < 0 || H < 1 || D < 1 || W < 2 || S < 1 || (fl & ~F_ALL))
    return ORC_ERR_INVALID_ARG;
  if (norm_on && !(d->norm_eps > 0.0f && std::isfinite(d->norm_eps)))
    return ORC_ERR_INVALID_ARG;
  if ((fl & F_BOUNDED_GATE) &&
      !(raw_gates && ex->lower_bound < 0.0f && std::isfinite(ex->lower_bound)))
    return ORC_ERR_INVALID_ARG;
  if (B == 0) return ORC_OK;
  if (!qkv || !conv_w || !conv_state || !rec_state || !state_idx || !out ||
      (norm_on && (!gate || !norm_w)))
    return ORC_ERR_INVALID_ARG;
  if (raw_gates ? (!ex->raw_beta || !ex->A_log || !ex->dt_bias)
                : (!g || !beta))
    return ORC_ERR_INVALID_ARG;
  const int64_t C = H * D;
  const T eps = T(d->norm_eps);
  const int64_t units = B * H;
  const bool update = !(fl & F_NO_CONV_UPDATE);
  // element (s, c, t) of the conv state
  const int64_t cs_slot = 3 * C * (W - 1);
  const int64_t cs_chan = (fl & F_CONV_TAP_MAJOR) ? 1 : (W - 1);
  const int64_t cs_tap = (fl & F_CONV_TAP_MAJOR) ? 3 * C : 1;
  const float* conv_bias = ex ? ex->conv_bias : nullptr;
  if (nthreads < 1) nthreads = 1;

#pragma omp parallel num_threads(nthreads)
  {
    std::vector<T> q(D), k(D), v(D), gg(D), o(D), y(D);
#pragma omp for schedule(static)
    for (int64_t unit = 0; unit < units; ++unit) {
      const int64_t n = unit / H, h = unit % H;
      const int64_t s = state_idx[n];
      uint16_t* out_row = out + n * C + h * D;
      if (s <= 0 || s >= S) {
        for (int64_t j = 0; j < D; ++j) out_row[j] = 0;
        if (y_out)
          for (int64_t j = 0; j < D; ++j) y_out[n * C + h * D + j] = T(0);
        continue;
      }
      // stage 1: q, k, v for this head
      T* parts[3] = {q.data(), k.data(), v.data()};
      for (int64_t p = 0; p < 3; ++p)
        for (int64_t i = 0; i < D; ++i) {
          const int64_t c = p * C + h * D + i;
          uint16_t* cs = conv_state + s * cs_slot + c * cs_chan;
          const float* w = conv_w + p * W * C + h * D + i;
          const T bias = conv_bias ? T(conv_bias[c]) : T(0);
          parts[p][i] = conv_channel<T>(static_cast<int>(W), cs, cs_tap,
                                        qkv[n * 3 * C + c], w, C, bias,
                                        update);
        }
      if (fl & F_QK_L2NORM) {
        l2_normalize<T>(static_cast<int>(D), q.data(),
                        T(1) / std::sqrt(T(D)));
        l2_normalize<T>(static_cast<int>(D), k.data(), T(1));
      }
      // stage 2
      T beta_nh;
      if (raw_gates) {
        for (int64_t i = 0; i < D; ++i)
          gg[i] = gate_from_raw<T>(
              T(bf16_to_f32(ex->raw_g[(n * H + h) * D + i])), T(ex->A_log[h]),
              T(ex->dt_bias[h * D + i]), (fl & F_BOUNDED_GATE) ? 1 : 0,
              T(ex->lower_bound));
        beta_nh = sigmoid(T(bf16_to_f32(ex->raw_beta[n * H + h])));
      } else {
        for (int64_t i = 0; i < D; ++i) gg[i] = T(g[(n * H + h) * D + i]);
        beta_nh = T(beta[n * H + h]);
      }
      T* Sst = rec_state + (s * H + h) * D * D;
      recurrence<T>(static_cast<int>(D), Sst, q.data(), k.data(), v.data(),
                    gg.data(), beta_nh, o.data());
      // stage 3
      gated_norm<T>(static_cast<int>(D), o.data(),
                    norm_on ? gate + n * C + h * D : nullptr, norm_w, eps,
                    norm_on, (fl & F_GATE_SILU) ? 1 : 0, y.data());
      for (int64_t j = 0; j < D; ++j) {
        out_row[j] = f32_to_bf16(static_cast<float>(y[j]));
        if (y_out) y_out[n * C + h * D + j] = y[j];
      }
    }
  }
  return ORC_OK;
}

// ---- variable-length prefill: each sequence's tokens in order -------------
// Sequence n covers tokens cu[n] .. cu[n+1]-1 of the token-major inputs
// (qkv [tokens, 3C], g [tokens, H, D], beta [tokens, H], gate [tokens, C],
// out [tokens, C]) and uses slot state_idx[n]; the result is that of one
// single-token step per token, in order.  Sequences are independent.  The
// prefill page gives a variable-length batch by its offsets but no rule for
// offsets that go down; a pair with cu[n+1] < cu[n] is read as a sequence
// of no tokens, like an equal pair: no output, no state touched (the same
// reading as the chunk bookkeeping, where a negative length counts as
// empty).
template <typename T>
int prefill(const Dims* d, const int32_t* cu, const uint16_t* qkv,
            const float* conv_w, uint16_t* conv_state, T* rec_state,
            const float* g, const float* beta, const uint16_t* gate,
            const float* norm_w, const int32_t* state_idx, uint16_t* out,
            T* y_out, int nthreads, const Extras* ex) {
  if (!d || d->batch < 0 || !cu) return ORC_ERR_INVALID_ARG;
  const bool raw_gates = ex && ex->raw_g;
  const int64_t N = d->batch;
  const int64_t H = d->num_heads, D = d->head_dim;
  const int64_t C = H * D;
  for (int64_t n = 0; n < N; ++n) {
    const int64_t len = static_cast<int64_t>(cu[n + 1]) - cu[n];
    if (len <= 0) continue;
    const int32_t slot = state_idx[n];
    for (int64_t t = 0; t < len; ++t) {
      const int64_t tok = cu[n] + t;
      Dims one = *d;
      one.batch = 1;
      // token tok's rows of the per-token gate inputs
      Extras tex{};
      if (ex) {
        tex = *ex;
        if (raw_gates) {
          tex.raw_g = ex->raw_g + tok * H * D;
          tex.raw_beta = ex->raw_beta ? ex->raw_beta + tok * H : nullptr;
        }
      }
      const int rc = decode<T>(
          &one, qkv + tok * 3 * C, conv_w, conv_state, rec_state,
          raw_gates ? nullptr : g + tok * H * D,
          raw_gates ? nullptr : beta + tok * H,
          (d->flags & F_NORM) ? gate + tok * C : nullptr, norm_w, &slot,
          out + tok * C, y_out ? y_out + tok * C : nullptr, nthreads,
          ex ? &tex : nullptr);
      if (rc != ORC_OK) return rc;
    }
  }
  return ORC_OK;
}

}  // namespace

// ---- exported C entry points (host pointers) -------------------------------
extern "C" {

struct kda_oracle_dims {
  int32_t batch, num_heads, head_dim, conv_width, num_slots;
  uint32_t flags;
  float norm_eps;
};

// Optional inputs of the extended step (any field may be null / unused).
struct kda_oracle_extras {
  const float* conv_bias;   // fp32 [3C]
  const uint16_t* raw_g;    // bf16 [B, H, D]; when set g and beta are derived
  const uint16_t* raw_beta; // bf16 [B, H]
  const float* A_log;       // fp32 [H]
  const float* dt_bias;     // fp32 [H*D]
  float lower_bound;        // < 0, with flag 0x20
};

// Whole step, fp32 state and arithmetic.  y_out (optional, [B, H*D]) gets
// the fp32 output before bf16 rounding.  Returns 0 or 1 (invalid argument).
int kda_oracle_decode_f32(const kda_oracle_dims* d, const uint16_t* qkv,
                          const float* conv_w, uint16_t* conv_state,
                          float* rec_state, const float* g, const float* beta,
                          const uint16_t* gate, const float* norm_w,
                          const int32_t* state_idx, uint16_t* out,
                          float* y_out, int nthreads) {
  return decode<float>(reinterpret_cast<const Dims*>(d), qkv, conv_w,
                       conv_state, rec_state, g, beta, gate, norm_w, state_idx,
                       out, y_out, nthreads, nullptr);
}

// Whole step, fp64 state and arithmetic (rec_state is a double pool).  The
// bf16 output rounds through float, so it may differ from a direct
// double-to-bf16 rounding on exact ties; y_out carries the double values.
int kda_oracle_decode_f64(const kda_oracle_dims* d, const uint16_t* qkv,
                          const float* conv_w, uint16_t* conv_state,
                          double* rec_state, const float* g, const float* beta,
                          const uint16_t* gate, const float* norm_w,
                          const int32_t* state_idx, uint16_t* out,
                          double* y_out, int nthreads) {
  return decode<double>(reinterpret_cast<const Dims*>(d), qkv, conv_w,
                        conv_state, rec_state, g, beta, gate, norm_w,
                        state_idx, out, y_out, nthreads, nullptr);
}

// The same with the variant flags' extra inputs (conv bias, raw gates).
int kda_oracle_decode_ext_f32(const kda_oracle_dims* d, const uint16_t* qkv,
                              const float* conv_w, uint16_t* conv_state,
                              float* rec_state, const float* g,
                              const float* beta, const uint16_t* gate,
                              const float* norm_w, const int32_t* state_idx,
                              uint16_t* out, float* y_out, int nthreads,
                              const kda_oracle_extras* ex) {
  return decode<float>(reinterpret_cast<const Dims*>(d), qkv, conv_w,
                       conv_state, rec_state, g, beta, gate, norm_w, state_idx,
                       out, y_out, nthreads,
                       reinterpret_cast<const Extras*>(ex));
}
int kda_oracle_decode_ext_f64(const kda_oracle_dims* d, const uint16_t* qkv,
                              const float* conv_w, uint16_t* conv_state,
                              double* rec_state, const float* g,
                              const float* beta, const uint16_t* gate,
                              const float* norm_w, const int32_t* state_idx,
                              uint16_t* out, double* y_out, int nthreads,
                              const kda_oracle_extras* ex) {
  return decode<double>(reinterpret_cast<const Dims*>(d), qkv, conv_w,
                        conv_state, rec_state, g, beta, gate, norm_w,
                        state_idx, out, y_out, nthreads,
                        reinterpret_cast<const Extras*>(ex));
}

// Variable-length prefill (see prefill() above); dims->batch = number of
// sequences, cu_seqlens [batch + 1] token offsets (a decreasing pair is an
// empty sequence).
int kda_oracle_prefill_f32(const kda_oracle_dims* d, const int32_t* cu_seqlens,
                           const uint16_t* qkv, const float* conv_w,
                           uint16_t* conv_state, float* rec_state,
                           const float* g, const float* beta,
                           const uint16_t* gate, const float* norm_w,
                           const int32_t* state_idx, uint16_t* out,
                           float* y_out, int nthreads) {
  return prefill<float>(reinterpret_cast<const Dims*>(d), cu_seqlens, qkv,
                        conv_w, conv_state, rec_state, g, beta, gate, norm_w,
                        state_idx, out, y_out, nthreads, nullptr);
}

// The same with the extra inputs of kda_oracle_decode_ext_f32, token-major:
// raw_g [tokens, H, D] and raw_beta [tokens, H] (g and beta then unread).
int kda_oracle_prefill_ext_f32(const kda_oracle_dims* d,
                               const int32_t* cu_seqlens, const uint16_t* qkv,
                               const float* conv_w, uint16_t* conv_state,
                               float* rec_state, const float* g,
                               const float* beta, const uint16_t* gate,
                               const float* norm_w, const int32_t* state_idx,
                               uint16_t* out, float* y_out, int nthreads,
                               const kda_oracle_extras* ex) {
  return prefill<float>(reinterpret_cast<const Dims*>(d), cu_seqlens, qkv,
                        conv_w, conv_state, rec_state, g, beta, gate, norm_w,
                        state_idx, out, y_out, nthreads,
                        reinterpret_cast<const Extras*>(ex));
}

// Stage 1 over nch channels: channel c has W-1 stored inputs, tap t at
// cs[c * cs_chan + t * cs_tap], input x[c], taps w[t*wstride + c], optional
// bias[c]; the stored inputs shift only when `update`.
void kda_oracle_conv_f64(int nch, int W, const uint16_t* x, const float* w,
                         std::ptrdiff_t wstride, uint16_t* cs,
                         std::ptrdiff_t cs_chan, std::ptrdiff_t cs_tap,
                         const float* bias, int update, double* y) {
  for (int c = 0; c < nch; ++c)
    y[c] = conv_channel<double>(W, cs + c * cs_chan, cs_tap, x[c], w + c,
                                wstride, bias ? double(bias[c]) : 0.0,
                                update != 0);
}
void kda_oracle_conv_f32(int nch, int W, const uint16_t* x, const float* w,
                         std::ptrdiff_t wstride, uint16_t* cs,
                         std::ptrdiff_t cs_chan, std::ptrdiff_t cs_tap,
                         const float* bias, int update, float* y) {
  for (int c = 0; c < nch; ++c)
    y[c] = conv_channel<float>(W, cs + c * cs_chan, cs_tap, x[c], w + c,
                               wstride, bias ? bias[c] : 0.0f, update != 0);
}

// Stage 2 on one [D, D] state (updated in place).
void kda_oracle_recurrence_f64(int D, double* S, const double* q,
                               const double* k, const double* v,
                               const double* g, double beta, double* o) {
  recurrence<double>(D, S, q, k, v, g, beta, o);
}
void kda_oracle_recurrence_f32(int D, float* S, const float* q, const float* k,
                               const float* v, const float* g, float beta,
                               float* o) {
  recurrence<float>(D, S, q, k, v, g, beta, o);
}

// Stage 3 on one unit's D outputs.
void kda_oracle_gated_norm_f64(int D, const double* o, const uint16_t* gate,
                               const float* norm_w, double eps, int norm_on,
                               int gate_silu, double* y) {
  gated_norm<double>(D, o, gate, norm_w, eps, norm_on, gate_silu, y);
}
void kda_oracle_gated_norm_f32(int D, const float* o, const uint16_t* gate,
                               const float* norm_w, float eps, int norm_on,
                               int gate_silu, float* y) {
  gated_norm<float>(D, o, gate, norm_w, eps, norm_on, gate_silu, y);
}

// q/k normalisation stage: x <- x / sqrt(sum x^2 + 1e-6) * scale.
void kda_oracle_l2norm_f64(int D, double* x, double scale) {
  l2_normalize<double>(D, x, scale);
}

// Raw-gate stage: D gates of one (row, head) and the activated beta.
void kda_oracle_raw_gates_f64(int D, const uint16_t* raw_g, float a_log,
                              const float* dt_bias, int bounded,
                              float lower_bound, uint16_t raw_beta, double* g,
                              double* beta) {
  for (int i = 0; i < D; ++i)
    g[i] = gate_from_raw<double>(double(bf16_to_f32(raw_g[i])), double(a_log),
                                 double(dt_bias[i]), bounded,
                                 double(lower_bound));
  *beta = sigmoid(double(bf16_to_f32(raw_beta)));
}

// bf16 conversions, element-wise over n values.
void kda_oracle_bf16_from_f32(const float* x, uint16_t* y, std::size_t n) {
  for (std::size_t i = 0; i < n; ++i) y[i] = f32_to_bf16(x[i]);
}
void kda_oracle_f32_from_bf16(const uint16_t* x, float* y, std::size_t n) {
  for (std::size_t i = 0; i < n; ++i) y[i] = bf16_to_f32(x[i]);
}

}  // extern "C"
