// Sequential CPU oracle for the Gated DeltaNet recurrent forward step.
//
// TEST INFRASTRUCTURE ONLY. This file is the checker the HIP path is compared
// against. Only the tests, the smoke check and the benchmark's CPU-baseline leg
// may load it; the product path never links, imports or calls it, and it shares
// no code, header, table or helper with the HIP library.
//
// What it computes (mlx-native 0.9.2, "gated_delta_net_decode_capture.metal",
// the token loop of gated_delta_net_decode_capture_impl; recurrence also stated
// in mlx-native 0.4.0 "src/ops/gated_delta_net.rs", module doc): for every
// sequence s and value head vh, a D_v x D_k state X (row i = the D_k keys of
// value channel i) is carried across tokens t. Per token:
//
//   alpha   = exp(-g[s,t,vh]),  b = beta[s,t,vh]
//   X[i,:]  = alpha * X[i,:]                       (decay first)
//   sk_i    = sum_j X[i,j] * k[s,t,kh,j]           (read-out of the decayed state)
//   d_i     = (v[s,t,vh,i] - sk_i) * b
//   X[i,:]  = X[i,:] + d_i * k[s,t,kh,:]           (rank-1 delta write)
//   y_i     = sum_j X[i,j] * q[s,t,kh,j]           (read-out of the updated state)
//   out[s,t,vh,i] = y_i * q_scale
//
// with q_scale = 1 when the params word q_scale_bits is 0 and the IEEE-754
// binary32 value of those bits otherwise (mlx-native 0.21.1
// "src/ops/gated_delta_net_decode.rs", module doc "Buffer / params contract";
// capture kernel, q_scale fold-in). When a capture buffer is given, the state
// after token t's update is copied to capture[s,t,vh] (capture kernel header,
// "Memory layout for state_capture"). The final state goes to state_out.
//
// The GQA key head kh is chosen by an explicit head-map argument because the
// pages show two maps: kh = vh % n_k_heads (capture kernel) and
// kh = vh / (n_v_heads / n_k_heads) (0.4.0 module doc "GQA broadcast" and its
// scalar CPU reference).
//
// Layouts are the pages' innermost-first ones (0.4.0 module doc "Memory layouts"):
//   q, k          [D_k, n_k_heads, n_tokens, n_seqs]   (d_k fastest)
//   v, output     [D_v, n_v_heads, n_tokens, n_seqs]
//   g, beta       [n_v_heads, n_tokens, n_seqs]
//   state_in/out  [D_k, D_v, n_v_heads, n_seqs]
//   state_capture [D_k, D_v, n_v_heads, n_tokens, n_seqs]
//
// Arithmetic: one template, instantiated for float (the oracle proper: every
// operation rounded to binary32, sums taken over j in increasing order, built
// with -ffp-contract=off so no multiply-add is fused) and for double (a shadow
// that widens the f32 inputs once and keeps everything in binary64; it only
// measures the error of the f32 results).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "gdn_oracle.h"

namespace {

template <typename real>
real decay_factor(float g);

template <>
float decay_factor<float>(float g) {
  return expf(-g);
}

template <>
double decay_factor<double>(float g) {
  return exp(-static_cast<double>(g));
}

float scale_from_bits(uint32_t bits) {
  if (bits == 0u) return 1.0f;
  float f;
  std::memcpy(&f, &bits, sizeof f);
  return f;
}

// kreal: element type of the key array the recurrence reads (the caller's f32
// keys, or keys normalised in the oracle's own precision).
// The (sequence, value head) pairs are independent: [pair_begin, pair_end)
// selects which ones run, in the order s * n_v_heads + vh (all of them for a
// whole call; the timing harness splits that range over threads).
template <typename real, typename kreal>
int run(const float *q, const kreal *k, const float *v, const float *g,
        const float *beta, const float *state_in, const oracle_gdn_shape *p,
        int head_map, real *output, real *state_out, real *capture,
        uint64_t pair_begin = 0, uint64_t pair_end = UINT64_MAX) {
  if (p == nullptr || q == nullptr || k == nullptr || v == nullptr ||
      g == nullptr || beta == nullptr || state_in == nullptr ||
      output == nullptr || state_out == nullptr)
    return 1;
  if (p->d_k == 0 || p->d_v == 0 || p->n_k_heads == 0 || p->n_v_heads == 0 ||
      p->n_tokens == 0 || p->n_seqs == 0)
    return 2;
  if (p->n_v_heads % p->n_k_heads != 0) return 3;
  if (head_map != ORACLE_HEAD_MAP_MOD && head_map != ORACLE_HEAD_MAP_DIV)
    return 4;

  const uint64_t Dk = p->d_k, Dv = p->d_v, Hk = p->n_k_heads,
                 Hv = p->n_v_heads, T = p->n_tokens, S = p->n_seqs;
  const uint64_t group_ratio = Hv / Hk;
  const real q_scale = static_cast<real>(scale_from_bits(p->q_scale_bits));

  // Flat offsets of the innermost-first layouts.
  auto at_qk = [&](uint64_t s, uint64_t t, uint64_t kh, uint64_t j) {
    return ((s * T + t) * Hk + kh) * Dk + j;
  };
  auto at_v = [&](uint64_t s, uint64_t t, uint64_t vh, uint64_t i) {
    return ((s * T + t) * Hv + vh) * Dv + i;
  };
  auto at_scalar = [&](uint64_t s, uint64_t t, uint64_t vh) {
    return (s * T + t) * Hv + vh;
  };
  auto at_state = [&](uint64_t s, uint64_t vh, uint64_t i, uint64_t j) {
    return ((s * Hv + vh) * Dv + i) * Dk + j;
  };
  auto at_capture = [&](uint64_t s, uint64_t t, uint64_t vh, uint64_t i,
                        uint64_t j) {
    return (((s * T + t) * Hv + vh) * Dv + i) * Dk + j;
  };

  std::vector<real> X(Dv * Dk);
  if (pair_end > S * Hv) pair_end = S * Hv;
  for (uint64_t pair = pair_begin; pair < pair_end; ++pair) {
    const uint64_t s = pair / Hv, vh = pair % Hv;
    const uint64_t kh =
        head_map == ORACLE_HEAD_MAP_MOD ? vh % Hk : vh / group_ratio;

    for (uint64_t i = 0; i < Dv; ++i)
      for (uint64_t j = 0; j < Dk; ++j)
        X[i * Dk + j] = static_cast<real>(state_in[at_state(s, vh, i, j)]);

    for (uint64_t t = 0; t < T; ++t) {
      const real alpha = decay_factor<real>(g[at_scalar(s, t, vh)]);
      const real b = static_cast<real>(beta[at_scalar(s, t, vh)]);

      for (uint64_t i = 0; i < Dv; ++i) {
        real *row = &X[i * Dk];

        real sk = 0;
        for (uint64_t j = 0; j < Dk; ++j) {
          row[j] = alpha * row[j];
          sk = sk + row[j] * static_cast<real>(k[at_qk(s, t, kh, j)]);
        }

        const real d = (static_cast<real>(v[at_v(s, t, vh, i)]) - sk) * b;

        real y = 0;
        for (uint64_t j = 0; j < Dk; ++j) {
          row[j] = row[j] + d * static_cast<real>(k[at_qk(s, t, kh, j)]);
          y = y + row[j] * static_cast<real>(q[at_qk(s, t, kh, j)]);
        }

        output[at_v(s, t, vh, i)] = y * q_scale;
      }

      if (capture != nullptr)
        for (uint64_t i = 0; i < Dv; ++i)
          for (uint64_t j = 0; j < Dk; ++j)
            capture[at_capture(s, t, vh, i, j)] = X[i * Dk + j];
    }

    for (uint64_t i = 0; i < Dv; ++i)
      for (uint64_t j = 0; j < Dk; ++j)
        state_out[at_state(s, vh, i, j)] = X[i * Dk + j];
  }
  return 0;
}

// Key normalisation option (in the benchmark configurations' input recipe,
// not on the pages): every key row k[s,t,kh,:] is replaced by
//   k / sqrt(sum_j k_j^2 + eps),  eps = 1e-6 (the binary32 value),
// the plain L2 normalisation with an epsilon that keeps an all-zero row at
// zero. Computed in the oracle's precision, sum over j in increasing order.
constexpr float kNormEps = 1e-6f;

template <typename real>
std::vector<real> normalized_keys(const float *k, const oracle_gdn_shape *p) {
  const uint64_t Dk = p->d_k;
  const uint64_t rows = (uint64_t)p->n_seqs * p->n_tokens * p->n_k_heads;
  std::vector<real> out(rows * Dk);
  for (uint64_t r = 0; r < rows; ++r) {
    const float *kr = k + r * Dk;
    real ss = 0;
    for (uint64_t j = 0; j < Dk; ++j)
      ss = ss + static_cast<real>(kr[j]) * static_cast<real>(kr[j]);
    const real inv = real(1) / std::sqrt(ss + static_cast<real>(kNormEps));
    for (uint64_t j = 0; j < Dk; ++j) out[r * Dk + j] = static_cast<real>(kr[j]) * inv;
  }
  return out;
}

// Option bits of the _ex entry points.
constexpr uint32_t kOptNormalizeK = 2u;

template <typename real>
int run_ex(const float *q, const float *k, const float *v, const float *g,
           const float *beta, const float *state_in, const oracle_gdn_shape *p,
           int head_map, uint32_t options, real *output, real *state_out,
           real *capture) {
  if ((options & ~kOptNormalizeK) != 0u) return 5;
  if (!(options & kOptNormalizeK))
    return run<real, float>(q, k, v, g, beta, state_in, p, head_map, output,
                            state_out, capture);
  if (p == nullptr || k == nullptr) return 1;
  const std::vector<real> kn = normalized_keys<real>(k, p);
  return run<real, real>(q, kn.data(), v, g, beta, state_in, p, head_map,
                         output, state_out, capture);
}

// bfloat16 is the top half of an IEEE binary32 value (sign, 8 exponent bits,
// 7 fraction bits). Widening is exact; narrowing rounds to nearest, ties to
// even on the 16 dropped bits; NaN stays NaN (quiet, sign kept).
float bf16_to_f32(uint16_t h) {
  const uint32_t bits = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &bits, sizeof f);
  return f;
}

uint16_t f32_to_bf16(float f) {
  uint32_t bits;
  std::memcpy(&bits, &f, sizeof bits);
  if ((bits & 0x7FFFFFFFu) > 0x7F800000u)  // NaN
    return (uint16_t)((bits >> 16) | 0x0040u);
  const uint32_t dropped = bits & 0xFFFFu;
  uint32_t kept = bits >> 16;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1;
  return (uint16_t)kept;
}

}  // namespace

extern "C" {

int oracle_gdn_forward_f32(const float *q, const float *k, const float *v,
                           const float *g, const float *beta,
                           const float *state_in, const oracle_gdn_shape *p,
                           int head_map, float *output, float *state_out,
                           float *state_capture) {
  return run<float, float>(q, k, v, g, beta, state_in, p, head_map, output,
                           state_out, state_capture);
}

int oracle_gdn_forward_f64(const float *q, const float *k, const float *v,
                           const float *g, const float *beta,
                           const float *state_in, const oracle_gdn_shape *p,
                           int head_map, double *output, double *state_out,
                           double *state_capture) {
  return run<double, float>(q, k, v, g, beta, state_in, p, head_map, output,
                            state_out, state_capture);
}

// oracle_gdn_forward_f32 restricted to the (sequence, value head) pairs
// [pair_begin, pair_end) in the order s * n_v_heads + vh: the same loop body,
// so disjoint ranges run on separate threads give the whole call's result bit
// for bit. Only the selected pairs' outputs, state and capture are written.
int oracle_gdn_forward_range_f32(const float *q, const float *k, const float *v,
                                 const float *g, const float *beta,
                                 const float *state_in,
                                 const oracle_gdn_shape *p, int head_map,
                                 uint64_t pair_begin, uint64_t pair_end,
                                 float *output, float *state_out,
                                 float *state_capture) {
  return run<float, float>(q, k, v, g, beta, state_in, p, head_map, output,
                           state_out, state_capture, pair_begin, pair_end);
}

// The binary64 shadow over a range of pairs, as above.
int oracle_gdn_forward_range_f64(const float *q, const float *k, const float *v,
                                 const float *g, const float *beta,
                                 const float *state_in,
                                 const oracle_gdn_shape *p, int head_map,
                                 uint64_t pair_begin, uint64_t pair_end,
                                 double *output, double *state_out,
                                 double *state_capture) {
  return run<double, float>(q, k, v, g, beta, state_in, p, head_map, output,
                            state_out, state_capture, pair_begin, pair_end);
}

// As the two above, with option bits: 2 = normalise every key row first
// (normalized_keys). Other bits are an error (5).
int oracle_gdn_forward_ex_f32(const float *q, const float *k, const float *v,
                              const float *g, const float *beta,
                              const float *state_in, const oracle_gdn_shape *p,
                              int head_map, uint32_t options, float *output,
                              float *state_out, float *state_capture) {
  return run_ex<float>(q, k, v, g, beta, state_in, p, head_map, options, output,
                       state_out, state_capture);
}

int oracle_gdn_forward_ex_f64(const float *q, const float *k, const float *v,
                              const float *g, const float *beta,
                              const float *state_in, const oracle_gdn_shape *p,
                              int head_map, uint32_t options, double *output,
                              double *state_out, double *state_capture) {
  return run_ex<double>(q, k, v, g, beta, state_in, p, head_map, options,
                        output, state_out, state_capture);
}

// bf16 inputs and output (the "future add" of mlx-native 0.4.0
// src/ops/gated_delta_net.rs, module doc "Dtype / precision"): q, k, v are
// widened exactly, the recurrence runs in f32 as above, and each output is
// rounded to the nearest bf16. State and capture stay f32.
int oracle_gdn_forward_ex_bf16(const uint16_t *q, const uint16_t *k,
                               const uint16_t *v, const float *g,
                               const float *beta, const float *state_in,
                               const oracle_gdn_shape *p, int head_map,
                               uint32_t options, uint16_t *output,
                               float *state_out, float *state_capture) {
  if (p == nullptr || q == nullptr || k == nullptr || v == nullptr ||
      output == nullptr)
    return 1;
  const uint64_t nqk = (uint64_t)p->d_k * p->n_k_heads * p->n_tokens * p->n_seqs;
  const uint64_t nv = (uint64_t)p->d_v * p->n_v_heads * p->n_tokens * p->n_seqs;
  std::vector<float> qf(nqk), kf(nqk), vf(nv), of(nv);
  for (uint64_t e = 0; e < nqk; ++e) {
    qf[e] = bf16_to_f32(q[e]);
    kf[e] = bf16_to_f32(k[e]);
  }
  for (uint64_t e = 0; e < nv; ++e) vf[e] = bf16_to_f32(v[e]);
  const int rc = run_ex<float>(qf.data(), kf.data(), vf.data(), g, beta,
                               state_in, p, head_map, options, of.data(),
                               state_out, state_capture);
  if (rc != 0) return rc;
  for (uint64_t e = 0; e < nv; ++e) output[e] = f32_to_bf16(of[e]);
  return 0;
}

int oracle_gdn_forward_bf16(const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const float *g,
                            const float *beta, const float *state_in,
                            const oracle_gdn_shape *p, int head_map,
                            uint16_t *output, float *state_out,
                            float *state_capture) {
  return oracle_gdn_forward_ex_bf16(q, k, v, g, beta, state_in, p, head_map, 0u,
                                    output, state_out, state_capture);
}

// The oracle's f32 -> bf16 rounding on its own, for the pins.
void oracle_f32_to_bf16(const float *in, uint16_t *out, uint64_t n) {
  for (uint64_t e = 0; e < n; ++e) out[e] = f32_to_bf16(in[e]);
}

// Accepted-prefix rollback (mlx-native 0.21.1,
// dispatch_gated_delta_net_decode_with_capture doc; 0.9.2 capture kernel
// header): after a call with capture, sequence s continues from the state
// after its accepted token accepted[s], i.e. capture[s, accepted[s]]. An index
// at or past n_tokens leaves that sequence's state as it was.
int oracle_gdn_rollback(const float *state_capture, const uint32_t *accepted,
                        const oracle_gdn_shape *p, float *state) {
  if (p == nullptr || state_capture == nullptr || accepted == nullptr ||
      state == nullptr)
    return 1;
  if (p->d_k == 0 || p->d_v == 0 || p->n_v_heads == 0 || p->n_tokens == 0 ||
      p->n_seqs == 0)
    return 2;
  const uint64_t head_state = (uint64_t)p->d_k * p->d_v * p->n_v_heads;
  for (uint64_t s = 0; s < p->n_seqs; ++s) {
    if (accepted[s] >= p->n_tokens) continue;
    const float *src =
        state_capture + (s * p->n_tokens + accepted[s]) * head_state;
    float *dst = state + s * head_state;
    for (uint64_t e = 0; e < head_state; ++e) dst[e] = src[e];
  }
  return 0;
}

}  // extern "C"
