// C ABI of the Gated DeltaNet forward library (include/gdn.h): argument
// validation, then one kernel launch. Mirrors the pages' validate-then-encode
// dispatchers (mlx-native 0.21.1 src/ops/gated_delta_net_decode.rs: validate,
// validate_params_buf, dispatch_gated_delta_net_decode[_with_capture]); the
// element-count and dtype checks on tensors live in the Python binding, since
// raw pointers carry neither.

#include <stdint.h>
#include <string.h>

#include "gdn.h"
#include "gdn_launch.h"

namespace {

bool mul_ok(uint64_t a, uint64_t b, uint64_t *out) {
  return !__builtin_mul_overflow(a, b, out);
}

// Element counts of every array for params p (false on 64-bit overflow).
struct Counts {
  uint64_t qk, v, scalar, state, capture;
};

bool counts_of(const gdn_params *p, Counts *c) {
  const uint64_t ts = (uint64_t)p->n_tokens * p->n_seqs;  // < 2^64
  if (!mul_ok((uint64_t)p->d_k * p->n_k_heads, ts, &c->qk)) return false;
  if (!mul_ok((uint64_t)p->d_v * p->n_v_heads, ts, &c->v)) return false;
  if (!mul_ok((uint64_t)p->n_v_heads, ts, &c->scalar)) return false;
  if (!mul_ok((uint64_t)p->d_k * p->d_v, (uint64_t)p->n_v_heads * p->n_seqs,
              &c->state))
    return false;
  if (!mul_ok(c->state, p->n_tokens, &c->capture)) return false;
  // Byte sizes must fit a signed 64-bit offset.
  const uint64_t max_elems = (uint64_t)INT64_MAX / sizeof(float);
  for (uint64_t n : {c->qk, c->v, c->scalar, c->state, c->capture})
    if (n > max_elems) return false;
  return true;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void *p, uint64_t elems, uint64_t elem_bytes = sizeof(float)) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)(elems * elem_bytes)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void *p, uintptr_t n) {
  return (reinterpret_cast<uintptr_t>(p) % n) == 0;
}

// Shared by the f32 and bf16 entry points. io_bytes is the element size of q,
// k, v and output (4 for f32, 2 for bf16); the state, capture, g and beta
// arrays are always f32.
gdn_status forward(const void *q, const void *k, const void *v, const float *g,
                   const float *beta, const float *state_in, void *output,
                   float *state_out, float *capture, const gdn_params *p,
                   void *stream, uint32_t io_bytes, bool normalize_k = false) {
  gdn_status st = gdn_check_params(p);
  if (st != GDN_OK) return st;
  if (!q || !k || !v || !g || !beta || !state_in || !output || !state_out)
    return GDN_ERR_NULL_POINTER;

  // q and k are read as vectors of four elements, the state as 4-float
  // vectors; v and output element by element.
  const uintptr_t vec = 4 * io_bytes;
  if (!aligned(q, vec) || !aligned(k, vec) || !aligned(state_in, 16) ||
      !aligned(state_out, 16) || (capture && !aligned(capture, 16)) ||
      !aligned(v, io_bytes) || !aligned(g, 4) || !aligned(beta, 4) ||
      !aligned(output, io_bytes))
    return GDN_ERR_MISALIGNED;

  Counts c;
  counts_of(p, &c);  // cannot fail after gdn_check_params
  const Range inputs[] = {range_of(q, c.qk, io_bytes), range_of(k, c.qk, io_bytes),
                          range_of(v, c.v, io_bytes),  range_of(g, c.scalar),
                          range_of(beta, c.scalar),    range_of(state_in, c.state)};
  const Range r_out = range_of(output, c.v, io_bytes);
  const Range r_state = range_of(state_out, c.state);
  const Range r_cap = range_of(capture, capture ? c.capture : 0);
  for (int i = 0; i < 6; ++i) {
    const bool in_place = (i == 5) && state_out == state_in;
    if (overlap(r_out, inputs[i]) || (!in_place && overlap(r_state, inputs[i])) ||
        (capture && overlap(r_cap, inputs[i])))
      return GDN_ERR_ALIASING;
  }
  if (overlap(r_out, r_state) ||
      (capture && (overlap(r_cap, r_out) || overlap(r_cap, r_state))))
    return GDN_ERR_ALIASING;

  float q_scale = 1.0f;  // params[8] == 0: q pre-scaled (mlx-native 0.21.1 doc)
  if (p->q_scale_bits != 0u) memcpy(&q_scale, &p->q_scale_bits, sizeof q_scale);

  gdn::ForwardArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.state_in = state_in;
  a.output = output;
  a.state_out = state_out;
  a.capture = capture;
  a.d_k = p->d_k;
  a.d_v = p->d_v;
  a.n_k_heads = p->n_k_heads;
  a.n_v_heads = p->n_v_heads;
  a.n_tokens = p->n_tokens;
  a.n_seqs = p->n_seqs;
  a.q_scale = q_scale;
  a.bf16 = io_bytes == 2;
  a.normalize_k = normalize_k;
  if (gdn::enqueue_forward(a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return GDN_ERR_LAUNCH;
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_rollback(const float *state_capture, const uint32_t *accepted,
                        float *state, const gdn_params *p, void *stream) {
  gdn_status st = gdn_check_params(p);
  if (st != GDN_OK) return st;
  if (!state_capture || !accepted || !state) return GDN_ERR_NULL_POINTER;
  if (!aligned(state_capture, 16) || !aligned(state, 16) || !aligned(accepted, 4))
    return GDN_ERR_MISALIGNED;
  Counts c;
  counts_of(p, &c);
  const Range r_cap = range_of(state_capture, c.capture);
  const Range r_state = range_of(state, c.state);
  const Range r_acc = Range{reinterpret_cast<uintptr_t>(accepted),
                            reinterpret_cast<uintptr_t>(accepted) +
                                (uintptr_t)p->n_seqs * sizeof(uint32_t)};
  if (overlap(r_state, r_cap) || overlap(r_state, r_acc)) return GDN_ERR_ALIASING;
  if (gdn::enqueue_rollback(state_capture, accepted, state, p->d_k, p->d_v,
                            p->n_v_heads, p->n_tokens, p->n_seqs,
                            static_cast<hipStream_t>(stream)) != hipSuccess)
    return GDN_ERR_LAUNCH;
  return GDN_OK;
}

gdn_status gdn_check_params(const gdn_params *p) {
  if (p == nullptr) return GDN_ERR_NULL_POINTER;
  if (p->d_k == 0 || p->d_v == 0 || p->n_k_heads == 0 || p->n_v_heads == 0)
    return GDN_ERR_ZERO_DIM;
  if (p->n_tokens == 0 || p->n_seqs == 0) return GDN_ERR_ZERO_EXTENT;
  if (p->n_v_heads % p->n_k_heads != 0) return GDN_ERR_GQA_RATIO;
  if (p->d_k != 32 && p->d_k != 64 && p->d_k != 128)
    return GDN_ERR_UNSUPPORTED_DK;
  if (p->reserved6 != 0 || p->reserved7 != 0) return GDN_ERR_RESERVED_NONZERO;
  Counts c;
  if (!counts_of(p, &c)) return GDN_ERR_SIZE_OVERFLOW;
  // The kernels address one head's state (d_v * d_k floats) through a buffer
  // descriptor whose size in bytes is a 32-bit field, and step through up to
  // 64 + 8 tokens of k/q or v/output with 32-bit scalar byte offsets.
  if ((uint64_t)p->d_v * p->d_k >= (uint64_t(1) << 30)) return GDN_ERR_SIZE_OVERFLOW;
  if ((uint64_t)p->n_v_heads * p->d_v >= (uint64_t(1) << 23) ||
      (uint64_t)p->n_k_heads * p->d_k >= (uint64_t(1) << 23))
    return GDN_ERR_SIZE_OVERFLOW;
  // The grid (one-token and short calls: key heads padded to a power of two,
  // at least 8, or on the memory-order and wide one-token grids a head's row
  // blocks) times the threads per block must stay below 2^32 work-items, for
  // every kernel, with or without capture. Blocks have at most 256 threads,
  // except the multi-token kernel's 512-thread geometry, which is chosen only
  // for grids of at most 256 blocks.
  for (bool cap : {false, true}) {
    const uint64_t blocks = gdn::grid_blocks(p->d_k, p->d_v, p->n_k_heads, p->n_v_heads,
                                             p->n_seqs, p->n_tokens, cap);
    if (blocks >= (uint64_t(1) << 32) / 256u) return GDN_ERR_SIZE_OVERFLOW;
  }
  return GDN_OK;
}

gdn_status gdn_forward(const float *q, const float *k, const float *v,
                       const float *g, const float *beta,
                       const float *state_in, float *output, float *state_out,
                       const gdn_params *p, void *stream) {
  return forward(q, k, v, g, beta, state_in, output, state_out, nullptr, p,
                 stream, 4);
}

gdn_status gdn_forward_capture(const float *q, const float *k, const float *v,
                               const float *g, const float *beta,
                               const float *state_in, float *output,
                               float *state_out, float *state_capture,
                               const gdn_params *p, void *stream) {
  return forward(q, k, v, g, beta, state_in, output, state_out, state_capture,
                 p, stream, 4);
}

gdn_status gdn_forward_bf16(const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const float *g,
                            const float *beta, const float *state_in,
                            uint16_t *output, float *state_out,
                            float *state_capture, const gdn_params *p,
                            void *stream) {
  return forward(q, k, v, g, beta, state_in, output, state_out, state_capture,
                 p, stream, 2);
}

gdn_status gdn_forward_ex(const void *q, const void *k, const void *v,
                          const float *g, const float *beta,
                          const float *state_in, void *output,
                          float *state_out, float *state_capture,
                          const gdn_params *p, uint32_t options, void *stream) {
  if (p == nullptr) return GDN_ERR_NULL_POINTER;
  if ((options & ~(GDN_OPT_BF16_IO | GDN_OPT_NORMALIZE_K)) != 0u)
    return GDN_ERR_OPTION;
  return forward(q, k, v, g, beta, state_in, output, state_out, state_capture,
                 p, stream, (options & GDN_OPT_BF16_IO) ? 2 : 4,
                 (options & GDN_OPT_NORMALIZE_K) != 0u);
}

const char *gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "success";
    case GDN_ERR_NULL_POINTER: return "params or a required array pointer is NULL";
    case GDN_ERR_ZERO_DIM: return "dims must all be > 0 (d_k, d_v, n_k_heads, n_v_heads)";
    case GDN_ERR_ZERO_EXTENT: return "n_tokens and n_seqs must be > 0";
    case GDN_ERR_GQA_RATIO: return "n_v_heads must be a multiple of n_k_heads";
    case GDN_ERR_UNSUPPORTED_DK: return "d_k must be 32, 64 or 128";
    case GDN_ERR_RESERVED_NONZERO: return "params words 6 and 7 are reserved and must be 0";
    case GDN_ERR_SIZE_OVERFLOW: return "array sizes or launch grid exceed 64-bit/32-bit limits";
    case GDN_ERR_MISALIGNED: return "an array breaks the alignment rule (f32: q, k, state, capture 16 bytes; bf16: q, k 8 bytes; every array its element size)";
    case GDN_ERR_ALIASING: return "an output array overlaps another array (only state_out == state_in is allowed)";
    case GDN_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
    case GDN_ERR_OPTION: return "an unknown bit is set in the options word";
  }
  return "unknown gdn_status";
}

}  // extern "C"
