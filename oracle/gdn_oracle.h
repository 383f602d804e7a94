/* Sequential CPU oracle for the Gated DeltaNet recurrent forward step.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the HIP library, with which it shares
 * nothing (this header is the oracle's own, not the library's).
 *
 * All arrays are host memory in the innermost-first layouts of mlx-native 0.4.0
 * "src/ops/gated_delta_net.rs" (module doc "Memory layouts"); the capture layout
 * is that of mlx-native 0.9.2 "gated_delta_net_decode_capture.metal" (header
 * "Memory layout for state_capture"). state_capture may be NULL.
 *
 * Return value: 0 on success, 1 for a NULL array, 2 for a zero dimension or
 * extent, 3 when n_v_heads is not a multiple of n_k_heads, 4 for an unknown
 * head map. Any positive sizes are accepted (no D_k restriction).
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct oracle_gdn_shape {
  uint32_t d_k, d_v, n_k_heads, n_v_heads, n_tokens, n_seqs;
  uint32_t q_scale_bits; /* 0: q already scaled; else binary32 bits of q_scale */
} oracle_gdn_shape;

enum {
  ORACLE_HEAD_MAP_MOD = 0, /* kh = vh % n_k_heads                 */
  ORACLE_HEAD_MAP_DIV = 1  /* kh = vh / (n_v_heads / n_k_heads)   */
};

int oracle_gdn_forward_f32(const float *q, const float *k, const float *v,
                           const float *g, const float *beta,
                           const float *state_in, const oracle_gdn_shape *p,
                           int head_map, float *output, float *state_out,
                           float *state_capture);

/* binary64 shadow: same inputs (f32), every operation in double. */
int oracle_gdn_forward_f64(const float *q, const float *k, const float *v,
                           const float *g, const float *beta,
                           const float *state_in, const oracle_gdn_shape *p,
                           int head_map, double *output, double *state_out,
                           double *state_capture);

/* oracle_gdn_forward_f32 (and _f64) over the (sequence, value head) pairs
 * [pair_begin, pair_end) only, numbered s * n_v_heads + vh (the end is clamped
 * to n_seqs * n_v_heads). Disjoint ranges may run concurrently on the same
 * arrays; together they write what one whole call writes, bit for bit. */
int oracle_gdn_forward_range_f32(const float *q, const float *k, const float *v,
                                 const float *g, const float *beta,
                                 const float *state_in,
                                 const oracle_gdn_shape *p, int head_map,
                                 uint64_t pair_begin, uint64_t pair_end,
                                 float *output, float *state_out,
                                 float *state_capture);

int oracle_gdn_forward_range_f64(const float *q, const float *k, const float *v,
                                 const float *g, const float *beta,
                                 const float *state_in,
                                 const oracle_gdn_shape *p, int head_map,
                                 uint64_t pair_begin, uint64_t pair_end,
                                 double *output, double *state_out,
                                 double *state_capture);

/* bf16 q, k, v and output (raw 16-bit patterns); g, beta, state and capture
 * f32. Inputs widened exactly, f32 recurrence, output rounded to nearest-even
 * bf16 (NaN kept as a quiet NaN). */
int oracle_gdn_forward_bf16(const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const float *g,
                            const float *beta, const float *state_in,
                            const oracle_gdn_shape *p, int head_map,
                            uint16_t *output, float *state_out,
                            float *state_capture);

/* The oracle's f32 -> bf16 rounding alone (round to nearest, ties to even). */
void oracle_f32_to_bf16(const float *in, uint16_t *out, uint64_t n);

/* As oracle_gdn_forward_f32 / _f64 / _bf16 with option bits: 2 = normalise
 * every key row k[s,t,kh,:] to k / sqrt(sum k^2 + 1e-6) before the recurrence
 * (in the oracle's precision). Any other bit returns 5. */
int oracle_gdn_forward_ex_f32(const float *q, const float *k, const float *v,
                              const float *g, const float *beta,
                              const float *state_in, const oracle_gdn_shape *p,
                              int head_map, uint32_t options, float *output,
                              float *state_out, float *state_capture);
int oracle_gdn_forward_ex_f64(const float *q, const float *k, const float *v,
                              const float *g, const float *beta,
                              const float *state_in, const oracle_gdn_shape *p,
                              int head_map, uint32_t options, double *output,
                              double *state_out, double *state_capture);
int oracle_gdn_forward_ex_bf16(const uint16_t *q, const uint16_t *k,
                               const uint16_t *v, const float *g,
                               const float *beta, const float *state_in,
                               const oracle_gdn_shape *p, int head_map,
                               uint32_t options, uint16_t *output,
                               float *state_out, float *state_capture);

/* Accepted-prefix rollback: state[s] = state_capture[s, accepted[s]] for every
 * sequence whose accepted[s] < n_tokens (others untouched). Uses d_k, d_v,
 * n_v_heads, n_tokens, n_seqs of p. */
int oracle_gdn_rollback(const float *state_capture, const uint32_t *accepted,
                        const oracle_gdn_shape *p, float *state);

#ifdef __cplusplus
}
#endif

#endif /* GDN_ORACLE_H */
