/* gdn.h - Gated DeltaNet recurrent forward step on AMD Instinct MI355X (gfx950).
 *
 * The operation (mlx-native 0.9.2, gated_delta_net_decode_capture.metal, token
 * loop of gated_delta_net_decode_capture_impl; also the recurrence in the module
 * doc of mlx-native 0.4.0 src/ops/gated_delta_net.rs). For every sequence s and
 * value head vh a D_v x D_k f32 state X is carried across tokens. Row i of X
 * holds the D_k key-dimension cells of value channel i. Per token t, with
 * kh = vh % n_k_heads (GQA broadcast of key/query heads):
 *
 *     alpha = exp(-g[s,t,vh]),  b = beta[s,t,vh]
 *     X[i,:] *= alpha                                  decay first
 *     sk     = X[i,:] . k[s,t,kh,:]
 *     delta  = (v[s,t,vh,i] - sk) * b
 *     X[i,:] += delta * k[s,t,kh,:]                    rank-1 write
 *     output[s,t,vh,i] = (X[i,:] . q[s,t,kh,:]) * q_scale
 *
 * and optionally state_capture[s,t,vh] = X after token t's update.
 *
 * Layouts (innermost-first, f32, mlx-native 0.4.0 module doc "Memory layouts";
 * the capture layout from the 0.9.2 kernel header "Memory layout for
 * state_capture"). As row-major C arrays:
 *     q, k            [n_seqs][n_tokens][n_k_heads][d_k]
 *     v, output       [n_seqs][n_tokens][n_v_heads][d_v]
 *     g, beta         [n_seqs][n_tokens][n_v_heads]
 *     state_in/out    [n_seqs][n_v_heads][d_v][d_k]
 *     state_capture   [n_seqs][n_tokens][n_v_heads][d_v][d_k]
 *
 * Conventions of every entry point:
 *   - Every array pointer is device memory owned by the caller. The library
 *     allocates nothing, keeps no global state and is reentrant.
 *   - q, k, state_in, state_out and state_capture must be 16-byte aligned
 *     (they are read and written as 4-float vectors; bf16 q and k, 8-byte);
 *     v, g, beta and output aligned to their element size.
 *   - The call only enqueues work on `stream` (a hipStream_t; NULL means the
 *     null stream) and returns without waiting for it. Every argument error is
 *     detected and returned before anything is enqueued; nothing is launched
 *     after a failed check (as the pages validate before encoding, mlx-native
 *     0.21.1 encode_decode).
 *   - state_out may be the same pointer as state_in (in-place update: each
 *     state cell is read and written by one lane only). Any other overlap of an
 *     output (output, state_out, state_capture) with another array is refused
 *     with GDN_ERR_ALIASING.
 */
#ifndef GDN_H
#define GDN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The pages' 9-word params block (mlx-native 0.9.2 kernel header, buffer(8):
 * D_k, D_v, n_k_heads, n_v_heads, n_tokens, n_seqs, 0, 0, q_scale_bits). Host
 * memory, read during the call only. */
typedef struct gdn_params {
  uint32_t d_k;          /* key/query head dim: 32, 64 or 128                  */
  uint32_t d_v;          /* value head dim, >= 1 (any value)                   */
  uint32_t n_k_heads;    /* >= 1                                               */
  uint32_t n_v_heads;    /* >= 1, a multiple of n_k_heads                      */
  uint32_t n_tokens;     /* >= 1 tokens per sequence in this call              */
  uint32_t n_seqs;       /* >= 1 independent sequences                         */
  uint32_t reserved6;    /* must be 0 (always written as 0 on the pages)       */
  uint32_t reserved7;    /* must be 0                                          */
  uint32_t q_scale_bits; /* 0: q is pre-scaled and q_scale = 1; otherwise the
                            IEEE-754 binary32 bits of q_scale, applied to each
                            output at writeback (mlx-native 0.21.1 module doc,
                            "Buffer / params contract"). Nonzero bits are read
                            literally, so 0x80000000 means q_scale = -0.0.   */
} gdn_params;

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL_POINTER = 1,     /* params or a required array pointer is NULL */
  GDN_ERR_ZERO_DIM = 2,         /* d_k, d_v, n_k_heads or n_v_heads is 0      */
  GDN_ERR_ZERO_EXTENT = 3,      /* n_tokens or n_seqs is 0 (an error, not a
                                   no-op, as on the pages)                    */
  GDN_ERR_GQA_RATIO = 4,        /* n_v_heads % n_k_heads != 0                 */
  GDN_ERR_UNSUPPORTED_DK = 5,   /* d_k not in {32, 64, 128}                    */
  GDN_ERR_RESERVED_NONZERO = 6, /* reserved6 or reserved7 is not 0            */
  GDN_ERR_SIZE_OVERFLOW = 7,    /* an array's byte size or the launch grid
                                   does not fit the 64-bit / 32-bit limits    */
  GDN_ERR_MISALIGNED = 8,       /* an array breaks the alignment rule above   */
  GDN_ERR_ALIASING = 9,         /* an output overlaps another array (other
                                   than state_out == state_in exactly)        */
  GDN_ERR_LAUNCH = 10,          /* the HIP runtime refused the launch         */
  GDN_ERR_OPTION = 11           /* an unknown bit is set in the options word  */
} gdn_status;

/* Option bits of gdn_forward_ex. */
#define GDN_OPT_BF16_IO 1u     /* q, k, v and output are bf16 (as gdn_forward_bf16) */
#define GDN_OPT_NORMALIZE_K 2u /* L2-normalise every key row in the kernel       */

/* Validate a params block (the checks on dims, extents, GQA ratio, D_k,
 * reserved words and sizes; mlx-native 0.21.1 validate / validate_params_buf).
 * Host-only: needs no GPU and touches no device state. */
gdn_status gdn_check_params(const gdn_params *p);

/* One forward call over n_tokens tokens of n_seqs sequences: reads q, k, v, g,
 * beta and state_in, writes output and state_out (mlx-native 0.21.1
 * dispatch_gated_delta_net_decode; buffer order of its slots 0-8). */
gdn_status gdn_forward(const float *q, const float *k, const float *v,
                       const float *g, const float *beta,
                       const float *state_in, float *output, float *state_out,
                       const gdn_params *p, void *stream);

/* As gdn_forward, and also writes the state after each token's update to
 * state_capture, which must hold exactly n_tokens * d_k * d_v * n_v_heads *
 * n_seqs floats (mlx-native 0.21.1 dispatch_gated_delta_net_decode_with_capture;
 * slot 9). state_capture[..., n_tokens-1, ...] equals state_out bit for bit.
 * state_capture == NULL makes the call identical to gdn_forward. */
gdn_status gdn_forward_capture(const float *q, const float *k, const float *v,
                               const float *g, const float *beta,
                               const float *state_in, float *output,
                               float *state_out, float *state_capture,
                               const gdn_params *p, void *stream);

/* As gdn_forward_capture with q, k, v and output in bfloat16 (the pages call
 * bf16 variants a future addition: mlx-native 0.4.0 src/ops/gated_delta_net.rs,
 * module doc "Dtype / precision"). Each bf16 element is the high 16 bits of an
 * IEEE binary32 value; inputs are widened exactly to f32, all arithmetic and
 * the state (state_in, state_out, state_capture), g and beta stay f32, and each
 * output is rounded to nearest-even bf16 at writeback. q and k need 8-byte
 * alignment, v and output 2-byte. state_capture may be NULL. */
gdn_status gdn_forward_bf16(const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const float *g,
                            const float *beta, const float *state_in,
                            uint16_t *output, float *state_out,
                            float *state_capture, const gdn_params *p,
                            void *stream);

/* gdn_forward_capture / gdn_forward_bf16 with an options word.
 * GDN_OPT_BF16_IO: q, k, v and output hold bf16 (uint16_t) elements, with the
 * conventions of gdn_forward_bf16; otherwise f32.
 * GDN_OPT_NORMALIZE_K: every key row k[s,t,kh,:] is used as
 *     k / sqrt(sum_j k_j^2 + 1e-6)
 * (the in-kernel form of the L2 normalisation that models apply to keys
 * before this step; not a step of the pages' kernels, which take k as given).
 * The caller's k array is not modified. Sums are taken in f32 in a
 * reduction order of the library's choosing.
 * state_capture may be NULL. Unknown option bits: GDN_ERR_OPTION, checked
 * before anything else after params. */
gdn_status gdn_forward_ex(const void *q, const void *k, const void *v,
                          const float *g, const float *beta,
                          const float *state_in, void *output,
                          float *state_out, float *state_capture,
                          const gdn_params *p, uint32_t options, void *stream);

/* Accepted-prefix rollback for speculative decoding (mlx-native 0.21.1,
 * dispatch_gated_delta_net_decode_with_capture doc: on a partial reject the
 * caller continues from state_capture[..., accepted_idx, ...]). For every
 * sequence s with accepted[s] < n_tokens, copies the capture slice
 * state_capture[s][accepted[s]] (n_v_heads x d_v x d_k floats) into
 * state[s]; sequences with accepted[s] >= n_tokens keep their state.
 * state_capture is a gdn_forward_capture output for the same params (exactly
 * n_tokens * d_k * d_v * n_v_heads * n_seqs floats); accepted is device memory
 * holding n_seqs uint32 indexes (so it can come from a device-side acceptance
 * step without a host round trip); state holds d_k * d_v * n_v_heads * n_seqs
 * floats and must not overlap state_capture or accepted (GDN_ERR_ALIASING).
 * state_capture and state need 16-byte alignment, accepted 4-byte. */
gdn_status gdn_rollback(const float *state_capture, const uint32_t *accepted,
                        float *state, const gdn_params *p, void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *gdn_status_string(gdn_status s);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
