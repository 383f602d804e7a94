// Internal interface between the C ABI (gdn_api.cpp) and the gfx950 kernels
// (gdn_kernels.hip). Not installed, not part of the public header.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace gdn {

// Validated arguments of one forward call. Pointers are device memory in the
// innermost-first layouts of include/gdn.h; capture may be null. q, k, v and
// output hold f32, or bf16 when bf16 is set.
struct ForwardArgs {
  const void *q, *k, *v;
  const float *g, *beta, *state_in;
  void *output;
  float *state_out, *capture;
  uint32_t d_k, d_v, n_k_heads, n_v_heads, n_tokens, n_seqs;
  float q_scale;
  bool bf16;
  bool normalize_k;  // use k / sqrt(sum k^2 + 1e-6) per key row
};

// Number of workgroups the chosen launch geometry needs (for the host-side
// overflow check; 0 when d_k is unsupported).
uint64_t grid_blocks(uint32_t d_k, uint32_t d_v, uint32_t n_k_heads, uint32_t n_v_heads,
                     uint32_t n_seqs, uint32_t n_tokens, bool capture);

// Pick the launch geometry for (d_k, n_tokens, capture) and enqueue the kernel
// on `stream`. Returns the runtime's status of the launch.
hipError_t enqueue_forward(const ForwardArgs &a, hipStream_t stream);

// Enqueue the accepted-prefix rollback copy (validated arguments).
hipError_t enqueue_rollback(const float *capture, const uint32_t *accepted,
                            float *state, uint32_t d_k, uint32_t d_v,
                            uint32_t n_v_heads, uint32_t n_tokens,
                            uint32_t n_seqs, hipStream_t stream);

}  // namespace gdn
