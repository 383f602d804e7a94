// Accepted-prefix rollback for speculative decoding (mlx-native 0.21.1,
// dispatch_gated_delta_net_decode_with_capture doc; mlx-native 0.9.2 capture
// kernel header): after a verify call with per-token state capture, sequence s
// continues from the state after its last accepted token a = accepted[s], the
// capture slice state_capture[s, a]. This kernel copies that slice into the
// sequence's state slot. An index at or past n_tokens leaves the slot as is.
//
// The copy is HBM-bound: every byte of the slice is read once and written
// once, as 16-byte vectors, non-temporal, four per lane in flight when the copy
// is large and one per lane (four times the workgroups) when four per lane
// would leave fewer than four workgroups per compute unit.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_launch.h"

namespace gdn {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// Grid: x = block within a sequence (blocks_per_seq of them), y = sequence
// within the launch (the host moves every base to the launch's first
// sequence), so the index read needs no division. kVecsPerThread: float4s per
// lane per pass.
template <int kVecsPerThread>
__global__ __launch_bounds__(kThreads) void gdn_rollback_kernel(
    const float *capture, const uint32_t *accepted, float *state,
    uint32_t n_tokens, uint64_t seq_vecs, uint32_t blocks_per_seq) {
  const uint32_t s = blockIdx.y;
  const uint32_t b = blockIdx.x;
  const uint32_t a = accepted[s];  // same address in every lane
  if (a >= n_tokens) return;       // uniform: the whole block leaves
  const f4 *src = reinterpret_cast<const f4 *>(capture) +
                  ((uint64_t)s * n_tokens + a) * seq_vecs;
  f4 *dst = reinterpret_cast<f4 *>(state) + (uint64_t)s * seq_vecs;
  const uint64_t stride = (uint64_t)blocks_per_seq * kThreads * kVecsPerThread;
  for (uint64_t i0 = ((uint64_t)b * kThreads * kVecsPerThread) + threadIdx.x;
       i0 < seq_vecs; i0 += stride) {
    f4 v[kVecsPerThread];
#pragma unroll
    for (int u = 0; u < kVecsPerThread; ++u) {
      const uint64_t i = i0 + (uint64_t)u * kThreads;
      if (i < seq_vecs) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kVecsPerThread; ++u) {
      const uint64_t i = i0 + (uint64_t)u * kThreads;
      if (i < seq_vecs) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

}  // namespace

hipError_t enqueue_rollback(const float *capture, const uint32_t *accepted,
                            float *state, uint32_t d_k, uint32_t d_v,
                            uint32_t n_v_heads, uint32_t n_tokens,
                            uint32_t n_seqs, hipStream_t stream) {
  // One sequence's state: n_v_heads * d_v * d_k floats, a multiple of 4
  // because d_k is 32, 64 or 128.
  const uint64_t seq_vecs = (uint64_t)n_v_heads * d_v * d_k / 4;
  // Four float4s per lane, unless that leaves fewer than 4 workgroups per
  // compute unit of an MI355X (256 of them): 3 MiB (one dense-shape layer)
  // and 4 MiB (the 8-sequence verify) copies then run one per lane.
  constexpr uint64_t kMinBlocks = 4 * 256;
  const uint64_t blocks4 = ((seq_vecs + kThreads * 4 - 1) / (kThreads * 4)) * n_seqs;
  const int vpt = blocks4 >= kMinBlocks ? 4 : 1;
  const void *kernel = vpt == 4 ? reinterpret_cast<const void *>(&gdn_rollback_kernel<4>)
                                : reinterpret_cast<const void *>(&gdn_rollback_kernel<1>);
  const uint64_t per_block = (uint64_t)kThreads * vpt;
  uint64_t blocks_per_seq = (seq_vecs + per_block - 1) / per_block;
  if (blocks_per_seq > 1024) blocks_per_seq = 1024;  // the loop covers the rest
  const uint64_t blocks = blocks_per_seq * n_seqs;
  if (blocks == 0 || blocks >= (uint64_t(1) << 31)) return hipErrorInvalidValue;
  uint32_t bps = (uint32_t)blocks_per_seq;
  // One launch per 65535 sequences (the limit of a grid's y dimension).
  constexpr uint32_t kMaxY = 65535;
  for (uint32_t s0 = 0; s0 < n_seqs; s0 += kMaxY) {
    const uint32_t ny = n_seqs - s0 < kMaxY ? n_seqs - s0 : kMaxY;
    const float *cap = capture + (uint64_t)s0 * n_tokens * seq_vecs * 4;
    const uint32_t *acc = accepted + s0;
    float *st = state + (uint64_t)s0 * seq_vecs * 4;
    void *args[] = {&cap, &acc, &st, &n_tokens, const_cast<uint64_t *>(&seq_vecs), &bps};
    const hipError_t e = hipLaunchKernel(kernel, dim3(bps, ny), dim3(kThreads), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gdn
