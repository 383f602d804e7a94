// Gated DeltaNet recurrent forward step: gfx950 (CDNA4, wave64) kernels.
//
// The recurrence (mlx-native 0.9.2, gated_delta_net_decode_capture.metal,
// token loop of gated_delta_net_decode_capture_impl): per (sequence, value
// head, value channel i) the D_k state cells of row i are decayed by
// alpha = exp(-g), read out against k (sk), corrected by
// delta = (v_i - sk) * beta along k, and read out against q (y_i).
//
// Mapping to the hardware.
//   * A state row (D_k contiguous f32) is owned by L = D_k / C lanes of one
//     wavefront; each lane keeps its C cells in VGPRs for the whole token loop,
//     so state is read from HBM once and written once per call, whatever the
//     number of tokens (the "Threading" note of mlx-native 0.4.0
//     src/ops/gated_delta_net.rs makes the same point for its thread-per-row
//     design).
//   * The lane's cells are C/4 float4 vectors at columns m*4L + 4*sub (sub =
//     lane index within its row group). For every vector index m the L lanes of
//     a row touch 4L consecutive floats, so each load/store instruction of a
//     wave covers whole 128-byte lines: fully coalesced dwordx4 traffic.
//   * sk and y are sums over the L lanes of a row: butterfly DPP adds
//     (quad_perm, row_half_mirror, row_mirror; a ds_swizzle for 32-lane
//     groups). No barriers. Each butterfly step adds a value to its partner's,
//     so every lane of the row ends with the same bits. With two rows per lane
//     the halves of a row group hold the rows in swapped order, so that one
//     butterfly reduces both rows (see partner()). In multi-token calls with
//     two rows per lane y needs no butterfly per token: the partials of a
//     batch of tokens are reduced together by one reduce-scatter that leaves
//     token t0+j's y in lane j (see scatter_sum()).
//   * In multi-token calls every row group of a wave, and every wave of a
//     workgroup, needs the same k and q columns; each token's k and q rows
//     are loaded once per workgroup (each wave a share of a ring group's
//     tokens; once per wave at D_k = 32 and with capture) and handed out
//     through LDS, so the vector memory unit sees each byte once per
//     workgroup instead of once per row group.
//   * A workgroup covers rows of one (sequence, value head), so g and beta are
//     uniform: the per-token factors of 64 tokens are computed once per wave
//     (lane j holds token t0+j), parked in LDS and read per ring group.
//   * Multi-token calls without capture carry the state divided by a running
//     product of alphas inside each ring group (the lazy form of step()): one
//     multiply per cell and token fewer, the same recurrence reassociated.
//   * The next ring group's k and q rows are requested at the start of a
//     group (or, per wave, token t+NB-1's while token t computes: a ring of
//     NB register sets); v is requested once per ring group, a group ahead,
//     for all rows of the wave.
//   * Every access goes through a buffer resource (a 128-bit scalar
//     descriptor: base address and size in bytes) plus a 32-bit per-lane byte
//     offset that is fixed for the whole loop; per-token bases advance with
//     scalar arithmetic only. Every load offset is computed in range (rows
//     past d_v read a valid row); the one-token and short kernels give the
//     stores of such rows the offset of the descriptor's size, which the
//     hardware drops, so that no store sits in a branch.
//   * Optionally (NK) every key row is used L2-normalised, its factor folded
//     into sk and delta: computed per token, or a ring group ahead in calls of
//     16 tokens or more (with shared staging, by the wave that stages the row,
//     which stages it scaled).
// Kernels: gdn_decode for a single decode token (HBM-bound on the state read
// and write; straight-line code, every input base and its sizes preloaded
// into scalar registers), gdn_decode_wide for one-token calls with sizes
// past gdn_decode's size word, gdn_short for 2 to 8 tokens (9 to 16 on small
// grids; the one-token kernel's form, every input requested before an
// unrolled token loop), and gdn_recurrent for longer multi-token calls
// (bound by VALU issue; two rows per lane share each k/q register).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "gdn_launch.h"

namespace gdn {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

// DPP_CTRL encodings (AMD CDNA3/CDNA4 ISA, "DPP" modifier).
constexpr int kDppXor1 = 0xB1;        // quad_perm:[1,0,3,2]  lane ^ 1
constexpr int kDppXor2 = 0x4E;        // quad_perm:[2,3,0,1]  lane ^ 2
constexpr int kDppHalfMirror = 0x141; // row_half_mirror: lane -> 7 - lane (per 8)
constexpr int kDppMirror = 0x140;     // row_mirror: lane -> 15 - lane (per 16)
constexpr int kDppRor8 = 0x128;       // row_ror:8: lane -> lane ^ 8 (per 16)
constexpr int kDppShr1 = 0x111;       // row_shr:1: lane - 1 (per 16)
constexpr int kDppShr2 = 0x112;       // row_shr:2: lane - 2 (per 16)
constexpr int kDppShr4 = 0x114;       // row_shr:4: lane - 4 (per 16)
constexpr int kDppBcast15 = 0x142;    // row_bcast:15: lane 15 of the row below
// ds_swizzle bit mode (offset bit 15 = 0): and_mask 0x1f, or_mask 0,
// xor_mask 0x10 -> lane ^ 16 within each group of 32.
constexpr int kSwizzleXor16 = 0x1F | (0x10 << 10);

// Lane value of the partner selected by CTRL (all source lanes are active).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF,
                                      0xF, true));
}

// Sum over the L consecutive lanes of a row group (L a power of two, 2..32).
// The result is bit-identical in all L lanes.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(L == 2 || L == 4 || L == 8 || L == 16 || L == 32,
                "row groups of 2..32 lanes");
  x += dpp<kDppXor1>(x);
  if constexpr (L >= 4) x += dpp<kDppXor2>(x);
  if constexpr (L >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (L >= 16) x += dpp<kDppMirror>(x);
  if constexpr (L >= 32)
    x += __builtin_bit_cast(
        float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x),
                                           kSwizzleXor16));
  return x;
}

// Two rows per lane, paired. A row group of L lanes holds rows P and Q; the
// low half of the group keeps row P in its first register set ("A") and row Q
// in its second ("B"), the high half the other way round. Each lane pairs
// with a partner in the other half, whose B cells are the same row as its own
// A cells. Adding the partner's B partial to one's own A partial leaves a
// partial of the lane's A row over both lanes' columns; a butterfly over the
// L/2 lanes of the half then completes it. Both rows are reduced with
// log2(L) adds per lane instead of 2*log2(L), and each half ends holding the
// sum of its own A row.
template <int L>
__device__ __forceinline__ float partner(float x) {
  static_assert(L == 4 || L == 8 || L == 16, "paired rows need 4, 8 or 16 lanes");
  if constexpr (L == 4) return dpp<kDppXor2>(x);        // lane ^ 2
  if constexpr (L == 8) return dpp<kDppHalfMirror>(x);  // lane -> 7 - lane
  if constexpr (L == 16) return dpp<kDppRor8>(x);       // lane ^ 8
}

// Partial of the lane's A row over its own and its partner's columns, given
// the A and B partials (paired layout).
template <int L>
__device__ __forceinline__ float pair_part(float a, float b) {
  return a + partner<L>(b);
}

// Sum of the lane's A row given the A and B partials (paired layout).
template <int L>
__device__ __forceinline__ float pair_sum(float a, float b) {
  return group_sum<L / 2>(pair_part<L>(a, b));
}

// Reduce-scatter over H aligned lanes (H = 2, 4 or 8): on entry w[i] holds
// the lane's partial of item i (i < H); on return w[0] of lane h (the lane's
// index within its H lanes) holds item h summed over the H lanes. Each level
// halves the items a lane keeps: with span S, a lane keeps the items whose
// bit S equals its own bit S and sends the others to a lane with the
// opposite bit (S = 4: lane -> 7 - lane, S = 2: lane ^ 2, S = 1: lane ^ 1),
// so H - 1 cross-lane adds reduce all H items instead of H * log2(H).
template <int S, int H>
__device__ __forceinline__ void scatter_sum(float (&w)[H], uint32_t h) {
  static_assert(S == 1 || S == 2 || S == 4, "span of 1, 2 or 4 lanes");
  const bool hi = (h & S) != 0;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const float keep = hi ? w[S + i] : w[i];
    const float send = hi ? w[i] : w[S + i];
    if constexpr (S == 4) w[i] = keep + dpp<kDppHalfMirror>(send);
    if constexpr (S == 2) w[i] = keep + dpp<kDppXor2>(send);
    if constexpr (S == 1) w[i] = keep + dpp<kDppXor1>(send);
  }
  if constexpr (S > 1) scatter_sum<S / 2>(w, h);
}

// ---------------------------------------------------------------- buffers

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Word 3 of a raw (untyped, stride 0) buffer descriptor on the gfx9 family.
constexpr int kBufferWord3 = 0x00020000;
// Cache-policy bit of buffer loads and stores for non-temporal (streaming)
// accesses.
constexpr int kNonTemporal = 2;

// s_waitcnt operand (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8) that waits for every outstanding vector-memory
// request and for nothing else.
constexpr int kWaitVmAll = 0x0F70;

// Descriptor over `bytes` bytes from `base` (bytes < 2^32).
__device__ __forceinline__ rsrc_t buffer(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes,
                                           kBufferWord3);
}

// A value the compiler cannot prove wave-uniform but that is (scalar operand).
__device__ __forceinline__ uint32_t uniform(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane(x);
}

// The same for a pointer: both 32-bit halves through readfirstlane, widened
// without sign extension (readfirstlane returns a signed int).
template <typename P>
__device__ __forceinline__ P *uniform(P *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<P *>((hi << 32) | lo);
}

// Descriptor size for `bytes` bytes, clamped to the 32-bit size field.
__device__ __forceinline__ uint32_t extent_bytes(uint64_t bytes) {
  return bytes < 0xFFFFFFFFull ? (uint32_t)bytes : 0xFFFFFFFFu;
}

// Loads and stores at lane byte offset `off` plus wave-uniform byte offset
// `soff` (the descriptor's scalar offset operand).
__device__ __forceinline__ f4 load4(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(f4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}

__device__ __forceinline__ float load1(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0));
}

// The state is read once per call: a streaming (non-temporal) load keeps it
// from displacing the k/q rows that other value heads reread.
__device__ __forceinline__ f4 load4_stream(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(
      f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal));
}

__device__ __forceinline__ void store1(rsrc_t r, uint32_t off, uint32_t soff, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, x), r,
                                        off, soff, 0);
}

__device__ __forceinline__ void store4_stream(rsrc_t r, uint32_t byte_off, f4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, x), r, byte_off,
                                         0, kNonTemporal);
}

// Element access for the arrays that take the caller's I/O type (q, k, v,
// output): f32, or bf16 widened exactly to f32 on load (the 16 bits become
// the high half of the f32) and rounded to nearest-even on store. State,
// capture, g and beta are always f32.
typedef unsigned int u2 __attribute__((ext_vector_type(2)));

template <typename IO>
struct Io;

// raw4/raw1 request the bytes and widen4/widen1 turn them into f32, so that
// a caller can issue every request before any widening waits for its data.
template <>
struct Io<float> {
  static constexpr uint32_t bytes = 4;
  typedef f4 R4;
  typedef float R1;
  static __device__ __forceinline__ R4 raw4(rsrc_t r, uint32_t off, uint32_t soff) {
    return ::gdn::load4(r, off, soff);
  }
  static __device__ __forceinline__ f4 widen4(R4 x) { return x; }
  static __device__ __forceinline__ R1 raw1(rsrc_t r, uint32_t off, uint32_t soff) {
    return ::gdn::load1(r, off, soff);
  }
  static __device__ __forceinline__ float widen1(R1 x) { return x; }
  static __device__ __forceinline__ f4 load4(rsrc_t r, uint32_t off, uint32_t soff) {
    return ::gdn::load4(r, off, soff);
  }
  static __device__ __forceinline__ float load1(rsrc_t r, uint32_t off, uint32_t soff) {
    return ::gdn::load1(r, off, soff);
  }
  static __device__ __forceinline__ void store1(rsrc_t r, uint32_t off, uint32_t soff,
                                                float x) {
    ::gdn::store1(r, off, soff, x);
  }
};

template <>
struct Io<__bf16> {
  static constexpr uint32_t bytes = 2;
  static __device__ __forceinline__ float widen(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
  }
  typedef u2 R4;
  typedef uint32_t R1;
  static __device__ __forceinline__ R4 raw4(rsrc_t r, uint32_t off, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
  }
  static __device__ __forceinline__ f4 widen4(R4 w) {
    return f4{__builtin_bit_cast(float, w.x << 16),
              __builtin_bit_cast(float, w.x & 0xFFFF0000u),
              __builtin_bit_cast(float, w.y << 16),
              __builtin_bit_cast(float, w.y & 0xFFFF0000u)};
  }
  static __device__ __forceinline__ R1 raw1(rsrc_t r, uint32_t off, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0);
  }
  static __device__ __forceinline__ float widen1(R1 x) { return widen(x); }
  static __device__ __forceinline__ f4 load4(rsrc_t r, uint32_t off, uint32_t soff) {
    return widen4(raw4(r, off, soff));
  }
  static __device__ __forceinline__ float load1(rsrc_t r, uint32_t off, uint32_t soff) {
    return widen1(raw1(r, off, soff));
  }
  static __device__ __forceinline__ void store1(rsrc_t r, uint32_t off, uint32_t soff,
                                                float x) {
    __builtin_amdgcn_raw_buffer_store_b16(
        __builtin_bit_cast(unsigned short, static_cast<__bf16>(x)), r, off, soff, 0);
  }
};

// Raw per-lane bytes of a staged row load (RB bytes per lane).
template <int RB>
struct Raw;
template <>
struct Raw<8> {
  typedef u2 T;
  static __device__ __forceinline__ T load(rsrc_t r, uint32_t off, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
  }
};
template <>
struct Raw<4> {
  typedef uint32_t T;
  static __device__ __forceinline__ T load(rsrc_t r, uint32_t off, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
  }
};
template <>
struct Raw<2> {
  typedef uint16_t T;
  static __device__ __forceinline__ T load(rsrc_t r, uint32_t off, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0);
  }
};
// The EPL staged elements (raw bits of IO type) as f32 values.
template <typename IO, uint32_t EPL, typename R>
__device__ __forceinline__ void widen(R raw, float (&out)[EPL]) {
  static_assert(EPL == 1 || EPL == 2, "one or two elements per lane");
  if constexpr (sizeof(IO) == 4) {
    if constexpr (EPL == 2) {
      // Element reads as values (raw[i]): bit-casting a vector member access
      // (raw.y) has been seen to read element 0 with this compiler.
      out[0] = __builtin_bit_cast(float, (uint32_t)raw[0]);
      out[1] = __builtin_bit_cast(float, (uint32_t)raw[1]);
    } else {
      out[0] = __builtin_bit_cast(float, (uint32_t)raw);
    }
  } else if constexpr (EPL == 2) {
    const uint32_t w = raw;  // two bf16
    out[0] = __builtin_bit_cast(float, w << 16);
    out[1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
  } else {
    out[0] = __builtin_bit_cast(float, (uint32_t)raw << 16);
  }
}

// Sum over all 64 lanes of a wave, as a wave-uniform value: DPP sums within
// each 16-lane row, then the four row sums read out lane by lane.
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  auto lane_value = [&](int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
  };
  return (lane_value(0) + lane_value(16)) + (lane_value(32) + lane_value(48));
}

// The multi-token kernel's arguments that its workgroup-index split and its
// state loads do not need; those come first, as scalar parameters, so that
// they are among the 13 kernel-argument dwords the dispatch preloads into
// scalar registers (a by-value struct is not preloaded), and the split and
// the state requests wait for no kernel-argument memory.
struct KernelArgs {
  const void *q, *k, *v;  // IO type
  const float *g, *beta;
  void *output;           // IO type
  float *state_out, *capture;
  float q_scale;
  // Descriptor sizes of the k/q and v rows of a whole sequence (the first
  // rebase), the same for every workgroup.
  uint32_t kq_ext0, v_ext0;
};

// Epsilon of the key-normalisation option (binary32 value of 1e-6).
constexpr float kNormEps = 1e-6f;

// DK: key dim. C: cells per lane per row. R: rows per lane. WAVES: waves per
// workgroup. NB: token buffers in the prefetch ring (token t + NB - 1 is
// requested while token t computes), at least 2: one-token calls take
// gdn_decode. CAPTURE: also write the per-token state. IO: element
// type of q, k, v and output (float or __bf16). NK: 0, or use every key row
// as k / sqrt(sum k^2 + kNormEps), its factor computed per token (1) or a ring
// group ahead (2; see GNORM and SNORM).
// Leading parameters (preloaded): the state base; d_v, n_k_heads, n_v_heads,
// n_tokens; row_blocks (workgroups per (sequence, value head)) and groups
// (value heads per key head) with host-computed reciprocals for the
// workgroup index split, x / d == (x * magic) >> shift for every x < 2^24
// (the grid size), d = row_blocks, groups, n_k_heads, the three shifts in
// bits 0-7, 8-15 and 16-23 of shifts; and n_blocks, the grid size (the
// grid's own size lives in kernel-argument memory).
template <int DK, int C, int R, int WAVES, int NB, bool CAPTURE, typename IO, int NK>
__global__ __launch_bounds__(WAVES * 64) void gdn_recurrent(
    const float *state_in, uint32_t d_v, uint32_t n_k_heads, uint32_t n_v_heads,
    uint32_t n_tokens, uint32_t row_blocks, uint32_t groups, uint32_t rb_magic,
    uint32_t g_magic, uint32_t kh_magic, uint32_t shifts, uint32_t n_blocks, KernelArgs a) {
  static_assert(NB >= 4 && NB % 4 == 0, "a ring of a multiple of four tokens");
  constexpr bool NORMK = NK != 0;
  constexpr int L = DK / C;      // lanes sharing one state row
  constexpr int G = 64 / L;      // row groups per wave
  constexpr int NV = C / 4;      // float4 vectors per lane per row
  constexpr int ROWS_PER_WAVE = G * R;
  constexpr int ROWS = WAVES * ROWS_PER_WAVE;
  constexpr uint32_t ROW_BYTES = DK * 4;       // one f32 state row
  constexpr uint32_t IB = Io<IO>::bytes;       // bytes per q/k/v/output element
  static_assert(DK % C == 0 && C % 4 == 0 && 64 % L == 0, "bad geometry");
  static_assert(R <= L, "one output lane per row");
  // R == 2 uses the paired layout (see partner()): register set 0 is the
  // lane's A row, whose sums, v and output the lane handles; set 1 its B row.
  constexpr bool PAIRED = R == 2;
  constexpr int NY = PAIRED ? 1 : R;  // rows whose v and output a lane handles

  // Workgroup -> (sequence s, value head vh, block of rows); all uniform.
  // Every token's k and q rows are read once per key head, so workgroups are
  // ordered (s, kh, g, block) with vh = kh + g * n_k_heads (the value heads of
  // the modulo GQA map that share key head kh) and renumbered so that each of
  // the 8 XCDs, which receive workgroups round-robin and each have their own
  // L2, runs one contiguous range of that order: a key head's k/q rows are
  // then fetched into one L2 instead of several.
  uint32_t s, vh, rb, kh;
  {
    const uint32_t n = n_blocks, xcd = blockIdx.x % 8u, local = blockIdx.x / 8u;
    const uint32_t per = n / 8u, extra = n % 8u;
    const uint32_t bid = xcd * per + (xcd < extra ? xcd : extra) + local;
    // bid = ((s * n_k_heads + kh) * groups + g) * row_blocks + rb, split by
    // multiplies with the host's reciprocals (no integer division).
    auto divmod = [](uint32_t x, uint32_t d, uint32_t magic, uint32_t shift, uint32_t &r) {
      const uint32_t q = (uint32_t)(((uint64_t)x * magic) >> shift);
      r = x - q * d;
      return q;
    };
    uint32_t g, khead;
    uint32_t rest = divmod(bid, row_blocks, rb_magic, shifts & 0xFFu, rb);
    rest = divmod(rest, groups, g_magic, (shifts >> 8) & 0xFFu, g);
    s = divmod(rest, n_k_heads, kh_magic, shifts >> 16, khead);
    vh = khead + g * n_k_heads;
    kh = khead;  // vh % n_k_heads
  }
  // s * n_v_heads + vh is below the grid size (host-checked < 2^24).
  const uint32_t hs = s * n_v_heads + vh;

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t grp = lane / L;
  const uint32_t sub = lane % L;

  const uint32_t Dv = d_v;
  const uint32_t T = n_tokens;
  const uint64_t Hv = n_v_heads, Hk = n_k_heads;

  // This lane's rows. Rows past D_v compute on a clamped (valid) row and
  // store nothing; all lanes stay active for the cross-lane sums. The high
  // half of a paired group holds the group's two rows in swapped order.
  const bool high = PAIRED && sub >= L / 2;
  uint32_t row[R];
  bool ok[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t slot = high ? R - 1 - r : r;
    const uint32_t i = rb * ROWS + wave * ROWS_PER_WAVE + slot * G + grp;
    ok[r] = i < Dv;
    row[r] = ok[r] ? i : Dv - 1;
  }

  // The state rows first: their requests need only preloaded arguments, and
  // the scheduling barrier keeps every read of kernel-argument memory (the
  // other arrays' bases) behind them. Per-lane byte offsets, fixed for the
  // whole call: vector m of row r starts at column m*4L + 4*sub (state: 16
  // bytes per vector; k/q: 4*IB bytes).
  const uint32_t head_bytes = Dv * ROW_BYTES;
  const rsrc_t s_in = buffer(state_in + (uint64_t)hs * Dv * DK, head_bytes);
  const uint32_t col = 16 * sub;
  uint32_t cell[R];
#pragma unroll
  for (int r = 0; r < R; ++r) cell[r] = row[r] * ROW_BYTES + col;
  f4 st[R][NV];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < NV; ++m) st[r][m] = load4_stream(s_in, cell[r] + m * 16 * L);
  __builtin_amdgcn_sched_barrier(0);

  // Wave-uniform bases of this (s, vh): token-0 addresses and per-token
  // strides, in elements. The k/q/v descriptors start at a token's row and
  // reach the end of the sequence (see rebase); state and capture descriptors
  // cover one head (D_v x D_k floats; the host guarantees d_v * d_k * 4 <
  // 2^32).
  const uint64_t tok0 = (uint64_t)s * T;                   // first token of s
  const char *k_tok = static_cast<const char *>(a.k) + ((tok0 * Hk + kh) * DK) * IB;
  const char *q_tok = static_cast<const char *>(a.q) + ((tok0 * Hk + kh) * DK) * IB;
  const uint64_t kq_step = Hk * DK;
  const char *v_tok = static_cast<const char *>(a.v) + ((tok0 * Hv + vh) * Dv) * IB;
  char *o_tok = static_cast<char *>(a.output) + ((tok0 * Hv + vh) * Dv) * IB;
  const uint64_t v_step = Hv * Dv;
  const float *g_tok = a.g + tok0 * Hv + vh;
  const float *b_tok = a.beta + tok0 * Hv + vh;
  float *c_tok = CAPTURE ? a.capture + (tok0 * Hv + vh) * (uint64_t)Dv * DK : nullptr;
  const uint64_t cap_step = Hv * Dv * DK;
  const rsrc_t s_out = buffer(a.state_out + (uint64_t)hs * Dv * DK, head_bytes);

  uint32_t vrow[NY];
#pragma unroll
  for (int r = 0; r < NY; ++r) vrow[r] = row[r] * IB;
  // Outputs are written TB tokens at a time, TB being the number of lanes
  // that hold a row's sums (L, or L/2 when paired): lane j of them keeps the
  // row's output of token t0 + j (t0 a multiple of TB) in yk, and one store
  // per row writes the TB tokens. Stores share the in-order memory counter
  // with the prefetch loads, so one store per token would hold back every
  // later prefetch behind its write acknowledgement.
  constexpr uint32_t TB = PAIRED ? L / 2 : L;  // divides 64
  const uint32_t slot_t = sub % TB;            // token slot of this lane
  // Paired multi-token calls defer the sums: token slot j keeps the lane's
  // pair-level partial of y (yp[j]), and one reduce-scatter over the TB lanes
  // of each half per TB tokens leaves token t0 + j's output in lane j. The
  // per-token butterfly (log2(TB) dependent cross-lane adds) leaves the
  // token's instruction stream.
  constexpr bool DEFER = PAIRED;
  static_assert(!DEFER || NB % TB == 0, "ring groups hold whole output batches");
  // yp keeps the lane's A-row partial and yq its B-row partial of each token
  // slot; the flush pairs them (a + partner's b), so the pairing adds of a
  // batch are independent of each other instead of one per token on that
  // token's dependent chain.
  float yp[DEFER ? TB : 1], yq[DEFER ? TB : 1];
#pragma unroll
  for (uint32_t j = 0; j < (DEFER ? TB : 1); ++j) yp[j] = yq[j] = 0.f;
  float yk[NY];
  uint32_t yoff[NY];  // lane's output address: row r of token t0 + slot_t
#pragma unroll
  for (int r = 0; r < NY; ++r) {
    yk[r] = 0.f;
    yoff[r] = vrow[r] + slot_t * (uint32_t)(Hv * Dv * IB);
  }

  // Register element e of a cell vector holds column (e + ROT) % 4 of its four
  // columns. The k/q column vectors arrive in aligned register quads, as the
  // state does, so with ROT = 0 every multiply-add would read cell and key (or
  // query) element e from the same VGPR bank, and a quarter of them a third
  // operand from that bank too, which costs the VALU a second cycle. ROT = 1
  // puts them in different banks (multi-token calls without capture; capture
  // stores the cells every token and keeps ROT = 0).
  constexpr int ROT = CAPTURE ? 0 : 1;
  if constexpr (ROT == 1)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < NV; ++m) st[r][m] = st[r][m].yzwx;

  // k and q are staged through LDS. All G row groups of a wave
  // need the same k and q columns, so direct per-lane loads would pull every
  // byte through the vector memory unit G times. Instead the wave reads each
  // token's k and q rows once (RB bytes per lane), parks them in a per-wave
  // LDS slot, and every lane reads its own columns from there.
  // Lane j loads elements EPL*j .. EPL*j+EPL-1 of each row (lanes past the
  // row repeat its last part and write nothing) and stores them widened to
  // f32, so the column reads need no conversion.
  constexpr uint32_t EPL = DK >= 64 ? DK / 64 : 1;  // elements per lane
  constexpr uint32_t SLANES = DK / EPL;              // lanes holding a part
  constexpr int RB = EPL * IB;                       // staged bytes per lane
  static_assert(RB == 2 || RB == 4 || RB == 8, "staged row size");
  typedef typename Raw<RB>::T RawT;
  __shared__ __attribute__((aligned(16))) float kq_lds[WAVES][2 * DK];
  float *const kq_row = kq_lds[wave];  // k row, then q row (f32)
  const uint32_t slane = lane < SLANES ? lane : SLANES - 1;
  struct Tok {
    RawT kr, qr;  // this lane's part of the token's k and q rows (raw bytes)
  };
  struct KQ {
    f4 k[NV], q[NV];
    float inv;  // NK: 1 / sqrt(sum k^2 + kNormEps) of the token's key row
  };
  // k, q, v and output are read through descriptors based at token base_t
  // that reach to the end of this sequence; token t's row is at scalar byte
  // offset (t - base_t) * stride. Rebased every 64 tokens, so the scalar
  // offsets stay far below 2^32 (the host bounds the per-token strides).
  const uint32_t kq_bytes = (uint32_t)kq_step * IB, v_bytes = (uint32_t)v_step * IB;
  uint32_t base_t = 0, kq_ext = 0, v_ext = 0;
  const char *k_b = nullptr, *q_b = nullptr, *v_b = nullptr;
  char *o_b = nullptr;
  auto rebase = [&](uint32_t t0) {
    base_t = uniform(t0);
    const uint64_t rest = T - t0 - 1;  // tokens after t0
    k_b = uniform(k_tok + t0 * kq_step * IB);
    q_b = uniform(q_tok + t0 * kq_step * IB);
    v_b = uniform(v_tok + t0 * v_step * IB);
    o_b = uniform(o_tok + t0 * v_step * IB);
    kq_ext = uniform(extent_bytes((rest * kq_step + DK) * IB));
    v_ext = uniform(extent_bytes((rest * v_step + Dv) * IB));
  };
  // Token 0: the bases themselves, sizes from the host.
  base_t = 0;
  k_b = uniform(k_tok);
  q_b = uniform(q_tok);
  v_b = uniform(v_tok);
  o_b = uniform(o_tok);
  kq_ext = a.kq_ext0;
  v_ext = a.v_ext0;

  // Token rows at byte offset kq_off from base_t's row.
  auto load_token_at = [&](uint32_t kq_off, Tok &x) {
    const rsrc_t k_rs = buffer(k_b, kq_ext), q_rs = buffer(q_b, kq_ext);
    x.kr = Raw<RB>::load(k_rs, slane * RB, kq_off);
    x.qr = Raw<RB>::load(q_rs, slane * RB, kq_off);
  };
  auto load_token = [&](uint32_t t, Tok &x) {
    load_token_at(uniform((t - base_t) * kq_bytes), x);
  };

  // Multi-token calls read v once per ring group: the wave's ROWS_PER_WAVE
  // rows (consecutive) times the group's NB tokens are at most 64 values, so
  // lane j requests token t0 + j / ROWS_PER_WAVE of row j % ROWS_PER_WAVE
  // (clamped to the last token and row), parks it in a per-wave LDS slot laid
  // out row by row, and every lane reads its rows' NB values back. One
  // vector-memory request per group instead of one per token.
  constexpr uint32_t VT = ROWS_PER_WAVE * NB;
  static_assert(VT <= 64, "one value per lane per ring group");
  __shared__ __attribute__((aligned(16))) float v_lds[WAVES][VT];
  float *const vslot = v_lds[wave];
  const uint32_t vl = lane < VT ? lane : VT - 1;
  const uint32_t vl_row = rb * ROWS + wave * ROWS_PER_WAVE + vl % ROWS_PER_WAVE;
  const uint32_t vl_off = (vl_row < Dv ? vl_row : Dv - 1) * IB;
  const uint32_t vl_tok = vl / ROWS_PER_WAVE;
  auto load_vgroup = [&](uint32_t t0) {
    const uint32_t tk = t0 + vl_tok < T ? t0 + vl_tok : T - 1;  // >= base_t
    return Io<IO>::load1(buffer(v_b, v_ext), vl_off + (tk - base_t) * v_bytes, 0);
  };
  // Park a group's raw v and return this lane's rows' NB values.
  auto park_vgroup = [&](float raw, float (&vg)[NY][NB]) {
    if (lane < VT) vslot[(vl % ROWS_PER_WAVE) * NB + vl_tok] = raw;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < NY; ++r) {
      const uint32_t slot = PAIRED ? (high ? 1u : 0u) : (uint32_t)r;
#pragma unroll
      for (int u = 0; u < NB; ++u) vg[r][u] = vslot[(slot * G + grp) * NB + u];
    }
  };

  // Shared staging (multi-token calls without capture, and without the
  // per-token key normalisation, which sums each key row in the wave that
  // loads it; the group-ahead normalisation computes each row's factor in
  // the wave that stages it, see staged_norms). All waves of a workgroup need the same k and q rows, so
  // instead of every wave loading every token's rows, each wave loads NB /
  // WAVES tokens of the next ring group and stages them, widened to f32, in
  // a workgroup LDS block (two of them, one per alternate group); one
  // workgroup barrier per group publishes the block. Every wave of a
  // workgroup runs the same token loop, so every wave reaches every barrier.
  // Four times fewer row requests, and no staging write per token: the
  // 512-token prefill went from 177 to 169 us, its key-normalised form from
  // 204 to 187 us. Not at D_k = 32, where a wave's rows are a quarter as
  // long and the per-group barrier costs more than the loads it saves
  // (a D_k = 32 prefill ran 106 us without it, 118 us with it).
  constexpr bool SHARE = !CAPTURE && NK != 1 && DK >= 64 && NB % WAVES == 0;
  constexpr int TPW = SHARE ? NB / WAVES : 1;  // tokens a wave stages per group
  // Group-ahead key normalisation with shared staging: the staged keys are
  // scaled by their factors, and step() runs as without normalisation.
  constexpr bool SNORM = SHARE && NK == 2;

  // Key normalisation in multi-token calls without shared staging (D_k = 32,
  // capture): the factors 1 / sqrt(sum k^2 + kNormEps) of a ring group's NB
  // key rows are computed one group ahead.
  // LPT = 64 / NB lanes share a token's row, each summing the squares of EPT
  // consecutive elements; a butterfly over the LPT lanes and one reciprocal
  // square root give the token's factor, parked in a per-wave LDS slot and
  // read back as broadcasts when the group starts. One butterfly and one
  // square root per group instead of a wave-wide sum per token. A lane's
  // slice is requested in KP parts (two when it holds 8 or more elements, at
  // the group's start and middle) to bound the registers in flight.
  constexpr bool GNORM = NK == 2 && !SHARE;
  constexpr uint32_t LPT = 64 / NB;
  constexpr uint32_t EPT = DK / LPT;
  static_assert(!GNORM || EPT == 2 || EPT % 4 == 0, "key row split");
  constexpr uint32_t KP = EPT >= 8 ? 2 : 1;          // parts per slice
  constexpr uint32_t KV = EPT >= 4 ? EPT / 4 / KP : 1;  // float4 per part
  __shared__ __attribute__((aligned(16))) float inv_lds[GNORM ? WAVES : 1][GNORM ? NB : 1];
  float *const inv_slot = inv_lds[GNORM ? wave : 0];
  struct KRow {
    f4 x[KV];
    float y[2];
  };
  auto load_krow = [&](uint32_t t0, uint32_t part, KRow &kr) {
    const uint32_t tk = t0 + lane / LPT < T ? t0 + lane / LPT : T - 1;  // >= base_t
    const uint32_t off = (tk - base_t) * kq_bytes + ((lane % LPT) * EPT + part * (EPT / KP)) * IB;
    const rsrc_t rs = buffer(k_b, kq_ext);
    if constexpr (EPT >= 4) {
#pragma unroll
      for (uint32_t i = 0; i < KV; ++i) kr.x[i] = Io<IO>::load4(rs, off + i * 4 * IB, 0);
    } else {
#pragma unroll
      for (uint32_t i = 0; i < 2; ++i) kr.y[i] = Io<IO>::load1(rs, off + i * IB, 0);
    }
  };
  auto add_krow = [&](const KRow &kr, float ss) {
    if constexpr (EPT >= 4) {
#pragma unroll
      for (uint32_t i = 0; i < KV; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss = __builtin_fmaf(kr.x[i][e], kr.x[i][e], ss);
    } else {
#pragma unroll
      for (uint32_t i = 0; i < 2; ++i) ss = __builtin_fmaf(kr.y[i], kr.y[i], ss);
    }
    return ss;
  };
  auto park_krow = [&](float ss) {
    ss = group_sum<LPT>(ss);
    if (lane % LPT == 0) inv_slot[lane / LPT] = __builtin_amdgcn_rsqf(ss + kNormEps);
  };
  auto read_krow = [&](float (&inv)[GNORM ? NB : 1]) {
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (uint32_t u = 0; u < (GNORM ? NB : 1); ++u) inv[u] = inv_slot[u];
  };

  // This lane's k and q columns of a token, through the staged LDS slot. The
  // slot is rewritten per token; LDS operations of a wave run in order, so
  // the reads of one token complete before the next token's write.
  auto columns = [&](const Tok &x) {
    KQ c;
    c.inv = 1.f;
    float kw[EPL], qw[EPL];
    widen<IO, EPL>(x.kr, kw);
    widen<IO, EPL>(x.qr, qw);
    if constexpr (NORMK && !GNORM) {
      // The wave holds the whole key row: its sum of squares over all lanes
      // (lanes past the row repeat its last part and count zero). The keys
      // stay unscaled; step() folds the factor into sk and delta, so this
      // reduction overlaps the LDS round trip instead of preceding it.
      float ss = 0.f;
#pragma unroll
      for (uint32_t e = 0; e < EPL; ++e) ss = __builtin_fmaf(kw[e], kw[e], ss);
      c.inv = __builtin_amdgcn_rsqf(wave_sum(lane < SLANES ? ss : 0.f) + kNormEps);
    }
    if (SLANES == 64 || lane < SLANES) {
#pragma unroll
      for (uint32_t e = 0; e < EPL; ++e) {
        kq_row[EPL * lane + e] = kw[e];
        kq_row[DK + EPL * lane + e] = qw[e];
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      c.k[m] = *reinterpret_cast<const f4 *>(kq_row + m * 4 * L + 4 * sub);
      c.q[m] = *reinterpret_cast<const f4 *>(kq_row + DK + m * 4 * L + 4 * sub);
    }
    return c;
  };

  __shared__ __attribute__((aligned(16)))
  float grp_lds[SHARE ? 2 : 1][SHARE ? NB : 1][SHARE ? 2 * DK : 1];
  // This lane's part of a token's rows, widened, into a staged row pair; the
  // key row scaled by ks (SNORM).
  auto stage_rows = [&](const Tok &x, float *dst, float ks) {
    float kw[EPL], qw[EPL];
    widen<IO, EPL>(x.kr, kw);
    widen<IO, EPL>(x.qr, qw);
    if (SLANES == 64 || lane < SLANES) {
#pragma unroll
      for (uint32_t e = 0; e < EPL; ++e) {
        dst[EPL * lane + e] = SNORM ? kw[e] * ks : kw[e];
        dst[DK + EPL * lane + e] = qw[e];
      }
    }
  };
  // SNORM: the factors 1 / sqrt(sum k^2 + kNormEps) of the TPW (1, 2 or 4)
  // key rows this wave stages, from the parts its lanes hold. Each lane sums
  // the squares of its part of every row; swapping the wave halves of rows 2i
  // and 2i+1 and adding leaves row 2i's partials in lanes 0-31 and row
  // 2i+1's in lanes 32-63 of one register (one row: the row with itself).
  // With four rows, swapping the odd 16-lane rows of the first such register
  // with the even ones of the second and adding gives one register whose
  // 16-lane rows hold the partials of key rows 0, 2, 1 and 3; a butterfly
  // within 16 lanes completes every sum. With one or two rows the butterfly
  // leaves half sums, and adding the row below's lane 15 completes them in
  // lanes 31 and 63. Wave-uniform results, a few cross-lane steps per group
  // for the wave's rows instead of a butterfly and a factor multiply per
  // token.
  auto staged_norms = [&](const Tok (&b)[TPW], float (&inv)[TPW]) {
    static_assert(!SNORM || TPW == 1 || TPW == 2 || TPW == 4, "1, 2 or 4 staged rows");
    if constexpr (SNORM) {
      float ss[TPW];
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        float kw[EPL];
        widen<IO, EPL>(b[i].kr, kw);
        ss[i] = 0.f;
#pragma unroll
        for (uint32_t e = 0; e < EPL; ++e) ss[i] = __builtin_fmaf(kw[e], kw[e], ss[i]);
        if (SLANES < 64 && lane >= SLANES) ss[i] = 0.f;  // repeated parts
      }
      // The swap's results are vector elements: each is cast to a plain value
      // before the bit cast, which otherwise reads the vector's first element
      // whatever the index (clang 22).
      constexpr int NH = TPW > 1 ? TPW / 2 : 1;  // row pairs
      float h[NH];
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        const float odd = ss[TPW > 1 ? 2 * i + 1 : 0];
        const auto w = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, ss[2 * i]),
                                                        __builtin_bit_cast(uint32_t, odd), false,
                                                        false);
        h[i] = __builtin_bit_cast(float, (uint32_t)w[0]) +
               __builtin_bit_cast(float, (uint32_t)w[1]);
      }
      auto lane_value = [](float x, int l) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
      };
      if constexpr (TPW <= 2) {
        float x = group_sum<16>(h[0]);
        x += dpp<kDppBcast15>(x);
        x = __builtin_amdgcn_rsqf(x + kNormEps);
        inv[0] = lane_value(x, 31);
        if constexpr (TPW == 2) inv[1] = lane_value(x, 63);
      } else {
        const auto w = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, h[0]),
                                                        __builtin_bit_cast(uint32_t, h[1]),
                                                        false, false);
        float x = group_sum<16>(__builtin_bit_cast(float, (uint32_t)w[0]) +
                                __builtin_bit_cast(float, (uint32_t)w[1]));
        x = __builtin_amdgcn_rsqf(x + kNormEps);
        inv[0] = lane_value(x, 0);
        inv[1] = lane_value(x, 32);
        inv[2] = lane_value(x, 16);
        inv[3] = lane_value(x, 48);
      }
    }
  };
  // This lane's columns of a staged row pair.
  auto columns_at = [&](const float *rows) {
    KQ c;
    c.inv = 1.f;
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      c.k[m] = *reinterpret_cast<const f4 *>(rows + m * 4 * L + 4 * sub);
      c.q[m] = *reinterpret_cast<const f4 *>(rows + DK + m * 4 * L + 4 * sub);
    }
    return c;
  };

  // Factor table of the current 64-token chunk (see next_chunk below): alpha,
  // b, c and beta of its tokens, each in its own array, so that a ring group
  // reads each factor of its NB tokens with NB / 4 16-byte reads.
  __shared__ __attribute__((aligned(16))) float ab_lds[WAVES][4][64];
  float *const fa = ab_lds[wave][0], *const fb = ab_lds[wave][1];
  float *const fc = ab_lds[wave][2], *const fbeta = ab_lds[wave][3];

  // One token. With decay set (c = 1, b = beta): the cells are multiplied by
  // alpha, then sk, delta = (v - sk) * beta, the rank-1 write and y, as the
  // recurrence is written. Lazy tokens (decay clear)
  // keep the state divided by c, the product of the alphas of the ring
  // group's tokens after its first, up to this one, and leave the cells
  // undecayed: sk = c * (cells . k), the write adds delta / c along k
  // (b = beta / c), y = c * (cells . q). The same recurrence reassociated,
  // one multiply per cell and token fewer. decay is wave-uniform.
  // j: the token's output slot t % TB when ring groups hold whole output
  // batches (NB % TB == 0), a constant after unrolling. may_end: t may be the
  // last token (in a ring group only the last token can be, and it then ends
  // an output batch anyway).
  // hold: a batch that this token ends is not stored here but by
  // store_held(), after the ring group's staging wait (see there).
  uint32_t held = 0, held_soff = 0;  // wave-uniform
  // alpha_at: read the token's alpha from the factor table at index t & 63
  // when it decays (a lazy group's tokens after its first do not decay, and
  // then read nothing), instead of the alpha argument.
  auto step = [&](uint32_t t, uint32_t j, bool may_end, const KQ &kq, const float (&v)[NY],
                  uint32_t decay, float alpha, bool alpha_at, float b, float c, bool raise,
                  bool hold) {
    // The sk chain (decay, dot products, butterfly, delta) is what the rest
    // of the token, and the next token, wait for; the rank-1 write and y are
    // throughput work the other waves of the SIMD can interleave with. The
    // wave's issue priority is raised for the chain and dropped after delta
    // (512-token prefill 183.5 -> 178.5 us; dropping it after the write
    // instead: 185.4 us). raise: not raised yet by the caller.
    if (raise) __builtin_amdgcn_s_setprio(1);
    // Normalised keys (NK, unless the staged keys are already scaled): sk =
    // c * inv * (cells . k) and the write adds delta * inv along the raw k,
    // the same as using k * inv throughout.
    float cs = c, bs = b;
    if constexpr (NORMK && !SNORM) {
      cs = c * kq.inv;
      bs = b * kq.inv;
    }
    if (decay != 0) {
      const float a = alpha_at ? fa[t & 63u] : alpha;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < NV; ++m) st[r][m] *= a;
    }
    float part[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      part[r] = 0.f;
#pragma unroll
      for (int m = 0; m < NV; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          part[r] = __builtin_fmaf(st[r][m][e], kq.k[m][(e + ROT) % 4], part[r]);
        }
    }
    float d[R];
    if constexpr (PAIRED) {
      d[0] = __builtin_fmaf(-cs, pair_sum<L>(part[0], part[1]), v[0]) * bs;
      d[1] = partner<L>(d[0]);  // the partner's A row is this lane's B row
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) d[r] = __builtin_fmaf(-cs, group_sum<L>(part[r]), v[r]) * bs;
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      part[r] = 0.f;
#pragma unroll
      for (int m = 0; m < NV; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          st[r][m][e] = __builtin_fmaf(d[r], kq.k[m][(e + ROT) % 4], st[r][m][e]);
          part[r] = __builtin_fmaf(st[r][m][e], kq.q[m][(e + ROT) % 4], part[r]);
        }
    }
    if constexpr (CAPTURE) {
      // The token's capture slice is stored before y's cross-lane sum, so
      // its writes run under that sum (stores keep program order). The
      // empty asm keeps the compiler from sinking the partials' arithmetic
      // below the stores.
#pragma unroll
      for (int r = 0; r < R; ++r) asm volatile("" : "+v"(part[r]));
      const rsrc_t ct = buffer(c_tok + t * cap_step, head_bytes);
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (ok[r])
#pragma unroll
          for (int m = 0; m < NV; ++m) store4_stream(ct, cell[r] + m * 16 * L, st[r][m]);
    }
    const bool mine = slot_t == (t & (TB - 1));
    if constexpr (DEFER) {
      // Only the flush reads the partial; the empty asm keeps the compiler
      // from sinking the token's dot product there, which would hold every
      // token's cells live until the end of the batch. The partial is kept
      // without the token's c: the flush applies c once to the lane's sum.
      float ya = part[0], yb = part[1];
      asm volatile("" : "+v"(ya), "+v"(yb));
#pragma unroll
      for (uint32_t i = 0; i < TB; ++i) {
        yp[i] = i == j ? ya : yp[i];
        yq[i] = i == j ? yb : yq[i];
      }
    } else if constexpr (PAIRED) {
      const float y = c * pair_sum<L>(part[0], part[1]);
      yk[0] = mine ? y : yk[0];
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float y = c * group_sum<L>(part[r]);
        yk[r] = mine ? y : yk[r];
      }
    }
    // Ring groups that hold whole batches end one only at a known token.
    const bool flush = NB % TB == 0 ? j == TB - 1 || (may_end && t + 1 == T)
                                    : (t & (TB - 1)) == TB - 1 || t + 1 == T;
    if (flush) {
      // The batch's reduce-scatter and store are a dependent chain as well:
      // raised priority (512-token prefill -1.2%).
      __builtin_amdgcn_s_setprio(1);
      // Token slots 0 .. t % TB hold tokens t0 .. t. base_t is a multiple of
      // 64 and at most t, so t0 - base_t >= 0. q_scale is applied here.
      const uint32_t t0 = t & ~(TB - 1);
      const rsrc_t o_rs = buffer(o_b, v_ext);
      const uint32_t soff = uniform((t0 - base_t) * v_bytes);
      if constexpr (DEFER) {
        float w[TB];
#pragma unroll
        for (uint32_t i = 0; i < TB; ++i) w[i] = pair_part<L>(yp[i], yq[i]);
        scatter_sum<TB / 2>(w, slot_t);
        // Token t0 + slot_t's c: from the factor table in a ring group (1
        // when the group ran eagerly); tokens after the last whole group run
        // with c = 1.
        yk[0] = may_end ? w[0] : w[0] * fc[(t0 & 63u) + slot_t];
      }
      if (hold) {
        held = 1;
        held_soff = soff;
      } else if (slot_t <= (t & (TB - 1))) {
#pragma unroll
        for (int r = 0; r < NY; ++r)
          if (ok[r]) Io<IO>::store1(o_rs, yoff[r], soff, yk[r] * a.q_scale);
      }
      __builtin_amdgcn_s_setprio(0);
    }
  };
  // The held batch (it ended a ring group, so every token slot is filled).
  // The memory counter runs in issue order, so a wait for the rows that
  // were requested at the group's start also waits for every store issued
  // after them; and when a store is issued on some paths only, the
  // compiler's bookkeeping waits as if it were (for its write
  // acknowledgement). Issued after that wait, the store is not waited for
  // until the next group's end, long after it has completed.
  auto store_held = [&]() {
    if (held != 0) {
      const rsrc_t o_rs = buffer(o_b, v_ext);
#pragma unroll
      for (int r = 0; r < NY; ++r)
        if (ok[r]) Io<IO>::store1(o_rs, yoff[r], held_soff, yk[r] * a.q_scale);
      held = 0;
    }
  };

  {
    // Raw g and beta of the 64-token chunk starting at t0: lane j holds token
    // t0 + j (clamped to the last token; lanes past the end are never read).
    auto load_chunk = [&](uint32_t t0, float &gr, float &br) {
      const uint32_t t = lane < T - t0 ? t0 + lane : T - 1;
      gr = *(g_tok + (uint64_t)t * Hv);
      br = *(b_tok + (uint64_t)t * Hv);
    };

    // Per-token factors of the current 64-token chunk live in a small
    // per-wave LDS slot (fa, fb, fc, fbeta), computed once per chunk (lane j:
    // token t0 + j) and read per ring group as broadcasts: alpha = exp(-g),
    // b, c and beta.
    // In a ring group that runs lazily, c is the product of the alphas of the
    // group's tokens 1 .. u (1 at u = 0) and b = beta / c. A group runs
    // eagerly (every token decays; c = 1, b = beta) if any of its c or
    // beta / c, or the alpha of its first token, would leave [2^-63, 2^63]
    // or is not finite (strong decay or growth, special values), and always
    // when the state is captured. A lazy group's first token decays by
    // kappa * alpha (kappa: the previous group's last c, or 1), so both
    // factors within [2^-63, 2^63] keep that product a normal number. The
    // raw g/beta of the next chunk are requested a chunk ahead into registers
    // that nothing else reads.
    float g_raw, b_raw;
    load_chunk(0, g_raw, b_raw);
    // Bit j set: token t0 + j belongs to an eager group (wave-uniform).
    uint64_t eager_mask = ~0ull;
    auto next_chunk = [&](uint32_t t) {
      if ((t & 63u) == 0) {
        const float al = expf(-g_raw), be = b_raw;
        if constexpr (CAPTURE) {
          fa[lane] = al;
          fb[lane] = be;
          fc[lane] = 1.f;
          fbeta[lane] = be;
        } else {
          fa[lane] = al;
          const uint32_t q0 = lane & ~(NB - 1u), u = lane & (NB - 1u);
          // c: the product of the alphas of the group's tokens 1 .. u, as an
          // inclusive prefix product over the group's lanes (lane u holds 1
          // at u = 0, its alpha otherwise; the step of span S multiplies in
          // the partial product of the lane S below, which lies in the same
          // NB-lane-aligned group when u >= S). Every lane reads its
          // neighbour (the DPP moves stand outside the selects, so no lane
          // reads from a disabled one).
          static_assert(NB <= 8, "prefix product within a 16-lane DPP row");
          float c = u == 0 ? 1.f : al;
          const float p1 = dpp<kDppShr1>(c);
          c = u >= 1 ? c * p1 : c;
          if constexpr (NB >= 4) {
            const float p2 = dpp<kDppShr2>(c);
            c = u >= 2 ? c * p2 : c;
          }
          if constexpr (NB >= 8) {
            const float p4 = dpp<kDppShr4>(c);
            c = u >= 4 ? c * p4 : c;
          }
          const float bc = be / c;
          const bool lazy_ok = c >= 0x1p-63f && c <= 0x1p63f &&
                               __builtin_fabsf(bc) <= 0x1p63f &&
                               (u != 0 || (al >= 0x1p-63f && al <= 0x1p63f));
          const uint64_t bad = __builtin_amdgcn_ballot_w64(!lazy_ok);
          eager_mask =
              (uint64_t)uniform((uint32_t)(bad >> 32)) << 32 | uniform((uint32_t)bad);
          const bool eager = (eager_mask >> q0) & ((1ull << NB) - 1u);
          fb[lane] = eager ? be : bc;
          fc[lane] = eager ? 1.f : c;
          fbeta[lane] = be;
        }
        // After the last use of this chunk's raw values, so that the requests
        // can land in the same registers without a copy (and a wait).
        if (T - t > 64) load_chunk(t + 64, g_raw, b_raw);
        __builtin_amdgcn_wave_barrier();
      }
    };
    auto run = [&](uint32_t t, uint32_t j, const KQ &kq, const float (&v)[NY]) {
      next_chunk(t);
      step(t, j, true, kq, v, true, fa[t & 63u], false, fbeta[t & 63u], 1.f, true, false);
    };

    // base_t moves in steps of 64 only if every group starts on a multiple
    // of NB that divides 64.
    static_assert(64 % NB == 0, "ring groups align with 64-token chunks");
    // Prefetch ring. Invariant at the top of each group: buf[0 .. NB-2] hold
    // tokens t .. t+NB-2. Requests past the last token are clamped to it
    // (they are never used): every request is unconditional, because a
    // request that some paths skip makes the compiler's memory-counter
    // bookkeeping wait for all outstanding loads, the prefetches included.
    // v of the group starting at t, requested before the ring so that the
    // first group's wait for it leaves the ring's requests in flight.
    float v_raw = load_vgroup(0);
    Tok buf[SHARE ? TPW : NB];
    uint32_t gb = 0;  // SHARE: the staged block of the current group
    if constexpr (SHARE) {
      // The first group's rows (this wave's share), staged and published.
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const uint32_t tk = wave * TPW + i;
        load_token(tk < T ? tk : T - 1, buf[i]);
      }
      float ks[TPW] = {};
      if constexpr (SNORM) staged_norms(buf, ks);
#pragma unroll
      for (int i = 0; i < TPW; ++i) stage_rows(buf[i], grp_lds[0][wave * TPW + i], ks[i]);
      __syncthreads();
      // Every request so far (state, the first chunk's g and beta, the first
      // group's v) completes before the loop. The compiler orders these
      // requests freely; one of them still in flight on entry would make its
      // bookkeeping at the loop's first wait for v (every group) cover the
      // requests issued after it in the loop, such as the next chunk's g and
      // beta or the held output store.
      __builtin_amdgcn_s_waitcnt(kWaitVmAll);
    } else {
#pragma unroll
      for (int u = 0; u < NB - 1; ++u) load_token(u < T ? u : T - 1, buf[u]);
    }
    float vg[NY][NB];
    uint32_t t = 0;
    // Columns of the current token. Without capture each step stages the next
    // token's k and q rows through LDS before computing its own, so the LDS
    // round trip runs under the current token's arithmetic (512-token prefill
    // -2%); capture calls, bound by their writes, stage each token in its own
    // step (4-token verify +2% the other way).
    constexpr bool AHEAD = !CAPTURE;
    KQ kq;
    if constexpr (SHARE) {
      kq = columns_at(grp_lds[0][0]);
    } else if constexpr (AHEAD) {
      kq = columns(buf[0]);
    }
    KRow kn;
    float kss = 0.f;  // sum of squares of the parts already received
    float invg[GNORM ? NB : 1];
    if constexpr (GNORM) {
#pragma unroll
      for (uint32_t p = 0; p < KP; ++p) {
        load_krow(0, p, kn);
        kss = add_krow(kn, kss);
      }
      park_krow(kss);
    }
    // The cells hold the state divided by kappa: the c of the previous
    // group's last token when that group ran lazily, else 1. A group's first
    // token decays by kappa * alpha, which makes the cells the state again
    // (c = 1) before the group's lazy tokens.
    float kappa = 1.f;
    while (T - t >= NB) {
      if (t - base_t >= 64) rebase(t);
      // A group starts on a multiple of NB, so a chunk boundary can only fall
      // on its first token; the factors of the group's NB tokens are read
      // from LDS together, one wait per group.
      next_chunk(t);
      // b and c of the group's tokens, and its first token's alpha (the
      // others' are read only by tokens that decay, in an eager group).
      const float alpha0 = fa[t & 63u];
      float fbl[NB], fcl[NB];
#pragma unroll
      for (int v4 = 0; v4 < NB / 4; ++v4) {
        const uint32_t at = (t & 63u) + 4 * v4;
        const f4 b4 = *reinterpret_cast<const f4 *>(fb + at);
        const f4 c4 = *reinterpret_cast<const f4 *>(fc + at);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          fbl[4 * v4 + e] = b4[e];
          fcl[4 * v4 + e] = c4[e];
        }
      }
      // Nonzero: the group runs eagerly. An integer, not a bool: a bool live
      // across the group's token branches is kept as a lane mask and turned
      // into a VGPR and back for every branch.
      const uint32_t eager =
          CAPTURE ? 1u : uniform((uint32_t)(eager_mask >> (t & 63u)) & ((1u << NB) - 1u));
      if (!CAPTURE && eager != 0 && uniform(__builtin_bit_cast(uint32_t, kappa)) != 0x3F800000u) {
        // An eager group after a lazy one: back to the plain state first, so
        // that the first token's alpha (possibly extreme: that is one reason
        // to run eagerly) is not multiplied into kappa.
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int m = 0; m < NV; ++m) st[r][m] *= kappa;
        kappa = 1.f;
      }
      park_vgroup(v_raw, vg);
      v_raw = load_vgroup(t + NB);
      if constexpr (GNORM) {
        read_krow(invg);
        load_krow(t + NB, 0, kn);
      }
      if constexpr (SHARE) {
        // This wave's share of the next group's rows (clamped to the last
        // token; at most 2 NB - 1 tokens past t, within 64 + 2 NB of base_t).
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          const uint32_t tk = t + NB + wave * TPW + i;
          load_token(tk < T ? tk : T - 1, buf[i]);
        }
      }
      // The group's prefetch requests (tokens t + NB - 1 .. t + 2 NB - 2),
      // each clamped to the last token, at byte offsets from base_t's row: a
      // running offset and one minimum per token. Requests reach at most
      // 63 + 2 NB - 2 tokens past base_t, so clamping the last token's
      // distance to 96 changes no request and keeps the products below 2^32
      // (the host bounds the row stride below 2^25 bytes).
      const uint32_t last_rel = T - 1 - base_t;
      const uint32_t kq_last = uniform((last_rel < 96u ? last_rel : 96u) * kq_bytes);
      uint32_t kq_next = uniform((t + NB - 1 - base_t) * kq_bytes);
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        float vu[NY];
#pragma unroll
        for (int r = 0; r < NY; ++r) vu[r] = vg[r][u];
        // The next group's factors, parked after this group's were read.
        if constexpr (GNORM) {
          if (KP == 2 && u == NB / 2) {
            kss = add_krow(kn, 0.f);
            load_krow(t - u + NB, 1, kn);
          }
          if (u == NB - 1) park_krow(add_krow(kn, KP == 2 ? kss : 0.f));
        }
        // Raised issue priority from here through delta (step drops it):
        // the prefetch request and the next token's staging are issued
        // ahead of the other waves' throughput work (-1%).
        __builtin_amdgcn_s_setprio(1);
        KQ nxt, cur;
        if constexpr (SHARE) {
          // The next token's columns, from this group's block; the next
          // group's first token is read after the barrier.
          nxt = u + 1 < NB ? columns_at(grp_lds[gb][u + 1]) : kq;
          cur = kq;
        } else {
          load_token_at(kq_next < kq_last ? kq_next : kq_last, buf[(u + NB - 1) % NB]);
          kq_next += kq_bytes;
          // buf[(u + 1) % NB] holds token t + 1, or a clamped repeat of the
          // last token when t is the last one.
          nxt = columns(buf[AHEAD ? (u + 1) % NB : u]);
          cur = AHEAD ? kq : nxt;
        }
        if constexpr (GNORM) cur.inv = invg[u];
        step(t, u % TB, false, cur, vu, u == 0 ? 1u : eager,
             kappa * alpha0, u != 0, fbl[u], fcl[u], false, SHARE && u == NB - 1);
        kq = nxt;
        ++t;
      }
      if constexpr (SHARE) {
        // Stage this wave's share of the next group, publish, switch blocks.
        float ks[TPW] = {};
        if constexpr (SNORM) staged_norms(buf, ks);
#pragma unroll
        for (int i = 0; i < TPW; ++i) stage_rows(buf[i], grp_lds[gb ^ 1][wave * TPW + i], ks[i]);
        store_held();
        __syncthreads();
        gb ^= 1;
        kq = columns_at(grp_lds[gb][0]);
      }
      kappa = fcl[NB - 1];  // 1 after an eager group
    }
    // Back to the plain state for the remaining tokens and the final store.
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < NV; ++m) st[r][m] *= kappa;
    // Fewer than NB tokens remain, all already requested.
    if (t < T) {
      park_vgroup(v_raw, vg);
      if constexpr (GNORM) read_krow(invg);
    }
#pragma unroll
    for (int u = 0; u < NB - 1; ++u)
      if (t < T) {
        float vu[NY];
#pragma unroll
        for (int r = 0; r < NY; ++r) vu[r] = vg[r][u];
        if constexpr (SHARE) {
          KQ nxt = kq;
          if (t + 1 < T) nxt = columns_at(grp_lds[gb][u + 1]);
          KQ cur = kq;
          if constexpr (GNORM) cur.inv = invg[u];
          run(t, u % TB, cur, vu);
          kq = nxt;
        } else if constexpr (AHEAD) {
          KQ nxt = kq;
          if (t + 1 < T) nxt = columns(buf[u + 1]);
          KQ cur = kq;
          if constexpr (GNORM) cur.inv = invg[u];
          run(t, u % TB, cur, vu);
          kq = nxt;
        } else {
          KQ cur = columns(buf[u]);
          if constexpr (GNORM) cur.inv = invg[u];
          run(t, u % TB, cur, vu);
        }
        ++t;
      }
  }

#pragma unroll
  for (int r = 0; r < R; ++r)
    if (ok[r])
#pragma unroll
      for (int m = 0; m < NV; ++m)
        store4_stream(s_out, cell[r] + m * 16 * L, ROT == 1 ? st[r][m].wxyz : st[r][m]);
}

// ---------------------------------------------------------------- one token

// The arrays of one one-token launch, every base moved to the launch's first
// sequence; q, k, v and output hold the IO type, capture may be null.
struct DecodePtrs {
  const float *state_in;
  const void *k, *q;
  const float *g, *beta;
  const void *v;
  void *output;
  float *state_out, *capture;
};

// One decode token (n_tokens == 1) of the workgroup's row block rb of value
// head vh (key head kh) of sequence s: straight-line code, the state
// streamed in and out once (HBM-bound). DK, C, R, WAVES, IO and NK as for
// gdn_recurrent (NK: 0 or 1).
template <int DK, int C, int R, int WAVES, bool CAPTURE, typename IO, int NK>
__device__ __forceinline__ void decode_token(const DecodePtrs &p, uint32_t d_v,
                                             uint32_t n_v_heads, uint32_t n_k_heads,
                                             uint32_t s, uint32_t vh, uint32_t kh,
                                             uint32_t rb, float q_scale) {
  constexpr bool NORMK = NK != 0;
  constexpr int L = DK / C;
  constexpr int G = 64 / L;
  constexpr int NV = C / 4;
  constexpr int ROWS_PER_WAVE = G * R;
  constexpr uint32_t ROWS = WAVES * ROWS_PER_WAVE;
  constexpr uint32_t ROW_BYTES = DK * 4;
  constexpr uint32_t IB = Io<IO>::bytes;
  static_assert(DK % C == 0 && C % 4 == 0 && 64 % L == 0, "bad geometry");
  static_assert(R == 1 || R == 2, "one row per lane, or two paired");
  constexpr bool PAIRED = R == 2;
  constexpr int NY = PAIRED ? 1 : R;           // rows whose v and output a lane handles
  constexpr uint32_t TB = PAIRED ? L / 2 : L;  // lanes that hold a row's sums

  if (rb * ROWS >= d_v) return;  // padding of the row blocks: the whole workgroup
  const uint32_t hs = s * n_v_heads + vh;  // (s, vh) and its g/beta index (T = 1)

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t grp = lane / L;
  const uint32_t sub = lane % L;
  // Rows past d_v compute on a clamped (valid) row and store nothing; the
  // high half of a paired group holds the group's two rows in swapped order.
  const bool high = PAIRED && sub >= L / 2;
  uint32_t row[R];
  bool ok[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t slot = high ? R - 1 - r : r;
    const uint32_t i = rb * ROWS + wave * ROWS_PER_WAVE + slot * G + grp;
    ok[r] = i < d_v;
    row[r] = ok[r] ? i : d_v - 1;
  }

  // The loads, all addressed from preloaded arguments in gdn_decode: g,
  // beta and v first, then the state rows and this lane's k and q columns.
  // Vector-memory loads complete in the order issued, so the decay factor
  // is computed while the state is still arriving instead of after it.
  const float g = load1(buffer(p.g + hs, 4), 0);
  const float beta = load1(buffer(p.beta + hs, 4), 0);
  const rsrc_t v_rs = buffer(static_cast<const char *>(p.v) + (uint64_t)hs * d_v * IB, d_v * IB);
  typename Io<IO>::R1 v_raw[NY];
#pragma unroll
  for (int r = 0; r < NY; ++r) v_raw[r] = Io<IO>::raw1(v_rs, row[r] * IB, 0);
  // head_bytes: host-checked < 2^32, and a multiple of ROW_BYTES.
  const uint32_t head_bytes = d_v * ROW_BYTES;
  const uint64_t head = (uint64_t)hs * d_v * DK;
  const uint32_t col = 16 * sub, col_io = 4 * IB * sub;
  uint32_t cell[R];
#pragma unroll
  for (int r = 0; r < R; ++r) cell[r] = row[r] * ROW_BYTES + col;
  const rsrc_t s_in = buffer(p.state_in + head, head_bytes);
  f4 st[R][NV];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < NV; ++m) st[r][m] = load4_stream(s_in, cell[r] + m * 16 * L);
  // (Kept ahead of the k and q requests, which the scheduler would otherwise
  // hoist above them.) Every value is requested as raw bytes and widened
  // (bf16 I/O) only after the decay factor: a widening placed among the
  // requests would wait for its data before issuing the rest.
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t kq = ((uint64_t)s * n_k_heads + kh) * DK * IB;
  const rsrc_t k_rs = buffer(static_cast<const char *>(p.k) + kq, DK * IB);
  typename Io<IO>::R4 k_raw[NV], q_raw[NV];
#pragma unroll
  for (int m = 0; m < NV; ++m) k_raw[m] = Io<IO>::raw4(k_rs, col_io + m * 4 * IB * L, 0);
  const rsrc_t q_rs = buffer(static_cast<const char *>(p.q) + kq, DK * IB);
#pragma unroll
  for (int m = 0; m < NV; ++m) q_raw[m] = Io<IO>::raw4(q_rs, col_io + m * 4 * IB * L, 0);
  __builtin_amdgcn_sched_barrier(0);
  const float alpha = expf(-g);
  __builtin_amdgcn_sched_barrier(0);
  f4 kc[NV];
  float v[NY];
#pragma unroll
  for (int m = 0; m < NV; ++m) kc[m] = Io<IO>::widen4(k_raw[m]);
#pragma unroll
  for (int r = 0; r < NY; ++r) v[r] = Io<IO>::widen1(v_raw[r]);
  // Then the arguments that may come from kernel-argument memory (the store
  // addresses and q_scale): requested here, and waited for once (the empty
  // asm takes them as operands, so that no read is left for its first use,
  // after the arithmetic).
  void *const out = p.output;
  float *const s_out_p = p.state_out, *const cap_p = p.capture;
  const float qsc = q_scale;
  asm volatile("" ::"s"(out), "s"(s_out_p), "s"(cap_p), "s"(qsc));

  // Normalised keys (NK): the L lanes of a row group hold the whole key row;
  // 1 / sqrt(sum k^2 + kNormEps) is folded into sk and delta.
  float inv = 1.f;
  if constexpr (NORMK) {
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < NV; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = __builtin_fmaf(kc[m][e], kc[m][e], ss);
    inv = __builtin_amdgcn_rsqf(group_sum<L>(ss) + kNormEps);
  }
  const float bs = beta * inv;

  // The step as written: decay, sk, delta = (v - sk) * beta, the rank-1
  // write, y on the updated state.
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < NV; ++m) st[r][m] *= alpha;
  float part[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    part[r] = 0.f;
#pragma unroll
    for (int m = 0; m < NV; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) part[r] = __builtin_fmaf(st[r][m][e], kc[m][e], part[r]);
  }
  float d[R];
  if constexpr (PAIRED) {
    d[0] = __builtin_fmaf(-inv, pair_sum<L>(part[0], part[1]), v[0]) * bs;
    d[1] = partner<L>(d[0]);  // the partner's A row is this lane's B row
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) d[r] = __builtin_fmaf(-inv, group_sum<L>(part[r]), v[r]) * bs;
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < NV; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) st[r][m][e] = __builtin_fmaf(d[r], kc[m][e], st[r][m][e]);

  // The state (and the capture slice, the state after the token) is stored
  // before y is formed: the call ends when its last store completes, so the
  // state's writes run under y's arithmetic instead of after it. The stores
  // are unconditional: a row past d_v gets the offset head_bytes, outside
  // the descriptor's range, and the hardware drops it (no wrap-around: the
  // largest immediate offset added, (NV - 1) * 16 * L, is below ROW_BYTES,
  // and head_bytes <= 2^32 - ROW_BYTES). A branch around them would make
  // the compiler wait for their completion before the loads y needs.
  uint32_t sc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) sc[r] = ok[r] ? cell[r] : head_bytes;
  if constexpr (CAPTURE) {
    const rsrc_t ct = buffer(cap_p + head, head_bytes);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < NV; ++m) store4_stream(ct, sc[r] + m * 16 * L, st[r][m]);
  }
  const rsrc_t s_out = buffer(s_out_p + head, head_bytes);
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < NV; ++m) store4_stream(s_out, sc[r] + m * 16 * L, st[r][m]);
  __builtin_amdgcn_sched_barrier(0);

  f4 qc[NV];
#pragma unroll
  for (int m = 0; m < NV; ++m) qc[m] = Io<IO>::widen4(q_raw[m]);
  float part_y[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    part_y[r] = 0.f;
#pragma unroll
    for (int m = 0; m < NV; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) part_y[r] = __builtin_fmaf(st[r][m][e], qc[m][e], part_y[r]);
  }
  float y[NY];
  if constexpr (PAIRED) {
    y[0] = pair_sum<L>(part_y[0], part_y[1]);
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) y[r] = group_sum<L>(part_y[r]);
  }
  // Lane 0 of each set of TB lanes writes its rows' outputs, q_scale applied.
  const rsrc_t o_rs =
      buffer(static_cast<char *>(out) + (uint64_t)hs * d_v * IB, d_v * IB);
  if (sub % TB == 0)
#pragma unroll
    for (int r = 0; r < NY; ++r)
      if (ok[r]) Io<IO>::store1(o_rs, row[r] * IB, 0, y[r] * qsc);
}

// Arguments of the one-token kernels that only the stores need: read from
// kernel-argument memory (the others are preloaded into scalar registers at
// dispatch, see below) once the loads are issued, a round trip that
// completes under theirs.
struct DecodeTail {
  void *output;  // IO type
  float *state_out, *capture;
  float q_scale;
};

// Sizes of a one-token launch in one 32-bit word: d_v in bits 0-10,
// kh_bits in 11-14, n_k_heads in 15-24, n_v_heads / n_k_heads in 25-31.
constexpr uint32_t kPackDv = 11, kPackRb = 4, kPackNk = 10, kPackGroups = 7;

// Key-head bits of a one-token or short launch's grid x = (row block <<
// kh_bits) | key head: at least 3, so that the row blocks of a head
// (2^kh_bits apart in x, and the y stride a multiple of that) run on one of
// the 8 XCDs, which take workgroups round-robin, and its k, q and v rows
// are fetched into one L2 instead of all eight. Padding key heads exit at
// once.
uint32_t xcd_kh_bits(uint32_t n_k_heads) {
  uint32_t b = 3;
  while ((1u << b) < n_k_heads) ++b;
  return b;
}

// The one-token kernel. The six arrays that the loads address (state, k,
// q, g, v, beta) and the size word are the first 13 kernel-argument dwords,
// which the dispatch preloads into scalar registers (the library is built
// with that preload count): no load waits for kernel-argument memory.
// Reading v and beta's bases from it cost single-layer decode 2.75 against
// 2.69 us; q's, 2.76 (y waits for q). The grid's own sizes would be such a
// read too (they live in the implicit kernel arguments), hence the size
// word. Grid: XO (XCD order): x = (row block << kh_bits) | key head kh
// (see xcd_kh_bits); else x = (kh << rb_shift) | row block, the order of
// the state in memory, a head's row blocks padded to a power of two. y = g,
// one of the n_v_heads / n_k_heads value heads of a key head; z = sequence
// within the launch. vh = kh + g * n_k_heads (the modulo GQA map, no
// division). XCD order against memory order: single-layer decode (one row
// per lane, then 768 two-wave workgroups) 2.61 -> 2.52 us, bf16 2.68 ->
// 2.57 us; the 64-sequence batch (two rows per lane, 8,192 workgroups)
// 41.8 -> 42.0 us, so that grid keeps the memory order.
template <int DK, int C, int R, int WAVES, bool CAPTURE, typename IO, int NK, bool XO>
__global__ __launch_bounds__(WAVES * 64) void gdn_decode(
    const float *state_in, const void *k_in, const void *q_in, const float *g_in,
    const void *v_in, const float *beta_in, uint32_t sizes, DecodeTail a) {
  const uint32_t d_v = sizes & ((1u << kPackDv) - 1u);
  const uint32_t bits = (sizes >> kPackDv) & ((1u << kPackRb) - 1u);  // kh_bits or rb_shift
  const uint32_t n_k_heads = (sizes >> (kPackDv + kPackRb)) & ((1u << kPackNk) - 1u);
  const uint32_t n_v_heads = (sizes >> (kPackDv + kPackRb + kPackNk)) * n_k_heads;
  const uint32_t lo = blockIdx.x & ((1u << bits) - 1u), hi = blockIdx.x >> bits;
  const uint32_t kh = XO ? lo : hi, rb = XO ? hi : lo;
  if (XO && kh >= n_k_heads) return;  // padding of the key heads: the whole workgroup
  const uint32_t vh = kh + n_k_heads * blockIdx.y;
  const DecodePtrs p{state_in, k_in, q_in, g_in, beta_in, v_in, a.output, a.state_out, a.capture};
  decode_token<DK, C, R, WAVES, CAPTURE, IO, NK>(p, d_v, n_v_heads, n_k_heads, blockIdx.z, vh,
                                                 kh, rb, a.q_scale);
}

// The one-token kernel for sizes past the size word's fields (d_v above
// 2047, more than 1023 key heads or 127 value heads per key head). Grid: x =
// (value head << rb_shift) | row block, y = sequence within the launch.
// shifts: kh_shift in bits 0-7, rb_shift in bits 8-15; vh / n_k_heads ==
// (vh * kh_magic) >> kh_shift for every value head (host-computed, exact
// below 2^23 heads). Its sizes come from kernel-argument memory.
template <int DK, int C, int R, int WAVES, bool CAPTURE, typename IO, int NK>
__global__ __launch_bounds__(WAVES * 64) void gdn_decode_wide(
    const float *state_in, const void *k_in, const void *q_in, const float *g_in,
    const void *v_in, const float *beta_in, uint32_t d_v, uint32_t n_v_heads,
    uint32_t n_k_heads, uint32_t kh_magic, uint32_t shifts, DecodeTail a) {
  const uint32_t rb_shift = shifts >> 8, kh_shift = shifts & 0xFFu;
  const uint32_t rb = blockIdx.x & ((1u << rb_shift) - 1u);
  const uint32_t vh = blockIdx.x >> rb_shift;
  const uint32_t kh = vh - n_k_heads * (uint32_t)(((uint64_t)vh * kh_magic) >> kh_shift);
  const DecodePtrs p{state_in, k_in, q_in, g_in, beta_in, v_in, a.output, a.state_out, a.capture};
  decode_token<DK, C, R, WAVES, CAPTURE, IO, NK>(p, d_v, n_v_heads, n_k_heads, blockIdx.y, vh,
                                                 kh, rb, a.q_scale);
}

// Sizes of a short multi-token launch in one 32-bit word: d_v in bits 0-10,
// kh_bits in 11-13, n_k_heads in 14-20, n_v_heads / n_k_heads in 21-27,
// n_tokens - 1 in 28-31.
constexpr uint32_t kShortKb = 3, kShortNk = 7, kShortGroups = 7, kShortTok = 4;

// f(std::integral_constant<int, I>{}) for each I in order: a token loop
// unrolled with each token's index a compile-time constant.
template <typename F, int... I>
__device__ __forceinline__ void for_tokens(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}


// Short multi-token calls (2 <= n_tokens <= NT; speculative
// verification): the one-token kernel's layout (preloaded arguments, L
// lanes per row, one row per lane, straight-line code) extended to NT
// tokens. Grid: x = (row block << kh_bits) | key head (see xcd_kh_bits),
// y = value head of the key head, z = sequence. Every input is requested before the token loop, in the order it
// is needed: g and beta (lane t holds token t's), each token's k and q rows
// (requested once per workgroup, 2 to 8 bytes a lane, the rows spread over
// the waves, and parked in LDS, from which each lane reads its columns), v,
// then the state rows last, whose HBM round trip covers the rest; the decay factors
// are one exp over the lanes and are read back as wave-uniform values. The
// loop then runs the tokens with nothing to wait for: decay, sk, delta, the
// rank-1 write, the capture slice (CAPTURE), y. Tokens past n_tokens (up to
// NT) request clamped, valid addresses and are skipped.
template <int DK, int C, int WAVES, int NT, bool CAPTURE, typename IO, int NK>
__global__ __launch_bounds__(WAVES * 64) void gdn_short(
    const float *state_in, const void *k_in, const void *q_in, const float *g_in,
    const void *v_in, const float *beta_in, uint32_t sizes, DecodeTail a) {
  constexpr bool NORMK = NK != 0;
  constexpr int L = DK / C;  // lanes per row
  constexpr int G = 64 / L;  // rows per wave
  constexpr int NV = C / 4;  // float4 per lane and row
  constexpr uint32_t ROWS = WAVES * G;
  constexpr uint32_t ROW_BYTES = DK * 4;
  constexpr uint32_t IB = Io<IO>::bytes;
  constexpr uint32_t KQ_BYTES = DK * IB;  // one k or q row (64 to 512 bytes)
  // It is staged by SL lanes of RB bytes (EPL elements) each: 64 lanes of
  // 8, 4 or 2 bytes, or 32 lanes of one element for the shortest rows.
  constexpr uint32_t RB = KQ_BYTES / 64 >= IB ? KQ_BYTES / 64 : IB;
  constexpr uint32_t SL = KQ_BYTES / RB;
  constexpr uint32_t EPL = RB / IB;
  static_assert((EPL == 1 || EPL == 2) && SL <= 64 && SL * RB == KQ_BYTES, "k/q staging");
  static_assert(NT >= 2 && NT <= 16, "2 to 16 tokens");
  // Past 8 tokens, each token's columns are read from LDS two tokens ahead
  // instead of all before the loop, and the state is requested before the
  // (larger) k/q staging.
  constexpr bool JIT = NT > 8;
  static_assert(DK % C == 0 && C % 4 == 0 && 64 % L == 0, "bad geometry");
  // Token t's k row is row 2t of the slot, its q row 2t + 1; wave w requests
  // rows w, w + WAVES, ... and parks them for the whole workgroup.
  __shared__ __attribute__((aligned(16))) float kq_lds[NT][2][DK];
  constexpr int RPW = (2 * NT + WAVES - 1) / WAVES;  // rows per wave

  const uint32_t d_v = sizes & ((1u << kPackDv) - 1u);
  const uint32_t kh_bits = (sizes >> kPackDv) & ((1u << kShortKb) - 1u);
  const uint32_t n_k = (sizes >> (kPackDv + kShortKb)) & ((1u << kShortNk) - 1u);
  const uint32_t groups = (sizes >> (kPackDv + kShortKb + kShortNk)) & ((1u << kShortGroups) - 1u);
  const uint32_t n_tok = (sizes >> (kPackDv + kShortKb + kShortNk + kShortGroups)) + 1u;
  const uint32_t n_v = groups * n_k;
  const uint32_t kh = blockIdx.x & ((1u << kh_bits) - 1u);
  const uint32_t rb = blockIdx.x >> kh_bits;
  const uint32_t vh = kh + n_k * blockIdx.y;
  const uint32_t s = blockIdx.z;
  if (kh >= n_k) return;  // padding of the key heads: the whole workgroup

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t grp = lane / L;
  const uint32_t sub = lane % L;
  const uint32_t i = rb * ROWS + wave * G + grp;
  const bool ok = i < d_v;
  const uint32_t row = ok ? i : d_v - 1;  // rows past d_v compute on a valid row
  const uint64_t tok0 = (uint64_t)s * n_tok;  // (s, token 0) in token-major order
  auto tclamp = [&](uint32_t t) { return t < n_tok ? t : n_tok - 1; };

  // The state rows (head_bytes is host-checked < 2^32, a multiple of
  // ROW_BYTES).
  const uint32_t head_bytes = d_v * ROW_BYTES;
  const uint64_t head = ((uint64_t)s * n_v + vh) * d_v * DK;
  const uint32_t cell = row * ROW_BYTES + 16 * sub;
  f4 st[NV];
  auto load_state = [&]() {
    const rsrc_t s_in = buffer(state_in + head, head_bytes);
#pragma unroll
    for (int m = 0; m < NV; ++m) st[m] = load4_stream(s_in, cell + m * 16 * L);
  };

  // g and beta: lane t requests token t's (clamped).
  const uint32_t gb_step = n_v * 4;
  const uint32_t gb_ext = (n_tok - 1) * gb_step + 4;
  const uint32_t tl = tclamp(lane);
  const float g_l = load1(buffer(g_in + tok0 * n_v + vh, gb_ext), tl * gb_step);
  const float b_l = load1(buffer(beta_in + tok0 * n_v + vh, gb_ext), tl * gb_step);
  if constexpr (JIT) {
    load_state();
    __builtin_amdgcn_sched_barrier(0);
  }
  // k and q rows: staging lane l holds elements EPL * l ... of each.
  const uint32_t kq_step = n_k * KQ_BYTES;
  const uint32_t kq_ext = (n_tok - 1) * kq_step + KQ_BYTES;
  const uint64_t kq0 = (tok0 * n_k + kh) * KQ_BYTES;
  const rsrc_t k_rs = buffer(static_cast<const char *>(k_in) + kq0, kq_ext);
  const rsrc_t q_rs = buffer(static_cast<const char *>(q_in) + kq0, kq_ext);
  typename Raw<RB>::T kr[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const uint32_t r = wave + j * WAVES;
    const uint32_t rr = r < 2 * NT ? r : 2 * NT - 1;
    const uint32_t off = uniform(tclamp(rr / 2) * kq_step);
    const uint32_t lo = (lane % SL) * RB;  // lanes past SL repeat the row
    kr[j] = (rr & 1) ? Raw<RB>::load(q_rs, lo, off) : Raw<RB>::load(k_rs, lo, off);
  }
  // v of this lane's row, every token.
  const uint32_t v_step = n_v * d_v * IB;
  const uint32_t v_ext = (n_tok - 1) * v_step + d_v * IB;
  const uint64_t v0 = (tok0 * n_v + vh) * d_v * IB;
  const rsrc_t v_rs = buffer(static_cast<const char *>(v_in) + v0, v_ext);
  typename Io<IO>::R1 vr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) vr[t] = Io<IO>::raw1(v_rs, row * IB, uniform(tclamp(t) * v_step));
  if constexpr (!JIT) load_state();
  __builtin_amdgcn_sched_barrier(0);
  const float alpha_l = expf(-g_l);
  __builtin_amdgcn_sched_barrier(0);

  // Park the wave's k and q rows (widened to f32) and, after the workgroup
  // barrier, read this lane's columns of every token.
  float(*const slot)[2][DK] = kq_lds;
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const uint32_t r = wave + j * WAVES;
    if (r < 2 * NT && (SL == 64 || lane < SL)) {
      float w[EPL];
      widen<IO, EPL>(kr[j], w);
#pragma unroll
      for (uint32_t e = 0; e < EPL; ++e) slot[r / 2][r & 1][EPL * lane + e] = w[e];
    }
  }
  __syncthreads();
  if constexpr (!JIT) {
    f4 kc[NT][NV], qc[NT][NV];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int m = 0; m < NV; ++m) {
        kc[t][m] = *reinterpret_cast<const f4 *>(&slot[t][0][m * 4 * L + 4 * sub]);
        qc[t][m] = *reinterpret_cast<const f4 *>(&slot[t][1][m * 4 * L + 4 * sub]);
      }
    // Per-token factors, wave-uniform: alpha, beta and (NK) the key row's
    // 1 / sqrt(sum k^2 + kNormEps), folded into sk and delta.
    float alpha[NT], bs[NT], inv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      alpha[t] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha_l), t));
      const float beta = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, b_l), t));
      inv[t] = 1.f;
      if constexpr (NORMK) {
        float ss = 0.f;
#pragma unroll
        for (int m = 0; m < NV; ++m)
#pragma unroll
          for (int e = 0; e < 4; ++e) ss = __builtin_fmaf(kc[t][m][e], kc[t][m][e], ss);
        inv[t] = __builtin_amdgcn_rsqf(group_sum<L>(ss) + kNormEps);
      }
      bs[t] = beta * inv[t];
    }
    float v[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) v[t] = Io<IO>::widen1(vr[t]);
    // The store addresses and q_scale, from kernel-argument memory: requested
    // here and waited for once.
    void *const out = a.output;
    float *const s_out_p = a.state_out, *const cap_p = a.capture;
    const float qsc = a.q_scale;
    asm volatile("" ::"s"(out), "s"(s_out_p), "s"(cap_p), "s"(qsc));
    // Every request has completed before the first store (the loop waits for
    // no memory, so its stores, inside per-token branches, never delay a
    // load's wait).
    __builtin_amdgcn_s_waitcnt(kWaitVmAll);

    // A row past d_v stores at offset head_bytes, outside its descriptor: the
    // hardware drops it (the immediate offsets added stay below ROW_BYTES).
    const uint32_t sc = ok ? cell : head_bytes;
    const rsrc_t o_rs = buffer(static_cast<char *>(out) + v0, v_ext);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= (int)n_tok) break;
#pragma unroll
      for (int m = 0; m < NV; ++m) st[m] *= alpha[t];
      float part = 0.f;
#pragma unroll
      for (int m = 0; m < NV; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) part = __builtin_fmaf(st[m][e], kc[t][m][e], part);
      const float d = __builtin_fmaf(-inv[t], group_sum<L>(part), v[t]) * bs[t];
#pragma unroll
      for (int m = 0; m < NV; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[m][e] = __builtin_fmaf(d, kc[t][m][e], st[m][e]);
      if constexpr (CAPTURE) {
        const rsrc_t ct = buffer(cap_p + ((tok0 + t) * n_v + vh) * d_v * DK, head_bytes);
#pragma unroll
        for (int m = 0; m < NV; ++m) store4_stream(ct, sc + m * 16 * L, st[m]);
      }
      float py = 0.f;
#pragma unroll
      for (int m = 0; m < NV; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) py = __builtin_fmaf(st[m][e], qc[t][m][e], py);
      const float y = group_sum<L>(py);
      if (sub == 0 && ok) Io<IO>::store1(o_rs, row * IB, uniform(t * v_step), y * qsc);
    }
    const rsrc_t s_out = buffer(s_out_p + head, head_bytes);
#pragma unroll
    for (int m = 0; m < NV; ++m) store4_stream(s_out, sc + m * 16 * L, st[m]);
  } else {
    // The store addresses and q_scale, then every request complete (as above).
    void *const out = a.output;
    float *const s_out_p = a.state_out, *const cap_p = a.capture;
    const float qsc = a.q_scale;
    asm volatile("" ::"s"(out), "s"(s_out_p), "s"(cap_p), "s"(qsc));
    __builtin_amdgcn_s_waitcnt(kWaitVmAll);
    const uint32_t sc = ok ? cell : head_bytes;
    const rsrc_t o_rs = buffer(static_cast<char *>(out) + v0, v_ext);
    f4 kc[NT][NV], qc[NT][NV];  // indexed by compile-time tokens: a few live
    auto cols = [&](int t) {
#pragma unroll
      for (int m = 0; m < NV; ++m) {
        kc[t][m] = *reinterpret_cast<const f4 *>(&slot[t][0][m * 4 * L + 4 * sub]);
        qc[t][m] = *reinterpret_cast<const f4 *>(&slot[t][1][m * 4 * L + 4 * sub]);
      }
    };
    cols(0);
    cols(1);
    float v[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) v[t] = Io<IO>::widen1(vr[t]);
    for_tokens(
        [&](auto tc) {
          constexpr int t = decltype(tc)::value;
          if (t >= (int)n_tok) return;
          if constexpr (t + 2 < NT) cols(t + 2);
          const float alpha =
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha_l), t));
          const float beta =
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, b_l), t));
          float inv = 1.f;
          if constexpr (NORMK) {
            float ss = 0.f;
#pragma unroll
            for (int m = 0; m < NV; ++m)
#pragma unroll
              for (int e = 0; e < 4; ++e) ss = __builtin_fmaf(kc[t][m][e], kc[t][m][e], ss);
            inv = __builtin_amdgcn_rsqf(group_sum<L>(ss) + kNormEps);
          }
#pragma unroll
          for (int m = 0; m < NV; ++m) st[m] *= alpha;
          float part = 0.f;
#pragma unroll
          for (int m = 0; m < NV; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) part = __builtin_fmaf(st[m][e], kc[t][m][e], part);
          const float d = __builtin_fmaf(-inv, group_sum<L>(part), v[t]) * (beta * inv);
#pragma unroll
          for (int m = 0; m < NV; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) st[m][e] = __builtin_fmaf(d, kc[t][m][e], st[m][e]);
          if constexpr (CAPTURE) {
            const rsrc_t ct = buffer(cap_p + ((tok0 + t) * n_v + vh) * d_v * DK, head_bytes);
#pragma unroll
            for (int m = 0; m < NV; ++m) store4_stream(ct, sc + m * 16 * L, st[m]);
          }
          float py = 0.f;
#pragma unroll
          for (int m = 0; m < NV; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) py = __builtin_fmaf(st[m][e], qc[t][m][e], py);
          const float y = group_sum<L>(py);
          if (sub == 0 && ok) Io<IO>::store1(o_rs, row * IB, uniform(t * v_step), y * qsc);
        },
        std::make_integer_sequence<int, NT>{});
    const rsrc_t s_out = buffer(s_out_p + head, head_bytes);
#pragma unroll
    for (int m = 0; m < NV; ++m) store4_stream(s_out, sc + m * 16 * L, st[m]);
  }
}

// ---------------------------------------------------------------- geometry

struct Geometry {
  int rows_per_block;  // WAVES * (64 / L) * R
  int threads;
  const void *kernel;
  bool decode;  // gdn_decode (one token) rather than gdn_recurrent
  const void *wide = nullptr;  // one token, GQA ratio above 65535: gdn_decode_wide
  // Multi-token calls of 2 to 8 tokens: gdn_short (short_rows rows per
  // block) when the sizes fit its size word, else `kernel`.
  const void *shortk = nullptr;
  int short_rows = 0, short_threads = 0;
  bool xcd_order = false;  // gdn_decode's grid order (its XO)
};

template <int DK, int C, int R, int WAVES, int NB, bool CAPTURE, typename IO, int NK>
constexpr Geometry make_geometry() {
  return Geometry{WAVES * (64 / (DK / C)) * R, WAVES * 64,
                  reinterpret_cast<const void *>(
                      &gdn_recurrent<DK, C, R, WAVES, NB, CAPTURE, IO, NK>),
                  false};
}

// A multi-token geometry with gdn_short (at most NT tokens) beside it.
template <int DK, int C, int WAVES, int NT, bool CAPTURE, typename IO, int NK>
constexpr Geometry with_short(Geometry geo) {
  geo.shortk = reinterpret_cast<const void *>(&gdn_short<DK, C, WAVES, NT, CAPTURE, IO, NK>);
  geo.short_rows = WAVES * (64 / (DK / C));
  geo.short_threads = WAVES * 64;
  return geo;
}

template <int DK, int C, int R, int WAVES, bool CAPTURE, typename IO, int NK, bool XO>
constexpr Geometry make_decode_geometry() {
  Geometry geo{
      WAVES * (64 / (DK / C)) * R, WAVES * 64,
      reinterpret_cast<const void *>(&gdn_decode<DK, C, R, WAVES, CAPTURE, IO, NK, XO>), true,
      reinterpret_cast<const void *>(&gdn_decode_wide<DK, C, R, WAVES, CAPTURE, IO, NK>)};
  geo.xcd_order = XO;
  return geo;
}

// Launch geometries, chosen by measurement on MI355X (graph-replayed calls on
// HBM-resident inputs; D_k = 128 workloads of one-token decode, 64-sequence
// batched decode, 4-token capture and 512-token prefill):
//   one token  : gdn_decode. 16 lanes per row, 4 waves, straight-line code;
//                pure streaming of the state, read with non-temporal loads
//                (single decode 3.58 -> 3.23 us, 64-sequence decode 48.3 ->
//                43.0 us). Its own kernel with preloaded leading arguments:
//                single decode 2.93 -> 2.88 us.
//                At D_k = 128 two rows per lane (paired): 3.23 -> 3.13 us;
//                other cell counts and wave counts measured no better, except
//                where that grid has fewer workgroups than the chip has
//                compute units: one sequence of the dense shape (192
//                workgroups) runs 3.14 -> 2.93 us with one row per lane and
//                two waves (768 workgroups; one wave since, below); from two
//                sequences on the two-row grid is faster again (4.05 vs
//                4.29 us).
//   2 to 8 tokens: gdn_short, one row per lane (8 cells at D_k = 128, 4
//                below), 4 waves, every input requested before the token
//                loop and the k/q rows staged once per workgroup (general
//                kernel -> gdn_short: 4-token verify with capture 5.21 ->
//                5.15 us, without capture 4.77 -> 3.57 us; 2 tokens with
//                capture 4.08 -> 3.71 us; 8 tokens without capture 5.38 ->
//                4.56 us; one dense-shape sequence of 4 tokens 4.19 -> 3.19
//                us; the 64-sequence batch of 4 tokens with capture 150.5 ->
//                137.9 us; the 8-token D_k = 32 case 3.97 -> 2.58 us; a
//                4-token D_k = 64 verify 3.43 -> 2.64 us). Staging the rows
//                per wave instead of per workgroup put four times the row
//                requests ahead of the state's in each compute unit's
//                queue (4-token verify 5.29 us, 8 tokens 9.12 us). 9 to 16
//                tokens: the unrolled 16-token instance on grids of at most
//                16,384 rows (see kShort16MaxRows); a rolled token loop
//                reading each token's columns during the previous one had
//                lost to the general kernel (16 tokens 8.38 against 6.88 us).
//   longer     : two rows per lane (each k/q register feeds two rows, which
//                halves k/q operand traffic per cell: 418 -> 289 us at 512
//                tokens against one row per lane), 16 lanes per row, 4 waves
//                (at D_k = 128 eight while the grid fits the chip in one
//                round, and one row per lane on grids below one workgroup per
//                compute unit; see pick()).
//                Without capture an eight-token prefetch ring and lazy group
//                (512-token prefill 221 -> 206 us against four tokens without
//                the lazy form). With capture, which runs eagerly and is bound
//                by its writes, one row per lane (twice the waves) and a
//                four-token ring: 4-token verify 5.88 -> 5.64 us. Among this
//                kernel's geometries the two-row one was best or within 2% of
//                the best measured variant from 2 tokens up (2 to 512). At
//                D_k = 64, 16 lanes per row (4 cells each), two waves and an
//                eight-token ring (twice the waves of 8 lanes per row with
//                8 cells): 512-token prefill 139 -> 96 us, 16 tokens 8.1 ->
//                7.1 us, a 4-token verify with capture 4.6 -> 3.8 us; four
//                waves without capture (512 tokens of 16 sequences 213 ->
//                199 us, of 64 sequences 800 -> 720 us, D_v = 128 115 ->
//                103 us, key-normalised 91 -> 87 us, 1 to 4 sequences 1-3%
//                faster; capture calls ~3% slower, so they keep two). At
//                D_k = 32, 8 lanes per row and two waves (32 rows, so a D_v
//                = 32 head has no padding waves; four waves had two of them):
//                512 tokens of 16 sequences 118 -> 108 us, of 64 sequences
//                399 -> 250 us, of 1 to 4 sequences 1-2% faster.
// Compute units of an MI355X.
constexpr uint64_t kComputeUnits = 256;

// Calls of 9 to 16 tokens take gdn_short only up to this many rows (n_v_heads
// * n_seqs * d_v), and at D_k = 128 only without capture: past it the general
// kernel's two-row layout does more work per request (the 64-sequence batch
// of 16 tokens: 97.0 against 79.1 us; a 12-token D_k = 64 batch 25.7 against
// 23.1 us); below it gdn_short (4-token-verify shape at 9, 12 and 16 tokens:
// 5.70 -> 4.96, 6.44 -> 5.50, 6.90 -> 6.26 us; D_k = 64 at 12 tokens 4.97 ->
// 4.03 us, with capture 5.44 -> 4.42 us). D_k = 128 capture calls of 12 or
// 16 tokens measured 2-5% slower on it.
constexpr uint64_t kShort16MaxRows = 16384;

// heads: n_v_heads * n_seqs.
template <bool CAPTURE, typename IO, int NK>
Geometry pick(uint32_t d_k, uint32_t d_v, uint64_t heads, uint32_t n_tokens) {
  const bool short16 = n_tokens <= 16 && heads * d_v <= kShort16MaxRows;
  const bool one_token = n_tokens == 1;
  constexpr int NK1 = NK == 2 ? 1 : NK;  // one-token calls have no ring group
  switch (d_k) {
    case 32: {
      if (one_token) return make_decode_geometry<32, 4, 1, 4, CAPTURE, IO, NK1, true>();
      const Geometry geo = make_geometry<32, 4, 2, 2, 4, CAPTURE, IO, NK>();
      if (n_tokens <= 4) return with_short<32, 4, 4, 4, CAPTURE, IO, NK1>(geo);
      if (n_tokens <= 8) return with_short<32, 4, 4, 8, CAPTURE, IO, NK1>(geo);
      if (short16) return with_short<32, 4, 4, 16, CAPTURE, IO, NK1>(geo);
      return geo;
    }
    case 64: {
      if (one_token) {
        // Two rows per lane once that grid fills the chip (64-sequence
        // batch of the MoE shape at D_k = 64: 12.9 -> 12.4 us); one row per
        // lane below (one dense-shape sequence: 2.19 vs 2.25 us).
        if (heads * ((d_v + 31) / 32) < kComputeUnits)
          return make_decode_geometry<64, 4, 1, 4, CAPTURE, IO, NK1, true>();
        return make_decode_geometry<64, 4, 2, 4, CAPTURE, IO, NK1, false>();
      }
      // Four waves without capture (each staging wave loads two tokens of a
      // ring group instead of four); two with capture.
      Geometry geo;
      if constexpr (CAPTURE)
        geo = make_geometry<64, 4, 2, 2, 8, CAPTURE, IO, NK>();
      else
        geo = make_geometry<64, 4, 2, 4, 8, CAPTURE, IO, NK>();
      if (n_tokens <= 4) return with_short<64, 4, 4, 4, CAPTURE, IO, NK1>(geo);
      if (n_tokens <= 8) return with_short<64, 4, 4, 8, CAPTURE, IO, NK1>(geo);
      if (short16) return with_short<64, 4, 4, 16, CAPTURE, IO, NK1>(geo);
      return geo;
    }
    case 128: {
      if (one_token) {
        // A grid of two-row workgroups that leaves compute units idle (one
        // dense-shape layer of one sequence: 192 workgroups) is spread over
        // eight times as many workgroups of one row per lane and one wave
        // (1,536 workgroups; two waves: 2.52 against 2.50 us, four: 2.63).
        if (heads * ((d_v + 31) / 32) < kComputeUnits)
          return make_decode_geometry<128, 8, 1, 1, CAPTURE, IO, NK1, true>();
        return make_decode_geometry<128, 8, 2, 4, CAPTURE, IO, NK1, false>();
      }
      Geometry geo;
      if constexpr (CAPTURE) {
        geo = make_geometry<128, 8, 1, 4, 4, CAPTURE, IO, NK>();
      } else {
        // Below one two-row workgroup per compute unit the waves run their
        // token loops nearly alone: one row per lane (half the work per wave
        // and token). One dense-shape sequence of 512 tokens: 125.4 -> 116.9
        // us; of 64 tokens: 19.4 -> 18.9 us. Four waves per workgroup rather
        // than two (each staging wave loads two tokens of a ring group
        // instead of four): 512 tokens 105.4 -> 102.6 us, 2048 tokens 407 ->
        // 397 us, key-normalised 112.2 -> 108.6 us, the MoE head count 103.5
        // -> 97.4 us.
        // Two rows per lane from one two-row workgroup per compute unit on:
        // eight waves per workgroup while that grid (64 rows each) fits the
        // chip in one round (each staging wave loads one token of a ring
        // group; 512 tokens of two dense-shape sequences 111.5 -> 106.5 us,
        // of three and four MoE-shape sequences 111.5 -> 106.0 and 113.6 ->
        // 108.8 us), four past it (one 512-thread workgroup fits a compute
        // unit: three dense-shape sequences took 209 against 132 us).
        if (heads * ((d_v + 31) / 32) < kComputeUnits)
          geo = make_geometry<128, 8, 1, 4, 8, CAPTURE, IO, NK>();
        else if (heads * ((d_v + 63) / 64) <= kComputeUnits)
          geo = make_geometry<128, 8, 2, 8, 8, CAPTURE, IO, NK>();
        else
          geo = make_geometry<128, 8, 2, 4, 8, CAPTURE, IO, NK>();
      }
      if (n_tokens <= 4) return with_short<128, 8, 4, 4, CAPTURE, IO, NK1>(geo);
      if (n_tokens <= 8) return with_short<128, 8, 4, 8, CAPTURE, IO, NK1>(geo);
      if constexpr (!CAPTURE) {
        if (short16) return with_short<128, 8, 4, 16, CAPTURE, IO, NK1>(geo);
      }
      return geo;
    }
    default:
      return Geometry{0, 0, nullptr, false};
  }
}

template <int NK>
Geometry pick_io(uint32_t d_k, uint32_t d_v, uint64_t heads, uint32_t n_tokens, bool capture,
                 bool bf16) {
  if (bf16)
    return capture ? pick<true, __bf16, NK>(d_k, d_v, heads, n_tokens)
                   : pick<false, __bf16, NK>(d_k, d_v, heads, n_tokens);
  return capture ? pick<true, float, NK>(d_k, d_v, heads, n_tokens)
                 : pick<false, float, NK>(d_k, d_v, heads, n_tokens);
}

// Key normalisation takes the group-ahead factors from this many tokens on:
// they save ~25 ns per token on the 512-token prefill but put one key-row
// round trip before the first token (~0.3 us on a 4-token verify).
constexpr uint32_t kGroupNormMinTokens = 16;

Geometry pick_geometry(uint32_t d_k, uint32_t d_v, uint64_t heads, uint32_t n_tokens,
                       bool capture, bool bf16, bool normalize_k) {
  if (!normalize_k) return pick_io<0>(d_k, d_v, heads, n_tokens, capture, bf16);
  return n_tokens >= kGroupNormMinTokens
             ? pick_io<2>(d_k, d_v, heads, n_tokens, capture, bf16)
             : pick_io<1>(d_k, d_v, heads, n_tokens, capture, bf16);
}

// Smallest s with 2^s >= x (x >= 1).
uint32_t ceil_log2(uint64_t x) {
  uint32_t s = 0;
  while ((uint64_t(1) << s) < x) ++s;
  return s;
}

}  // namespace

namespace {

// Whether a multi-token call takes gdn_short (its sizes fit the size word).
bool short_fits(const Geometry &geo, uint32_t d_v, uint32_t n_k_heads, uint32_t n_v_heads) {
  if (geo.shortk == nullptr) return false;
  const uint32_t groups = n_v_heads / n_k_heads;
  const uint32_t row_blocks = (d_v + geo.short_rows - 1) / geo.short_rows;
  return d_v >> kPackDv == 0 && row_blocks <= 128 && n_k_heads >> kShortNk == 0 &&
         groups >> kShortGroups == 0;
}

}  // namespace

uint64_t grid_blocks(uint32_t d_k, uint32_t d_v, uint32_t n_k_heads, uint32_t n_v_heads,
                     uint32_t n_seqs, uint32_t n_tokens, bool capture) {
  const Geometry geo =
      pick_geometry(d_k, d_v, (uint64_t)n_v_heads * n_seqs, n_tokens, capture, false, false);
  if (geo.kernel == nullptr) return 0;
  // One-token and short grids pad each head's row blocks to a power of two.
  if (short_fits(geo, d_v, n_k_heads, n_v_heads)) {
    // Short grids pad the key heads to a power of two (at least 8).
    const uint64_t row_blocks = (d_v + geo.short_rows - 1) / geo.short_rows;
    return (row_blocks << xcd_kh_bits(n_k_heads)) * (n_v_heads / n_k_heads) * n_seqs;
  }
  const uint64_t row_blocks = (d_v + geo.rows_per_block - 1) / geo.rows_per_block;
  if (geo.decode) {
    const uint32_t groups = n_v_heads / n_k_heads;
    const bool wide = d_v >> kPackDv != 0 || n_k_heads >> kPackNk != 0 ||
                      groups >> kPackGroups != 0;
    // One-token grids pad the key heads to a power of two (at least 8), or
    // (past the size word) each head's row blocks.
    if (!wide && geo.xcd_order) return (row_blocks << xcd_kh_bits(n_k_heads)) * groups * n_seqs;
    return (uint64_t(1) << ceil_log2(row_blocks)) * n_v_heads * n_seqs;
  }
  return row_blocks * n_v_heads * n_seqs;
}

hipError_t enqueue_forward(const ForwardArgs &f, hipStream_t stream) {
  const bool capture = f.capture != nullptr;
  const Geometry geo = pick_geometry(f.d_k, f.d_v, (uint64_t)f.n_v_heads * f.n_seqs, f.n_tokens,
                                     capture, f.bf16, f.normalize_k);
  if (geo.kernel == nullptr) return hipErrorInvalidValue;
  const uint32_t row_blocks =
      (f.d_v + geo.rows_per_block - 1) / geo.rows_per_block;
  const uint64_t blocks = (uint64_t)row_blocks * f.n_v_heads * f.n_seqs;

  const uint64_t io = f.bf16 ? 2 : 4;
  if (geo.decode) {
    // One token: grid x = (row block << kh_bits) | key head (XCD order) or
    // (key head << rb_shift) | row block; y = value head of the key head; z
    // = sequence, one launch per 65535 sequences with
    // every base moved to the launch's first sequence (sequences are
    // independent and T = 1). Sizes past the size word take
    // gdn_decode_wide: x = (value head << rb_shift) | row block, y =
    // sequence.
    constexpr uint32_t kMaxGrid = 65535;
    const uint32_t rb_shift = ceil_log2(row_blocks);
    const uint32_t groups = f.n_v_heads / f.n_k_heads;
    const bool wide = f.d_v >> kPackDv != 0 || rb_shift >> kPackRb != 0 ||
                      f.n_k_heads >> kPackNk != 0 || groups >> kPackGroups != 0;
    const uint32_t kh_shift = 23 + ceil_log2(f.n_k_heads);
    const uint32_t kh_magic =
        (uint32_t)(((uint64_t(1) << kh_shift) + f.n_k_heads - 1) / f.n_k_heads);
    const uint64_t state_seq = (uint64_t)f.n_v_heads * f.d_v * f.d_k;  // floats
    const uint64_t kq_seq = (uint64_t)f.n_k_heads * f.d_k * io;       // bytes
    const uint64_t v_seq = (uint64_t)f.n_v_heads * f.d_v * io;        // bytes
    for (uint32_t s0 = 0; s0 < f.n_seqs; s0 += kMaxGrid) {
      const uint32_t ns = f.n_seqs - s0 < kMaxGrid ? f.n_seqs - s0 : kMaxGrid;
      const float *state_in = f.state_in + s0 * state_seq;
      const void *k = static_cast<const char *>(f.k) + s0 * kq_seq;
      const float *g = f.g + (uint64_t)s0 * f.n_v_heads;
      const void *v = static_cast<const char *>(f.v) + s0 * v_seq;
      const float *beta = f.beta + (uint64_t)s0 * f.n_v_heads;
      const void *q = static_cast<const char *>(f.q) + s0 * kq_seq;
      DecodeTail t;
      t.output = static_cast<char *>(f.output) + s0 * v_seq;
      t.state_out = f.state_out + s0 * state_seq;
      t.capture = f.capture != nullptr ? f.capture + s0 * state_seq : nullptr;
      t.q_scale = f.q_scale;
      hipError_t e;
      if (!wide) {
        const uint32_t bits = geo.xcd_order ? xcd_kh_bits(f.n_k_heads) : rb_shift;
        const uint32_t gx = geo.xcd_order ? row_blocks << bits : f.n_k_heads << bits;
        uint32_t sizes = f.d_v | bits << kPackDv | f.n_k_heads << (kPackDv + kPackRb) |
                         groups << (kPackDv + kPackRb + kPackNk);
        void *args[] = {&state_in, &k, &q, &g, &v, &beta, &sizes, &t};
        e = hipLaunchKernel(geo.kernel, dim3(gx, groups, ns),
                            dim3(geo.threads), args, 0, stream);
      } else {
        uint32_t d_v = f.d_v, n_v = f.n_v_heads, n_k = f.n_k_heads, magic = kh_magic;
        uint32_t shifts = kh_shift | rb_shift << 8;
        void *args[] = {&state_in, &k, &q, &g, &v, &beta, &d_v, &n_v, &n_k, &magic, &shifts, &t};
        e = hipLaunchKernel(geo.wide, dim3(f.n_v_heads << rb_shift, ns), dim3(geo.threads), args,
                            0, stream);
      }
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }

  if (short_fits(geo, f.d_v, f.n_k_heads, f.n_v_heads)) {
    // At most 8 tokens: the one-token argument layout (see above), the
    // sizes word carrying kh_bits and n_tokens - 1; grid x = (row block <<
    // kh_bits) | key head; one launch per 65535 sequences.
    constexpr uint32_t kMaxGrid = 65535;
    const uint32_t row_blocks = (f.d_v + geo.short_rows - 1) / geo.short_rows;
    const uint32_t kh_bits = xcd_kh_bits(f.n_k_heads);
    const uint32_t groups = f.n_v_heads / f.n_k_heads;
    uint32_t sizes = f.d_v | kh_bits << kPackDv | f.n_k_heads << (kPackDv + kShortKb) |
                     groups << (kPackDv + kShortKb + kShortNk) |
                     (f.n_tokens - 1) << (kPackDv + kShortKb + kShortNk + kShortGroups);
    const uint64_t state_seq = (uint64_t)f.n_v_heads * f.d_v * f.d_k;                // floats
    const uint64_t kq_seq = (uint64_t)f.n_tokens * f.n_k_heads * f.d_k * io;         // bytes
    const uint64_t v_seq = (uint64_t)f.n_tokens * f.n_v_heads * f.d_v * io;          // bytes
    const uint64_t gb_seq = (uint64_t)f.n_tokens * f.n_v_heads;                      // floats
    for (uint32_t s0 = 0; s0 < f.n_seqs; s0 += kMaxGrid) {
      const uint32_t ns = f.n_seqs - s0 < kMaxGrid ? f.n_seqs - s0 : kMaxGrid;
      const float *state_in = f.state_in + s0 * state_seq;
      const void *k = static_cast<const char *>(f.k) + s0 * kq_seq;
      const float *g = f.g + s0 * gb_seq;
      const void *v = static_cast<const char *>(f.v) + s0 * v_seq;
      const float *beta = f.beta + s0 * gb_seq;
      const void *q = static_cast<const char *>(f.q) + s0 * kq_seq;
      DecodeTail t;
      t.output = static_cast<char *>(f.output) + s0 * v_seq;
      t.state_out = f.state_out + s0 * state_seq;
      t.capture = f.capture != nullptr ? f.capture + s0 * f.n_tokens * state_seq : nullptr;
      t.q_scale = f.q_scale;
      void *args[] = {&state_in, &k, &q, &g, &v, &beta, &sizes, &t};
      const hipError_t e = hipLaunchKernel(geo.shortk, dim3(row_blocks << kh_bits, groups, ns),
                                           dim3(geo.short_threads), args, 0, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }

  KernelArgs a;
  a.q = f.q;
  a.k = f.k;
  a.v = f.v;
  a.g = f.g;
  a.beta = f.beta;
  a.output = f.output;
  a.state_out = f.state_out;
  a.capture = f.capture;
  a.q_scale = f.q_scale;
  const uint64_t kq_row = (uint64_t)f.n_k_heads * f.d_k, v_row = (uint64_t)f.n_v_heads * f.d_v;
  const uint64_t last = f.n_tokens - 1u;
  const uint64_t kq_bytes = (last * kq_row + f.d_k) * io, v_bytes = (last * v_row + f.d_v) * io;
  a.kq_ext0 = kq_bytes < 0xFFFFFFFFull ? (uint32_t)kq_bytes : 0xFFFFFFFFu;
  a.v_ext0 = v_bytes < 0xFFFFFFFFull ? (uint32_t)v_bytes : 0xFFFFFFFFu;
  // Reciprocals for the workgroup index split (every quotient's numerator is
  // below the grid size, < 2^24): shift = 24 + ceil(log2 d), magic =
  // ceil(2^shift / d) <= 2^25, exact because x * (magic * d - 2^shift) <
  // 2^24 * d <= 2^shift.
  if (blocks >= (uint64_t(1) << 24)) return hipErrorInvalidValue;
  auto recip = [](uint32_t d, uint32_t &magic) {
    const uint32_t shift = 24 + ceil_log2(d);
    magic = (uint32_t)(((uint64_t(1) << shift) + d - 1) / d);
    return shift;
  };
  const float *state_in = f.state_in;
  uint32_t d_v = f.d_v, n_k = f.n_k_heads, n_v = f.n_v_heads, n_tok = f.n_tokens;
  uint32_t rbs = row_blocks, groups = f.n_v_heads / f.n_k_heads;
  uint32_t rb_magic, g_magic, kh_magic;
  uint32_t shifts = recip(row_blocks, rb_magic) | recip(groups, g_magic) << 8 |
                    recip(f.n_k_heads, kh_magic) << 16;
  uint32_t n_blocks = (uint32_t)blocks;
  void *args[] = {&state_in, &d_v,     &n_k,      &n_v,    &n_tok,    &rbs,      &groups,
                  &rb_magic, &g_magic, &kh_magic, &shifts, &n_blocks, &a};
  return hipLaunchKernel(geo.kernel, dim3(n_blocks), dim3(geo.threads), args, 0, stream);
}

}  // namespace gdn
