// Device-side building blocks shared by the route, decode and grouped kernels.
//
// Kernel layout of a quantised matrix W[O, K] (written by the host packer):
//   * O is cut into tiles of 64 output rows ("lanes"); a wave of 64 lanes
//     owns one tile, lane l owning one output row.
//   * codes: per tile, chunk-major: chunk c holds codes k in [32c, 32c+32)
//     of every row of the tile, rows (lanes) contiguous. A chunk is CB bytes
//     per lane (4-bit: 16, 3-bit: 12, 8-bit: 32 stored as two 16-byte
//     sub-blocks), so one wave-wide load of a chunk is a contiguous block.
//   * inside a lane's chunk, the 32 codes form 16 pairs (k = 2p, 2p+1); the
//     two codes of a pair sit at the same bit offset of the low and high
//     16-bit halves of a word, so one shift and one and-or turn a pair into
//     two exact fp16 values 1 + q/M (M = 16 for 3- and 4-bit codes, 256 for
//     8-bit) that v_dot2_f32_f16 takes directly:
//       4-bit: word w holds pairs 4w..4w+3 at bits 4j (and 16+4j);
//       8-bit: word w holds pairs 2w, 2w+1 at bits 8j (and 16+8j);
//       3-bit: word w (0..2) holds pairs 5w..5w+4 at bits 3j (and 16+3j);
//              pair 15 keeps bit b of its codes in bit 15 / bit 31 of word b.
//   * scales: per tile, per 256-k block, per lane: 256/G entries of
//     u32 (bf16 scale | bf16 bias << 16) for affine, u16 fp16 scale for
//     symmetric.
// With the pair value v = 1 + q/M and the group sum X = sum x, the group's
// contribution is s*sum(q x) + b*X = (M s) * sum(v x) + (b - M s) * X, which
// keeps every product exact and needs no per-weight scale multiply.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef _Float16 f16;
typedef f16 half2v __attribute__((ext_vector_type(2)));
typedef f16 half4v __attribute__((ext_vector_type(4)));
typedef f16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));

// kernel-side format ids
enum { F_Q4 = 0, F_Q3 = 1, F_Q8 = 2, F_S4 = 3, F_DENSE = 4 };

template <int F> struct Fmt;
template <> struct Fmt<F_Q4> {
  static constexpr int BITS = 4, G = 64, M = 16, CB = 16, WORDS = 4, SCB = 4;
  static constexpr bool AFF = true;
};
template <> struct Fmt<F_Q3> {
  // 3-bit codes use the 4-bit pair value 1 + q/16, so a 3-bit layer and the
  // same codes widened to 4-bit words run identical arithmetic
  static constexpr int BITS = 3, G = 64, M = 16, CB = 12, WORDS = 3, SCB = 4;
  static constexpr bool AFF = true;
};
template <> struct Fmt<F_Q8> {
  static constexpr int BITS = 8, G = 64, M = 256, CB = 32, WORDS = 8, SCB = 4;
  static constexpr bool AFF = true;
};
template <> struct Fmt<F_S4> {
  static constexpr int BITS = 4, G = 128, M = 16, CB = 16, WORDS = 4, SCB = 2;
  static constexpr bool AFF = false;
};

constexpr int KBLK = 256;   // k per scale block (and per decode wave slice)

// ---------------------------------------------------------------- bit casts
__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t as_u(half2v h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ float bf16_to_f(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f(uint32_t b) {
  return (float)__builtin_bit_cast(f16, (uint16_t)b);
}
__device__ __forceinline__ float act_to_f(uint16_t b, int act_fp16) {
  return act_fp16 ? f16_bits_to_f(b) : bf16_to_f(b);
}

// ------------------------------------------------------------------ unpack
// 16 packed fp16 pairs (1 + q/M) of one lane's chunk.
template <int F> __device__ __forceinline__ void unpack_chunk(const uint32_t* w, uint32_t* o);

template <> __device__ __forceinline__ void unpack_chunk<F_Q4>(const uint32_t* w, uint32_t* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v = w[i];
    o[4 * i + 0] = ((v << 6) & 0x03C003C0u) | 0x3C003C00u;
    o[4 * i + 1] = ((v << 2) & 0x03C003C0u) | 0x3C003C00u;
    o[4 * i + 2] = ((v >> 2) & 0x03C003C0u) | 0x3C003C00u;
    o[4 * i + 3] = ((v >> 6) & 0x03C003C0u) | 0x3C003C00u;
  }
}
template <> __device__ __forceinline__ void unpack_chunk<F_S4>(const uint32_t* w, uint32_t* o) {
  unpack_chunk<F_Q4>(w, o);
}
template <> __device__ __forceinline__ void unpack_chunk<F_Q8>(const uint32_t* w, uint32_t* o) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t v = w[i];
    o[2 * i + 0] = ((v << 2) & 0x03FC03FCu) | 0x3C003C00u;
    o[2 * i + 1] = ((v >> 6) & 0x03FC03FCu) | 0x3C003C00u;
  }
}
template <> __device__ __forceinline__ void unpack_chunk<F_Q3>(const uint32_t* w, uint32_t* o) {
  // code bits land in mantissa bits 6..8 (bit 9 stays 0): value 1 + q/16
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const uint32_t v = w[i];
    o[5 * i + 0] = ((v << 6) & 0x01C001C0u) | 0x3C003C00u;
    o[5 * i + 1] = ((v << 3) & 0x01C001C0u) | 0x3C003C00u;
    o[5 * i + 2] = (v & 0x01C001C0u) | 0x3C003C00u;
    o[5 * i + 3] = ((v >> 3) & 0x01C001C0u) | 0x3C003C00u;
    o[5 * i + 4] = ((v >> 6) & 0x01C001C0u) | 0x3C003C00u;
  }
  o[15] = ((w[0] >> 9) & 0x00400040u) | ((w[1] >> 8) & 0x00800080u) |
          ((w[2] >> 7) & 0x01000100u) | 0x3C003C00u;
}

// load one lane's chunk words (CB bytes) from a chunk block base
template <int F> __device__ __forceinline__ void load_chunk(const uint8_t* blk, int lane, uint32_t* w);
template <> __device__ __forceinline__ void load_chunk<F_Q4>(const uint8_t* blk, int lane, uint32_t* w) {
  const uint4 v = *reinterpret_cast<const uint4*>(blk + lane * 16);
  w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
}
template <> __device__ __forceinline__ void load_chunk<F_S4>(const uint8_t* blk, int lane, uint32_t* w) {
  load_chunk<F_Q4>(blk, lane, w);
}
template <> __device__ __forceinline__ void load_chunk<F_Q3>(const uint8_t* blk, int lane, uint32_t* w) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(blk + lane * 12);
  w[0] = p[0]; w[1] = p[1]; w[2] = p[2];
}
template <> __device__ __forceinline__ void load_chunk<F_Q8>(const uint8_t* blk, int lane, uint32_t* w) {
  const uint4 a = *reinterpret_cast<const uint4*>(blk + lane * 16);
  const uint4 b = *reinterpret_cast<const uint4*>(blk + 64 * 16 + lane * 16);
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// Byte offset of chunk c of tile t (K/32 chunks per row).
template <int F> __device__ __forceinline__ uint64_t chunk_off(int t, int c, int nchunks) {
  return ((uint64_t)t * nchunks + c) * (uint64_t)(64 * Fmt<F>::CB);
}
// Byte offset of the scale block kb of tile t (K/256 blocks per row).
template <int F> __device__ __forceinline__ uint64_t sblk_off(int t, int kb, int nkb) {
  return ((uint64_t)t * nkb + kb) * (uint64_t)(64 * (KBLK / Fmt<F>::G) * Fmt<F>::SCB);
}

// Multiplier M*s and offset (b - M s) of one group for one lane.
template <int F> __device__ __forceinline__ void group_coef(const uint8_t* sblk, int lane, int gi,
                                                            float& ms, float& bm) {
  if constexpr (Fmt<F>::AFF) {
    const uint32_t v = reinterpret_cast<const uint32_t*>(sblk)[lane * (KBLK / Fmt<F>::G) + gi];
    const float s = bf16_to_f(v & 0xFFFFu), b = bf16_to_f(v >> 16);
    ms = (float)Fmt<F>::M * s;
    bm = b - ms;
  } else {
    const uint16_t v = reinterpret_cast<const uint16_t*>(sblk)[lane * (KBLK / Fmt<F>::G) + gi];
    const float s = f16_bits_to_f(v);
    ms = (float)Fmt<F>::M * s;
    bm = -8.0f * s - ms;       // symmetric: w = s*(u - 8)
  }
}

// sum over the 16 pairs of a chunk: acc += v_p . a_p (fixed order p = 0..15)
__device__ __forceinline__ float dot_chunk(const uint32_t* v, const half2v* a, float acc) {
#pragma unroll
  for (int p = 0; p < 16; ++p) acc = __builtin_amdgcn_fdot2(as_h2(v[p]), a[p], acc, false);
  return acc;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  // silu(g) * u with silu(z) = z / (1 + exp(-z))
  return (g / (1.0f + expf(-g))) * u;
}

// comparator of the pick: NaN first, then larger value, then lower id
__device__ __forceinline__ bool pick_better(float a, int ia, float b, int ib) {
  const bool an = a != a, bn = b != b;
  if (an != bn) return an;
  if (!an && a != b) return a > b;
  return ia < ib;
}

}  // namespace moe
