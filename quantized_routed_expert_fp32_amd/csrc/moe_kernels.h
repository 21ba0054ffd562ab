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
//       2-bit: word w (0..1) holds pairs 8w..8w+7 at bits 2j (and 16+2j);
//       5-bit: word w (0..4) holds pairs 3w..3w+2 at bits 5j (and 16+5j);
//              pair 15 keeps bit b of its codes in bit 15 / bit 31 of word b;
//       6-bit: word w (0..5) holds pairs 2w, 2w+1 at bits 6j (and 16+6j);
//              pair 12+m keeps its low 4 bits in bits 12..15 (28..31) of
//              word m, its high 2 bits in bits 12+2(m%2) (28+2(m%2)) of
//              word 4+m/2;
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
enum { F_Q4 = 0, F_Q3 = 1, F_Q8 = 2, F_S4 = 3, F_DENSE = 4, F_Q2 = 5, F_Q5 = 6, F_Q6 = 7, F_MX4 = 8 };

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
template <> struct Fmt<F_Q2> {
  // 2-bit codes also use the pair value 1 + q/16 (read by the decode kernels)
  static constexpr int BITS = 2, G = 64, M = 16, CB = 8, WORDS = 2, SCB = 4;
  static constexpr bool AFF = true;
};
template <> struct Fmt<F_Q5> {
  // pair value 1 + q/32 (read by the decode kernels)
  static constexpr int BITS = 5, G = 64, M = 32, CB = 20, WORDS = 5, SCB = 4;
  static constexpr bool AFF = true;
};
template <> struct Fmt<F_Q6> {
  // pair value 1 + q/64 (read by the decode kernels)
  static constexpr int BITS = 6, G = 64, M = 64, CB = 24, WORDS = 6, SCB = 4;
  static constexpr bool AFF = true;
};
template <> struct Fmt<F_S4> {
  static constexpr int BITS = 4, G = 128, M = 16, CB = 16, WORDS = 4, SCB = 2;
  static constexpr bool AFF = false;
};
template <> struct Fmt<F_MX4> {
  // MXFP4: E2M1 elements whose pairs are the bytes of the canonical words,
  // one E8M0 exponent byte per group of 32 (M is unused: the pair values are
  // the elements themselves, the block scale multiplies the group's dot)
  static constexpr int BITS = 4, G = 32, M = 1, CB = 16, WORDS = 4, SCB = 1;
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

// comparator of the pick: NaN first, then larger value, then lower id.
// Branch-free (bitwise on the predicates) so it compiles to selects.
__device__ __forceinline__ bool pick_better(float a, int ia, float b, int ib) {
  const bool an = a != a, bn = b != b;
  const bool tie = (a == b) | (an & bn);
  return (an & !bn) | ((!an & !bn) & (a > b)) | (tie & (ia < ib));
}

// (x & m) | c in one v_and_or_b32. gfx9 VOP3 takes no literal constant, so
// the mask goes in an SGPR and the constant in a VGPR (hoisted once).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}

// ------------------------------------------------------------------ unpack
// 16 packed fp16 pairs (1 + q/M) of one lane's chunk.
template <int F> __device__ __forceinline__ void unpack_chunk(const uint32_t* w, uint32_t* o);

template <> __device__ __forceinline__ void unpack_chunk<F_Q4>(const uint32_t* w, uint32_t* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v = w[i];
    o[4 * i + 0] = and_or(v << 6, 0x03C003C0u, 0x3C003C00u);
    o[4 * i + 1] = and_or(v << 2, 0x03C003C0u, 0x3C003C00u);
    o[4 * i + 2] = and_or(v >> 2, 0x03C003C0u, 0x3C003C00u);
    o[4 * i + 3] = and_or(v >> 6, 0x03C003C0u, 0x3C003C00u);
  }
}
template <> __device__ __forceinline__ void unpack_chunk<F_S4>(const uint32_t* w, uint32_t* o) {
  unpack_chunk<F_Q4>(w, o);
}
template <> __device__ __forceinline__ void unpack_chunk<F_Q8>(const uint32_t* w, uint32_t* o) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t v = w[i];
    o[2 * i + 0] = and_or(v << 2, 0x03FC03FCu, 0x3C003C00u);
    o[2 * i + 1] = and_or(v >> 6, 0x03FC03FCu, 0x3C003C00u);
  }
}
template <> __device__ __forceinline__ void unpack_chunk<F_Q3>(const uint32_t* w, uint32_t* o) {
  // code bits land in mantissa bits 6..8 (bit 9 stays 0): value 1 + q/16
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const uint32_t v = w[i];
    o[5 * i + 0] = and_or(v << 6, 0x01C001C0u, 0x3C003C00u);
    o[5 * i + 1] = and_or(v << 3, 0x01C001C0u, 0x3C003C00u);
    o[5 * i + 2] = and_or(v, 0x01C001C0u, 0x3C003C00u);
    o[5 * i + 3] = and_or(v >> 3, 0x01C001C0u, 0x3C003C00u);
    o[5 * i + 4] = and_or(v >> 6, 0x01C001C0u, 0x3C003C00u);
  }
  o[15] = and_or(w[2] >> 7, 0x01000100u,
                 and_or(w[1] >> 8, 0x00800080u, and_or(w[0] >> 9, 0x00400040u, 0x3C003C00u)));
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

// Buffer resource of one byte range (an expert block, a router): loads
// through it take a per-lane offset in a VGPR and a uniform offset in an
// SGPR, and return 0 instead of touching memory past `bytes`.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // GFX9 raw buffer: stride 0, num_records in bytes, 32-bit data format word
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One lane's chunk words: voff = lane * CB (per lane), soff = byte offset of
// the chunk block inside the range (uniform).
template <int F> __device__ __forceinline__ void load_chunk_rs(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* w) {
  if constexpr (F == F_Q3) {
    const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(r, (int)voff, (int)soff, 0);
    w[0] = v.x; w[1] = v.y; w[2] = v.z;
  } else if constexpr (F == F_Q2) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (F == F_Q5) {
    const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(voff + 16), (int)soff, 0);
  } else if constexpr (F == F_Q6) {
    const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    const u32x2_t b = __builtin_amdgcn_raw_buffer_load_b64(r, (int)(voff + 16), (int)soff, 0);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y;
  } else if constexpr (F == F_Q8) {
    const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(voff / 2), (int)soff, 0);
    const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(voff / 2), (int)(soff + 64 * 16), 0);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
}
// One lane's scale words of a 256-wide block (see load_scales): voff = lane *
// (256/G) * SCB, soff = byte offset of the scale block inside the range.
template <int F> __device__ __forceinline__ void load_scales_rs(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* sc) {
  if constexpr (Fmt<F>::AFF) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    sc[0] = v.x; sc[1] = v.y; sc[2] = v.z; sc[3] = v.w;
  } else if constexpr (F == F_MX4) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
    sc[0] = v.x; sc[1] = v.y;
  } else {
    sc[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
  }
}
template <int F> __device__ __forceinline__ uint32_t chunk_voff(int lane) { return (uint32_t)lane * Fmt<F>::CB; }
template <int F> __device__ __forceinline__ uint32_t scale_voff(int lane) {
  return (uint32_t)lane * (KBLK / Fmt<F>::G) * Fmt<F>::SCB;
}

// Byte offset of chunk c of tile t (K/32 chunks per row).
template <int F> __device__ __forceinline__ uint64_t chunk_off(int t, int c, int nchunks) {
  return ((uint64_t)t * nchunks + c) * (uint64_t)(64 * Fmt<F>::CB);
}
// Byte offset of the scale block kb of tile t (K/256 blocks per row).
template <int F> __device__ __forceinline__ uint64_t sblk_off(int t, int kb, int nkb) {
  return ((uint64_t)t * nkb + kb) * (uint64_t)(64 * (KBLK / Fmt<F>::G) * Fmt<F>::SCB);
}

// sum over the 16 pairs of a chunk: acc += v_p . a_p (fixed order p = 0..15)
__device__ __forceinline__ float dot_chunk(const uint32_t* v, const half2v* a, float acc) {
#pragma unroll
  for (int p = 0; p < 16; ++p) acc = __builtin_amdgcn_fdot2(as_h2(v[p]), a[p], acc, false);
  return acc;
}

typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf2v as_b2(uint32_t u) { return __builtin_bit_cast(bf2v, u); }

// 16 packed bf16 pairs (1 + q/16) of one lane's chunk: the code sits in
// mantissa bits 3..6 of a bf16 1.0 (0x3F80). For 8-bit codes the low and high
// nibbles give two such sets (lo: o[0..15], hi: o[16..31]).
template <int F> __device__ __forceinline__ void unpack_chunk_bf(const uint32_t* w, uint32_t* o);
template <> __device__ __forceinline__ void unpack_chunk_bf<F_Q4>(const uint32_t* w, uint32_t* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v = w[i];
    o[4 * i + 0] = and_or(v << 3, 0x00780078u, 0x3F803F80u);
    o[4 * i + 1] = and_or(v >> 1, 0x00780078u, 0x3F803F80u);
    o[4 * i + 2] = and_or(v >> 5, 0x00780078u, 0x3F803F80u);
    o[4 * i + 3] = and_or(v >> 9, 0x00780078u, 0x3F803F80u);
  }
}
template <> __device__ __forceinline__ void unpack_chunk_bf<F_S4>(const uint32_t* w, uint32_t* o) {
  unpack_chunk_bf<F_Q4>(w, o);
}
template <> __device__ __forceinline__ void unpack_chunk_bf<F_Q3>(const uint32_t* w, uint32_t* o) {
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const uint32_t v = w[i];
    o[5 * i + 0] = and_or(v << 3, 0x00380038u, 0x3F803F80u);
    o[5 * i + 1] = and_or(v, 0x00380038u, 0x3F803F80u);
    o[5 * i + 2] = and_or(v >> 3, 0x00380038u, 0x3F803F80u);
    o[5 * i + 3] = and_or(v >> 6, 0x00380038u, 0x3F803F80u);
    o[5 * i + 4] = and_or(v >> 9, 0x00380038u, 0x3F803F80u);
  }
  o[15] = and_or(w[2] >> 10, 0x00200020u,
                 and_or(w[1] >> 11, 0x00100010u, and_or(w[0] >> 12, 0x00080008u, 0x3F803F80u)));
}
template <> __device__ __forceinline__ void unpack_chunk_bf<F_Q8>(const uint32_t* w, uint32_t* o) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t v = w[i];
    o[2 * i + 0] = and_or(v << 3, 0x00780078u, 0x3F803F80u);        // low nibbles
    o[2 * i + 1] = and_or(v >> 5, 0x00780078u, 0x3F803F80u);
    o[16 + 2 * i + 0] = and_or(v >> 1, 0x00780078u, 0x3F803F80u);   // high nibbles
    o[16 + 2 * i + 1] = and_or(v >> 9, 0x00780078u, 0x3F803F80u);
  }
}

// acc += sum_p v_p . a_p over 16 bf16 pairs (fixed order)
__device__ __forceinline__ float dot_chunk_bf(const uint32_t* v, const uint32_t* a, float acc) {
#pragma unroll
  for (int p = 0; p < 16; ++p) acc = __builtin_amdgcn_fdot2_f32_bf16(as_b2(v[p]), as_b2(a[p]), acc, false);
  return acc;
}
// same with fp16 pairs held as uint32
__device__ __forceinline__ float dot_chunk_h(const uint32_t* v, const uint32_t* a, float acc) {
#pragma unroll
  for (int p = 0; p < 16; ++p) acc = __builtin_amdgcn_fdot2(as_h2(v[p]), as_h2(a[p]), acc, false);
  return acc;
}

// ------------------------------------------------------------- DPP moves
// VALU-only lane moves (no LDS round trip). dpp_ctrl codes of the GCN/CDNA
// DPP encoding: quad_perm(1,0,3,2) = 0xB1, quad_perm(2,3,0,1) = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
// Sum over each aligned group of 8 lanes; every lane of a group gets the
// same bits (the pairings are symmetric and addition commutes).
__device__ __forceinline__ float sum8(float s) {
  s += dpp_f<0xB1>(s);
  s += dpp_f<0x4E>(s);
  s += dpp_f<0x141>(s);
  return s;
}
// Sum over each row of 16 lanes, same bits in every lane of the row.
__device__ __forceinline__ float sum16(float s) {
  s = sum8(s);
  s += dpp_f<0x140>(s);
  return s;
}

// Order-preserving key of a logit for the pick: NaN above +inf above every
// finite value, -0.0 equal to +0.0; larger key = better.
__device__ __forceinline__ uint32_t pick_key(float v) {
  const float z = v + 0.0f;
  const uint32_t b = __float_as_uint(z);
  if (z != z) return 0xFFFFFFFFu;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
// wave-wide max / min of a uint32: 16-lane rows by DPP, then the 4 rows
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<0xB1>((int)v));
  v = max(v, (uint32_t)dpp_i<0x4E>((int)v));
  v = max(v, (uint32_t)dpp_i<0x141>((int)v));
  v = max(v, (uint32_t)dpp_i<0x140>((int)v));
  uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  m = max(m, (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  m = max(m, (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
  m = max(m, (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return m;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)dpp_i<0xB1>((int)v));
  v = min(v, (uint32_t)dpp_i<0x4E>((int)v));
  v = min(v, (uint32_t)dpp_i<0x141>((int)v));
  v = min(v, (uint32_t)dpp_i<0x140>((int)v));
  uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  m = min(m, (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  m = min(m, (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
  m = min(m, (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return m;
}

// Wave-wide best (value, id) under pick_better; every lane gets the result.
// Within 16-lane rows by DPP, then across the 4 rows through readlane.
__device__ __forceinline__ void wave_best(float& v, int& id) {
  {
    const float ov = dpp_f<0xB1>(v); const int oi = dpp_i<0xB1>(id);
    if (pick_better(ov, oi, v, id)) { v = ov; id = oi; }
  }
  {
    const float ov = dpp_f<0x4E>(v); const int oi = dpp_i<0x4E>(id);
    if (pick_better(ov, oi, v, id)) { v = ov; id = oi; }
  }
  {
    const float ov = dpp_f<0x141>(v); const int oi = dpp_i<0x141>(id);
    if (pick_better(ov, oi, v, id)) { v = ov; id = oi; }
  }
  {
    const float ov = dpp_f<0x140>(v); const int oi = dpp_i<0x140>(id);
    if (pick_better(ov, oi, v, id)) { v = ov; id = oi; }
  }
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bi = __builtin_amdgcn_readlane(id, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
    const int oi = __builtin_amdgcn_readlane(id, 16 * r);
    if (pick_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  v = bv;
  id = bi;
}

// Lane's scale words of one 256-wide K block, loaded ahead of use: affine
// formats 4 u32 (bf16 s | bf16 b << 16, one per group of 64), symmetric one
// u32 (two fp16 scales, groups of 128).
template <int F> __device__ __forceinline__ void load_scales(const uint8_t* sblk, int lane, uint32_t* sc) {
  if constexpr (Fmt<F>::AFF) {
    const uint4 v = *reinterpret_cast<const uint4*>(sblk + lane * 16);
    sc[0] = v.x; sc[1] = v.y; sc[2] = v.z; sc[3] = v.w;
  } else {
    sc[0] = *reinterpret_cast<const uint32_t*>(sblk + lane * 4);
  }
}
// The E8M0 block scale 2^(e - 127) as fp32: e = 0 is the subnormal 2^-127,
// e = 255 NaN (OCP MX v1.0).
__device__ __forceinline__ float e8m0_to_f(uint32_t e) {
  const uint32_t bits = e == 0u ? 0x00400000u : e == 255u ? 0x7FC00000u : e << 23;
  return __uint_as_float(bits);
}

// Multiplier M*s and offset (b - M s) of group gi of a block from its words
// (MXFP4: the block scale and 0; the pair values are the elements).
template <int F> __device__ __forceinline__ void coef_reg(const uint32_t* sc, int gi, float& ms, float& bm) {
  if constexpr (F == F_MX4) {
    ms = e8m0_to_f((sc[gi >> 2] >> (8 * (gi & 3))) & 0xFFu);
    bm = 0.f;
  } else if constexpr (Fmt<F>::AFF) {
    const uint32_t v = sc[gi];
    const float s = bf16_to_f(v & 0xFFFFu), b = bf16_to_f(v >> 16);
    ms = (float)Fmt<F>::M * s;
    bm = b - ms;
  } else {
    const float s = f16_bits_to_f((sc[0] >> (16 * gi)) & 0xFFFFu);
    ms = (float)Fmt<F>::M * s;
    bm = -8.0f * s - ms;       // symmetric: w = s*(u - 8)
  }
}

// Sum of a lane's 4 consecutive activations (fixed order).
template <int ACT16> __device__ __forceinline__ float sum4(uint2 v) {
  float s = act_to_f((uint16_t)(v.x & 0xFFFFu), ACT16);
  s += act_to_f((uint16_t)(v.x >> 16), ACT16);
  s += act_to_f((uint16_t)(v.y & 0xFFFFu), ACT16);
  s += act_to_f((uint16_t)(v.y >> 16), ACT16);
  return s;
}

// One group of one row: acc = sum over the group's chunks of the pair dots
// (chunks in K order, pairs in order), then out = fma(M s, acc, out),
// out = fma(b - M s, X, out) with X the group's activation sum (8-bit codes
// with bf16 activations: two nibble sets). v: the unpacked pairs of the
// group's chunks, a: pointer to the row's activation pairs of the first
// chunk (16 u32 per chunk), X: the group's chunk sums added in order.
template <int F, int ACT16, int CPG>
__device__ __forceinline__ float group_dot(const uint32_t (*v)[F == F_Q8 ? 32 : 16], const uint32_t* a,
                                           float X, float ms, float bm, float out) {
  float acc = 0.f, acc2 = 0.f;
#pragma unroll
  for (int cc = 0; cc < CPG; ++cc) {
    uint32_t av[16];
    const uint4* q = reinterpret_cast<const uint4*>(a + 16 * cc);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 t = q[u];
      av[4 * u] = t.x; av[4 * u + 1] = t.y; av[4 * u + 2] = t.z; av[4 * u + 3] = t.w;
    }
    if constexpr (ACT16) {
      acc = dot_chunk_h(v[cc], av, acc);
    } else {
      acc = dot_chunk_bf(v[cc], av, acc);
      if constexpr (F == F_Q8) acc2 = dot_chunk_bf(v[cc] + 16, av, acc2);
    }
  }
  if constexpr (F == F_Q8 && !ACT16) {
    // q = lo + 16 hi: s*sum(q a) + b*X = 16s*A_lo + 256s*A_hi + (b - 272 s)*X
    const float s = ms * (1.0f / 256.0f), b = bm + ms;
    out = fmaf(16.0f * s, acc, out);
    out = fmaf(256.0f * s, acc2, out);
    return fmaf(b - 272.0f * s, X, out);
  }
  out = fmaf(ms, acc, out);
  return fmaf(bm, X, out);
}

// unpack of one chunk in the pair format the activations need
template <int F, int ACT16>
__device__ __forceinline__ void unpack_for(const uint32_t* w, uint32_t* v) {
  if constexpr (ACT16) unpack_chunk<F>(w, v); else unpack_chunk_bf<F>(w, v);
}

// One wave, one 256-wide K slice: for up to NR activation rows, the dot of
// each lane's weight row with the row's slice. w: the lane's 8 chunks of
// codes; sc: the slice's scale words (load_scales); xv[i]: the lane's 4
// activations of row i's slice (lane l holds elements 4l..4l+3), loaded by
// the caller; lx: this wave's LDS staging area (NR x 512 bytes). Each lane
// writes its activations to LDS and sums them; the dot then reads each
// chunk's 16 pairs back as a broadcast. Only this wave touches lx, and LDS
// serves one wave's operations in order, so no barrier. Chunk sums: 4
// consecutive activations per lane, then over aligned groups of 8 lanes.
template <int F, int NR, int ACT16>
__device__ __forceinline__ void slice_dot(const uint32_t (&w)[8][Fmt<F>::WORDS], const uint32_t* sc,
                                          int lane, const uint2* xv, int nr, uint32_t* lx, float* out) {
  constexpr int GPS = KBLK / Fmt<F>::G, CPG = Fmt<F>::G / 32;
  float csum[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    out[i] = 0.f;
    csum[i] = 0.f;
    if (i < nr) {
      reinterpret_cast<uint2*>(lx + i * 128)[lane] = xv[i];
      csum[i] = sum8(sum4<ACT16>(xv[i]));
    }
  }
#pragma unroll
  for (int gi = 0; gi < GPS; ++gi) {
    float ms, bm;
    coef_reg<F>(sc, gi, ms, bm);
    uint32_t v[CPG][F == F_Q8 ? 32 : 16];
#pragma unroll
    for (int cc = 0; cc < CPG; ++cc) unpack_for<F, ACT16>(w[gi * CPG + cc], v[cc]);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (i < nr) {
        float X = 0.f;
#pragma unroll
        for (int cc = 0; cc < CPG; ++cc)
          X += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(csum[i]), 8 * (gi * CPG + cc)));
        out[i] = group_dot<F, ACT16, CPG>(v, lx + i * 128 + 16 * gi * CPG, X, ms, bm, out[i]);
      }
    }
  }
}

// The k best of up to 64 * NC candidates held by one wave (lane l holds
// column i's candidate with its order key and id; key 0 = absent), ranked by
// (key desc, id asc); ids must grow with (column, lane) so that lane order
// settles ties. Every lane must be active. Steps:
//  1. T = the k-th largest key, two bits at a time from the top: of the four
//     digits the largest is kept for which at least k keys are >= the prefix
//     with it (three ballots per candidate column and step, all issued before
//     the counts are read);
//  2. the picks are every key > T plus the lowest ids among the keys == T;
//  3. they are compacted in id order into the wave's LDS scratch (8 entries)
//     and lane j < k reads entry j, then takes its slot from the other
//     picks' keys and ids.
// On return lane j < k holds slot s_j (distinct, 0..k-1) with its id and
// value; lanes >= k hold slot k.
template <int NC>
__device__ __forceinline__ void wave_topk_ids(const uint32_t (&key)[NC], const float (&val)[NC],
                                              const int (&idv)[NC], int lane, int k,
                                              uint32_t* scratch /* wave-private LDS, 24 u32 */, int& slot,
                                              int& id, float& v) {
  // T = the largest key with at least k keys >= T (the k-th largest key),
  // two bits per step: the counts for the three candidate digits of a step
  // are independent, and they do not increase with the digit
  uint32_t T = 0;
#pragma unroll
  for (int b = 30; b >= 0; b -= 2) {
    const uint32_t c1 = T | (1u << b), c2 = T | (2u << b), c3 = T | (3u << b);
    // all compares of the step issue before the first count reads one
    uint64_t m[NC][3];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      m[i][0] = __ballot(key[i] >= c1);
      m[i][1] = __ballot(key[i] >= c2);
      m[i][2] = __ballot(key[i] >= c3);
    }
    __builtin_amdgcn_sched_barrier(0);
    int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      n1 += __popcll(m[i][0]);
      n2 += __popcll(m[i][1]);
      n3 += __popcll(m[i][2]);
    }
    T = n3 >= k ? c3 : n2 >= k ? c2 : n1 >= k ? c1 : T;
  }
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int need = k, before = 0;
#pragma unroll
  for (int i = 0; i < NC; ++i) need -= __popcll(__ballot(key[i] > T));
  bool sel[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const uint64_t eq = __ballot(key[i] == T);
    const int tie_rank = before + __popcll(eq & lt);
    sel[i] = key[i] > T || (key[i] == T && tie_rank < need);
    before += __popcll(eq);
  }
  int pos = 0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const uint64_t sm = __ballot(sel[i]);
    if (sel[i]) {
      const int p = pos + __popcll(sm & lt);
      scratch[p] = key[i];
      scratch[8 + p] = (uint32_t)idv[i];
      scratch[16 + p] = __float_as_uint(val[i]);
    }
    pos += __popcll(sm);
  }
  __builtin_amdgcn_wave_barrier();
  const int e = lane < k ? lane : 0;
  const uint32_t mk = scratch[e];
  id = (int)scratch[8 + e];
  v = __uint_as_float(scratch[16 + e]);
  int s = 0;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m < k) {
      const uint32_t km = (uint32_t)__builtin_amdgcn_readlane((int)mk, m);
      const int im = __builtin_amdgcn_readlane(id, m);
      s += (km > mk || (km == mk && im < id)) ? 1 : 0;
    }
  }
  slot = lane < k ? s : k;
}
// 256 candidates, lane l holding ids l + 64 i
__device__ __forceinline__ void wave_topk(const uint32_t (&key)[4], const float (&val)[4], int lane, int k,
                                          uint32_t* scratch, int& slot, int& id, float& v) {
  const int idv[4] = {lane, lane + 64, lane + 128, lane + 192};
  wave_topk_ids<4>(key, val, idv, lane, k, scratch, slot, id, v);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  // silu(g) * u with silu(z) = z / (1 + exp(-z))
  return (g / (1.0f + expf(-g))) * u;
}


// The pair unpack of one chunk for the matrix-core form: the same values
// as unpack_for, written as plain code on masks the compiler cannot see as
// constants, so it still selects one v_and_or_b32 per pair and, unlike for
// inline asm, tracks the wait states a VALU write needs before a matrix-core
// read of the same register.
struct PairMasks {
  uint32_t m, c, q0, q1, q2;   // field mask, 1.0 pair, 3-bit last-pair masks
};
template <int F, int ACT16>
__device__ __forceinline__ PairMasks pair_masks() {
  PairMasks k;
  if constexpr (F == F_Q8) {
    k.m = ACT16 ? 0x03FC03FCu : 0x00780078u;   // fp16: the byte; bf16: a nibble
    k.q0 = k.q1 = k.q2 = 0u;
  } else if constexpr (F == F_Q2) {
    k.m = ACT16 ? 0x00C000C0u : 0x00180018u;
    k.q0 = k.q1 = k.q2 = 0u;
  } else if constexpr (F == F_Q5) {
    k.m = ACT16 ? 0x03E003E0u : 0x007C007Cu;
    k.q0 = k.q1 = k.q2 = 0u;
  } else if constexpr (F == F_Q6) {
    k.m = ACT16 ? 0x03F003F0u : 0x007E007Eu;
    k.q0 = ACT16 ? 0x00F000F0u : 0x001E001Eu;   // low 4 bits of pairs 12..15
    k.q1 = ACT16 ? 0x03000300u : 0x00600060u;   // their high 2 bits
    k.q2 = 0u;
  } else if constexpr (F == F_Q3) {
    k.m = ACT16 ? 0x01C001C0u : 0x00380038u;
    k.q0 = ACT16 ? 0x00400040u : 0x00080008u;
    k.q1 = ACT16 ? 0x00800080u : 0x00100010u;
    k.q2 = ACT16 ? 0x01000100u : 0x00200020u;
  } else {
    k.m = ACT16 ? 0x03C003C0u : 0x00780078u;
    k.q0 = k.q1 = k.q2 = 0u;
  }
  k.c = ACT16 ? 0x3C003C00u : 0x3F803F80u;
  asm volatile("" : "+s"(k.m), "+s"(k.q0), "+s"(k.q1), "+s"(k.q2), "+v"(k.c));
  return k;
}
// One nibble set of 8-bit codes for bf16 activations (HI = 0: the low
// nibbles, 1: the high ones), 16 pairs 1 + n/16: unpack_pairs' o[0..15] or
// o[16..31], for code that runs one set's dots before unpacking the other.
template <int HI>
__device__ __forceinline__ void unpack_q8_nibbles(const uint32_t* w, const PairMasks& k, uint32_t* o) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t v = w[i];
    o[2 * i] = ((HI ? v >> 1 : v << 3) & k.m) | k.c;
    o[2 * i + 1] = ((HI ? v >> 9 : v >> 5) & k.m) | k.c;
  }
}

// 8-bit codes: with fp16 activations 16 pairs 1 + q/256; with bf16 ones
// (7 mantissa bits) the low nibbles' 16 pairs in o[0..15] and the high
// nibbles' in o[16..31], each 1 + n/16.
// The two E2M1 elements of byte B of v as an fp16 (ACT16) or bf16 pair,
// element 2B's low nibble in the low half.
template <int ACT16>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t v, int b) {
  if constexpr (ACT16) {
    switch (b) {
      case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 0));
      case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 1));
      case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 2));
      default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 3));
    }
  } else {
    switch (b) {
      case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 0));
      case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 1));
      case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 2));
      default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 3));
    }
  }
}

template <int F, int ACT16>
__device__ __forceinline__ void unpack_pairs(const uint32_t* w, const PairMasks& k, uint32_t* o) {
  if constexpr (F == F_Q8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t v = w[i];
      if constexpr (ACT16) {
        o[2 * i] = ((v << 2) & k.m) | k.c;
        o[2 * i + 1] = ((v >> 6) & k.m) | k.c;
      } else {
        o[2 * i] = ((v << 3) & k.m) | k.c;
        o[2 * i + 1] = ((v >> 5) & k.m) | k.c;
        o[16 + 2 * i] = ((v >> 1) & k.m) | k.c;
        o[16 + 2 * i + 1] = ((v >> 9) & k.m) | k.c;
      }
    }
  } else if constexpr (F == F_Q2) {
    // pair j of word i at bits 2j: moved to mantissa bit 6 (fp16) or 3 (bf16)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t v = w[i];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        constexpr int T = ACT16 ? 6 : 3;
        const uint32_t sv = 2 * j <= T ? v << (T - 2 * j) : v >> (2 * j - T);
        o[8 * i + j] = (sv & k.m) | k.c;
      }
    }
  } else if constexpr (F == F_Q5) {
    // value 1 + q/32: code bit 0 to mantissa bit 5 (fp16) or 2 (bf16)
    constexpr int T = ACT16 ? 5 : 2;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const uint32_t v = w[i];
      o[3 * i + 0] = ((v << T) & k.m) | k.c;
      o[3 * i + 1] = ((ACT16 ? v : v >> 3) & k.m) | k.c;
      o[3 * i + 2] = ((v >> (10 - T)) & k.m) | k.c;
    }
    uint32_t t = k.c;
#pragma unroll
    for (int b = 0; b < 5; ++b) t |= (w[b] >> (15 - T - b)) & (0x00010001u << (T + b));
    o[15] = t;
  } else if constexpr (F == F_Q6) {
    // value 1 + q/64: code bit 0 to mantissa bit 4 (fp16) or 1 (bf16)
    constexpr int T = ACT16 ? 4 : 1;
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const uint32_t v = w[i];
      o[2 * i + 0] = ((v << T) & k.m) | k.c;
      o[2 * i + 1] = ((v >> (6 - T)) & k.m) | k.c;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
      o[12 + m] = ((w[4 + m / 2] >> (8 + 2 * (m % 2) - T)) & k.q1) | (((w[m] >> (12 - T)) & k.q0) | k.c);
  } else if constexpr (F == F_Q3) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const uint32_t v = w[i];
      o[5 * i + 0] = ((ACT16 ? v << 6 : v << 3) & k.m) | k.c;
      o[5 * i + 1] = ((ACT16 ? v << 3 : v) & k.m) | k.c;
      o[5 * i + 2] = ((ACT16 ? v : v >> 3) & k.m) | k.c;
      o[5 * i + 3] = ((ACT16 ? v >> 3 : v >> 6) & k.m) | k.c;
      o[5 * i + 4] = ((ACT16 ? v >> 6 : v >> 9) & k.m) | k.c;
    }
    const uint32_t t0 = ((w[0] >> (ACT16 ? 9 : 12)) & k.q0) | k.c;
    const uint32_t t1 = ((w[1] >> (ACT16 ? 8 : 11)) & k.q1) | t0;
    o[15] = ((w[2] >> (ACT16 ? 7 : 10)) & k.q2) | t1;
  } else if constexpr (F == F_MX4) {
    // pair p = byte p of the chunk (elements 2p in the low nibble, 2p + 1 in
    // the high one), converted exactly by the FP4 unit at scale 1
#pragma unroll
    for (int p = 0; p < 16; ++p) o[p] = fp4_pair<ACT16>(w[p >> 2], p & 3);
    (void)k;
  } else {   // 4-bit affine or symmetric
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = w[i];
      o[4 * i + 0] = ((ACT16 ? v << 6 : v << 3) & k.m) | k.c;
      o[4 * i + 1] = ((ACT16 ? v << 2 : v >> 1) & k.m) | k.c;
      o[4 * i + 2] = ((ACT16 ? v >> 2 : v >> 5) & k.m) | k.c;
      o[4 * i + 3] = ((ACT16 ? v >> 6 : v >> 9) & k.m) | k.c;
    }
  }
}

}  // namespace moe
