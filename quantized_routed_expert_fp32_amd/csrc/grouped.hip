// Grouped (prompt-chunk) path: the prefill form for chunks of many rows.
//
//  1. k_grp_sort: one workgroup sorts the slots (row r, pick j) by expert:
//     per-wave expert histograms (one LDS atomic per slot), an exclusive
//     scan, and a scatter into expert-major order (the shared expert follows
//     as expert E with every row). A slot's place inside its expert's run
//     comes from the LDS atomic that counts it, so it can differ from call to
//     call; nothing downstream depends on it (every row of an M-tile is
//     computed from its own activations alone, and outputs go back to the
//     slot's own place). Then the work list: each expert's
//     run is cut into M-tiles of 128 rows, the last one 32, 64, 96 or 128
//     rows tall; the list holds every 128-row tile first, then the 96-, 64-
//     and 32-row ones, so the longest work starts first and the short tiles
//     fill the end. Extra workgroups of the same launch convert bf16
//     activations to fp16 for the GEMMs.
//  2. k_grp_gemm<GU>: a persistent grid (two workgroups per CU) takes
//     (M-tile, 256-column block) items from a device queue. Wave w owns one
//     64-row layout tile of the gate/up matrix (32 gate rows and the 32 up
//     rows of the same intermediate indices), so gate and up of an output
//     land in the same lane and SwiGLU runs in registers. Both operands go
//     from memory straight into a three-stage LDS ring (global_load_lds, one
//     64-k step ahead): A, the tile's activation rows gathered by the sort's
//     permutation (XOR-swizzled 16-byte segments), and per wave B, the packed
//     codes and scale words of its layout tile. B is dequantised to fp16
//     right before use (affine: s*q + b; symmetric: s*(u - 8));
//     v_mfma_f32_32x32x16_f16 accumulates in fp32. Output h in fp16,
//     expert-major.
//  3. k_grp_gemm<DN>: the same on h and the down matrices; output e in fp32
//     per slot.
//  4. k_grp_combine: y = sum_j p_j e_j + sigma e_shared, slots in pick order.
// ("Sage-A1.5 ... #1329", Proposal: grouped MoE and prompt chunks on the
//  matrix engines; Limits to agree on: the grouped form adds in another
//  order than the per-row form, so it is judged by tolerance, not bits.)
#include "moe_kernels.h"
#include "moe_launch.h"
#include "moe_dispatch.h"

#include <algorithm>

namespace moe {

typedef f16 half8v_t __attribute__((ext_vector_type(8)));
typedef float f16v_t __attribute__((ext_vector_type(16)));

// meta layout (int32): [0] M-tiles in the work list, [1] gate/up queue
// counter, [2] down queue counter, [8 .. E+10) expert offsets (E+2 entries)
constexpr int META_OFF = 8;

// ------------------------------------------------------------------ sort
// Exclusive prefix sum of n <= 320 LDS counters by one wave (lane l owns
// entries 5l .. 5l+4); returns the total.
__device__ __forceinline__ int wave_exclusive_scan(const int* in, int* out, int n, int lane) {
  int v[5], loc = 0;
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    const int i = 5 * lane + q;
    v[q] = i < n ? in[i] : 0;
    loc += v[q];
  }
  int inc = loc;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  int run = inc - loc;
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    const int i = 5 * lane + q;
    if (i < n) out[i] = run;
    run += v[q];
  }
  return __shfl(inc, 63);
}

// Workgroup 0: the sort and the work list (1024 threads, 16 waves; wave w
// owns the contiguous slot range [w S, (w+1) S), S = ceil(R k / 16)):
//  1. per-wave expert histograms (one LDS atomic per slot);
//  2. exclusive scan over the experts (shared expert E with every row), then
//     each wave's base per expert: the offset plus the earlier waves' counts;
//  3. the same walk again scatters each slot to the position its wave's
//     running count for the expert returns;
//  4. the work list of M-tiles (expert, first position, rows), 128-row tiles
//     first, then 96-, 64- and 32-row ones, each class laid out by a scan
//     over the experts; the queue counters of the two GEMMs are reset. With
//     blk16 (the exact chunk form) the list holds instead each expert's run
//     cut into blocks of 16 rows (the last one shorter), in expert order.
// Workgroups 1.. (bf16 activations only): x -> fp16 copy for the gate/up GEMM.
__global__ __launch_bounds__(1024) void k_grp_sort(GroupedArgs a) {
  __shared__ int cnt[320];
  __shared__ int off[320];
  __shared__ int nt[4][320];             // M-tiles per expert in each height class, then their offsets
  __shared__ int wh[16][258];            // per-wave counts, then per-wave running positions
  __shared__ int s_tot[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (blockIdx.x > 0) {
    // bf16 -> fp16 (exact for |x| >= 2^-17 and below 65504), 8 values a thread
    const uint64_t n8 = (uint64_t)a.R * a.H / 8;
    const uint4* src = reinterpret_cast<const uint4*>(a.x);
    uint4* dst = reinterpret_cast<uint4*>(const_cast<uint16_t*>(a.x16));
    for (uint64_t i = (uint64_t)(blockIdx.x - 1) * 1024 + tid; i < n8; i += (uint64_t)(gridDim.x - 1) * 1024) {
      const uint4 v = src[i];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        half2v h;
        h.x = (f16)bf16_to_f(u[q] & 0xFFFFu);
        h.y = (f16)bf16_to_f(u[q] >> 16);
        o[q] = as_u(h);
      }
      dst[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    return;
  }
  const int E = a.E, k = a.k, R = a.R, nslot = R * k;
  const int S = (nslot + 15) / 16, s0 = w * S, s1 = min(nslot, s0 + S);
  for (int q = tid; q < 16 * 258; q += 1024) (&wh[0][0])[q] = 0;
  __syncthreads();
  // 1. histograms (the ids of 16 rounds are loaded at once: one memory
  // latency per 1024 slots of a wave)
  for (int bb = s0; bb < s1; bb += 1024) {
    int ev[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int i = bb + 64 * q + lane;
      ev[q] = i < s1 ? a.ids[i] : -1;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = ev[q];
      if (e >= 0 && e < E) atomicAdd(&wh[w][e], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    int c = 0;
    for (int q = 0; q < 16; ++q) c += wh[q][e];
    cnt[e] = c;
  }
  __syncthreads();
  // 2. offsets, per-wave bases
  if (w == 0) {
    if (lane == 0) cnt[E] = R;
    __builtin_amdgcn_wave_barrier();
    const int tot = wave_exclusive_scan(cnt, off, E + 1, lane);
    if (lane == 0) off[E + 1] = tot;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    int run = off[e];
    for (int q = 0; q < 16; ++q) {
      const int c = wh[q][e];
      wh[q][e] = run;
      run += c;
    }
  }
  for (int e = tid; e <= E + 1; e += 1024) a.meta[META_OFF + e] = off[e];
  for (int e = tid; e <= E; e += 1024) {
    const int c = cnt[e];
    const int mtr = ((c & 127) + 31) >> 5;       // height of the last tile in 32-row units (0: none)
    nt[0][e] = a.blk16 ? (c + 15) >> 4 : (c >> 7) + (mtr == 4);
    nt[1][e] = !a.blk16 && mtr == 3;
    nt[2][e] = !a.blk16 && mtr == 2;
    nt[3][e] = !a.blk16 && mtr == 1;
  }
  __syncthreads();
  // 3. scatter (positions from the wave's own LDS row)
  for (int bb = s0; bb < s1; bb += 1024) {
    int ev[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int i = bb + 64 * q + lane;
      ev[q] = i < s1 ? a.ids[i] : -1;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int i = bb + 64 * q + lane;
      const int e = ev[q];
      if (e >= 0 && e < E) a.perm[atomicAdd(&wh[w][e], 1)] = (i / k) * (k + 1) + i % k;
    }
  }
  for (int r = tid; r < R; r += 1024) a.perm[off[E] + r] = r * (k + 1) + k;
  // 4. work list: one scan per height class (waves 0..3)
  if (w < 4) {
    const int tot = wave_exclusive_scan(nt[w], nt[w], E + 1, lane);
    if (lane == 0) s_tot[w] = tot;
  }
  __syncthreads();
  const int b1 = s_tot[0], b2 = b1 + s_tot[1], b3 = b2 + s_tot[2];
  for (int e = tid; e <= E && a.blk16; e += 1024) {
    // the exact chunk form: blocks of 16 rows, the last one shorter
    const int c = cnt[e];
    int* t = a.tiles + 3 * nt[0][e];
    for (int m = 0; 16 * m < c; ++m, t += 3) {
      t[0] = e;
      t[1] = off[e] + 16 * m;
      t[2] = min(16, c - 16 * m);
    }
  }
  for (int e = tid; e <= E && !a.blk16; e += 1024) {
    const int c = cnt[e];
    const int full = c >> 7, rem = c & 127, mtr = (rem + 31) >> 5;
    int* t = a.tiles + 3 * nt[0][e];
    for (int m = 0; m < full; ++m, t += 3) {
      t[0] = e;
      t[1] = off[e] + 128 * m;
      t[2] = 128;
    }
    if (mtr > 0) {
      if (mtr != 4) t = a.tiles + 3 * (mtr == 3 ? b1 + nt[1][e] : mtr == 2 ? b2 + nt[2][e] : b3 + nt[3][e]);
      t[0] = e;
      t[1] = off[e] + 128 * full;
      t[2] = rem;
    }
  }
  if (tid == 0) {
    a.meta[0] = b3 + s_tot[3];
    a.meta[1] = 0;
    a.meta[2] = 0;
  }
}

// ------------------------------------------------------------------ GEMM
// fp16 pair dequantisation of one code word (8 codes of one weight row):
// 4 packed fp16 pairs w = s*q + b (affine) or s*(u - 8) (symmetric), for
// the pair layout of the packed codes (pairs of consecutive k).
template <int F>
__device__ __forceinline__ void deq_word(const uint32_t* wv, half2v s2, half2v b2, uint32_t* o);

template <>
__device__ __forceinline__ void deq_word<F_Q4>(const uint32_t* wv, half2v s16, half2v b2, uint32_t* o) {
  // 1 + q/16 -> q/16 (exact) -> fma with (16 s, b): one rounding
  const uint32_t v = wv[0];
  const uint32_t p[4] = {and_or(v << 6, 0x03C003C0u, 0x3C003C00u), and_or(v << 2, 0x03C003C0u, 0x3C003C00u),
                         and_or(v >> 2, 0x03C003C0u, 0x3C003C00u), and_or(v >> 6, 0x03C003C0u, 0x3C003C00u)};
  const half2v one = {(f16)1.0f, (f16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v q16 = as_h2(p[i]) - one;
    o[i] = as_u(__builtin_elementwise_fma(q16, s16, b2));
  }
}
template <>
__device__ __forceinline__ void deq_word<F_S4>(const uint32_t* wv, half2v s16, half2v b2, uint32_t* o) {
  // 1 + u/16 - 1.5 = (u - 8)/16 exactly, times 16 s: one rounding
  const uint32_t v = wv[0];
  const uint32_t p[4] = {and_or(v << 6, 0x03C003C0u, 0x3C003C00u), and_or(v << 2, 0x03C003C0u, 0x3C003C00u),
                         and_or(v >> 2, 0x03C003C0u, 0x3C003C00u), and_or(v >> 6, 0x03C003C0u, 0x3C003C00u)};
  const half2v off = {(f16)1.5f, (f16)1.5f};
  (void)b2;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = as_u((as_h2(p[i]) - off) * s16);
}

// MXFP4: the word's 4 bytes are the pairs (consecutive k, low nibble first);
// the FP4 converter scales each by the block scale 2^(e - 127) and rounds to
// fp16, exactly for the exponents the grouped call accepts (104..140, 255).
__device__ __forceinline__ void deq_word_mx(uint32_t v, float scale, uint32_t* o) {
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, scale, 0));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, scale, 1));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, scale, 2));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, scale, 3));
}

// Widths read through the generic B layout (the chunk block copied to LDS
// as it is packed, every lane unpacking its row's whole chunk).
template <int F> constexpr bool gen_fmt() { return F == F_Q2 || F == F_Q5 || F == F_Q6 || F == F_Q8; }

// For the 3-bit layout and the generic widths, the 8 codes k = 8v..8v+7 of
// a chunk (v = 0..3) sit in pairs 4v..4v+3 of the chunk's full unpack.
template <int F>
__device__ __forceinline__ void deq_chunk_half(const uint32_t* cw, int wsel, half2v s16, half2v b2,
                                               uint32_t* o) {
  if constexpr (gen_fmt<F>()) {
    // pairs 1 + q/M of the whole chunk, then the 4 of this lane's k range
    uint32_t v[16];
    unpack_pairs<F, 1>(cw, pair_masks<F, 1>(), v);
    const half2v one = {(f16)1.0f, (f16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t pv = v[i];
#pragma unroll
      for (int q = 1; q < 4; ++q) pv = (wsel == q) ? v[4 * q + i] : pv;
      o[i] = as_u(__builtin_elementwise_fma(as_h2(pv) - one, s16, b2));
    }
  } else if constexpr (F == F_Q3) {
    uint32_t v[16];
    unpack_chunk<F_Q3>(cw, v);   // 1 + q/16 pairs
    const half2v one = {(f16)1.0f, (f16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t pv = v[0];
#pragma unroll
      for (int q = 0; q < 4; ++q) pv = (wsel == q) ? v[4 * q + i] : pv;
      o[i] = as_u(__builtin_elementwise_fma(as_h2(pv) - one, s16, b2));
    }
  } else {
    uint32_t wv[1];
    wv[0] = cw[0];
#pragma unroll
    for (int q = 1; q < 4; ++q) wv[0] = (wsel == q) ? cw[q] : wv[0];
    deq_word<F>(wv, s16, b2, o);
  }
}

enum { GU = 0, DN = 1 };

// The LDS ring of the GEMMs: 3 stages, each the A tile of one 64-k step
// (128 rows x 64 k fp16, 16 KiB) and, per wave, the B codes of its layout
// tile for that step (two chunk blocks of 64 rows) and the rows' scale
// words. Every load of a step goes straight from memory into its stage
// (global_load_lds), so nothing of the pipeline sits in registers; loads run
// one step ahead.
constexpr int NST = 3;
constexpr int A_STAGE = 128 * 64;        // halves of the A tile of one step

// LDS bytes of one chunk block (64 weight rows of one 32-k chunk): 12-byte
// rows land at a 16-byte lane stride, the generic widths keep the packed
// layout (64 rows of CB bytes, see row_word).
template <int F> constexpr int chunk_lds() { return gen_fmt<F>() ? 64 * Fmt<F>::CB : 1024; }
// Word q of weight row r inside a chunk block as packed: rows of CB bytes
// one after another, except 8-bit rows, whose first and second 16 bytes sit
// in two 1 KiB halves of the block (rows 0..63 each).
template <int F> __device__ __forceinline__ int row_word(int r, int q) {
  if constexpr (F == F_Q8) return (q >> 2) * 256 + 4 * r + (q & 3);
  else return r * Fmt<F>::WORDS + q;
}
// One wave's B area: the codes of 2 chunk blocks, then the 64 rows' scale words.
template <int F> constexpr int b_scale_off() { return 2 * chunk_lds<F>(); }
template <int F> constexpr int b_wave() { return b_scale_off<F>() + 256; }
// B loads per thread and step: 2 chunk blocks (one load each, or CB / 4
// loads of 4 bytes each for the generic widths) and 1 scale word.
template <int F> constexpr int b_loads() { return gen_fmt<F>() ? 2 * (Fmt<F>::CB / 4) + 1 : 3; }
template <int FR, int FS> constexpr int stage_b_wave() { return b_wave<FR>() > b_wave<FS>() ? b_wave<FR>() : b_wave<FS>(); }
template <int FR, int FS> constexpr int stage_bytes() { return 2 * A_STAGE + 4 * stage_b_wave<FR, FS>(); }

// 4-bit codes: the lane of half hsel takes words 2 hsel, 2 hsel + 1 of each
// chunk row (8 contiguous bytes), i.e. k = 16 hsel .. 16 hsel + 15 of the
// chunk, and the A fragments follow the same k. The 3-bit rows hold a
// chunk's codes across all 3 words, so their lanes take the full row.
template <int F> struct BFrag {
  static constexpr bool HALF = F == F_Q4 || F == F_S4 || F == F_MX4;
  static constexpr int W = HALF ? 2 : Fmt<F>::WORDS;   // words per chunk per lane
};

// Codes (per n-tile and chunk) and scale words (per n-tile) of the wave's
// layout tile for one 64-k step, as the lane uses them.
template <int F>
struct BStage {
  uint32_t w[2][2][BFrag<F>::W];
  uint32_t sr[2];
};

// At most N vector-memory operations of this wave still in flight (expcnt
// and lgkmcnt not waited for).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS byte address of a __shared__ pointer
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// XOR swizzle of the A tile's 16-byte segments: row r's segment s sits at
// position s ^ swz(r), so the 8 (32 banks) or 16 (64 banks) lanes served
// together read distinct bank groups.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// The B loads of one step into the wave's area bw (exactly b_loads<F>() loads:
// the wait counts rely on it): lane l copies row l of the layout tile's two
// chunk blocks (CB bytes each) and row l's scale word: affine, the (s, b)
// word of the step's group; symmetric, the word holding both fp16 scales of
// the row's 256-wide block. Every load to LDS here moves whole dwords; a
// 16- or 4-byte load puts lane l's data at l times its size, a 12-byte load
// (3-bit rows) at 16 l, so a chunk block takes 1 KiB in LDS either way.
template <int F>
__device__ __forceinline__ void issue_b(uint8_t* bw, const uint8_t* blk, uint32_t codes, uint32_t scales, int T,
                                       int nch, int nkb, int lane, int step) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int GPS = KBLK / Fmt<F>::G, CB = Fmt<F>::CB;
  const int kk0 = 64 * step;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if constexpr (gen_fmt<F>()) {
      // the chunk block as packed: CB / 4 pieces of 256 bytes, a dword a lane
#pragma unroll
      for (int q = 0; q < CB / 4; ++q)
        __builtin_amdgcn_global_load_lds(blk + codes + chunk_off<F>(T, kk0 / 32 + c, nch) + 256 * q + 4 * lane,
                                         (__attribute__((address_space(3))) void*)(bw + chunk_lds<F>() * c + 256 * q),
                                         4, 0, 0);
    } else {
      __builtin_amdgcn_global_load_lds(blk + codes + chunk_off<F>(T, kk0 / 32 + c, nch) + lane * CB,
                                       (__attribute__((address_space(3))) void*)(bw + 1024 * c), CB, 0, 0);
    }
  }
  const uint8_t* sb = blk + scales + sblk_off<F>(T, kk0 / KBLK, nkb);
  if constexpr (F == F_MX4) {
    // the row's 8 exponent bytes of the block: the word of groups 4 h .. 4 h + 3
    // that holds this step's two (h = the step's half of the block)
    __builtin_amdgcn_global_load_lds(sb + lane * 8 + ((kk0 % KBLK) / 128) * 4,
                                     (__attribute__((address_space(3))) void*)(bw + b_scale_off<F>()), 4, 0, 0);
  } else if constexpr (Fmt<F>::AFF) {
    const int gi = (kk0 % KBLK) / Fmt<F>::G;
    __builtin_amdgcn_global_load_lds(sb + (lane * GPS + gi) * 4,
                                     (__attribute__((address_space(3))) void*)(bw + b_scale_off<F>()), 4, 0, 0);
  } else {
    static_assert(GPS == 2, "two fp16 scales per row and block");
    __builtin_amdgcn_global_load_lds(sb + lane * 4, (__attribute__((address_space(3))) void*)(bw + b_scale_off<F>()),
                                     4, 0, 0);
  }
#endif
}

// The A loads of one step: MT loads of 16 bytes per thread straight into
// the stage's A tile (wave w's instruction i fills the 1 KiB at segment
// 256 i + 64 w; lane l's segment is row q / 8, position q % 8, holding the
// row's source segment (q % 8) ^ swz(row)).
template <int MT>
__device__ __forceinline__ void issue_a(const uint16_t* const* asrc, uint16_t* buf, int w, int step) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int i = 0; i < MT; ++i)
    __builtin_amdgcn_global_load_lds(asrc[i] + 64 * step,
                                     (__attribute__((address_space(3))) void*)(buf + (256 * i + 64 * w) * 8), 16, 0,
                                     0);
#endif
}

// The reads below are inline asm, each block waiting for its own results:
// the compiler would otherwise guard every LDS read against the loads into
// LDS still in flight (the prefetched stage included) by waiting for all of
// them. What they read has landed: the step's wait and barrier came first.
// Every output is early-clobber ("=&v"): a block issues several reads before
// its one wait, so an output register shared with an address input of the
// same block can be overwritten while the block still reads through it (a
// W4A16 instantiation whose scale outputs took the address registers read
// wrong scales for whole k-steps).
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v3u __attribute__((ext_vector_type(3)));

// The lane's B words of one step from the wave's area at byte address bw:
// codes of rows col and 32 + col (half hsel for 4-bit codes, the whole row
// for 3-bit ones) of both chunks, and the two rows' scale entries (a
// symmetric row's word holds the scales of groups 0 and 1 of its block; the
// step's group is step % 4 / 2).
template <int F>
__device__ __forceinline__ void read_b(BStage<F>& st, uint32_t bw, int col, int hsel, int step) {
  uint32_t s0, s1;
  if constexpr (gen_fmt<F>()) {
    // generic widths: plain LDS reads of the two rows' whole chunks (the
    // compiler waits for every load to LDS in flight before them)
    typedef const __attribute__((address_space(3))) uint32_t* lds_u32;
    const lds_u32 b = (lds_u32)(uintptr_t)bw;
    constexpr int WD = Fmt<F>::WORDS, CW = chunk_lds<F>() / 4;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int q = 0; q < WD; ++q) st.w[nt][c][q] = b[c * CW + row_word<F>(col + 32 * nt, q)];
    s0 = b[b_scale_off<F>() / 4 + col];
    s1 = b[b_scale_off<F>() / 4 + 32 + col];
  } else if constexpr (BFrag<F>::HALF) {
    const uint32_t ac = bw + col * 16 + 8 * hsel;
    v2u c00, c10, c01, c11;
    if constexpr (Fmt<F>::AFF) {
      asm volatile("ds_read_b64 %0, %6\n\tds_read_b64 %1, %6 offset:512\n\tds_read_b64 %2, %6 offset:1024\n\t"
                   "ds_read_b64 %3, %6 offset:1536\n\tds_read_b32 %4, %7\n\tds_read_b32 %5, %7 offset:128\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(c00), "=&v"(c10), "=&v"(c01), "=&v"(c11), "=&v"(s0), "=&v"(s1)
                   : "v"(ac), "v"(bw + 2048 + col * 4));
    } else {
      asm volatile("ds_read_b64 %0, %6\n\tds_read_b64 %1, %6 offset:512\n\tds_read_b64 %2, %6 offset:1024\n\t"
                   "ds_read_b64 %3, %6 offset:1536\n\tds_read_b32 %4, %7\n\tds_read_b32 %5, %7 offset:128\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(c00), "=&v"(c10), "=&v"(c01), "=&v"(c11), "=&v"(s0), "=&v"(s1)
                   : "v"(ac), "v"(bw + 2048 + col * 4));
      // symmetric: the fp16 scale of the step's group (half (step % 4) / 2);
      // MXFP4: the exponent bytes of the step's two chunks in the low half
      const int sh = F == F_MX4 ? 16 * (step & 1) : 16 * ((step & 3) >> 1);
      s0 >>= sh;
      s1 >>= sh;
    }
    st.w[0][0][0] = c00.x; st.w[0][0][1] = c00.y;
    st.w[1][0][0] = c10.x; st.w[1][0][1] = c10.y;
    st.w[0][1][0] = c01.x; st.w[0][1][1] = c01.y;
    st.w[1][1][0] = c11.x; st.w[1][1][1] = c11.y;
  } else {
    // 3-bit rows: 12 bytes at a 16-byte lane stride
    static_assert(Fmt<F>::CB == 12, "row layout");
    const uint32_t ac = bw + col * 16;
    v3u r0, r1, r2, r3;
    asm volatile("ds_read_b96 %0, %6\n\tds_read_b96 %1, %6 offset:512\n\tds_read_b96 %2, %6 offset:1024\n\t"
                 "ds_read_b96 %3, %6 offset:1536\n\tds_read_b32 %4, %7\n\tds_read_b32 %5, %7 offset:128\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(s0), "=&v"(s1)
                 : "v"(ac), "v"(bw + 2048 + col * 4));
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      st.w[0][0][q] = r0[q];
      st.w[1][0][q] = r1[q];
      st.w[0][1][q] = r2[q];
      st.w[1][1][q] = r3[q];
    }
  }
  st.sr[0] = s0;
  st.sr[1] = s1;
}

template <int F>
__device__ __forceinline__ int a_seg(int i, int hsel) {
  const int c = i >> 1, j = i & 1;
  return BFrag<F>::HALF ? 4 * c + 2 * hsel + j : 4 * c + 2 * j + hsel;
}

// The MT A fragments of k-step i (rows 32 mt + col) from the A tile at
// byte address buf.
template <int F, int MT>
__device__ __forceinline__ void read_a(half8v_t (&ah)[MT], uint32_t buf, int i, int col, int hsel) {
  const uint32_t ad = buf + col * 128 + 16 * (a_seg<F>(i, hsel) ^ swz(col));
  v4u r0, r1, r2, r3;
  if constexpr (MT == 4)
    asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:4096\n\tds_read_b128 %2, %4 offset:8192\n\t"
                 "ds_read_b128 %3, %4 offset:12288\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3) : "v"(ad));
  else if constexpr (MT == 3)
    asm volatile("ds_read_b128 %0, %3\n\tds_read_b128 %1, %3 offset:4096\n\tds_read_b128 %2, %3 offset:8192\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r0), "=&v"(r1), "=&v"(r2) : "v"(ad));
  else if constexpr (MT == 2)
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:4096\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(r0), "=&v"(r1) : "v"(ad));
  else
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r0) : "v"(ad));
  ah[0] = __builtin_bit_cast(half8v_t, r0);
  if constexpr (MT > 1) ah[1] = __builtin_bit_cast(half8v_t, r1);
  if constexpr (MT > 2) ah[2] = __builtin_bit_cast(half8v_t, r2);
  if constexpr (MT > 3) ah[3] = __builtin_bit_cast(half8v_t, r3);
}

// The MFMAs of one 64-k step: 4 k-steps of 16 over the step's 2 chunks; the
// A fragments of k-step i + 1 are read while those of k-step i are in use.
template <int F, int MT>
__device__ __forceinline__ void step_mma(f16v_t (&acc)[MT][2], const BStage<F>& st, uint32_t abuf, int col,
                                         int hsel) {
  half2v s16[2], b2[2];
  float mxs[2][2];   // MXFP4: block scale per n-tile and chunk
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if constexpr (F == F_MX4) {
      mxs[nt][0] = e8m0_to_f(st.sr[nt] & 0xFFu);
      mxs[nt][1] = e8m0_to_f((st.sr[nt] >> 8) & 0xFFu);
      continue;
    }
    float sc, bi;
    if constexpr (Fmt<F>::AFF) {
      sc = bf16_to_f(st.sr[nt] & 0xFFFFu);
      bi = bf16_to_f(st.sr[nt] >> 16);
    } else {
      sc = f16_bits_to_f(st.sr[nt] & 0xFFFFu);
      bi = 0.f;
    }
    const f16 sh = (f16)((float)Fmt<F>::M * sc), bh = (f16)bi;   // M s: pairs hold 1 + q/M
    s16[nt] = {sh, sh};
    b2[nt] = {bh, bh};
  }
  half8v_t ah[2][MT];
  read_a<F, MT>(ah[0], abuf, 0, col, hsel);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = i >> 1, j = i & 1;
    if (i + 1 < 4) read_a<F, MT>(ah[(i + 1) & 1], abuf, i + 1, col, hsel);
    half8v_t bf[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      uint32_t d[4];
      if constexpr (F == F_MX4) deq_word_mx(st.w[nt][c][j], mxs[nt][c], d);
      else if constexpr (BFrag<F>::HALF) deq_word<F>(&st.w[nt][c][j], s16[nt], b2[nt], d);
      else deq_chunk_half<F>(st.w[nt][c], 2 * j + hsel, s16[nt], b2[nt], d);
      bf[nt] = __builtin_bit_cast(half8v_t, *reinterpret_cast<uint4*>(d));
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i & 1][mt], bf[nt], acc[mt][nt], 0, 0, 0);
  }
}

// One item: rows [m0, m0 + mc) of expert e's run (mc <= 32 MT), column
// block nb (wave w: layout tile 4 nb + w). K in steps of 64: at step t the
// A and B loads of step t + 1 go out (past the last step, the last step's
// loads again, unused), then the wave waits until its own loads of step t
// have landed (at most the loads of step t + 1 in flight: the count is exact
// because every load here is one known instruction), and a bare barrier
// makes every wave's part of the stage visible and tells that every wave has
// finished step t - 1 (so the stage of step t - 2, which the loads of step
// t + 1 refill, is no longer read). __syncthreads would add a release fence,
// which waits for every load to LDS in flight, the prefetched stage
// included.
template <int F, int MODE, int MT, int BW>
__device__ __forceinline__ void gemm_item(const GroupedArgs& a, int e, int m0, int mc, int nb, uint8_t* const (&stg)[NST],
                                          int* slot_l) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = a.k, H = a.H;
  const bool shared = e == a.E;
  const ExpertClass& ec = shared ? a.sh : a.rt;
  const int K = MODE == GU ? H : ec.inter;   // contraction length
  const int T = nb * 4 + w;                  // this wave's layout tile
  const uint8_t* blk = a.base + ec.base_off + (shared ? 0 : (uint64_t)e * ec.stride);
  const uint32_t codes = (uint32_t)(MODE == GU ? ec.gu_codes : ec.dn_codes);
  const uint32_t scales = (uint32_t)(MODE == GU ? ec.gu_scales : ec.dn_scales);
  const int nch = K / 32, nkb = K / KBLK;
  const int col = lane & 31, hsel = lane >> 5;
  // A rows staged by this thread (rows past mc repeat the last row; their
  // results are not stored)
  const uint16_t* asrc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int q = 256 * i + tid;
    const int rr = q >> 3, pos = q & 7;
    const int rowc = min(rr, mc - 1);
    const int slot = a.perm[m0 + rowc];
    if (pos == 0) slot_l[rr] = slot;
    const uint16_t* src;
    if constexpr (MODE == GU) src = a.x16 + (uint64_t)(slot / (k + 1)) * H;
    else src = a.hbuf + (uint64_t)(m0 + rowc) * a.Imax;
    asrc[i] = src + 8 * (pos ^ swz(rr));
  }
  f16v_t acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][n][v] = 0.f;
  const int steps = K / 64;   // a multiple of 4 (K is a multiple of 256)
  uint8_t* bw[NST];
#pragma unroll
  for (int q = 0; q < NST; ++q) bw[q] = stg[q] + 2 * A_STAGE + BW * w;
  issue_a<MT>(asrc, reinterpret_cast<uint16_t*>(stg[0]), w, 0);
  issue_b<F>(bw[0], blk, codes, scales, T, nch, nkb, lane, 0);
  for (int base = 0; base < steps; base += NST) {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int t = base + s;
      if (t >= steps) break;
      const int tn = min(t + 1, steps - 1);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      issue_a<MT>(asrc, reinterpret_cast<uint16_t*>(stg[(s + 1) % NST]), w, tn);
      issue_b<F>(bw[(s + 1) % NST], blk, codes, scales, T, nch, nkb, lane, tn);
      asm volatile("" ::: "memory");
      wait_vm<MT + b_loads<F>()>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      BStage<F> bs;
      read_b<F>(bs, lds_addr(bw[s]), col, hsel, t);
      step_mma<F, MT>(acc, bs, lds_addr(stg[s]), col, hsel);
    }
  }
  wait_vm<0>();   // the repeated loads past the last step have landed before the stages are reused
  // ---- epilogue (slot indexes of the tile's rows from LDS; 32-bit offsets:
  // positions < R (k+1) <= 589824 and Imax, H <= 4096 keep them below 2^32)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 32 * mt + 8 * (v / 4) + 4 * hsel + (v % 4);
      if (row >= mc) continue;
      const uint32_t pos = (uint32_t)(m0 + row);
      if constexpr (MODE == GU) {
        const float g = acc[mt][0][v], u = acc[mt][1][v];
        // silu(g) u with the hardware exp and reciprocal (h is rounded to fp16)
        const float hv = g * __frcp_rn(1.0f + __expf(-g)) * u;
        const uint32_t j = 32 * T + col;
        a.hbuf[pos * (uint32_t)a.Imax + j] = __builtin_bit_cast(uint16_t, (f16)hv);
        if (a.tap_gu || a.tap_h) {
          const uint64_t s = (uint64_t)slot_l[row];
          if (a.tap_gu) {
            a.tap_gu[(s * 2 + 0) * a.Imax + j] = g;
            a.tap_gu[(s * 2 + 1) * a.Imax + j] = u;
          }
          if (a.tap_h) a.tap_h[s * a.Imax + j] = hv;
        }
      } else {
        const uint32_t s = (uint32_t)slot_l[row];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const uint32_t c = 64 * T + 32 * n + col;
          a.e_ws[s * (uint32_t)H + c] = acc[mt][n][v];
          if (a.tap_e) a.tap_e[(uint64_t)s * H + c] = acc[mt][n][v];
        }
      }
    }
  }
}

template <int F, int MODE, int BW>
__device__ __forceinline__ void gemm_item_mt(const GroupedArgs& a, int e, int m0, int mc, int nb,
                                             uint8_t* const (&stg)[NST], int* slot_l) {
  switch ((mc + 31) >> 5) {
    case 4: gemm_item<F, MODE, 4, BW>(a, e, m0, mc, nb, stg, slot_l); break;
    case 3: gemm_item<F, MODE, 3, BW>(a, e, m0, mc, nb, stg, slot_l); break;
    case 2: gemm_item<F, MODE, 2, BW>(a, e, m0, mc, nb, stg, slot_l); break;
    default: gemm_item<F, MODE, 1, BW>(a, e, m0, mc, nb, stg, slot_l); break;
  }
}

// Workgroups per CU the LDS ring allows (two when three stages fit twice).
template <int FR, int FS> constexpr int gemm_wg_per_cu() {
  return 2 * (NST * stage_bytes<FR, FS>() + 1024) <= 160 * 1024 ? 2 : 1;
}

// Persistent workgroups: each takes items q = (M-tile q / nblk, column block
// q % nblk) from the queue counter until the list is done. The work list is
// ordered by tile height, so the long items start first.
template <int FR, int FS, int MODE>
__global__ __launch_bounds__(256, (gemm_wg_per_cu<FR, FS>())) void k_grp_gemm(GroupedArgs a) {
  constexpr int SB = stage_bytes<FR, FS>(), BW = stage_b_wave<FR, FS>();
  __shared__ __align__(16) uint8_t stg0[SB];
  __shared__ __align__(16) uint8_t stg1[SB];
  __shared__ __align__(16) uint8_t stg2[SB];
  uint8_t* const stg[NST] = {stg0, stg1, stg2};
  __shared__ int slot_l[128];
  __shared__ int s_item[2];
  int* ctr = a.meta + (MODE == GU ? 1 : 2);
  const int nlt_max = MODE == GU ? 2 * a.Imax / 64 : a.H / 64;   // layout tiles along N (widest class)
  const int nblk = (nlt_max + 3) / 4;
  const int n_items = a.meta[0] * nblk;
  int par = 0;
  for (;;) {
    if (threadIdx.x == 0) s_item[par] = atomicAdd(ctr, 1);
    __syncthreads();
    const int q = s_item[par];
    par ^= 1;
    if (q >= n_items) break;
    const int* t = a.tiles + 3 * (q / nblk);
    const int nb = q % nblk;
    const int e = t[0], m0 = t[1], mc = t[2];
    if (e < 0 || e > a.E || mc <= 0) continue;
    const bool shared = e == a.E;
    const int I = shared ? a.sh.inter : a.rt.inter;
    const int nlt = MODE == GU ? 2 * I / 64 : a.H / 64;
    if (nb * 4 >= nlt) continue;
    if (shared) gemm_item_mt<FS, MODE, BW>(a, e, m0, mc, nb, stg, slot_l);
    else gemm_item_mt<FR, MODE, BW>(a, e, m0, mc, nb, stg, slot_l);
  }
}

// ------------------------------------------------------------------ combine
// y = sum_j p_j e_j + sigma e_shared, slots in pick order; 4 columns per
// thread (16-byte loads of the slot outputs).
__global__ __launch_bounds__(256) void k_grp_combine(GroupedArgs a) {
  const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;   // 4-column group
  const int H = a.H, k = a.k, H4 = H / 4;
  if (i >= (uint64_t)a.R * H4) return;
  const int r = (int)(i / H4), n = (int)(i % H4) * 4;
  const float* e = a.e_ws + (uint64_t)r * (k + 1) * H + n;
  float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    // a slot whose id is outside [0, E) has no expert output (the sort
    // skipped it): it adds nothing, as in the decode form
    const int id = a.ids[r * k + j];
    if (id < 0 || id >= a.E) continue;
    const float pj = a.p[r * k + j];
    const float4 v = *reinterpret_cast<const float4*>(e + (uint64_t)j * H);
    y.x = fmaf(pj, v.x, y.x);
    y.y = fmaf(pj, v.y, y.y);
    y.z = fmaf(pj, v.z, y.z);
    y.w = fmaf(pj, v.w, y.w);
  }
  const float sg = a.sg[r];
  const float4 v = *reinterpret_cast<const float4*>(e + (uint64_t)k * H);
  y.x = fmaf(sg, v.x, y.x);
  y.y = fmaf(sg, v.y, y.y);
  y.z = fmaf(sg, v.z, y.z);
  y.w = fmaf(sg, v.w, y.w);
  *reinterpret_cast<float4*>(a.y + (uint64_t)r * H + n) = y;
}

// ------------------------------------------------------------------ launch
static int gemm_grid(int wg_per_cu) {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256 * wg_per_cu;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev] * wg_per_cu;
}

hipError_t launch_grp_sort(const GroupedArgs& a, hipStream_t s, hipEvent_t* ev) {
  launch_k(k_grp_sort, dim3(1), dim3(1024), 0, s, ev, 0, a);
  return hipGetLastError();
}

template <int FR, int FS>
static hipError_t launch_grouped_t(const GroupedArgs& a, hipStream_t s, hipEvent_t* ev) {
  // sort workgroup, plus conversion workgroups for bf16 activations
  const uint64_t n8 = (uint64_t)a.R * a.H / 8;
  const int nconv = a.act_fp16 ? 0 : (int)std::min<uint64_t>(256, (n8 + 1023) / 1024);
  launch_k(k_grp_sort, dim3(1 + nconv), dim3(1024), 0, s, ev, 0, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int G = gemm_grid(gemm_wg_per_cu<FR, FS>());
  launch_k(k_grp_gemm<FR, FS, GU>, dim3(G), dim3(256), 0, s, ev, 2, a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  launch_k(k_grp_gemm<FR, FS, DN>, dim3(G), dim3(256), 0, s, ev, 4, a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const uint64_t n = (uint64_t)a.R * (a.H / 4);
  launch_k(k_grp_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ev, 6, a);
  return hipGetLastError();
}

// Routed / shared format pairs the grouped GEMMs read (grouped_pair_supported):
// the 3- and 4-bit formats in any pairing, the other widths with a shared
// expert of the same width or 4-bit affine.
template <int FR>
static hipError_t launch_grouped_s(int fs, const GroupedArgs& a, hipStream_t s, hipEvent_t* ev) {
  if constexpr (FR == F_Q4 || FR == F_Q3 || FR == F_S4) {
    switch (fs) {
      case F_Q4: return launch_grouped_t<FR, F_Q4>(a, s, ev);
      case F_Q3: return launch_grouped_t<FR, F_Q3>(a, s, ev);
      case F_S4: return launch_grouped_t<FR, F_S4>(a, s, ev);
    }
  } else {
    if (fs == FR) return launch_grouped_t<FR, FR>(a, s, ev);
    if (fs == F_Q4) return launch_grouped_t<FR, F_Q4>(a, s, ev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_grouped(int fr, int fs, const GroupedArgs& a, hipStream_t s, hipEvent_t* ev) {
  switch (fr) {
    case F_Q4: return launch_grouped_s<F_Q4>(fs, a, s, ev);
    case F_Q3: return launch_grouped_s<F_Q3>(fs, a, s, ev);
    case F_S4: return launch_grouped_s<F_S4>(fs, a, s, ev);
    case F_Q2: return launch_grouped_s<F_Q2>(fs, a, s, ev);
    case F_Q5: return launch_grouped_s<F_Q5>(fs, a, s, ev);
    case F_Q6: return launch_grouped_s<F_Q6>(fs, a, s, ev);
    case F_Q8: return launch_grouped_s<F_Q8>(fs, a, s, ev);
    case F_MX4: return launch_grouped_s<F_MX4>(fs, a, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
