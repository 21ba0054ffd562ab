// Grouped (prompt-chunk) path: the prefill form for chunks of many rows.
//
//  1. k_grp_sort (one workgroup): expert histogram of the picks, exclusive
//     prefix scan, scatter of the slots (row r, pick j) into
//     expert-major order; the shared expert follows as expert E with every
//     row. Then the tile lists: experts with many rows get 128-row M-tiles,
//     the rest 32-row M-tiles (the Zipf-skewed chunk has one hot expert
//     with most rows and a long tail of small ones).
//  2. k_grp_gemm<GU>: per (M-tile, 256-column block) a workgroup of 4 waves;
//     wave w owns one 64-row layout tile of the gate/up matrix (32 gate rows
//     + the 32 up rows of the same intermediate indices), so gate and up of
//     an output land in the same lane and SwiGLU runs in registers. A (the
//     activations of the tile's slots, gathered by the sort's permutation)
//     is staged through LDS as fp16; B (the packed codes) goes from memory
//     straight to registers and is dequantised there to fp16
//     (affine: s*q + b; symmetric: s*(u - 8)); v_mfma_f32_32x32x16_f16
//     accumulates in fp32. Output h in fp16, expert-major. The 128-row and
//     32-row tile lists share one launch, so the few large tiles (the shared
//     expert, hot experts) run beside the many small ones.
//  3. k_grp_gemm<DN>: the same on h and the down matrices; output e in fp32
//     in slot order.
//  4. k_grp_combine: y = sum_j p_j e_j + sigma e_shared, slots in pick order.
// ("Sage-A1.5 ... #1329", Proposal: grouped MoE and XMX prompt chunks;
//  Limits to agree on: the grouped form has a different sum order than the
//  per-row form, so it is judged by tolerance, not bits.)
#include "moe_kernels.h"
#include "moe_launch.h"
#include "moe_dispatch.h"

namespace moe {

typedef f16 half8v_t __attribute__((ext_vector_type(8)));
typedef float f16v_t __attribute__((ext_vector_type(16)));

constexpr int BIG_MIN_ROWS = 96;   // experts with at least this many rows take 128-row tiles

// meta layout (int32): [0] n_big, [1] n_small, [2 .. E+3) offsets (E+2 entries)
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

// One workgroup of 1024 threads (16 waves). Wave w owns the contiguous slot
// range [w S, (w+1) S), S = ceil(R k / 16), read 1024 slots at a time:
//  1. per-wave expert histograms (LDS atomics on the wave's own row);
//  2. exclusive scan over the experts (shared expert E with every row), then
//     each wave's base per expert: the offset plus the earlier waves' counts;
//  3. the same walk again scatters each slot (row r, pick j) to the position
//     its atomic increment of the wave's counter returns. Rows of one expert
//     stay within the wave's range in slot order only up to the order the
//     hardware serves one instruction's lanes; a row's output does not depend
//     on its position in a tile, so results are the same either way;
//  4. the tile lists: experts with many rows get 128-row M-tiles, the rest
//     32-row M-tiles (the Zipf-skewed chunk has one hot expert with most rows
//     and a long tail of small ones), each list laid out by a scan over the
//     experts' tile counts.
__global__ __launch_bounds__(1024) void k_grp_sort(GroupedArgs a) {
  __shared__ int cnt[320];
  __shared__ int off[320];
  __shared__ int tb[320], ts[320];       // tiles per expert (big / small lists), then their offsets
  __shared__ int wh[16][258];            // per-wave counts, then per-wave running positions
  __shared__ int s_tot[2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int E = a.E, k = a.k, R = a.R, nslot = R * k;
  const int S = (nslot + 15) / 16, s0 = w * S, s1 = min(nslot, s0 + S);
  for (int q = tid; q < 16 * 258; q += 1024) (&wh[0][0])[q] = 0;
  __syncthreads();
  // 1. histograms: the picks of 16 rounds are loaded at once (one latency
  // per 1024 slots of a wave)
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
    const bool big = c >= BIG_MIN_ROWS;
    tb[e] = big ? (c + 127) / 128 : 0;
    ts[e] = big ? 0 : (c + 31) / 32;
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
  // 4. tile lists: entry = (expert, first position, rows)
  if (w == 0) {
    const int nb = wave_exclusive_scan(tb, tb, E + 1, lane);
    if (lane == 0) s_tot[0] = nb;
  } else if (w == 1) {
    const int ns = wave_exclusive_scan(ts, ts, E + 1, lane);
    if (lane == 0) s_tot[1] = ns;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += 1024) {
    const int c = cnt[e];
    if (c == 0) continue;
    const bool big = c >= BIG_MIN_ROWS;
    const int bm = big ? 128 : 32;
    int* t = big ? a.tiles + 3 * tb[e] : a.tiles + 3 * (a.max_tiles + ts[e]);
    for (int m0 = 0; m0 < c; m0 += bm, t += 3) {
      t[0] = e;
      t[1] = off[e] + m0;
      t[2] = min(bm, c - m0);
    }
  }
  if (tid == 0) {
    a.meta[0] = s_tot[0];
    a.meta[1] = s_tot[1];
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

// For the 3-bit layout, the 8 codes k = 8v..8v+7 of a chunk (v = 0..3) sit
// in pairs 4v..4v+3; the chunk's full unpack gives them.
template <int F>
__device__ __forceinline__ void deq_chunk_half(const uint32_t* cw, int wsel, half2v s16, half2v b2,
                                               uint32_t* o) {
  if constexpr (F == F_Q3) {
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

constexpr int AST = 72;    // LDS row stride of the A tile in halves (64 + 8 pad)

// 4-bit codes: the lane of half hsel takes words 2 hsel, 2 hsel + 1 of each
// chunk row (8 contiguous bytes), i.e. k = 16 hsel .. 16 hsel + 15 of the
// chunk, and the A fragments follow the same k. The 3-bit rows hold a
// chunk's codes across all 3 words, so their lanes load the full row.
template <int F> struct BFrag {
  static constexpr bool HALF = F == F_Q4 || F == F_S4;
  static constexpr int W = HALF ? 2 : Fmt<F>::WORDS;   // words per chunk per lane
};

// One pipeline stage: the A segments a thread stages, the code words and
// the scale word (per n-tile) of the wave's layout tile for one 64-k step.
template <int F, int SPT>
struct GrpStage {
  uint4 av[SPT];
  uint32_t bw[2][2][BFrag<F>::W];
  uint32_t sr[2];
};

template <int F, int SPT>
__device__ __forceinline__ void grp_issue(GrpStage<F, SPT>& st, const uint16_t* const (&arow)[SPT],
                                          const int (&aseg)[SPT], const uint8_t* codes, const uint8_t* scales,
                                          int T, int nch, int nkb, int col, int hsel, int kk0) {
  constexpr int GPS = KBLK / Fmt<F>::G;
#pragma unroll
  for (int q = 0; q < SPT; ++q) st.av[q] = *reinterpret_cast<const uint4*>(arow[q] + kk0 + 8 * aseg[q]);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint8_t* blk = codes + chunk_off<F>(T, kk0 / 32 + c, nch);
      if constexpr (BFrag<F>::HALF) {
        const uint2 v = *reinterpret_cast<const uint2*>(blk + (32 * nt + col) * Fmt<F>::CB + 8 * hsel);
        st.bw[nt][c][0] = v.x;
        st.bw[nt][c][1] = v.y;
      } else {
        load_chunk<F>(blk, 32 * nt + col, st.bw[nt][c]);
      }
    }
  const int gi = (kk0 % KBLK) / Fmt<F>::G;
  const uint8_t* sblk = scales + sblk_off<F>(T, kk0 / KBLK, nkb);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if constexpr (Fmt<F>::AFF) st.sr[nt] = reinterpret_cast<const uint32_t*>(sblk)[(32 * nt + col) * GPS + gi];
    else st.sr[nt] = reinterpret_cast<const uint16_t*>(sblk)[(32 * nt + col) * GPS + gi];
  }
}

// A segments of a stage into one LDS buffer (bf16 -> fp16 on the way: exact
// for |x| in fp16's normal range)
template <int MODE, int ACT16, int SPT>
__device__ __forceinline__ void grp_store_a(const uint4 (&av)[SPT], uint16_t* buf, const int (&arr)[SPT],
                                            const int (&aseg)[SPT]) {
#pragma unroll
  for (int q = 0; q < SPT; ++q) {
    uint4 v = av[q];
    if constexpr (MODE == GU && !ACT16) {
      uint32_t* u = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        half2v h;
        h.x = (f16)bf16_to_f(u[i] & 0xFFFFu);
        h.y = (f16)bf16_to_f(u[i] >> 16);
        u[i] = as_u(h);
      }
    }
    *reinterpret_cast<uint4*>(buf + arr[q] * AST + 8 * aseg[q]) = v;
  }
}

// The MFMAs of one 64-k step: 4 k-steps of 16 over the step's 2 chunks; the
// A fragments of a k-step are read from LDS ahead of the dequantisation.
template <int F, int MT, int SPT>
__device__ __forceinline__ void grp_mma(f16v_t (&acc)[MT][2], const GrpStage<F, SPT>& st, const uint16_t* buf,
                                        int col, int hsel) {
  half2v s16[2], b2[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float sc, bi;
    if constexpr (Fmt<F>::AFF) {
      sc = bf16_to_f(st.sr[nt] & 0xFFFFu);
      bi = bf16_to_f(st.sr[nt] >> 16);
    } else {
      sc = f16_bits_to_f(st.sr[nt]);
      bi = 0.f;
    }
    const f16 sh = (f16)(16.0f * sc), bh = (f16)bi;
    s16[nt] = {sh, sh};
    b2[nt] = {bh, bh};
  }
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // k offset of this lane's 8 values inside the 64-k step
      const int koff = BFrag<F>::HALF ? 32 * c + 16 * hsel + 8 * j : 32 * c + 16 * j + 8 * hsel;
      half8v_t ah[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        ah[mt] = __builtin_bit_cast(half8v_t, *reinterpret_cast<const uint4*>(buf + (32 * mt + col) * AST + koff));
      half8v_t bf[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        uint32_t d[4];
        if constexpr (BFrag<F>::HALF) deq_word<F>(&st.bw[nt][c][j], s16[nt], b2[nt], d);
        else deq_chunk_half<F>(st.bw[nt][c], 2 * j + hsel, s16[nt], b2[nt], d);
        bf[nt] = __builtin_bit_cast(half8v_t, *reinterpret_cast<uint4*>(d));
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[mt], bf[nt], acc[mt][nt], 0, 0, 0);
    }
}

// One workgroup: (tile, column block of 4 layout tiles); wave w = layout tile.
// BM = 32 * MT rows. K walked in steps of 64 (two code chunks) through a ring
// of NS register stages: the loads of step t + NS - 1 are issued before the
// MFMAs of step t. The A tile alternates between two LDS buffers, so one
// barrier per step orders both the buffer's writes before its reads and the
// reads of step t - 1 before the writes of step t + 1.
template <int F, int MODE, int MT, int ACT16, int NS>
__device__ __forceinline__ void grp_tile(const GroupedArgs& a, const uint16_t* __restrict__ x,
                                         int e, int m0, int mc, int nb, uint16_t* lds_a, int* slot_l) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = a.k, H = a.H;
  const bool shared = e == a.E;
  const ExpertClass& ec = shared ? a.sh : a.rt;
  const int I = ec.inter;
  const int K = MODE == GU ? H : I;          // contraction length
  const int T = nb * 4 + w;                  // this wave's layout tile
  const uint8_t* blk = a.base + ec.base_off + (shared ? 0 : (uint64_t)e * ec.stride);
  const uint8_t* codes = blk + (MODE == GU ? ec.gu_codes : ec.dn_codes);
  const uint8_t* scales = blk + (MODE == GU ? ec.gu_scales : ec.dn_scales);
  const int nch = K / 32, nkb = K / KBLK;
  constexpr int BM = 32 * MT;
  // ---- A rows this thread stages: BM rows x 64 halves per step, as
  // (row, 8-half segment) pairs
  constexpr int SEGS = BM * 8;               // 8 halves per segment
  constexpr int SPT = SEGS / 256;            // segments per thread
  const uint16_t* arow[SPT];
  int aseg[SPT], arr[SPT];
#pragma unroll
  for (int q = 0; q < SPT; ++q) {
    const int sidx = tid + 256 * q;
    const int rr = sidx / 8, sg = sidx % 8;
    const int rowc = min(rr, mc - 1);
    const int slot = a.perm[m0 + rowc];
    if (sg == 0) slot_l[rr] = slot;       // the tile's slot indexes, for the epilogue
    const uint16_t* src;
    if constexpr (MODE == GU) src = x + (uint64_t)(slot / (k + 1)) * H;
    else src = a.hbuf + (uint64_t)(m0 + rowc) * a.Imax;
    arow[q] = src;
    aseg[q] = sg;
    arr[q] = rr;
  }
  f16v_t acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][nt][v] = 0.f;
  const int col = lane & 31, hsel = lane >> 5;
  // K is a multiple of 256, so the step count is a multiple of NS (2 or 4);
  // the prefetches past the last step re-read it (clamped, never used)
  const int steps = K / 64;
  GrpStage<F, SPT> st[NS];
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    grp_issue<F, SPT>(st[s], arow, aseg, codes, scales, T, nch, nkb, col, hsel, 64 * min(s, steps - 1));
  for (int base = 0; base < steps; base += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int step = base + s;
      uint16_t* buf = lds_a + (s & 1) * (BM * AST);
      grp_store_a<MODE, ACT16, SPT>(st[s].av, buf, arr, aseg);
      grp_issue<F, SPT>(st[(s + NS - 1) % NS], arow, aseg, codes, scales, T, nch, nkb, col, hsel,
                        64 * min(step + NS - 1, steps - 1));
      __syncthreads();
      grp_mma<F, MT, SPT>(acc, st[s], buf, col, hsel);
    }
  }
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
        for (int nt = 0; nt < 2; ++nt) {
          const uint32_t n = 64 * T + 32 * nt + col;
          a.e_ws[s * (uint32_t)H + n] = acc[mt][nt][v];
          if (a.tap_e) a.tap_e[(uint64_t)s * H + n] = acc[mt][nt][v];
        }
      }
    }
  }
}

// One launch for both tile lists, so the two run side by side: workgroups
// [0, nbig) take the 128-row list (tile wg / nblk, column block wg % nblk),
// the rest the 32-row list. Each list is sized for its worst case; the
// workgroups past a list's tile count exit at once.
template <int FR, int FS, int MODE, int MT, int ACT16>
__device__ __forceinline__ void grp_list(const GroupedArgs& a, const uint16_t* __restrict__ x, int list, int wg,
                                         uint16_t* lds_a, int* slot_l) {
  constexpr int NS = MT == 1 ? 4 : 2;        // pipeline stages
  const int nblk = a.gemm_nblk;
  const int ti = wg / nblk, nb = wg % nblk;
  const int ntiles = a.meta[list];
  if (ti >= ntiles) return;
  const int* t = a.tiles + 3 * (list ? a.max_tiles + ti : ti);
  const int e = t[0], m0 = t[1], mc = t[2];
  if (e < 0 || e > a.E || mc <= 0) return;
  const bool shared = e == a.E;
  const int I = shared ? a.sh.inter : a.rt.inter;
  const int nlt = MODE == GU ? 2 * I / 64 : a.H / 64;   // layout tiles of this expert along N
  if (nb * 4 >= nlt) return;
  if (shared) grp_tile<FS, MODE, MT, ACT16, NS>(a, x, e, m0, mc, nb, lds_a, slot_l);
  else grp_tile<FR, MODE, MT, ACT16, NS>(a, x, e, m0, mc, nb, lds_a, slot_l);
}

template <int FR, int FS, int MODE, int ACT16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_grp_gemm(GroupedArgs a, const uint16_t* __restrict__ x, int nbig) {
  __shared__ __align__(16) uint16_t lds_a[2 * 128 * AST];
  __shared__ int slot_l[128];
  const int wg = blockIdx.x;
  if (wg < nbig) grp_list<FR, FS, MODE, 4, ACT16>(a, x, 0, wg, lds_a, slot_l);
  else grp_list<FR, FS, MODE, 1, ACT16>(a, x, 1, wg - nbig, lds_a, slot_l);
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
template <int FR, int FS, int MODE, int ACT16>
static hipError_t launch_gemm(const GroupedArgs& a, hipStream_t s, int nblk, hipEvent_t* ev, int i) {
  GroupedArgs b = a;
  b.gemm_nblk = nblk;
  // upper bounds of the two lists: every expert's rows split in tiles; an
  // expert of c >= 96 rows takes ceil(c / 128) <= c / 128 + c / 96 tiles
  const int slots = a.R * (a.k + 1);
  const int max_big = slots / 128 + slots / BIG_MIN_ROWS + 1;
  const int max_small = slots / 32 + a.E + 1;
  const int nbig = max_big * nblk;
  launch_k(k_grp_gemm<FR, FS, MODE, ACT16>, dim3(nbig + max_small * nblk), dim3(256), 0, s, ev, i, b, a.x, nbig);
  return hipGetLastError();
}

template <int FR, int FS, int ACT16>
static hipError_t launch_grouped_t(const GroupedArgs& a, hipStream_t s, hipEvent_t* ev) {
  const int Imax = a.Imax;
  launch_k(k_grp_sort, dim3(1), dim3(1024), 0, s, ev, 0, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_gemm<FR, FS, GU, ACT16>(a, s, (2 * Imax / 64 + 3) / 4, ev, 2);
  if (err != hipSuccess) return err;
  err = launch_gemm<FR, FS, DN, ACT16>(a, s, (a.H / 64 + 3) / 4, ev, 4);
  if (err != hipSuccess) return err;
  const uint64_t n = (uint64_t)a.R * (a.H / 4);
  launch_k(k_grp_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ev, 6, a);
  return hipGetLastError();
}

template <int FR, int FS>
static hipError_t launch_grouped_a(const GroupedArgs& a, hipStream_t s, hipEvent_t* ev) {
  return a.act_fp16 ? launch_grouped_t<FR, FS, 1>(a, s, ev) : launch_grouped_t<FR, FS, 0>(a, s, ev);
}

template <int FR>
static hipError_t launch_grouped_s(int fs, const GroupedArgs& a, hipStream_t s, hipEvent_t* ev) {
  switch (fs) {
    case F_Q4: return launch_grouped_a<FR, F_Q4>(a, s, ev);
    case F_Q3: return launch_grouped_a<FR, F_Q3>(a, s, ev);
    case F_S4: return launch_grouped_a<FR, F_S4>(a, s, ev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_grouped(int fr, int fs, const GroupedArgs& a, hipStream_t s, hipEvent_t* ev) {
  switch (fr) {
    case F_Q4: return launch_grouped_s<F_Q4>(fs, a, s, ev);
    case F_Q3: return launch_grouped_s<F_Q3>(fs, a, s, ev);
    case F_S4: return launch_grouped_s<F_S4>(fs, a, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
