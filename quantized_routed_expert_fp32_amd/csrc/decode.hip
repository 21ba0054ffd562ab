// Decode path: routed + shared experts for up to 16 independent rows.
//
// gate/up (k_dec_gateup): a persistent grid. A unit is an expert picked by
// some row, found from the picks as the first slot (row r, pick j) that
// holds it, or the shared expert for up to four rows (one pass of the
// matrix-core dots serves four rows at the cost of one); an item is (unit,
// 64-row tile of the interleaved gate/up matrix). Workgroup b takes items b, b + G, ...;
// wave w owns the 256-wide K slice w, one weight row per lane, and streams
// the tile's packed codes once (coalesced 128-bit loads) for every row that
// picked the expert, so rows sharing an expert share its reads ("Native
// server: --backend xpu for Nemotron on Intel Arc", review comments: each
// extra row costs more because more distinct experts are read). The dots
// run on 4x4x4 MFMAs, up to four rows per pass. The codes
// and scale words of the next item are in flight while the current one is
// computed. The activations of all rows sit in LDS (loaded once per
// workgroup) with their 32-wide chunk sums. Output: h = silu(g)*u split into
// fp16 hi + lo parts (22 significant bits) plus per-32 chunk sums, for down.
//
// down + combine (k_dec_down): one workgroup per (row, 64-column tile of y)
// with KS waves per routed slot, each over 1/KS of the intermediate axis,
// plus a share of the shared expert's groups. Each wave loads the part of
// the row's h it reads ahead of its weights and stages it in its own LDS
// area, so it computes as soon as its own loads have landed; the dots run
// on 4x4x4 MFMAs with the hi and lo parts as two rows of one pass. The slot
// parts are added in part order, the shared parts in wave order; wave 0
// forms y = sum_j p_j e_j + sigma e_shared in slot order. Blocks are mapped
// so the rows of one tile run on one XCD and share expert tiles in its L2.
//
// Every row's arithmetic is fixed (K slices owned by fixed waves, chunks and
// groups in K order, slices reduced in slice order, slots combined in pick
// order, shared last; an MFMA output element is formed from its own row slot
// and column alone, whichever slot holds the row) and independent of the
// other rows, so a row's y is bit-identical alone or in a batch ("Sage-A1.5
// ... #1329", Limits to agree on: the per-row kernels keep one stream's sum
// order).
#include "moe_kernels.h"
#include "moe_launch.h"
#include "moe_dispatch.h"

#include <algorithm>

namespace moe {

// Codes (8 chunks of one K slice, W words each) and scale words of one lane.
template <int W>
struct SliceBuf {
  uint32_t w[8][W];
  uint32_t sc[4];
};

// Codes and scale words of K slice sl of tile t of a matrix in the range
// behind r (codes / scales: byte offsets of the matrix's parts in it).
template <int F, typename SB>
__device__ __forceinline__ void load_slice(rsrc_t r, uint32_t codes, uint32_t scales, int t, int sl, int nch,
                                           int nkb, int lane, SB& b) {
  const uint32_t vc = chunk_voff<F>(lane), vs = scale_voff<F>(lane);
  // scale words first: group 0's arithmetic then waits only for its chunks
  load_scales_rs<F>(r, vs, scales + (uint32_t)sblk_off<F>(t, sl, nkb), b.sc);
#pragma unroll
  for (int cc = 0; cc < 8; ++cc)
    load_chunk_rs<F>(r, vc, codes + (uint32_t)chunk_off<F>(t, sl * 8 + cc, nch), b.w[cc]);
}

// The picks seen by one wave: lane l holds slots l and l + 64.
struct Picks {
  int id0, id1;
  bool first0, first1;   // the slot is the first to hold its expert
  int rank0, rank1;      // its unit index among the first slots
  int nrt;               // routed units
};

// Slot lanes holding the same expert, from one ballot per id bit (ids < 256).
__device__ __forceinline__ Picks find_units(int id0, int id1, int E, int lane) {
  Picks P;
  P.id0 = id0;
  P.id1 = id1;
  const bool v0 = P.id0 >= 0 && P.id0 < E, v1 = P.id1 >= 0 && P.id1 < E;
  uint64_t M0 = __ballot(v0), N0 = __ballot(v1), M1 = M0, N1 = N0;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool b0 = (P.id0 >> b) & 1, b1 = (P.id1 >> b) & 1;
    const uint64_t B0 = __ballot(v0 && b0), B1 = __ballot(v1 && b1);
    M0 &= b0 ? B0 : ~B0;
    N0 &= b0 ? B1 : ~B1;
    M1 &= b1 ? B0 : ~B0;
    N1 &= b1 ? B1 : ~B1;
  }
  (void)N0;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  P.first0 = v0 && (M0 & lt) == 0;
  P.first1 = v1 && M1 == 0 && (N1 & lt) == 0;
  const uint64_t F0 = __ballot(P.first0), F1 = __ballot(P.first1);
  P.rank0 = __popcll(F0 & lt);
  P.rank1 = __popcll(F0) + __popcll(F1 & lt);
  P.nrt = __popcll(F0) + __popcll(F1);
  return P;
}

// Expert of routed unit u (uniform).
__device__ __forceinline__ int unit_expert(const Picks& P, int u) {
  const uint64_t s0 = __ballot(P.first0 && P.rank0 == u);
  if (s0) return __builtin_amdgcn_readlane(P.id0, __ffsll((unsigned long long)s0) - 1);
  const uint64_t s1 = __ballot(P.first1 && P.rank1 == u);
  return __builtin_amdgcn_readlane(P.id1, __ffsll((unsigned long long)s1) - 1);
}

constexpr int GU_SHARED_ROWS = 4;   // rows per shared-expert unit (one pass)

struct GuItem {
  rsrc_t r;     // the expert block
  uint32_t codes, scales;   // gate/up codes and scale words inside it
  int t;        // layout tile (64 rows: 32 gate + 32 up)
  int tl;       // tile actually loaded (t clamped into the class)
  int shared;
  int e;        // expert (routed) or the shared unit (rows 4e .. 4e + 3)
};

// What an item needs of its expert class, read once from the arguments and
// held in registers (opaque to the compiler, which would otherwise reload
// the argument block with a wait for each item's address).
struct GuCls {
  uint64_t base_off, stride;
  uint32_t codes, scales, blk_bytes;
  int tlast;   // last gate/up tile of the class
};
__device__ __forceinline__ GuCls gu_cls(const ExpertClass& c) {
  GuCls g;
  g.base_off = c.base_off;
  g.stride = c.stride;
  g.codes = (uint32_t)c.gu_codes;
  g.scales = (uint32_t)c.gu_scales;
  g.blk_bytes = c.blk_bytes;
  g.tlast = 2 * c.inter / 64 - 1;
  asm volatile("" : "+s"(g.base_off), "+s"(g.stride), "+s"(g.codes), "+s"(g.scales), "+s"(g.blk_bytes),
               "+s"(g.tlast));
  return g;
}

__device__ __forceinline__ GuItem gu_item(const uint8_t* base, const GuCls& rc, const GuCls& sc, const Picks& P,
                                          int item, int Tmax) {
  GuItem it;
  const int u = item / Tmax;
  it.t = item % Tmax;
  it.shared = u >= P.nrt;
  it.e = it.shared ? u - P.nrt : unit_expert(P, u);
  const uint64_t off = it.shared ? sc.base_off : rc.base_off + (uint64_t)it.e * rc.stride;
  it.r = make_rsrc(base + off, it.shared ? sc.blk_bytes : rc.blk_bytes);
  it.codes = it.shared ? sc.codes : rc.codes;
  it.scales = it.shared ? sc.scales : rc.scales;
  it.tl = min(it.t, it.shared ? sc.tlast : rc.tlast);
  return it;
}

template <int FR, int FS, typename SB>
__device__ __forceinline__ void gu_issue(const GuItem& it, int wv, int nch, int nkb, int lane, SB& b) {
  if constexpr (FR == FS) {
    load_slice<FR>(it.r, it.codes, it.scales, it.tl, wv, nch, nkb, lane, b);
  } else {
    if (it.shared) load_slice<FS>(it.r, it.codes, it.scales, it.tl, wv, nch, nkb, lane, b);
    else load_slice<FR>(it.r, it.codes, it.scales, it.tl, wv, nch, nkb, lane, b);
  }
}

// Up to 4 rows of an item against the wave's K slice on the matrix cores.
// v_mfma_f32_4x4x4 (16 blocks): B = the weights, lane l = weight row l
// (block l/4, column l%4), 4 consecutive k per step from its own unpacked
// pairs; A = the activations, lane l supplies row slot l%4 of its block
// (every block sees the same rows); result register v of lane l = slot v's
// dot with weight row l. So each lane ends with its own row's dots for the
// four slots, and each output element is formed from its own row and slot
// alone. Per 64-wide group: acc = sum of the pair products over the group's
// chunks in k order, then out += ms*acc + bm*X (X: the group's activation
// sum), as the pair-dot form. xr: this lane's slot row in LDS; xs0..3: the
// four slots' rows of chunk sums.
typedef short s4v __attribute__((ext_vector_type(4)));
typedef _Float16 h4v __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));

template <int ACT16>
__device__ __forceinline__ f4v mfma4(uint32_t x0, uint32_t x1, uint32_t w0, uint32_t w1, f4v acc) {
  if constexpr (ACT16) {
    const h4v xa = __builtin_bit_cast(h4v, make_uint2(x0, x1));
    const h4v wb = __builtin_bit_cast(h4v, make_uint2(w0, w1));
    return __builtin_amdgcn_mfma_f32_4x4x4f16(xa, wb, acc, 0, 0, 0);
  } else {
    const s4v xa = __builtin_bit_cast(s4v, make_uint2(x0, x1));
    const s4v wb = __builtin_bit_cast(s4v, make_uint2(w0, w1));
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(xa, wb, acc, 0, 0, 0);
  }
}

template <int F, int ACT16, int W>
__device__ __forceinline__ f4v gu_slice_mfma(const uint32_t (*w)[W], const uint32_t* sc, const uint32_t* xr,
                                             const float* xs0, const float* xs1, const float* xs2,
                                             const float* xs3, int sl, f4v out) {
  constexpr int GPS = KBLK / Fmt<F>::G, CPG = Fmt<F>::G / 32;
  constexpr bool NIB = F == F_Q8 && !ACT16;   // two nibble sets, two sums
  const PairMasks pk = pair_masks<F, ACT16>();
#pragma unroll
  for (int gi = 0; gi < GPS; ++gi) {
    float ms, bm;
    coef_reg<F>(sc, gi, ms, bm);
    f4v acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
    float X0 = 0.f, X1 = 0.f, X2 = 0.f, X3 = 0.f;
#pragma unroll
    for (int cc = 0; cc < CPG; ++cc) {
      const int c = gi * CPG + cc;
      uint32_t v[16], av[16], wc[Fmt<F>::WORDS];
#pragma unroll
      for (int q = 0; q < Fmt<F>::WORDS; ++q) {
        wc[q] = w[c][q];
        // opaque to loop-invariant motion: the unpack stays beside its use
        // instead of being hoisted out of the pass loop for every chunk
        asm volatile("" : "+v"(wc[q]));
      }
      // two nibble sets: the low set's dots, then the high set unpacked into
      // the same registers (each accumulator keeps its order)
      if constexpr (NIB) unpack_q8_nibbles<0>(wc, pk, v);
      else unpack_pairs<F, ACT16>(wc, pk, v);
      const uint4* q = reinterpret_cast<const uint4*>(xr + (sl * KBLK + 32 * c) / 2);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 tq = q[u];
        av[4 * u] = tq.x; av[4 * u + 1] = tq.y; av[4 * u + 2] = tq.z; av[4 * u + 3] = tq.w;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = mfma4<ACT16>(av[2 * i], av[2 * i + 1], v[2 * i], v[2 * i + 1], acc);
      if constexpr (NIB) {
        unpack_q8_nibbles<1>(wc, pk, v);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          acc2 = mfma4<ACT16>(av[2 * i], av[2 * i + 1], v[2 * i], v[2 * i + 1], acc2);
      }
      X0 += xs0[sl * 8 + c];
      X1 += xs1[sl * 8 + c];
      X2 += xs2[sl * 8 + c];
      X3 += xs3[sl * 8 + c];
    }
    if constexpr (NIB) {
      // q = lo + 16 hi: s q + b = (ms/16)(1 + lo/16) + ms (1 + hi/16) + (bm - ms/16)
      const float m16 = ms * (1.0f / 16.0f), b16 = bm - m16;
      out[0] = fmaf(b16, X0, fmaf(ms, acc2[0], fmaf(m16, acc[0], out[0])));
      out[1] = fmaf(b16, X1, fmaf(ms, acc2[1], fmaf(m16, acc[1], out[1])));
      out[2] = fmaf(b16, X2, fmaf(ms, acc2[2], fmaf(m16, acc[2], out[2])));
      out[3] = fmaf(b16, X3, fmaf(ms, acc2[3], fmaf(m16, acc[3], out[3])));
    } else {
      out[0] = fmaf(bm, X0, fmaf(ms, acc[0], out[0]));
      out[1] = fmaf(bm, X1, fmaf(ms, acc[1], out[1]));
      out[2] = fmaf(bm, X2, fmaf(ms, acc[2], out[2]));
      out[3] = fmaf(bm, X3, fmaf(ms, acc[3], out[3]));
    }
  }
  return out;
}

// One wave after the barrier, for one row: g and u of the tile's 32
// intermediate indices (slices added in slice order), h = silu(g) u, split
// and stored.
__device__ __forceinline__ void gu_finish(const DecodeArgs& a, const float* red, int nw, int r, int j,
                                          int t, int lane) {
  const int k = a.k;
  const int c = lane & 31;
  float g = 0.f, u = 0.f;
  for (int q = 0; q < nw; ++q) {
    g += red[q * 64 + c];
    u += red[q * 64 + 32 + c];
  }
  const float hv = silu_mul(g, u);
  const f16 hi = (f16)hv, lo = (f16)(hv - (float)hi);
  // chunk sum of hi + lo over the 32 columns: 16-lane rows by DPP, then
  // the two rows in order (lanes 0..31 and 32..63 hold the same values)
  const float s16 = sum16((float)hi + (float)lo);
  const float sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 0)) +
                   __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 16));
  if (lane < 32) {
    const uint64_t rs = (uint64_t)r * (k + 1) + j;
    const int col = 32 * t + c;
    a.hhi[rs * a.Imax + col] = __builtin_bit_cast(uint16_t, hi);
    a.hlo[rs * a.Imax + col] = __builtin_bit_cast(uint16_t, lo);
    if (c == 0) a.hc[rs * (a.Imax / 32) + t] = sv;
    if (a.tap_gu) {
      a.tap_gu[(rs * 2 + 0) * a.Imax + col] = g;
      a.tap_gu[(rs * 2 + 1) * a.Imax + col] = u;
    }
    if (a.tap_h) a.tap_h[rs * a.Imax + col] = hv;
  }
}

__device__ __forceinline__ int pick4(int v, int a0, int a1, int a2, int a3) {
  return v == 0 ? a0 : v == 1 ? a1 : v == 2 ? a2 : a3;   // selects, not an indexed array (scratch)
}

// One pass: up to 4 rows of an item against the wave's K slices, the slice
// partials of every wave to LDS, one barrier, then wave v finishes the
// pass's slot v (with fewer waves than slots a wave finishes several). lr:
// the slots' rows in the LDS activation block (and their chunk-sum rows),
// rr / jj: the slots' rows and picks in the outputs; slots past m repeat
// slot 0 and their results are not used.
template <int F, int ACT16, typename SB>
__device__ __forceinline__ void gu_pass(const DecodeArgs& a, const GuItem& it, const SB& b, const uint32_t* xl,
                                        const float* cs, float* red, int& rb, int wv, int nw, int lane,
                                        const int (&lr)[4], const int (&rr)[4], const int (&jj)[4], int m) {
  const int H = a.H, nch = H / 32, nsl = H / KBLK;
  const int rl = pick4(lane & 3, lr[0], lr[1], lr[2], lr[3]);
  const uint32_t* xr = xl + (uint64_t)rl * (H / 2);
  const float *xs0 = cs + lr[0] * nch, *xs1 = cs + lr[1] * nch, *xs2 = cs + lr[2] * nch, *xs3 = cs + lr[3] * nch;
  f4v out = {0.f, 0.f, 0.f, 0.f};
  out = gu_slice_mfma<F, ACT16>(b.w, b.sc, xr, xs0, xs1, xs2, xs3, wv, out);
  for (int sl = wv + nw; sl < nsl; sl += nw) {     // hidden > 256 * waves: further slices in place
    SB c2;
    load_slice<F>(it.r, it.codes, it.scales, it.tl, sl, nch, nsl, lane, c2);
    out = gu_slice_mfma<F, ACT16>(c2.w, c2.sc, xr, xs0, xs1, xs2, xs3, sl, out);
  }
  float* rbuf = red + rb * (4 * nw * 64);
#pragma unroll
  for (int v = 0; v < 4; ++v)
    if (v < m) rbuf[(v * nw + wv) * 64 + lane] = out[v];
  __syncthreads();
  for (int v = wv; v < m; v += nw)    // fewer waves than slots: waves take several
    gu_finish(a, rbuf + v * nw * 64, nw, pick4(v, rr[0], rr[1], rr[2], rr[3]),
              pick4(v, jj[0], jj[1], jj[2], jj[3]), it.t, lane);
  rb ^= 1;   // the other buffer next: its readers passed this barrier
}

// gu_slice_mfma for NG groups of 4 rows at once (the exact chunk form):
// each chunk is unpacked once for every group, and each group's
// accumulators, chunk sums and folds are gu_slice_mfma's in its order, so
// every row's result is the same bit for bit. Group g's rows are LDS rows
// 4 g .. 4 g + 3 of the block (a row past m reads row 0; its results are
// not used); lane l supplies row slot l % 4.
template <int F, int ACT16, int W, int NG>
__device__ __forceinline__ void gu_slice_mfma_n(const uint32_t (*w)[W], const uint32_t* sc, const uint32_t* xl,
                                                const float* cs, int H, int m, int lane, int sl, f4v (&out)[NG]) {
  constexpr int GPS = KBLK / Fmt<F>::G, CPG = Fmt<F>::G / 32;
  constexpr bool NIB = F == F_Q8 && !ACT16;   // two nibble sets, two sums
  const int nch = H / 32;
  const PairMasks pk = pair_masks<F, ACT16>();
#pragma unroll
  for (int gi = 0; gi < GPS; ++gi) {
    float ms, bm;
    coef_reg<F>(sc, gi, ms, bm);
    f4v acc[NG], acc2[NG];
    float X[NG][4];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[g][i] = 0.f;
        acc2[g][i] = 0.f;
        X[g][i] = 0.f;
      }
#pragma unroll
    for (int cc = 0; cc < CPG; ++cc) {
      const int c = gi * CPG + cc;
      uint32_t v[NIB ? 32 : 16], wc[Fmt<F>::WORDS];
#pragma unroll
      for (int q = 0; q < Fmt<F>::WORDS; ++q) {
        wc[q] = w[c][q];
        asm volatile("" : "+v"(wc[q]));
      }
      unpack_pairs<F, ACT16>(wc, pk, v);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int lr = 4 * g + (lane & 3);
        const uint32_t* xr = xl + (uint64_t)(lr < m ? lr : 0) * (H / 2);
        const uint4* q = reinterpret_cast<const uint4*>(xr + (sl * KBLK + 32 * c) / 2);
        uint32_t av[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 tq = q[u];
          av[4 * u] = tq.x; av[4 * u + 1] = tq.y; av[4 * u + 2] = tq.z; av[4 * u + 3] = tq.w;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
          acc[g] = mfma4<ACT16>(av[2 * i], av[2 * i + 1], v[2 * i], v[2 * i + 1], acc[g]);
        if constexpr (NIB) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            acc2[g] = mfma4<ACT16>(av[2 * i], av[2 * i + 1], v[16 + 2 * i], v[16 + 2 * i + 1], acc2[g]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          X[g][i] += cs[(r < m ? r : 0) * nch + sl * 8 + c];
        }
      }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if constexpr (NIB) {
        const float m16 = ms * (1.0f / 16.0f), b16 = bm - m16;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          out[g][i] = fmaf(b16, X[g][i], fmaf(ms, acc2[g][i], fmaf(m16, acc[g][i], out[g][i])));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) out[g][i] = fmaf(bm, X[g][i], fmaf(ms, acc[g][i], out[g][i]));
      }
    }
  }
}

// Rows per exact-form pass: 16 while the partial sums fit beside the block's
// activations in LDS (hidden <= 3072), else 8.
__host__ __device__ constexpr int exact_pass_rows(int H) { return H <= 3072 ? 16 : 8; }

// One exact-form pass: the block's rows i0 .. i0 + m - 1 (m <= the pass
// rows, NG = ceil(m / 4) groups) against the wave's K slices; the partials
// of every wave to LDS, one barrier, then wave v finishes rows v, v + nw, ..
// (gu_finish), and a second barrier before the partials are rewritten.
template <int F, int ACT16, int NG, typename SB>
__device__ __forceinline__ void exact_pass(const DecodeArgs& a, const GuItem& it, const SB& b, const uint32_t* xl,
                                           const float* cs, float* red, int wv, int nw, int lane,
                                           const int* sslot, int m) {
  const int H = a.H, nch = H / 32, nsl = H / KBLK, k = a.k;
  constexpr int W = sizeof(b.w[0]) / sizeof(uint32_t);
  f4v out[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) out[g] = f4v{0.f, 0.f, 0.f, 0.f};
  gu_slice_mfma_n<F, ACT16, W, NG>(b.w, b.sc, xl, cs, H, m, lane, wv, out);
  for (int sl = wv + nw; sl < nsl; sl += nw) {     // hidden > 256 * waves: further slices in place
    SB c2;
    load_slice<F>(it.r, it.codes, it.scales, it.tl, sl, nch, nsl, lane, c2);
    gu_slice_mfma_n<F, ACT16, W, NG>(c2.w, c2.sc, xl, cs, H, m, lane, sl, out);
  }
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (4 * g + v < m) red[((4 * g + v) * nw + wv) * 64 + lane] = out[g][v];
  __syncthreads();
  for (int r = wv; r < m; r += nw) {
    const int slot = sslot[r];
    gu_finish(a, red + r * nw * 64, nw, slot / (k + 1), slot % (k + 1), it.t, lane);
  }
  __syncthreads();
}

// The rows of an item in passes of up to 4 (slot order = pick order); all
// rows of the batch sit in LDS, so a slot's LDS row is its row.
template <int F, int ACT16, typename SB>
__device__ __forceinline__ void gu_process_t(const DecodeArgs& a, const Picks& P, const GuItem& it,
                                             const SB& b, const uint32_t* xl, const float* cs,
                                             float* red, int& rb, int wv, int nw, int lane) {
  const int k = a.k;
  uint64_t m0 = 0, m1 = 0;
  int n = min(GU_SHARED_ROWS, a.R - GU_SHARED_ROWS * it.e);   // shared: rows 4e .. 4e + n - 1
  if (!it.shared) {
    m0 = __ballot(P.id0 == it.e);
    m1 = __ballot(P.id1 == it.e);
    n = __popcll(m0) + __popcll(m1);
  }
  for (int i = 0; i < n; i += 4) {
    const int m = min(4, n - i);
    int rr[4], jj[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      int r = GU_SHARED_ROWS * it.e + v, j = k;
      if (!it.shared && v < m) {
        int s;
        if (m0) { s = __ffsll((unsigned long long)m0) - 1; m0 &= m0 - 1; }
        else { s = 64 + __ffsll((unsigned long long)m1) - 1; m1 &= m1 - 1; }
        r = s / k;
        j = s % k;
      }
      rr[v] = (v == 0 || v < m) ? r : rr[0];
      jj[v] = (v == 0 || v < m) ? j : jj[0];
    }
    gu_pass<F, ACT16>(a, it, b, xl, cs, red, rb, wv, nw, lane, rr, rr, jj, m);
  }
}

template <int FR, int FS, int ACT16, typename SB>
__device__ __forceinline__ void gu_process(const DecodeArgs& a, const Picks& P, const GuItem& it,
                                           const SB& b, const uint32_t* xl, const float* cs,
                                           float* red, int& rb, int wv, int nw, int lane) {
  if (it.t != it.tl) return;      // tile beyond this class (intermediates differ)
  if constexpr (FR == FS) {        // one copy of the code when both classes share a format
    gu_process_t<FR, ACT16>(a, P, it, b, xl, cs, red, rb, wv, nw, lane);
  } else {
    if (it.shared) gu_process_t<FS, ACT16>(a, P, it, b, xl, cs, red, rb, wv, nw, lane);
    else gu_process_t<FR, ACT16>(a, P, it, b, xl, cs, red, rb, wv, nw, lane);
  }
}


// Prologue of the gate/up kernel: the picks (lane l: slots l, l + 64) and
// the units, the first item's loads, then the activations of all rows into
// LDS and their 32-wide chunk sums (4 consecutive activations per lane, then
// aligned 8-lane groups). With XV > 0 the activations come through XV
// unconditional 16-byte register loads per thread (indexes clamped), issued
// before the item's loads, so the compiler can count what is outstanding and
// the wait for them leaves the item's loads in flight; XV == 0 (many rows)
// copies them straight into LDS instead. LDS: activations [R][H] u16, chunk
// sums [R][H/32] f32, two reduction buffers [4][nw][64] f32.
struct GuCtx {
  uint32_t* xl;
  float* cs;
  float* red;
  int nw, wv, lane, nch, nsl, Tmax, n_items;
};

// Persistent grid G (a multiple of 8); block 64 * nw threads,
// nw = min(8, H / 256): wave w owns the K slices w, w + nw, ... Item
// i = (unit i / Tmax, tile i % Tmax); workgroup b takes items b, b + G, ...
// and the next item's loads are in flight during the current one's
// arithmetic. With Tmax and G multiples of 8, every item of tile t runs on
// XCD t % 8, so the shared units re-read the shared expert's tiles
// from that L2.
template <int FR, int FS, int ACT16, int XV>
__global__ __launch_bounds__(512) void k_dec_gateup(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  GuCtx c;
  const int H = a.H, R = a.R;
  const int tid = threadIdx.x, nthr = blockDim.x;
  c.nw = nthr >> 6;
  c.lane = tid & 63;
  c.wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  c.nch = H / 32;
  c.nsl = H / KBLK;
  c.xl = reinterpret_cast<uint32_t*>(smem);
  c.cs = reinterpret_cast<float*>(smem + (size_t)R * H * 2);
  c.red = c.cs + R * c.nch;
  const int nslot = R * a.k, nx = R * H / 8;     // slots, 16-byte activation pieces
  // four named registers (not an array, which would live in scratch)
  const uint4* xg = reinterpret_cast<const uint4*>(a.x);
  uint4 xv0, xv1, xv2, xv3;
  const int i0 = a.ids[min(c.lane, nslot - 1)];
  const int i1 = a.ids[min(c.lane + 64, nslot - 1)];
  if constexpr (XV > 0) {
    xv0 = xg[tid % nx];        // surplus threads re-read other pieces (distinct lines)
    xv1 = xg[(tid + nthr) % nx];
    xv2 = xg[(tid + 2 * nthr) % nx];
    xv3 = xg[(tid + 3 * nthr) % nx];
    asm volatile("" ::: "memory");   // these loads go out before the item's loads
  }
  Picks P = find_units(c.lane < nslot ? i0 : -1, c.lane + 64 < nslot ? i1 : -1, a.E, c.lane);
  c.Tmax = 2 * a.Imax / 64;
  c.n_items = (P.nrt + (R + GU_SHARED_ROWS - 1) / GU_SHARED_ROWS) * c.Tmax;
  int it_i = blockIdx.x;
  if (it_i >= c.n_items) return;
  const int G = gridDim.x;
  constexpr int SW = Fmt<FR>::WORDS > Fmt<FS>::WORDS ? Fmt<FR>::WORDS : Fmt<FS>::WORDS;
  SliceBuf<SW> A, B;
  const GuCls rcl = gu_cls(a.rt), scl = gu_cls(a.sh);
  const uint8_t* const base = a.base;
  GuItem ia = gu_item(base, rcl, scl, P, it_i, c.Tmax);
  gu_issue<FR, FS>(ia, c.wv, c.nch, c.nsl, c.lane, A);
  if constexpr (XV > 0) {
    // surplus threads rewrite a piece with the same bytes
    uint4* xd = reinterpret_cast<uint4*>(c.xl);
    xd[tid % nx] = xv0;
    xd[(tid + nthr) % nx] = xv1;
    xd[(tid + 2 * nthr) % nx] = xv2;
    xd[(tid + 3 * nthr) % nx] = xv3;
  } else {
    for (int base = c.wv * 64; base < nx; base += nthr) {
      if (base + c.lane < nx)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(a.x) + base + c.lane,
                                         (__attribute__((address_space(3))) void*)(reinterpret_cast<uint4*>(c.xl) + base),
                                         16, 0, 0);
    }
  }
  __syncthreads();
  for (int r = 0; r < R; ++r) {
    for (int sl = c.wv; sl < c.nsl; sl += c.nw) {
      const uint2 v = reinterpret_cast<const uint2*>(c.xl + (uint64_t)r * (H / 2) + sl * (KBLK / 2))[c.lane];
      const float sm = sum8(sum4<ACT16>(v));
      if ((c.lane & 7) == 0) c.cs[r * c.nch + sl * 8 + (c.lane >> 3)] = sm;
    }
  }
  __syncthreads();
  int rb = 0;
  for (;;) {
    // the next item's loads go out before this item's arithmetic; past the
    // end, the current item is re-issued (its lines are in L2)
    int nx1 = it_i + G;
    GuItem ib = nx1 < c.n_items ? gu_item(base, rcl, scl, P, nx1, c.Tmax) : ia;
    gu_issue<FR, FS>(ib, c.wv, c.nch, c.nsl, c.lane, B);
    gu_process<FR, FS, ACT16>(a, P, ia, A, c.xl, c.cs, c.red, rb, c.wv, c.nw, c.lane);
    if (nx1 >= c.n_items) break;
    it_i = nx1;
    int nx2 = it_i + G;
    ia = nx2 < c.n_items ? gu_item(base, rcl, scl, P, nx2, c.Tmax) : ib;
    gu_issue<FR, FS>(ia, c.wv, c.nch, c.nsl, c.lane, A);
    gu_process<FR, FS, ACT16>(a, P, ib, B, c.xl, c.cs, c.red, rb, c.wv, c.nw, c.lane);
    if (nx2 >= c.n_items) break;
    it_i = nx2;
  }
}

// The exact chunk form of gate/up: the same per-row arithmetic as
// k_dec_gateup (gu_pass: slices owned by fixed waves, chunks and groups in K
// order, slices reduced in slice order, each output element formed from its
// own row and column alone), on the expert blocks of the grouped sort
// (expert, first position, up to 16 rows) instead of a decode batch's units:
// every row's h is its one-row decode step's, however the prompt is cut,
// while an expert's weights are read once per block instead of once per
// 16-row window. Item = (block, group of GU_TG layout tiles); a workgroup
// stages the block's activations (16 rows) and their chunk sums in LDS once
// per item, then streams the group's tiles with the next tile's loads in
// flight, each tile in passes of 4 of the block's slots.
constexpr int GU_TG = 4;   // layout tiles per exact-form item
constexpr int GX_RB = 16;  // rows per expert block

// One tile of an exact-form item: the block's mc rows in passes of
// exact_pass_rows(H) (one pass for a block of 16 at hidden <= 3072); a
// row's LDS row is its place in the block. Layers with 5-, 6- or 8-bit
// experts, whose wider unpack leaves no registers for more groups, take
// passes of 4 (WIDE).
template <int F, int ACT16, bool WIDE, typename SB>
__device__ __forceinline__ void exact_tile_f(const DecodeArgs& a, const GuItem& it, const SB& b, const uint32_t* xl,
                                             const float* cs, float* red, int wv, int nw, int lane,
                                             const int* sslot, int mc) {
  const int rp = WIDE ? 4 : exact_pass_rows(a.H);
  for (int i = 0; i < mc; i += rp) {
    const int m = min(rp, mc - i);
    const uint32_t* xb = xl + (uint64_t)i * (a.H / 2);
    const float* cb = cs + (uint64_t)i * (a.H / 32);
    if constexpr (WIDE) {
      exact_pass<F, ACT16, 1>(a, it, b, xb, cb, red, wv, nw, lane, sslot + i, m);
    } else {
      if (m > 8) exact_pass<F, ACT16, 4>(a, it, b, xb, cb, red, wv, nw, lane, sslot + i, m);
      else if (m > 4) exact_pass<F, ACT16, 2>(a, it, b, xb, cb, red, wv, nw, lane, sslot + i, m);
      else exact_pass<F, ACT16, 1>(a, it, b, xb, cb, red, wv, nw, lane, sslot + i, m);
    }
  }
}
template <int FR, int FS, int ACT16, typename SB>
__device__ __forceinline__ void exact_tile(const DecodeArgs& a, const GuItem& it, const SB& b, const uint32_t* xl,
                                           const float* cs, float* red, int wv, int nw, int lane,
                                           const int* sslot, int mc) {
  constexpr bool WIDE = FR == F_Q5 || FR == F_Q6 || FR == F_Q8 || FS == F_Q5 || FS == F_Q6 || FS == F_Q8;
  if (it.shared) exact_tile_f<FS, ACT16, WIDE>(a, it, b, xl, cs, red, wv, nw, lane, sslot, mc);
  else exact_tile_f<FR, ACT16, WIDE>(a, it, b, xl, cs, red, wv, nw, lane, sslot, mc);
}

template <int FR, int FS, int ACT16>
__global__ __launch_bounds__(512) void k_exact_gateup(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int RB = GX_RB;   // rows per block
  const int H = a.H, k = a.k;
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63;
  const int nw = nthr >> 6, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = H / 32, nsl = H / KBLK;
  uint32_t* xl = reinterpret_cast<uint32_t*>(smem);
  float* cs = reinterpret_cast<float*>(smem + (size_t)RB * H * 2);
  float* red = cs + RB * nch;                  // [pass rows][nw][64]
  __shared__ int sslot[GX_RB];                  // the block's slot indexes

  const int Tmax = 2 * a.Imax / 64, ngr = (Tmax + GU_TG - 1) / GU_TG;
  const int n_items = *a.nblocks * ngr;
  const GuCls rcl = gu_cls(a.rt), scl = gu_cls(a.sh);
  constexpr int SW = Fmt<FR>::WORDS > Fmt<FS>::WORDS ? Fmt<FR>::WORDS : Fmt<FS>::WORDS;
  SliceBuf<SW> A, B;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int* blk = a.blocks + 3 * (item / ngr);
    const int e = blk[0], p0 = blk[1], mc = blk[2];
    const bool shared = e == a.E;
    const GuCls& cl = shared ? scl : rcl;
    const int t0 = (item % ngr) * GU_TG, t1 = min(t0 + GU_TG, cl.tlast + 1);
    if (t0 >= t1 || mc <= 0) continue;
    GuItem it;
    it.r = make_rsrc(a.base + (shared ? cl.base_off : cl.base_off + (uint64_t)e * cl.stride), cl.blk_bytes);
    it.codes = cl.codes;
    it.scales = cl.scales;
    it.shared = shared;
    it.e = e;
    it.t = it.tl = t0;
    gu_issue<FR, FS>(it, wv, nch, nsl, lane, A);
    // the block's slots, then its rows (the previous item's readers are past
    // its last barrier); the gather issues all of a thread's loads at once
    __syncthreads();
    if (tid < mc) sslot[tid] = a.perm[p0 + tid];
    __syncthreads();
    const uint4* xg = reinterpret_cast<const uint4*>(a.x);
    const int npc = mc * (H / 8);
    for (int q0 = 0; q0 < npc; q0 += 4 * nthr) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = min(q0 + u * nthr + tid, npc - 1);
        const int lr = q / (H / 8), c8 = q % (H / 8);
        v[u] = xg[(uint64_t)(sslot[lr] / (k + 1)) * (H / 8) + c8];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + u * nthr + tid;
        if (q < npc) reinterpret_cast<uint4*>(xl)[q] = v[u];
      }
    }
    __syncthreads();
    for (int r = 0; r < mc; ++r) {
      for (int sl = wv; sl < nsl; sl += nw) {
        const uint2 v = reinterpret_cast<const uint2*>(xl + (uint64_t)r * (H / 2) + sl * (KBLK / 2))[lane];
        const float sm = sum8(sum4<ACT16>(v));
        if ((lane & 7) == 0) cs[r * nch + sl * 8 + (lane >> 3)] = sm;
      }
    }
    __syncthreads();
    // tiles in pairs, A and B alternating; the next tile's loads go out
    // before this tile's arithmetic
    for (int t = t0; t < t1; t += 2) {
      GuItem nx = it;
      nx.t = nx.tl = t + 1;
      if (t + 1 < t1) gu_issue<FR, FS>(nx, wv, nch, nsl, lane, B);
      it.t = it.tl = t;
      exact_tile<FR, FS, ACT16>(a, it, A, xl, cs, red, wv, nw, lane, sslot, mc);
      if (t + 1 >= t1) break;
      nx.t = nx.tl = t + 2;
      if (t + 2 < t1) gu_issue<FR, FS>(nx, wv, nch, nsl, lane, A);
      it.t = it.tl = t + 1;
      exact_tile<FR, FS, ACT16>(a, it, B, xl, cs, red, wv, nw, lane, sslot, mc);
    }
  }
}

// ------------------------------------------------------------------ down
constexpr int DN_KS = 2;   // waves per routed slot (each 1/KS of the intermediate axis)

// The dots of down on 4x4x4 MFMAs, as in gate/up: B = the lane's weight
// row (one output column per lane), A = h with the fp16 high part in row
// slot 0 and the low part in slot 1 (slots 2, 3 repeat them; unused), so
// one pass gives both dots. Per group: out += ms*(dot_hi + dot_lo) + bm*X.
// hh/hl: the fp16 pairs of the part in LDS, hc: its chunk sums.
__device__ __forceinline__ const uint32_t* dn_slot_src(const uint32_t* hh, const uint32_t* hl) {
  return (threadIdx.x & 1) ? hl : hh;     // lane l supplies slot l % 4
}

template <int F>
__device__ __forceinline__ f4v dn_chunk(const uint32_t* wc, const PairMasks& pk, const uint32_t* src, f4v acc) {
  uint32_t v[16], av[16];
  unpack_pairs<F, 1>(wc, pk, v);
  const uint4* q = reinterpret_cast<const uint4*>(src);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint4 t = q[u];
    av[4 * u] = t.x; av[4 * u + 1] = t.y; av[4 * u + 2] = t.z; av[4 * u + 3] = t.w;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = mfma4<1>(av[2 * i], av[2 * i + 1], v[2 * i], v[2 * i + 1], acc);
  return acc;
}

// Routed part: one 256-wide block (8 chunks) of one slot's h against the
// lane's weight row.
template <int F>
__device__ __forceinline__ float dn_block(const uint32_t (&w)[8][Fmt<F>::WORDS], const uint32_t* sc,
                                          const uint32_t* hh, const uint32_t* hl, const float* hc,
                                          float out) {
  constexpr int GPS = KBLK / Fmt<F>::G, CPG = Fmt<F>::G / 32;
  const PairMasks pk = pair_masks<F, 1>();
  const uint32_t* src = dn_slot_src(hh, hl);
#pragma unroll
  for (int gi = 0; gi < GPS; ++gi) {
    float ms, bm;
    coef_reg<F>(sc, gi, ms, bm);
    f4v acc = {0.f, 0.f, 0.f, 0.f};
    float X = 0.f;
#pragma unroll
    for (int cc = 0; cc < CPG; ++cc) {
      const int c = gi * CPG + cc;
      acc = dn_chunk<F>(w[c], pk, src + 16 * c, acc);
      X += hc[c];
    }
    out = fmaf(ms, acc[0] + acc[1], out);
    out = fmaf(bm, X, out);
  }
  return out;
}

// One group (CPG chunks) of the shared expert: codes and its scale word.
template <int F>
__device__ __forceinline__ float dn_group(const uint32_t (*w)[Fmt<F>::WORDS], uint32_t scw, int gi,
                                          const uint32_t* hh, const uint32_t* hl, const float* hc) {
  constexpr int CPG = Fmt<F>::G / 32;
  uint32_t sc[4] = {scw, scw, scw, scw};
  float ms, bm;
  // the word holds this group's entry: affine one u32, symmetric the u16 at
  // gi % 2, MXFP4 the byte at gi % 4
  coef_reg<F>(sc, Fmt<F>::AFF ? 0 : F == F_MX4 ? (gi & 3) : (gi & 1), ms, bm);
  const PairMasks pk = pair_masks<F, 1>();
  const uint32_t* src = dn_slot_src(hh, hl);
  f4v acc = {0.f, 0.f, 0.f, 0.f};
  float X = 0.f;
#pragma unroll
  for (int cc = 0; cc < CPG; ++cc) {
    acc = dn_chunk<F>(w[cc], pk, src + 16 * cc, acc);
    X += hc[cc];
  }
  return fmaf(bm, X, fmaf(ms, acc[0] + acc[1], 0.f));
}

// Per-lane byte offset, inside its scale block, of the 4-byte word holding
// group g's entry: affine the group's u32, symmetric the u32 holding both
// fp16 scales of the block (the entry at half g % 2), MXFP4 the u32 of the
// lane's 8 exponent bytes that holds byte g % 8 (at byte g % 4).
template <int F>
__device__ __forceinline__ uint32_t group_word_voff(int g, int lane) {
  constexpr int GPS = KBLK / Fmt<F>::G;
  if constexpr (Fmt<F>::AFF) return (uint32_t)(lane * GPS + (g % GPS)) * 4;
  else if constexpr (F == F_MX4) return (uint32_t)lane * 8 + (uint32_t)((g % GPS) >> 2) * 4;
  else return (uint32_t)lane * 4;
}

// down + combine: one workgroup per (row, 64-column tile of y), k * KS waves.
// Every wave stages only the h it reads (its routed block of slot j and its
// shared groups) in a wave-private LDS area and starts as soon as its own
// loads have landed; one barrier before the combine.
constexpr int DN_WR = 128 + 128 + 8;   // routed block: hi pairs, lo pairs, chunk sums (words)
constexpr int DN_WS = 136;             // shared group: up to 64 + 64 pairs + 4 chunk sums
constexpr int DN_WW = DN_WR + DN_WS;   // words per wave

// h of slot s for the 256-wide block kb, loaded (lanes 0..31 the hi pairs,
// 32..63 the lo pairs, every lane one of the 8 sums), then stored to the
// wave area (hi at [0, 128), lo at [128, 256), sums at [256, 264)).
struct HBlk {
  uint4 v;
  uint32_t c;
};
__device__ __forceinline__ HBlk dn_load_block(const DecodeArgs& a, uint64_t s, int kb, int lane) {
  const int Ih = a.Imax / 2, Ic = a.Imax / 32;
  const uint32_t* src = (lane < 32 ? reinterpret_cast<const uint32_t*>(a.hhi) : reinterpret_cast<const uint32_t*>(a.hlo)) +
                        s * Ih + 128 * kb + 4 * (lane & 31);
  HBlk h;
  h.v = *reinterpret_cast<const uint4*>(src);
  h.c = reinterpret_cast<const uint32_t*>(a.hc)[s * Ic + 8 * kb + (lane & 7)];
  return h;
}
__device__ __forceinline__ void dn_store_block(const HBlk& h, uint32_t* w, int lane) {
  *reinterpret_cast<uint4*>(w + 4 * lane) = h.v;
  if (lane < 8) w[256 + lane] = h.c;
  __builtin_amdgcn_wave_barrier();
}

// h of the shared slot s for group g (G wide): hi pairs [0, G/2), lo pairs
// [G/2, G), sums [G, G + G/32) of the wave's shared area.
template <int G>
struct HGrp {
  uint32_t v[(G + G / 32 + 63) / 64];
};
template <int G>
__device__ __forceinline__ HGrp<G> dn_load_group(const DecodeArgs& a, uint64_t s, int g, int lane) {
  const int Ih = a.Imax / 2, Ic = a.Imax / 32;
  constexpr int NW = G + G / 32;
  const uint32_t* hh = reinterpret_cast<const uint32_t*>(a.hhi) + s * Ih + (G / 2) * g;
  const uint32_t* hl = reinterpret_cast<const uint32_t*>(a.hlo) + s * Ih + (G / 2) * g;
  const uint32_t* hc = reinterpret_cast<const uint32_t*>(a.hc) + s * Ic + (G / 32) * g;
  HGrp<G> h;
#pragma unroll
  for (int q = 0; q < (NW + 63) / 64; ++q) {
    const int i = min(lane + 64 * q, NW - 1);
    h.v[q] = i < G / 2 ? hh[i] : (i < G ? hl[i - G / 2] : hc[i - G]);
  }
  return h;
}
template <int G>
__device__ __forceinline__ void dn_store_group(const HGrp<G>& h, uint32_t* w, int lane) {
  constexpr int NW = G + G / 32;
#pragma unroll
  for (int q = 0; q < (NW + 63) / 64; ++q) w[min(lane + 64 * q, NW - 1)] = h.v[q];
  __builtin_amdgcn_wave_barrier();
}

template <int FR, int FS>
__global__ __launch_bounds__(1024) void k_dec_down(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int T = a.H / 64, R = a.R, k = a.k;
  const int nwv = k * DN_KS;
  uint32_t* wl = reinterpret_cast<uint32_t*>(smem);          // [nwv][DN_WW]
  float* es = reinterpret_cast<float*>(wl + nwv * DN_WW);    // [nwv][64]
  float* ps = es + nwv * 64;                                  // [nwv][64]
  const int wg = blockIdx.x;
  int t, r;
  if (T % 8 == 0) {          // rows of one tile on one XCD (round-robin dispatch over 8 XCDs)
    const int xcd = wg % 8, loc = wg / 8;
    t = xcd + 8 * (loc / R);
    r = loc % R;
  } else {
    t = wg / R;
    r = wg % R;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wi = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = wi / DN_KS, kp = wi % DN_KS;
  uint32_t* wr_l = wl + wi * DN_WW;      // this wave's routed block area
  uint32_t* ws_l = wr_l + DN_WR;          // and its shared group area
  // the slot's expert through the scalar cache (uniform)
  const int e = ((const __attribute__((address_space(4))) int32_t*)(a.ids))[r * k + j];
  const bool valid = e >= 0 && e < a.E;
  const rsrc_t rr = make_rsrc(a.base + a.rt.base_off + (uint64_t)(valid ? e : 0) * a.rt.stride, a.rt.blk_bytes);
  const uint32_t rcodes = (uint32_t)a.rt.dn_codes, rscales = (uint32_t)a.rt.dn_scales;
  const int rnch = a.rt.inter / 32, rnkb = a.rt.inter / KBLK;
  uint32_t wr[8][Fmt<FR>::WORDS], scr[4];
  // loads are unconditional (a wave without a block or group of its own
  // loads a valid one and ignores it) so that the wait counts stay exact
  const bool has_blk = kp < rnkb;
  const int kb0 = min(kp, rnkb - 1);
  const uint64_t srow = (uint64_t)r * (k + 1);
  constexpr int SG = Fmt<FS>::G;
  const int sng = a.sh.inter / SG;
  const int g0 = min(wi, sng - 1);
  // this wave's h first (the routed block, the first shared group): the
  // wait for it before the LDS stores leaves the weight loads in flight
  const HBlk hb = dn_load_block(a, srow + j, kb0, lane);
  const HGrp<SG> hg = dn_load_group<SG>(a, srow + k, g0, lane);
  asm volatile("" ::: "memory");
  load_scales_rs<FR>(rr, scale_voff<FR>(lane), rscales + (uint32_t)sblk_off<FR>(t, kb0, rnkb), scr);
#pragma unroll
  for (int cc = 0; cc < 8; ++cc)
    load_chunk_rs<FR>(rr, chunk_voff<FR>(lane), rcodes + (uint32_t)chunk_off<FR>(t, kb0 * 8 + cc, rnch), wr[cc]);
  // shared expert: groups wi, wi + nwv, ... (first one loaded here)
  constexpr int SCPG = Fmt<FS>::G / 32;
  const rsrc_t rs = make_rsrc(a.base + a.sh.base_off, a.sh.blk_bytes);
  const uint32_t scodes = (uint32_t)a.sh.dn_codes, sscales = (uint32_t)a.sh.dn_scales;
  const int snch = a.sh.inter / 32, snkb = a.sh.inter / KBLK;
  uint32_t wsh[SCPG][Fmt<FS>::WORDS], scs = 0;
  scs = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)group_word_voff<FS>(g0, lane),
                                             (int)(sscales + (uint32_t)sblk_off<FS>(t, g0 / (KBLK / Fmt<FS>::G), snkb)), 0);
#pragma unroll
  for (int cc = 0; cc < SCPG; ++cc)
    load_chunk_rs<FS>(rs, chunk_voff<FS>(lane), scodes + (uint32_t)chunk_off<FS>(t, g0 * SCPG + cc, snch), wsh[cc]);
  dn_store_block(hb, wr_l, lane);
  dn_store_group<SG>(hg, ws_l, lane);
  float e_out = 0.f;
  if (has_blk) {
    e_out = dn_block<FR>(wr, scr, wr_l, wr_l + 128, reinterpret_cast<const float*>(wr_l + 256), e_out);
    for (int kb = kp + DN_KS; kb < rnkb; kb += DN_KS) {
      load_scales_rs<FR>(rr, scale_voff<FR>(lane), rscales + (uint32_t)sblk_off<FR>(t, kb, rnkb), scr);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc)
        load_chunk_rs<FR>(rr, chunk_voff<FR>(lane), rcodes + (uint32_t)chunk_off<FR>(t, kb * 8 + cc, rnch), wr[cc]);
      dn_store_block(dn_load_block(a, srow + j, kb, lane), wr_l, lane);
      e_out = dn_block<FR>(wr, scr, wr_l, wr_l + 128, reinterpret_cast<const float*>(wr_l + 256), e_out);
    }
  }
  if (!valid) e_out = 0.f;
  float s_out = 0.f;
  for (int g = wi; g < sng; g += nwv) {
    if (g != wi) {
#pragma unroll
      for (int cc = 0; cc < SCPG; ++cc)
        load_chunk_rs<FS>(rs, chunk_voff<FS>(lane), scodes + (uint32_t)chunk_off<FS>(t, g * SCPG + cc, snch), wsh[cc]);
      scs = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)group_word_voff<FS>(g, lane),
                                                 (int)(sscales + (uint32_t)sblk_off<FS>(t, g / (KBLK / Fmt<FS>::G), snkb)), 0);
      dn_store_group<SG>(dn_load_group<SG>(a, srow + k, g, lane), ws_l, lane);
    }
    s_out += dn_group<FS>(wsh, scs, g, ws_l, ws_l + Fmt<FS>::G / 2, reinterpret_cast<const float*>(ws_l + Fmt<FS>::G));
  }
  es[wi * 64 + lane] = e_out;
  ps[wi * 64 + lane] = s_out;
  __syncthreads();
  if (wi == 0) {
    float sh = 0.f;
    for (int q = 0; q < nwv; ++q) sh += ps[q * 64 + lane];
    float y = 0.f;
    for (int q = 0; q < k; ++q) {
      float eq = 0.f;
#pragma unroll
      for (int p = 0; p < DN_KS; ++p) eq += es[(q * DN_KS + p) * 64 + lane];
      if (a.tap_e) a.tap_e[((uint64_t)r * (k + 1) + q) * a.H + 64 * t + lane] = eq;
      y = fmaf(a.p[r * k + q], eq, y);
    }
    if (a.tap_e) a.tap_e[((uint64_t)r * (k + 1) + k) * a.H + 64 * t + lane] = sh;
    y = fmaf(a.sg[r], sh, y);
    a.y[(uint64_t)r * a.H + 64 * t + lane] = y;
  }
}

// ------------------------------------------------------------------ exact down
// The exact chunk form of down: k_dec_down's per-(row, slot) arithmetic on
// the expert blocks, so an expert's down tiles are read once per block of
// up to 16 rows instead of once per row. Two rows share each 4x4x4 MFMA: row
// slots 0 / 1 hold the first row's high / low h parts, slots 2 / 3 the
// second row's (k_dec_down repeats one row's parts there); an output element
// depends on its own row slot alone, so each row's sums are k_dec_down's.
// Item = (block, group of DX_TG 64-column tiles); wave w takes tile w / 2 of
// the group and the K blocks w % 2, w % 2 + 2, ... (k_dec_down's two parts).
// A routed slot's output is (0 + part 0) + part 1, as k_dec_down adds them;
// the shared expert's is k_dec_down's sum over its k * DN_KS wave partials,
// each the sum of the groups that wave takes (dn_group per group). Outputs
// go to e_ws in slot order; k_exact_combine adds them as k_dec_down does.
constexpr int DX_TG = 4;        // 64-column tiles per exact-form down item
constexpr int DX_MAXG = 32;     // shared-expert groups kept per row and tile (the host refuses more)

template <int F>
__device__ __forceinline__ void dn_block2(const uint32_t (&w)[8][Fmt<F>::WORDS], const uint32_t* sc,
                                          const uint32_t* src, const float* hca, const float* hcb, float& oa,
                                          float& ob) {
  constexpr int GPS = KBLK / Fmt<F>::G, CPG = Fmt<F>::G / 32;
  const PairMasks pk = pair_masks<F, 1>();
#pragma unroll
  for (int gi = 0; gi < GPS; ++gi) {
    float ms, bm;
    coef_reg<F>(sc, gi, ms, bm);
    f4v acc = {0.f, 0.f, 0.f, 0.f};
    float Xa = 0.f, Xb = 0.f;
#pragma unroll
    for (int cc = 0; cc < CPG; ++cc) {
      const int c = gi * CPG + cc;
      acc = dn_chunk<F>(w[c], pk, src + 16 * c, acc);
      Xa += hca[c];
      Xb += hcb[c];
    }
    oa = fmaf(ms, acc[0] + acc[1], oa);
    oa = fmaf(bm, Xa, oa);
    ob = fmaf(ms, acc[2] + acc[3], ob);
    ob = fmaf(bm, Xb, ob);
  }
}

// The groups of one 256-wide K block of the shared expert for two rows:
// each group's value is dn_group's (its own fma chain from 0).
template <int F>
__device__ __forceinline__ void dn_groups2(const uint32_t (&w)[8][Fmt<F>::WORDS], const uint32_t* sc,
                                           const uint32_t* src, const float* hca, const float* hcb,
                                           float (&va)[KBLK / Fmt<F>::G], float (&vb)[KBLK / Fmt<F>::G]) {
  constexpr int GPS = KBLK / Fmt<F>::G, CPG = Fmt<F>::G / 32;
  const PairMasks pk = pair_masks<F, 1>();
#pragma unroll
  for (int gi = 0; gi < GPS; ++gi) {
    float ms, bm;
    coef_reg<F>(sc, gi, ms, bm);
    f4v acc = {0.f, 0.f, 0.f, 0.f};
    float Xa = 0.f, Xb = 0.f;
#pragma unroll
    for (int cc = 0; cc < CPG; ++cc) {
      const int c = gi * CPG + cc;
      acc = dn_chunk<F>(w[c], pk, src + 16 * c, acc);
      Xa += hca[c];
      Xb += hcb[c];
    }
    va[gi] = fmaf(bm, Xa, fmaf(ms, acc[0] + acc[1], 0.f));
    vb[gi] = fmaf(bm, Xb, fmaf(ms, acc[2] + acc[3], 0.f));
  }
}

// One class's part of an exact-form down item (F: the class's format). The
// block's slots are in LDS (sslot). Routed blocks: each wave's parts of all
// the block's slots go to LDS (pr: [16 slots][tiles][DN_KS][64]) and one
// barrier precedes the part sums; the shared expert's group values are
// summed per pass (sgp). The next pass's h is loaded during this pass's
// arithmetic when a wave has one K block (inter <= 512).
template <int F>
__device__ __forceinline__ void exact_down_item(const DecodeArgs& a, uint32_t (*hw)[264], float* pr, float* sgp,
                                                const int* sslot, int e, int mc, int t, int ti, int kp, int lane) {
  const bool shared = e == a.E;
  const ExpertClass& ec = shared ? a.sh : a.rt;
  const int k = a.k, H = a.H, inter = ec.inter;
  const int nch = inter / 32, nkb = inter / KBLK;
  constexpr int GPS = KBLK / Fmt<F>::G;
  const int sng = inter / Fmt<F>::G, nwv = k * DN_KS;
  const rsrc_t rs = make_rsrc(a.base + ec.base_off + (shared ? 0 : (uint64_t)e * ec.stride), ec.blk_bytes);
  const uint32_t codes = (uint32_t)ec.dn_codes, scales = (uint32_t)ec.dn_scales;
  uint32_t wr[8][Fmt<F>::WORDS], sc[4];
  const int kb0 = min(kp, nkb - 1);
  load_scales_rs<F>(rs, scale_voff<F>(lane), scales + (uint32_t)sblk_off<F>(t, kb0, nkb), sc);
#pragma unroll
  for (int cc = 0; cc < 8; ++cc)
    load_chunk_rs<F>(rs, chunk_voff<F>(lane), codes + (uint32_t)chunk_off<F>(t, kb0 * 8 + cc, nch), wr[cc]);
  // this lane's MFMA row slot: 0 / 1 the first row's hi / lo, 2 / 3 the second's
  const uint32_t* src = hw[(lane >> 1) & 1] + ((lane & 1) ? 128 : 0);
  const float* hca = reinterpret_cast<const float*>(hw[0] + 256);
  const float* hcb = reinterpret_cast<const float*>(hw[1] + 256);
  const bool one_kb = nkb <= DN_KS;
  int held = kb0;   // the K block whose weights wr holds (several per wave: reloaded per pass)
  HBlk ha, hb;
  if (one_kb && kp < nkb) {
    ha = dn_load_block(a, (uint64_t)sslot[0], kp, lane);
    hb = dn_load_block(a, (uint64_t)sslot[min(1, mc - 1)], kp, lane);
  }
  for (int i = 0; i < mc; i += 2) {
    const int m = min(2, mc - i);
    const int sa = sslot[i], sb = sslot[i + m - 1];
    float oa = 0.f, ob = 0.f;
    for (int kb = kp; kb < nkb; kb += DN_KS) {
      if (one_kb) {
        dn_store_block(ha, hw[0], lane);
        dn_store_block(hb, hw[1], lane);
        if (i + 2 < mc) {
          ha = dn_load_block(a, (uint64_t)sslot[i + 2], kb, lane);
          hb = dn_load_block(a, (uint64_t)sslot[min(i + 3, mc - 1)], kb, lane);
        }
      } else {
        if (kb != held) {
          load_scales_rs<F>(rs, scale_voff<F>(lane), scales + (uint32_t)sblk_off<F>(t, kb, nkb), sc);
#pragma unroll
          for (int cc = 0; cc < 8; ++cc)
            load_chunk_rs<F>(rs, chunk_voff<F>(lane), codes + (uint32_t)chunk_off<F>(t, kb * 8 + cc, nch), wr[cc]);
          held = kb;
        }
        dn_store_block(dn_load_block(a, (uint64_t)sa, kb, lane), hw[0], lane);
        dn_store_block(dn_load_block(a, (uint64_t)sb, kb, lane), hw[1], lane);
      }
      if (!shared) {
        dn_block2<F>(wr, sc, src, hca, hcb, oa, ob);
      } else {
        float va[GPS], vb[GPS];
        dn_groups2<F>(wr, sc, src, hca, hcb, va, vb);
#pragma unroll
        for (int gi = 0; gi < GPS; ++gi) {
          sgp[((0 * DX_TG + ti) * DX_MAXG + kb * GPS + gi) * 64 + lane] = va[gi];
          sgp[((1 * DX_TG + ti) * DX_MAXG + kb * GPS + gi) * 64 + lane] = vb[gi];
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    if (!shared) {
      pr[((i * DX_TG + ti) * DN_KS + kp) * 64 + lane] = oa;
      if (m > 1) pr[(((i + 1) * DX_TG + ti) * DN_KS + kp) * 64 + lane] = ob;
      continue;
    }
    __syncthreads();
    if (kp == 0) {
      for (int v = 0; v < m; ++v) {
        float o = 0.f;
        for (int q = 0; q < nwv; ++q) {
          float ps = 0.f;
          for (int g = q; g < sng; g += nwv) ps += sgp[((v * DX_TG + ti) * DX_MAXG + g) * 64 + lane];
          o += ps;
        }
        a.e_ws[(uint64_t)(v ? sb : sa) * H + 64 * t + lane] = o;
      }
    }
    __syncthreads();
  }
  if (!shared) {
    __syncthreads();
    if (kp == 0) {
      for (int sl = 0; sl < mc; ++sl) {
        float o = 0.f;
#pragma unroll
        for (int q = 0; q < DN_KS; ++q) o += pr[((sl * DX_TG + ti) * DN_KS + q) * 64 + lane];
        a.e_ws[(uint64_t)sslot[sl] * H + 64 * t + lane] = o;
      }
    }
  }
}

template <int FR, int FS>
__global__ __launch_bounds__(512) void k_exact_down(DecodeArgs a) {
  __shared__ __align__(16) uint32_t hw_all[8][2][264];           // per wave: the pass's two rows' h parts
  __shared__ float pr[GX_RB * DX_TG * DN_KS * 64];                // routed parts of the block's slots
  __shared__ float sgp[2 * DX_TG * DX_MAXG * 64];                 // shared-expert group values of the pass
  __shared__ int sslot[GX_RB];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ti = w >> 1, kp = w & 1;
  const int ngr = (a.H / 64) / DX_TG;
  const int n_items = *a.nblocks * ngr;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int* blk = a.blocks + 3 * (item / ngr);
    const int e = blk[0], p0 = blk[1], mc = blk[2];
    if (mc <= 0 || e < 0 || e > a.E) continue;
    // the previous item's readers of sslot and pr are past this barrier
    __syncthreads();
    if (tid < mc) sslot[tid] = a.perm[p0 + tid];
    __syncthreads();
    const int t = (item % ngr) * DX_TG + ti;
    if (e == a.E) exact_down_item<FS>(a, hw_all[w], pr, sgp, sslot, e, mc, t, ti, kp, lane);
    else exact_down_item<FR>(a, hw_all[w], pr, sgp, sslot, e, mc, t, ti, kp, lane);
  }
}

// y = sum_j p_j e_j + sigma e_shared per row, in k_dec_down's order (a slot
// whose id is outside [0, E) adds p_j * 0); 4 columns per thread.
__global__ __launch_bounds__(256) void k_exact_combine(DecodeArgs a) {
  const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  const int H = a.H, k = a.k, H4 = H / 4;
  if (i >= (uint64_t)a.R * H4) return;
  const int r = (int)(i / H4), n = (int)(i % H4) * 4;
  const float* e = a.e_ws + (uint64_t)r * (k + 1) * H + n;
  float y[4] = {0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < k; ++q) {
    const int id = a.ids[r * k + q];
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (id >= 0 && id < a.E) v = *reinterpret_cast<const float4*>(e + (uint64_t)q * H);
    const float pq = a.p[r * k + q];
    y[0] = fmaf(pq, v.x, y[0]);
    y[1] = fmaf(pq, v.y, y[1]);
    y[2] = fmaf(pq, v.z, y[2]);
    y[3] = fmaf(pq, v.w, y[3]);
    if (a.tap_e) *reinterpret_cast<float4*>(a.tap_e + ((uint64_t)r * (k + 1) + q) * H + n) = v;
  }
  const float4 v = *reinterpret_cast<const float4*>(e + (uint64_t)k * H);
  const float sg = a.sg[r];
  y[0] = fmaf(sg, v.x, y[0]);
  y[1] = fmaf(sg, v.y, y[1]);
  y[2] = fmaf(sg, v.z, y[2]);
  y[3] = fmaf(sg, v.w, y[3]);
  if (a.tap_e) *reinterpret_cast<float4*>(a.tap_e + ((uint64_t)r * (k + 1) + k) * H + n) = v;
  *reinterpret_cast<float4*>(a.y + (uint64_t)r * H + n) = make_float4(y[0], y[1], y[2], y[3]);
}

// ------------------------------------------------------------------ launch
constexpr int GU_GRID = 256;   // persistent gate/up workgroups (a multiple of 8)

size_t decode_gu_smem(int R, int H) {
  return (size_t)R * H * 2 + (size_t)R * (H / 32) * 4 + 2 * 4 * (size_t)std::min(8, H / KBLK) * 64 * 4;
}
size_t decode_dn_smem(int k, int Imax) {
  (void)Imax;
  return (size_t)k * DN_KS * (DN_WW * 4 + 2 * 64 * 4);
}

template <typename K>
static hipError_t allow_smem(K kern, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <int FR, int FS, int ACT16>
static hipError_t launch_gateup(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev, int nw, size_t gsm) {
  hipError_t err;
  if (a.R * a.H / 8 <= 4 * 64 * nw) {
    if ((err = allow_smem(k_dec_gateup<FR, FS, ACT16, 4>, gsm)) != hipSuccess) return err;
    launch_k(k_dec_gateup<FR, FS, ACT16, 4>, dim3(GU_GRID), dim3(64 * nw), (uint32_t)gsm, s, ev, 0, a);
  } else {
    if ((err = allow_smem(k_dec_gateup<FR, FS, ACT16, 0>, gsm)) != hipSuccess) return err;
    launch_k(k_dec_gateup<FR, FS, ACT16, 0>, dim3(GU_GRID), dim3(64 * nw), (uint32_t)gsm, s, ev, 0, a);
  }
  return hipGetLastError();
}

// The exact chunk form's experts: gate/up and down on the sort's expert
// blocks, then the combine of every row.
template <int FR, int FS>
static hipError_t launch_exact_t(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  const int nw = std::min(8, a.H / KBLK);
  const size_t gsm = (size_t)GX_RB * a.H * 2 + (size_t)GX_RB * (a.H / 32) * 4 +
                     (size_t)exact_pass_rows(a.H) * std::min(8, a.H / KBLK) * 64 * 4;
  const size_t dsm = decode_dn_smem(a.k, a.Imax);
  hipError_t err;
  if (a.act_fp16) {
    if ((err = allow_smem(k_exact_gateup<FR, FS, 1>, gsm)) != hipSuccess) return err;
    launch_k(k_exact_gateup<FR, FS, 1>, dim3(GU_GRID), dim3(64 * nw), (uint32_t)gsm, s, ev, 0, a);
  } else {
    if ((err = allow_smem(k_exact_gateup<FR, FS, 0>, gsm)) != hipSuccess) return err;
    launch_k(k_exact_gateup<FR, FS, 0>, dim3(GU_GRID), dim3(64 * nw), (uint32_t)gsm, s, ev, 0, a);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  (void)dsm;
  hipEvent_t e2[2] = {ev ? ev[2] : nullptr, nullptr}, e3[2] = {nullptr, ev ? ev[3] : nullptr};
  launch_k(k_exact_down<FR, FS>, dim3(GU_GRID), dim3(512), 0, s, e2, 0, a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const uint64_t n4 = (uint64_t)a.R * (a.H / 4);
  launch_k(k_exact_combine, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, e3, 0, a);
  return hipGetLastError();
}

template <int FR, int FS>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  const int nw = std::min(8, a.H / KBLK);
  const size_t gsm = decode_gu_smem(a.R, a.H), dsm = decode_dn_smem(a.k, a.Imax);
  hipError_t err = a.act_fp16 ? launch_gateup<FR, FS, 1>(a, s, ev, nw, gsm) : launch_gateup<FR, FS, 0>(a, s, ev, nw, gsm);
  if (err != hipSuccess) return err;
  const int dthr = 64 * a.k * DN_KS;
  if ((err = allow_smem(k_dec_down<FR, FS>, dsm)) != hipSuccess) return err;
  launch_k(k_dec_down<FR, FS>, dim3((a.H / 64) * a.R), dim3(dthr), (uint32_t)dsm, s, ev, 2, a);
  return hipGetLastError();
}

template <int FR>
static hipError_t launch_decode_s(int fs, const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  if constexpr (FR == F_Q5 || FR == F_Q6 || FR == F_MX4) {
    // 5/6-bit and MXFP4 routed experts: shared of the same format or 4-bit affine
    if (fs == FR) return launch_decode_t<FR, FR>(a, s, ev);
    if (fs == F_Q4) return launch_decode_t<FR, F_Q4>(a, s, ev);
  } else {
    switch (fs) {
      case F_Q4: return launch_decode_t<FR, F_Q4>(a, s, ev);
      case F_Q3: return launch_decode_t<FR, F_Q3>(a, s, ev);
      case F_S4: return launch_decode_t<FR, F_S4>(a, s, ev);
      case F_Q8: return launch_decode_t<FR, F_Q8>(a, s, ev);
      case F_Q2: return launch_decode_t<FR, F_Q2>(a, s, ev);
    }
  }
  return hipErrorInvalidValue;
}

template <int FR>
static hipError_t launch_exact_s(int fs, const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  if constexpr (FR == F_Q5 || FR == F_Q6 || FR == F_MX4) {
    if (fs == FR) return launch_exact_t<FR, FR>(a, s, ev);
    if (fs == F_Q4) return launch_exact_t<FR, F_Q4>(a, s, ev);
  } else {
    switch (fs) {
      case F_Q4: return launch_exact_t<FR, F_Q4>(a, s, ev);
      case F_Q3: return launch_exact_t<FR, F_Q3>(a, s, ev);
      case F_S4: return launch_exact_t<FR, F_S4>(a, s, ev);
      case F_Q8: return launch_exact_t<FR, F_Q8>(a, s, ev);
      case F_Q2: return launch_exact_t<FR, F_Q2>(a, s, ev);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_exact_experts(int fr, int fs, const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  switch (fr) {
    case F_Q4: return launch_exact_s<F_Q4>(fs, a, s, ev);
    case F_Q3: return launch_exact_s<F_Q3>(fs, a, s, ev);
    case F_S4: return launch_exact_s<F_S4>(fs, a, s, ev);
    case F_Q8: return launch_exact_s<F_Q8>(fs, a, s, ev);
    case F_Q2: return launch_exact_s<F_Q2>(fs, a, s, ev);
    case F_Q5: return launch_exact_s<F_Q5>(fs, a, s, ev);
    case F_Q6: return launch_exact_s<F_Q6>(fs, a, s, ev);
    case F_MX4: return launch_exact_s<F_MX4>(fs, a, s, ev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(int fr, int fs, const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  switch (fr) {
    case F_Q4: return launch_decode_s<F_Q4>(fs, a, s, ev);
    case F_Q3: return launch_decode_s<F_Q3>(fs, a, s, ev);
    case F_S4: return launch_decode_s<F_S4>(fs, a, s, ev);
    case F_Q8: return launch_decode_s<F_Q8>(fs, a, s, ev);
    case F_Q2: return launch_decode_s<F_Q2>(fs, a, s, ev);
    case F_Q5: return launch_decode_s<F_Q5>(fs, a, s, ev);
    case F_Q6: return launch_decode_s<F_Q6>(fs, a, s, ev);
    case F_MX4: return launch_decode_s<F_MX4>(fs, a, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
