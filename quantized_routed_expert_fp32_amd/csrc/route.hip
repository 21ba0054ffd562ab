// Router: fp32 logits over the experts and the shared expert's gate row,
// top-k with ties to the lower id, renormalised weights, sigmoid gate
// ("qwen3_5_moe on native CUDA with 3-bit routed experts #803", Activity,
// comment "Progress on the 4-bit gate").
//
// Logits: one workgroup per (tile of 64 experts, group of NR rows); lanes
// own router rows exactly as the expert kernels own weight rows, wave w sums
// the K slices w, w + nw, ... and the waves are added in wave order.
// Pick (wave_topk): a two-bits-a-step search for the k-th largest order key
// (NaN above +inf above every finite logit), the keys above it plus the
// lowest ids among its ties, slots by (key desc, id asc); then
// exp(l - l_top) / sum in slot order and sigmoid of the gate logit.
//  * decode batches (k_route): one launch; each tile workgroup picks its
//    own k best, sends them out with write-through stores, and tile 0's
//    workgroup waits for them and picks from the tiles' picks.
//  * prompt chunks: logits of 32 rows x 64 experts per workgroup on MFMA
//    (k_route_mfma, 4-bit router codes) or 8 rows per workgroup on the
//    vector units (k_route_logits), then one wave per row picks in a second
//    launch (k_route_pick).
// Each row's arithmetic is the same whatever NR and the other rows are, so
// picks and weights of a row do not depend on the batch.
#include "moe_kernels.h"
#include "moe_launch.h"
#include "moe_dispatch.h"

namespace moe {

// Gate-row logit part of one lane (chunks lane, lane+64, ...), before the
// wave sum. The row is stored as one tile row: chunk c at c * CB bytes.
template <int FG, int ACT16>
__device__ __forceinline__ float gate_row_part(const RouteArgs& a, const uint16_t* xr, int lane) {
  const int H = a.H, nch = H / 32;
  const uint8_t* codes = a.base + a.g_off;
  const uint8_t* scales = a.base + a.g_soff;
  float part = 0.f;
  for (int c = lane; c < nch; c += 64) {
    const uint16_t* xc = xr + 32 * c;
    uint32_t xp[16];
    {
      const uint4* q = reinterpret_cast<const uint4*>(xc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = q[i];
        xp[4 * i] = v.x; xp[4 * i + 1] = v.y; xp[4 * i + 2] = v.z; xp[4 * i + 3] = v.w;
      }
    }
    float contrib;
    if constexpr (FG == F_DENSE) {
      const uint4* wq = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(codes) + 32 * c);
      uint32_t wv[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = wq[i];
        wv[4 * i] = v.x; wv[4 * i + 1] = v.y; wv[4 * i + 2] = v.z; wv[4 * i + 3] = v.w;
      }
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc = fmaf(bf16_to_f(wv[i] & 0xFFFFu), act_to_f((uint16_t)(xp[i] & 0xFFFFu), ACT16), acc);
        acc = fmaf(bf16_to_f(wv[i] >> 16), act_to_f((uint16_t)(xp[i] >> 16), ACT16), acc);
      }
      contrib = acc;
    } else {
      uint32_t wd[8], v[32];
      const uint32_t* src = reinterpret_cast<const uint32_t*>(codes + (uint64_t)c * Fmt<FG>::CB);
#pragma unroll
      for (int i = 0; i < Fmt<FG>::WORDS; ++i) wd[i] = src[i];
      const int g = (32 * c) / Fmt<FG>::G;
      float s, b;
      if constexpr (Fmt<FG>::AFF) {
        const uint32_t sv = reinterpret_cast<const uint32_t*>(scales)[g];
        s = bf16_to_f(sv & 0xFFFFu);
        b = bf16_to_f(sv >> 16);
      } else {
        s = f16_bits_to_f(reinterpret_cast<const uint16_t*>(scales)[g]);
        b = -8.0f * s;
      }
      float X = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        X += act_to_f((uint16_t)(xp[i] & 0xFFFFu), ACT16);
        X += act_to_f((uint16_t)(xp[i] >> 16), ACT16);
      }
      if (ACT16) {
        unpack_chunk<FG>(wd, v);
        const float A = dot_chunk_h(v, xp, 0.f);
        const float M = (float)Fmt<FG>::M;
        contrib = fmaf(b - M * s, X, (M * s) * A);
      } else {
        unpack_chunk_bf<FG>(wd, v);
        const float A = dot_chunk_bf(v, xp, 0.f);
        if constexpr (FG == F_Q8) {
          const float A2 = dot_chunk_bf(v + 16, xp, 0.f);
          contrib = fmaf(b - 272.0f * s, X, fmaf(256.0f * s, A2, (16.0f * s) * A));
        } else {
          contrib = fmaf(b - 16.0f * s, X, (16.0f * s) * A);
        }
      }
    }
    part += contrib;
  }
  return part;
}

// Logits of NR rows for one tile of 64 experts. Wave w sums the K slices
// w, w + nw, ... in ascending order; the waves are added in wave order.
template <int FR, int ACT16, int NR>
__global__ __launch_bounds__(512) void k_route_logits(RouteArgs a, const uint16_t* __restrict__ x) {
  __shared__ float red[8][NR][64];
  __shared__ __align__(16) uint32_t lxs[8][NR * 128];    // per-wave activation slices
  const int H = a.H, E = a.E, nsl = H / KBLK, nch = H / 32;
  const int t = blockIdx.x, r0 = blockIdx.y * NR, tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int nw = blockDim.x >> 6;
  const int nr = min(NR, a.R - r0);
  const uint8_t* rc = a.base + a.r_off;
  const uint8_t* rs = a.base + a.r_soff;
  float out[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) out[i] = 0.f;
  for (int sl = w; sl < nsl; sl += nw) {
    // activations first, then codes and scale words: the wait for the
    // activations does not wait for the larger code loads
    uint2 xv[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i)
      xv[i] = *reinterpret_cast<const uint2*>(x + (uint64_t)(r0 + min(i, nr - 1)) * H + sl * KBLK + 4 * lane);
    uint32_t wc[8][Fmt<FR>::WORDS], sc[4];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) load_chunk<FR>(rc + chunk_off<FR>(t, sl * 8 + cc, nch), lane, wc[cc]);
    load_scales<FR>(rs + sblk_off<FR>(t, sl, nsl), lane, sc);
    float part[NR];
    slice_dot<FR, NR, ACT16>(wc, sc, lane, xv, nr, lxs[w], part);
#pragma unroll
    for (int i = 0; i < NR; ++i) out[i] += part[i];
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) red[w][i][lane] = out[i];
  __syncthreads();
  // wave i sums row i (rows beyond nw: waves take several)
  for (int i = w; i < nr; i += nw) {
    float l = 0.f;
    for (int q = 0; q < nw; ++q) l += red[q][i][lane];
    a.lg_ws[(uint64_t)(r0 + i) * E + 64 * t + lane] = l;
  }
}

// Top k of one row from its candidates (keys, values, expert ids; see
// wave_topk_ids), then weights exp(l_j - l_top) / sum over the k picks in
// slot order, and sigmoid of the gate logit c. One wave.
template <int NC>
__device__ __forceinline__ void pick_and_store_n(const RouteArgs& a, int row, const uint32_t (&key)[NC],
                                                 const float (&v)[NC], const int (&idv)[NC], float c, int lane,
                                                 uint32_t* scr) {
  const int k = a.k;
  int slot, id;
  float val;
  wave_topk_ids<NC>(key, v, idv, lane, k, scr, slot, id, val);
  // into slot order
  if (lane < k) {
    scr[slot] = (uint32_t)id;
    scr[8 + slot] = __float_as_uint(val);
  }
  __builtin_amdgcn_wave_barrier();
  const int my_i = (int)scr[lane < k ? lane : 0];
  const float my_v = __uint_as_float(scr[8 + (lane < k ? lane : 0)]);
  const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
  const float ex = expf(my_v - top);
  float S = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < k) S += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
  if (lane < k) {
    a.ids[(uint64_t)row * k + lane] = my_i;
    a.p[(uint64_t)row * k + lane] = ex / S;
  }
  if (lane == 0) a.sg[row] = 1.0f / (1.0f + expf(-c));
}
// all E <= 256 experts of a row, lane l holding experts l + 64 i
__device__ __forceinline__ void pick_and_store(const RouteArgs& a, int row, const uint32_t (&key)[4],
                                               const float (&v)[4], float c, int lane, uint32_t* scr) {
  const int idv[4] = {lane, lane + 64, lane + 128, lane + 192};
  pick_and_store_n<4>(a, row, key, v, idv, c, lane, scr);
}

// Decode batches: one workgroup per (tile of 64 experts, row) forms the
// tile's logits and picks the tile's own k best (the k best of a row are
// among the union of its tiles' k best under the same order). Tiles 1.. send
// their k entries to tile 0's workgroup of the row, each entry one 64-bit
// word (epoch << 40 | id << 32 | value bits) written through to memory;
// tile 0 polls those words (loads that bypass its XCD's L2) until each
// carries this call's epoch, then picks from its own entries and theirs.
// The epoch is a call counter kept in the workspace: every workgroup reads
// it at its start, and the last workgroup of the launch to finish (an
// integer completion counter) advances it, so a word left by an earlier
// call (or replay of a captured call) is never taken for this call's, and
// the words need no clearing between calls. Every workgroup of the launch
// is resident at once (E/64 * rows <= 128 workgroups), so the wait ends; it
// is bounded all the same: a row whose entries do not arrive within the
// bound gets ids -1 and NaN weights and gate, and the failure is counted in
// a sticky word of the workspace (moe_route_failures), which also makes
// every later call on that workspace report its rows the same way until the
// count is cleared. One wave past the slice waves forms the gate-row logit
// in tile 0, beside the slices.
constexpr uint32_t EPOCH_MOD = 0xFFFFFFu;   // epochs 1 .. 2^24 - 1 (0 never matches)

// Completion of one workgroup of k_route (wave 0, one lane): the last one
// of the launch resets the counter and advances the epoch state.
__device__ __forceinline__ void route_done(const RouteArgs& a, uint32_t state) {
  const uint32_t total = gridDim.x * gridDim.y;
  // every workgroup read the epoch state before it got here (its hand-off
  // words or its wait used the value), so the last one may advance it; the
  // next launch sees the new state after this kernel ends
  const uint32_t old = __hip_atomic_fetch_add(&a.sync[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old == total - 1) {
    __hip_atomic_store(&a.sync[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.sync[0], (state + 1) % EPOCH_MOD, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int FR, int FG, int ACT16>
__global__ __launch_bounds__(576) void k_route(RouteArgs a, const uint16_t* __restrict__ x) {
  __shared__ float red[8][64];
  __shared__ __align__(16) uint32_t lxs[8][128];
  __shared__ uint32_t scr[24];
  __shared__ float s_gate;
  const int H = a.H, E = a.E, nsl = H / KBLK, nch = H / 32, ntile = E / 64;
  const int t = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = (blockDim.x >> 6) - 1;          // slice waves; the last wave forms the gate logit
  const uint16_t* xr = x + (uint64_t)row * H;
  const uint8_t* rc = a.base + a.r_off;
  const uint8_t* rs = a.base + a.r_soff;
  // this call's epoch state (set by the previous launch's last workgroup)
  const uint32_t state = w == 0 ? __hip_atomic_load(&a.sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
  float out = 0.f;
  for (int sl = w; w < nw && sl < nsl; sl += nw) {
    uint2 xv[1];
    xv[0] = *reinterpret_cast<const uint2*>(xr + sl * KBLK + 4 * lane);
    uint32_t wc[8][Fmt<FR>::WORDS], sc[4];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) load_chunk<FR>(rc + chunk_off<FR>(t, sl * 8 + cc, nch), lane, wc[cc]);
    load_scales<FR>(rs + sblk_off<FR>(t, sl, nsl), lane, sc);
    float part[1];
    slice_dot<FR, 1, ACT16>(wc, sc, lane, xv, 1, lxs[w], part);
    out += part[0];
  }
  if (w < nw) red[w][lane] = out;
  if (t == 0 && w == nw) {
    const float s16 = sum16(gate_row_part<FG, ACT16>(a, xr, lane));
    float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 0));
    c += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 16));
    c += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 32));
    c += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 48));
    if (lane == 0) s_gate = c;
  }
  __syncthreads();
  if (w != 0) return;
  const int k = a.k;
  uint64_t* cand = a.cand + (uint64_t)row * 32;    // tile u's entries at 8 u .. 8 u + k - 1
  float l = 0.f;
  for (int q = 0; q < nw; ++q) l += red[q][lane];
  const int e = 64 * t + lane;
  const float v1[1] = {a.bias ? l + a.bias[e] : l};
  if (a.logits) a.logits[(uint64_t)row * (E + 1) + e] = v1[0];
  const uint32_t k1[1] = {pick_key(v1[0])};
  const int i1[1] = {e};
  int slot, id;
  float val;
  wave_topk_ids<1>(k1, v1, i1, lane, k, scr, slot, id, val);   // lane j < k: the tile's j-th pick by id
  const uint32_t ep = state % EPOCH_MOD + 1;
  if (t != 0) {
    if (lane < k)
      __hip_atomic_store(&cand[8 * t + lane],
                         ((uint64_t)((ep << 8) | (uint32_t)id) << 32) | __float_as_uint(val),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0) route_done(a, state);
    return;
  }
  // tile 0: lane j < k holds its own entry j; lane j in [k, ntile * k) waits
  // for entry j % k of tile j / k (a word of this call's epoch)
  const int nc = ntile * k;
  const bool remote = lane >= k && lane < nc;
  uint64_t* src = &cand[8 * (lane / k) + lane % k];
  uint64_t word = 0;
  bool have = !remote;
  // a failure recorded earlier on this workspace keeps every later call's
  // rows marked as failed until the caller clears it
  const bool sticky =
      a.sticky && __hip_atomic_load(&a.sync[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
  for (int spin = 0; spin < a.wait_limit && !sticky; ++spin) {
    if (!have) {
      word = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      have = (uint32_t)(word >> 40) == ep;
    }
    if (__ballot(!have) == 0) break;
    __builtin_amdgcn_s_sleep(1);
  }
  if (sticky || __ballot(!have) != 0) {
    // the wait bound ran out (the tile workgroups were not all resident) or
    // an earlier call failed: the row is marked invalid rather than picked
    // from missing entries
    if (lane < k) {
      a.ids[(uint64_t)row * k + lane] = -1;
      a.p[(uint64_t)row * k + lane] = __uint_as_float(0x7FC00000u);
    }
    if (lane == 0) {
      a.sg[row] = __uint_as_float(0x7FC00000u);
      __hip_atomic_fetch_add(&a.sync[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      route_done(a, state);
    }
    return;
  }
  const float cv = remote ? __uint_as_float((uint32_t)word) : val;
  const int ci = remote ? (int)((word >> 32) & 0xFFu) : id;
  const float c = s_gate;
  if (a.logits && lane == 0) a.logits[(uint64_t)row * (E + 1) + E] = c;
  const float vv[1] = {cv};
  const uint32_t kk[1] = {(lane < k || remote) ? pick_key(cv) : 0u};
  const int ii[1] = {ci};
  pick_and_store_n<1>(a, row, kk, vv, ii, c, lane, scr);
  if (lane == 0) route_done(a, state);
}

// Prompt chunks: logits of 32 rows x 64 experts per workgroup on 16-bit
// MFMA. The K axis is split over 8 waves by 256-wide scale blocks (wave w
// takes blocks w, w + 8, ...); a wave issues all loads of a block (32 rows of
// activations, 64 rows of codes, their scales) before its first MFMA, so one
// memory latency covers the block. The codes enter as exact fp16 values q/16
// (affine) or (u - 8)/16 (symmetric), the activations as fp16 (bf16 converts
// exactly in fp16's normal range), so every product is exact and each
// group's MFMA sum is scaled in fp32: logit += 16 s * acc_g, then for affine
// codes + b_g * sum_g x, group by group. The 8 wave partials are added in a
// fixed order. Same values as the per-row form up to the order of the fp32
// sums, and a row's value does not depend on the other rows of the chunk.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int RM_WAVES = 8;

// One 256-wide block kb of one wave: xr points at the lane's activation row
// (row col of the tile) at k offset 8 hsel.
template <int FR, int ACT16>
__device__ __forceinline__ void route_mfma_block(const RouteArgs& a, const uint16_t* xr, int t, int kb, int nch,
                                                 int nkb, int col, int hsel, float* xs, float16_t (&tot)[2]) {
  constexpr int G = Fmt<FR>::G, NG = KBLK / G, KPG = G / 16;
  const uint8_t* codes = a.base + a.r_off;
  const uint8_t* scales = a.base + a.r_soff + sblk_off<FR>(t, kb, nkb);
  uint4 xv[16];
  uint32_t cw[2][16];
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) xv[kk] = *reinterpret_cast<const uint4*>(xr + KBLK * kb + 16 * kk);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
      cw[nt][kk] = *reinterpret_cast<const uint32_t*>(codes + chunk_off<FR>(t, 8 * kb + kk / 2, nch) +
                                                      (uint64_t)(32 * nt + col) * Fmt<FR>::CB +
                                                      4 * (2 * (kk % 2) + hsel));
  // scales of rows 32 nt + col: NG groups each (bf16 scale/bias pairs, or fp16 scales)
  uint32_t sv[2][NG];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if constexpr (Fmt<FR>::AFF) {
      const uint4 q = reinterpret_cast<const uint4*>(scales)[32 * nt + col];
      sv[nt][0] = q.x; sv[nt][1] = q.y; sv[nt][2] = q.z; sv[nt][3] = q.w;
    } else {
      const uint32_t q = reinterpret_cast<const uint32_t*>(scales)[32 * nt + col];
      sv[nt][0] = q & 0xFFFFu;
      sv[nt][1] = q >> 16;
    }
  }
  __builtin_amdgcn_sched_barrier(0);    // every load of the block issued before the first MFMA
  static_assert(!Fmt<FR>::AFF || NG == 4, "affine router groups of 64");
  static_assert(Fmt<FR>::AFF || NG == 2, "symmetric router groups of 128");
  const half2v off = Fmt<FR>::AFF ? half2v{(f16)1.0f, (f16)1.0f} : half2v{(f16)1.5f, (f16)1.5f};
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    float16_t acc[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[nt][v] = 0.f;
    float xsum = 0.f;
#pragma unroll
    for (int j = 0; j < KPG; ++j) {
      const int kk = KPG * gi + j;
      const uint32_t xw[4] = {xv[kk].x, xv[kk].y, xv[kk].z, xv[kk].w};
      uint32_t ah[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = act_to_f((uint16_t)(xw[i] & 0xFFFFu), ACT16);
        const float hi = act_to_f((uint16_t)(xw[i] >> 16), ACT16);
        if constexpr (Fmt<FR>::AFF) {
          xsum += lo;
          xsum += hi;
        }
        if constexpr (ACT16) {
          ah[i] = xw[i];
        } else {
          half2v hp;
          hp.x = (f16)lo;
          hp.y = (f16)hi;
          ah[i] = as_u(hp);
        }
      }
      const half8_t A = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4*>(ah));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        uint32_t o[4], pv[16];
        const uint32_t wv[4] = {cw[nt][kk], 0u, 0u, 0u};
        unpack_chunk<F_Q4>(wv, pv);      // pairs 0..3 (this word): 1 + q/16
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = as_u(as_h2(pv[i]) - off);
        const half8_t B = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4*>(o));
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B, acc[nt], 0, 0, 0);
      }
    }
    if constexpr (Fmt<FR>::AFF) {
      const float xs_row = xsum + __shfl_xor(xsum, 32);
      if (hsel == 0) xs[32 * gi + col] = xs_row;
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float s16 = 16.0f * (Fmt<FR>::AFF ? bf16_to_f(sv[nt][gi] & 0xFFFFu) : f16_bits_to_f(sv[nt][gi]));
#pragma unroll
      for (int v = 0; v < 16; ++v) tot[nt][v] = fmaf(s16, acc[nt][v], tot[nt][v]);
    }
  }
  if constexpr (Fmt<FR>::AFF) {
    // + b_g * (sum over the group of the row's activations), accumulator rows
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float b = bf16_to_f(sv[nt][gi] >> 16);
#pragma unroll
        for (int v = 0; v < 16; ++v)
          tot[nt][v] = fmaf(b, xs[32 * gi + 8 * (v / 4) + 4 * hsel + (v % 4)], tot[nt][v]);
      }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int FR, int ACT16>
__global__ __launch_bounds__(64 * RM_WAVES) void k_route_mfma(RouteArgs a, const uint16_t* __restrict__ x) {
  static_assert(FR == F_Q4 || FR == F_S4, "16-bit MFMA router reads 4-bit codes");
  __shared__ float part[4][32][64];
  __shared__ float xs_all[RM_WAVES][128];
  const int H = a.H, E = a.E, nch = H / 32, nkb = H / KBLK;
  const int t = blockIdx.x, r0 = blockIdx.y * 32;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, hsel = lane >> 5;
  const int arow = min(r0 + col, a.R - 1);
  const uint16_t* xr = x + (uint64_t)arow * H + 8 * hsel;
  float16_t tot[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int v = 0; v < 16; ++v) tot[nt][v] = 0.f;
  for (int kb = w; kb < nkb; kb += RM_WAVES)
    route_mfma_block<FR, ACT16>(a, xr, t, kb, nch, nkb, col, hsel, xs_all[w], tot);
  // partials: waves 4..7 onto waves 0..3, then the four in order
  if (w >= 4) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) part[w - 4][16 * nt + v][lane] = tot[nt][v];
  }
  __syncthreads();
  if (w < 4) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) part[w][16 * nt + v][lane] = tot[nt][v] + part[w][16 * nt + v][lane];
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 32 * 64; q += 64 * RM_WAVES) {
    const int slot = q / 64, ln = q % 64;            // (nt, v) index and lane
    const int nt = slot / 16, v = slot % 16;
    const int rr = 8 * (v / 4) + 4 * (ln >> 5) + (v % 4);
    const int row = r0 + rr, e = t * 64 + 32 * nt + (ln & 31);
    float l = part[0][slot][ln];
    l += part[1][slot][ln];
    l += part[2][slot][ln];
    l += part[3][slot][ln];
    if (row < a.R && e < E) a.lg_ws[(uint64_t)row * E + e] = l;
  }
}

// One wave per row: gate-row logit, top k, weights, sigmoid gate.
template <int FG, int ACT16>
__global__ __launch_bounds__(256) void k_route_pick(RouteArgs a, const uint16_t* __restrict__ x) {
  const int E = a.E, k = a.k;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x * 4 + wv;
  __shared__ uint32_t scratch[4][24];
  uint32_t* scr = scratch[wv];
  if (row >= a.R) return;
  float v[4];
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    const int ec = min(e, E - 1);
    const float l = a.lg_ws[(uint64_t)row * E + ec];
    v[i] = a.bias ? l + a.bias[ec] : l;
    key[i] = e < E ? pick_key(v[i]) : 0u;     // key 0 marks taken / absent
  }
  // gate-row logit: lane parts, 16-lane rows by DPP, then the 4 rows in order
  const float s16 = sum16(gate_row_part<FG, ACT16>(a, x + (uint64_t)row * a.H, lane));
  float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 0));
  c += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 16));
  c += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 32));
  c += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 48));
  if (a.logits) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i < E) a.logits[(uint64_t)row * (E + 1) + lane + 64 * i] = v[i];
    if (lane == 0) a.logits[(uint64_t)row * (E + 1) + E] = c;
  }
  pick_and_store(a, row, key, v, c, lane, scr);
}

// decode batches up to this many rows take the one-launch router
constexpr int ROUTE_FUSED_MAX_ROWS = 32;

template <int FR, int FG, int ACT16>
static hipError_t launch_route_t(const RouteArgs& a, hipStream_t s, hipEvent_t* ev) {
  const int nw = min(8, a.H / KBLK);
  if (a.R <= ROUTE_FUSED_MAX_ROWS) {
    launch_k(k_route<FR, FG, ACT16>, dim3(a.E / 64, a.R), dim3(64 * (nw + 1)), 0, s, ev, 0, a, a.x);
    return hipGetLastError();
  }
  hipEvent_t e0[2] = {ev ? ev[0] : nullptr, nullptr}, e1[2] = {nullptr, ev ? ev[1] : nullptr};
  if constexpr (FR == F_Q4 || FR == F_S4) {
    if (a.H % KBLK == 0)     // whole 256-wide blocks over 8 waves
      launch_k(k_route_mfma<FR, ACT16>, dim3(a.E / 64, (a.R + 31) / 32), dim3(64 * RM_WAVES), 0, s, e0, 0, a, a.x);
    else
      launch_k(k_route_logits<FR, ACT16, 8>, dim3(a.E / 64, (a.R + 7) / 8), dim3(64 * nw), 0, s, e0, 0, a, a.x);
  } else {
    launch_k(k_route_logits<FR, ACT16, 8>, dim3(a.E / 64, (a.R + 7) / 8), dim3(64 * nw), 0, s, e0, 0, a, a.x);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  launch_k(k_route_pick<FG, ACT16>, dim3((a.R + 3) / 4), dim3(256), 0, s, e1, 0, a, a.x);
  return hipGetLastError();
}

// The exact chunk form: logits on the vector units (k_route_logits, whose
// per-row slice dots and wave sums are those of k_route) and the one-wave
// pick (the same order and weights as k_route's two-level pick), for any
// number of rows: every row's ids, weights and gate equal its one-row
// decode step's.
template <int FR, int FG, int ACT16>
static hipError_t launch_route_exact_t(const RouteArgs& a, hipStream_t s, hipEvent_t* ev) {
  const int nw = min(8, a.H / KBLK);
  hipEvent_t e0[2] = {ev ? ev[0] : nullptr, nullptr}, e1[2] = {nullptr, ev ? ev[1] : nullptr};
  launch_k(k_route_logits<FR, ACT16, 8>, dim3(a.E / 64, (a.R + 7) / 8), dim3(64 * nw), 0, s, e0, 0, a, a.x);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  launch_k(k_route_pick<FG, ACT16>, dim3((a.R + 3) / 4), dim3(256), 0, s, e1, 0, a, a.x);
  return hipGetLastError();
}

template <int FR, int ACT16>
static hipError_t launch_route_exact_g(int fg, const RouteArgs& a, hipStream_t s, hipEvent_t* ev) {
  switch (fg) {
    case F_Q4: return launch_route_exact_t<FR, F_Q4, ACT16>(a, s, ev);
    case F_Q8: return launch_route_exact_t<FR, F_Q8, ACT16>(a, s, ev);
    case F_S4: return launch_route_exact_t<FR, F_S4, ACT16>(a, s, ev);
    case F_DENSE: return launch_route_exact_t<FR, F_DENSE, ACT16>(a, s, ev);
  }
  return hipErrorInvalidValue;
}

template <int FR>
static hipError_t launch_route_exact_a(int fg, const RouteArgs& a, hipStream_t s, hipEvent_t* ev) {
  return a.act_fp16 ? launch_route_exact_g<FR, 1>(fg, a, s, ev) : launch_route_exact_g<FR, 0>(fg, a, s, ev);
}

hipError_t launch_route_exact(int fr, int fg, const RouteArgs& a, hipStream_t s, hipEvent_t* ev) {
  switch (fr) {
    case F_Q4: return launch_route_exact_a<F_Q4>(fg, a, s, ev);
    case F_Q8: return launch_route_exact_a<F_Q8>(fg, a, s, ev);
    case F_S4: return launch_route_exact_a<F_S4>(fg, a, s, ev);
  }
  return hipErrorInvalidValue;
}

template <int FR, int ACT16>
static hipError_t launch_route_g(int fg, const RouteArgs& a, hipStream_t s, hipEvent_t* ev) {
  switch (fg) {
    case F_Q4: return launch_route_t<FR, F_Q4, ACT16>(a, s, ev);
    case F_Q8: return launch_route_t<FR, F_Q8, ACT16>(a, s, ev);
    case F_S4: return launch_route_t<FR, F_S4, ACT16>(a, s, ev);
    case F_DENSE: return launch_route_t<FR, F_DENSE, ACT16>(a, s, ev);
  }
  return hipErrorInvalidValue;
}

template <int FR>
static hipError_t launch_route_a(int fg, const RouteArgs& a, hipStream_t s, hipEvent_t* ev) {
  return a.act_fp16 ? launch_route_g<FR, 1>(fg, a, s, ev) : launch_route_g<FR, 0>(fg, a, s, ev);
}

hipError_t launch_route(int fr, int fg, const RouteArgs& a, hipStream_t s, hipEvent_t* ev) {
  switch (fr) {
    case F_Q4: return launch_route_a<F_Q4>(fg, a, s, ev);
    case F_Q8: return launch_route_a<F_Q8>(fg, a, s, ev);
    case F_S4: return launch_route_a<F_S4>(fg, a, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
