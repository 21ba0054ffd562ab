// Decode path: routed + shared experts for up to 16 independent rows.
//
// gate/up (k_dec_gateup): one workgroup per (unit, 64-row tile of the
// interleaved gate/up matrix), one wave per 256-wide K slice. A unit is a
// slot (row r, pick j) whose expert no earlier slot picked, or the shared
// expert for one row: it streams the tile's packed codes once (coalesced 128-bit loads,
// lane = weight row) for every row that picked the expert, so rows sharing
// an expert share its reads ("Native server: --backend xpu for Nemotron on
// Intel Arc", review comments: each extra row costs more because more
// distinct experts are read; the gain needs expert reads shared across
// rows). Each wave finds its unit from the picks with one ballot (no LDS, no
// barrier) and reads activations with uniform loads straight into
// v_dot2_f32_bf16 / v_dot2_f32_f16. Output: h = silu(g)*u split into fp16
// hi + lo parts (22 significant bits) plus per-32 chunk sums, for down.
//
// down + combine (k_dec_down): one workgroup per (row, 64-column tile of y),
// k waves. Wave j computes routed slot j's output columns over the full
// intermediate axis plus 1/k of the shared expert's (added in wave order);
// wave 0 then forms y = sum_j p_j e_j + sigma e_shared in slot order. Blocks
// are mapped so the rows of one tile run on one XCD and share the shared
// expert's tile in that XCD's L2.
//
// Every row's arithmetic is fixed (K slices owned by fixed waves, chunks
// and groups in K order, slices reduced in slice order, slots combined in
// pick order, shared last) and independent of the other rows, so a row's y
// is bit-identical alone or in a batch ("Sage-A1.5 ... #1329", Limits to
// agree on: the per-row kernels keep one stream's sum order).
#include "moe_kernels.h"
#include "moe_launch.h"
#include "moe_dispatch.h"

namespace moe {

// Rows of one unit, one at a time: the wave's codes stay in registers (one
// K slice per wave when H <= 2048) and each row re-runs the unpack, which is
// free for the usual single-row unit.
template <int F, int ACT16>
__device__ __forceinline__ void gu_body(const DecodeArgs& a, const uint16_t* __restrict__ x,
                                        const uint8_t* codes, const uint8_t* scales,
                                        int t, int nrows, int shared_row, uint64_t m0, uint64_t m1,
                                        float* red, uint32_t* lx) {
  // wave wv owns the K slices wv, wv + nw, ...
  const int H = a.H, k = a.k, nsl = H / KBLK, nch = H / 32;
  const int tid = threadIdx.x, lane = tid & 63, nw = blockDim.x >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  uint32_t w[8][Fmt<F>::WORDS];
  if (wv < nsl) {
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) load_chunk<F>(codes + chunk_off<F>(t, wv * 8 + cc, nch), lane, w[cc]);
  }
  for (int i = 0; i < nrows; ++i) {
    int r = shared_row, j = k;
    if (shared_row < 0) {
      int s;
      if (m0) { s = __ffsll((unsigned long long)m0) - 1; m0 &= m0 - 1; }
      else { s = 64 + __ffsll((unsigned long long)m1) - 1; m1 &= m1 - 1; }
      r = s / k;
      j = s % k;
    }
    float out = 0.f;
    for (int sl = wv; sl < nsl; sl += nw) {
      if (sl != wv) {
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) load_chunk<F>(codes + chunk_off<F>(t, sl * 8 + cc, nch), lane, w[cc]);
      }
      const uint16_t* xs[1] = {x + (uint64_t)r * H + sl * KBLK};
      float part[1];
      slice_dot<F, 1, ACT16>(w, scales + sblk_off<F>(t, sl, nsl), lane, xs, 1, lx + wv * 128, part);
      out += part[0];
    }
    red[wv * 64 + lane] = out;
    __syncthreads();
    if (tid < 64) {
      const int c = tid & 31;
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
      if (tid < 32) {
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
    __syncthreads();
  }
}

// grid (gate/up tiles, R*k + R units): unit u < R*k is slot u when no earlier
// slot picked its expert; unit R*k + r is the shared expert for row r. With
// the linear block index t + 16u, every unit of tile t runs on XCD t % 8, so
// the shared expert's rows re-read its tile from that XCD's L2.
template <int FR, int FS, int ACT16>
__global__ __launch_bounds__(512) void k_dec_gateup(DecodeArgs a, const uint16_t* __restrict__ x) {
  extern __shared__ __align__(16) float red[];   // [waves][64], then per-wave x slices
  uint32_t* lx = reinterpret_cast<uint32_t*>(red + (blockDim.x >> 6) * 64);
  const int t = blockIdx.x, u = blockIdx.y, lane = threadIdx.x & 63;
  const int nslot = a.R * a.k;
  if (u < nslot) {
    const int e = a.ids[u];
    if (e < 0 || e >= a.E) return;
    if (t >= 2 * a.rt.inter / 64) return;
    const int id0 = lane < nslot ? a.ids[lane] : -1;
    const int id1 = lane + 64 < nslot ? a.ids[lane + 64] : -1;
    const uint64_t m0 = __ballot(id0 == e), m1 = __ballot(id1 == e);
    const int first = m0 ? __ffsll((unsigned long long)m0) - 1 : 64 + __ffsll((unsigned long long)m1) - 1;
    if (first != u) return;        // an earlier slot's unit serves this expert
    const uint8_t* blk = a.base + a.rt.base_off + (uint64_t)e * a.rt.stride;
    gu_body<FR, ACT16>(a, x, blk + a.rt.gu_codes, blk + a.rt.gu_scales, t, __popcll(m0) + __popcll(m1),
                       -1, m0, m1, red, lx);
  } else {
    if (t >= 2 * a.sh.inter / 64) return;
    const uint8_t* blk = a.base + a.sh.base_off;
    gu_body<FS, ACT16>(a, x, blk + a.sh.gu_codes, blk + a.sh.gu_scales, t, 1, u - nslot, 0, 0, red, lx);
  }
}

// Part of one slot's 64 output columns of tile t over chunks c0 .. c0+n-1 of
// the intermediate axis (chunk c covers 32 intermediate indices): load the
// codes (dn_load), then the dot in chunk order (dn_dot). n <= MAXC.
template <int F, int MAXC>
__device__ __forceinline__ void dn_load(const uint8_t* codes, int I, int t, int lane, int c0, int n,
                                        uint32_t (&w)[MAXC][Fmt<F>::WORDS]) {
  const int nch = I / 32;
#pragma unroll
  for (int q = 0; q < MAXC; ++q)
    if (q < n) load_chunk<F>(codes + chunk_off<F>(t, c0 + q, nch), lane, w[q]);
}
template <int F, int MAXC>
__device__ __forceinline__ float dn_dot(const uint32_t (&w)[MAXC][Fmt<F>::WORDS],
                                        const uint32_t* __restrict__ hh, const uint32_t* __restrict__ hl,
                                        const float* __restrict__ hc, const uint8_t* scales, int I,
                                        int t, int lane, int c0, int n) {
  constexpr int CPG = Fmt<F>::G / 32;
  const int nkb = I / KBLK;
  float out = 0.f;
#pragma unroll
  for (int q0 = 0; q0 < MAXC; q0 += CPG) {
    if (q0 < n) {
      // one group: CPG chunks from chunk c0 + q0 (c0 is a multiple of CPG)
      const int c = c0 + q0, sl = c / 8, gi = (c % 8) / CPG;
      float ms, bm;
      group_coef<F>(scales + sblk_off<F>(t, sl, nkb), lane, gi, ms, bm);
      float acc = 0.f, X = 0.f;
#pragma unroll
      for (int cc = 0; cc < CPG; ++cc) {
        uint32_t v[16], ph[16], pl[16];
        unpack_chunk<F>(w[q0 + cc], v);
#pragma unroll
        for (int p = 0; p < 16; ++p) { ph[p] = hh[16 * (c + cc) + p]; pl[p] = hl[16 * (c + cc) + p]; }
        acc = dot_chunk_h(v, ph, acc);
        acc = dot_chunk_h(v, pl, acc);
        X += hc[c + cc];
      }
      out = fmaf(ms, acc, out);
      out = fmaf(bm, X, out);
    }
  }
  return out;
}

// down + combine: one workgroup per (row, 64-column tile of y) with k waves.
// Wave j computes routed slot j over the full intermediate axis and 1/k of
// the shared expert's chunks; the k shared parts are added in wave order.
// Wave 0 then forms y = sum_j p_j e_j + sigma e_shared in slot order.
template <int FR, int FS>
__global__ __launch_bounds__(512) void k_dec_down(DecodeArgs a, const uint16_t* __restrict__ hhi,
                                                  const uint16_t* __restrict__ hlo,
                                                  const float* __restrict__ hcs) {
  __shared__ float es[8][64];
  __shared__ float ps[8][64];
  const int T = a.H / 64, R = a.R, k = a.k;
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
  const int j = __builtin_amdgcn_readfirstlane(tid >> 6);   // slot of this wave, uniform
  // routed slot j: all its chunks (blocks of 16 when inter > 512); the
  // wave's share of the shared expert (whole groups, split over k waves) is
  // loaded together with the first block
  const uint64_t rsj = (uint64_t)r * (k + 1) + j, rsk = (uint64_t)r * (k + 1) + k;
  const int e = a.ids[r * k + j];
  const bool valid = e >= 0 && e < a.E;
  const uint8_t* rblk = a.base + a.rt.base_off + (uint64_t)(valid ? e : 0) * a.rt.stride;
  const uint8_t* sblk = a.base + a.sh.base_off;
  const int gch = Fmt<FS>::G / 32, ngr = (a.sh.inter / 32) / gch, per = (ngr + k - 1) / k;
  const int g0 = min(ngr, j * per), g1 = min(ngr, g0 + per);
  const int sc0 = g0 * gch, sn = min(8, (g1 - g0) * gch);
  const int rn = a.rt.inter / 32;
  uint32_t wr[16][Fmt<FR>::WORDS], wsh[8][Fmt<FS>::WORDS];
  dn_load<FR, 16>(rblk + a.rt.dn_codes, a.rt.inter, t, lane, 0, min(16, rn), wr);
  dn_load<FS, 8>(sblk + a.sh.dn_codes, a.sh.inter, t, lane, sc0, sn, wsh);
  const uint32_t* hhj = reinterpret_cast<const uint32_t*>(hhi + rsj * a.Imax);
  const uint32_t* hlj = reinterpret_cast<const uint32_t*>(hlo + rsj * a.Imax);
  float e_out = dn_dot<FR, 16>(wr, hhj, hlj, hcs + rsj * (a.Imax / 32), rblk + a.rt.dn_scales,
                               a.rt.inter, t, lane, 0, min(16, rn));
  for (int cb = 16; cb < rn; cb += 16) {
    dn_load<FR, 16>(rblk + a.rt.dn_codes, a.rt.inter, t, lane, cb, min(16, rn - cb), wr);
    e_out += dn_dot<FR, 16>(wr, hhj, hlj, hcs + rsj * (a.Imax / 32), rblk + a.rt.dn_scales,
                            a.rt.inter, t, lane, cb, min(16, rn - cb));
  }
  if (!valid) e_out = 0.f;
  float s_out = 0.f;
  if (sn > 0) {
    const uint32_t* hhk = reinterpret_cast<const uint32_t*>(hhi + rsk * a.Imax);
    const uint32_t* hlk = reinterpret_cast<const uint32_t*>(hlo + rsk * a.Imax);
    s_out = dn_dot<FS, 8>(wsh, hhk, hlk, hcs + rsk * (a.Imax / 32), sblk + a.sh.dn_scales, a.sh.inter,
                          t, lane, sc0, sn);
    for (int cb = sc0 + sn; cb < g1 * gch; cb += 8) {
      const int m = min(8, g1 * gch - cb);
      dn_load<FS, 8>(sblk + a.sh.dn_codes, a.sh.inter, t, lane, cb, m, wsh);
      s_out += dn_dot<FS, 8>(wsh, hhk, hlk, hcs + rsk * (a.Imax / 32), sblk + a.sh.dn_scales,
                             a.sh.inter, t, lane, cb, m);
    }
  }
  es[j][lane] = e_out;
  ps[j][lane] = s_out;
  if (a.tap_e) a.tap_e[((uint64_t)r * (k + 1) + j) * a.H + 64 * t + lane] = e_out;
  __syncthreads();
  if (j == 0) {
    float sh = 0.f;
    for (int q = 0; q < k; ++q) sh += ps[q][lane];
    if (a.tap_e) a.tap_e[((uint64_t)r * (k + 1) + k) * a.H + 64 * t + lane] = sh;
    float y = 0.f;
    for (int q = 0; q < k; ++q) y = fmaf(a.p[r * k + q], es[q][lane], y);
    y = fmaf(a.sg[r], sh, y);
    a.y[(uint64_t)r * a.H + 64 * t + lane] = y;
  }
}

// ------------------------------------------------------------------ launch
template <int FR, int FS>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  const int nw = min(8, a.H / KBLK);
  const int units = a.R * a.k + a.R;
  const int gu_tiles = 2 * a.Imax / 64;
  const size_t smem = (size_t)nw * 64 * 4 + (size_t)nw * 512;
  if (a.act_fp16)
    launch_k(k_dec_gateup<FR, FS, 1>, dim3(gu_tiles, units), dim3(64 * nw), smem, s, ev, 0, a, a.x);
  else
    launch_k(k_dec_gateup<FR, FS, 0>, dim3(gu_tiles, units), dim3(64 * nw), smem, s, ev, 0, a, a.x);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  launch_k(k_dec_down<FR, FS>, dim3((a.H / 64) * a.R), dim3(64 * a.k), 0, s, ev, 2, a,
           (const uint16_t*)a.hhi, (const uint16_t*)a.hlo, (const float*)a.hc);
  return hipGetLastError();
}

template <int FR>
static hipError_t launch_decode_s(int fs, const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  switch (fs) {
    case F_Q4: return launch_decode_t<FR, F_Q4>(a, s, ev);
    case F_Q3: return launch_decode_t<FR, F_Q3>(a, s, ev);
    case F_S4: return launch_decode_t<FR, F_S4>(a, s, ev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(int fr, int fs, const DecodeArgs& a, hipStream_t s, hipEvent_t* ev) {
  switch (fr) {
    case F_Q4: return launch_decode_s<F_Q4>(fs, a, s, ev);
    case F_Q3: return launch_decode_s<F_Q3>(fs, a, s, ev);
    case F_S4: return launch_decode_s<F_S4>(fs, a, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
