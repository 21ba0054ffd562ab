// Router: fp32 logits over the experts and the shared expert's gate row,
// top-k with ties to the lower id, renormalised weights, sigmoid gate
// ("qwen3_5_moe on native CUDA with 3-bit routed experts #803", Activity,
// comment "Progress on the 4-bit gate").
//
// The logits are spread over the chip: one workgroup per (tile of 64
// experts, row), lanes owning router rows exactly as the expert kernels own
// weight rows, activations through scalar loads. The last tile workgroup of
// a row picks the top k as k rounds of a wave-wide arg-max under the total
// order (NaN, value desc, id asc) built from DPP moves, then forms
// exp(l - l_top) / sum and sigmoid(gate).
#include "moe_kernels.h"
#include "moe_launch.h"
#include "moe_dispatch.h"

namespace moe {

// gate-row logit part of one lane (chunks lane, lane+64, ...), before the
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

// One workgroup per (tile of 64 experts, row); wave w sums the slices
// w, w + nw, ... in ascending order, the waves are added in wave order. The
// last of a row's tile workgroups to finish (a per-row arrival counter in the
// workspace, reset by that workgroup) picks the row's top k.
template <int FR, int FG, int ACT16>
__global__ __launch_bounds__(512) void k_route(RouteArgs a, const uint16_t* __restrict__ x) {
  __shared__ float red[8][64];
  __shared__ int s_last;
  __shared__ __align__(16) uint32_t lxs[8][128];    // per-wave activation slice
  const int H = a.H, E = a.E, k = a.k, nsl = H / KBLK, nch = H / 32;
  const int t = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int nw = blockDim.x >> 6, ntile = E / 64;
  const uint16_t* xr = x + (uint64_t)row * H;
  const uint8_t* rc = a.base + a.r_off;
  const uint8_t* rs = a.base + a.r_soff;
  float gpart = 0.f;
  const bool gate_job = (t == 0 && w == nw - 1);
  if (gate_job) gpart = gate_row_part<FG, ACT16>(a, xr, lane);
  float out = 0.f;
  for (int sl = w; sl < nsl; sl += nw) {
    uint32_t wc[8][Fmt<FR>::WORDS];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) load_chunk<FR>(rc + chunk_off<FR>(t, sl * 8 + cc, nch), lane, wc[cc]);
    const uint16_t* xs[1] = {xr + sl * KBLK};
    float part[1];
    slice_dot<FR, 1, ACT16>(wc, rs + sblk_off<FR>(t, sl, nsl), lane, xs, 1, lxs[w], part);
    out += part[0];
  }
  red[w][lane] = out;
  if (gate_job) {
    // wave sum of the gate-row parts: 16-lane rows by DPP, then the 4 rows in order
    const float s16 = sum16(gpart);
    float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 0));
    c += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 16));
    c += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 32));
    c += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 48));
    if (lane == 0) a.gl_ws[row] = c;
  }
  __syncthreads();
  if (w == 0) {
    float l = 0.f;
    for (int q = 0; q < nw; ++q) l += red[q][lane];
    a.lg_ws[(uint64_t)row * E + 64 * t + lane] = l;
  }
  __threadfence();                         // logits visible device-wide before the arrival
  __syncthreads();
  if (tid == 0) {
    const unsigned old = atomicAdd(&a.cnt[row], 1u);
    s_last = old == (unsigned)(ntile - 1);
    if (s_last) a.cnt[row] = 0u;           // every tile of this row has arrived
  }
  __syncthreads();
  if (!s_last || w != 0) return;
  __threadfence();
  // wave 0 of the last tile workgroup: the pick
  float v[4], bias[4], lv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = min(lane + 64 * i, E - 1);
    lv[i] = __hip_atomic_load(&a.lg_ws[(uint64_t)row * E + e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bias[i] = a.bias ? a.bias[e] : 0.f;
  }
  const float c = __hip_atomic_load(&a.gl_ws[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // candidates of this lane: experts lane + 64 i; key 0 marks taken/absent
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    v[i] = a.bias ? lv[i] + bias[i] : lv[i];
    key[i] = e < E ? pick_key(v[i]) : 0u;
  }
  if (a.logits) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i < E) a.logits[(uint64_t)row * (E + 1) + lane + 64 * i] = v[i];
    if (lane == 0) a.logits[(uint64_t)row * (E + 1) + E] = c;
  }
  // k rounds (fully unrolled, k <= 8): the wave-wide largest key, ties to the
  // lowest id; lane j keeps the j-th pick
  float my_v = 0.f, top = 0.f;
  int my_i = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k) {
      const uint32_t bk = max(max(key[0], key[1]), max(key[2], key[3]));
      const uint32_t m = wave_max_u32(bk);
      // lowest id holding the best key (ids lane + 64 i grow with i)
      uint32_t cid = 0xFFFFFFFFu;
#pragma unroll
      for (int i = 3; i >= 0; --i) cid = key[i] == m ? (uint32_t)(lane + 64 * i) : cid;
      const int bi = (int)wave_min_u32(cid);
      float bv = v[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) bv = (bi == lane + 64 * i) ? v[i] : bv;
      bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), bi & 63));
#pragma unroll
      for (int i = 0; i < 4; ++i) key[i] = (bi == lane + 64 * i) ? 0u : key[i];
      if (j == 0) top = bv;
      my_v = lane == j ? bv : my_v;
      my_i = lane == j ? bi : my_i;
    }
  }
  // weights exp(l_j - l_top) / sum over the k picks, summed in pick order
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

template <int FR, int FG>
static hipError_t launch_route_t(const RouteArgs& a, hipStream_t s, hipEvent_t* ev) {
  const int nw = min(8, a.H / KBLK);
  if (a.act_fp16)
    launch_k(k_route<FR, FG, 1>, dim3(a.E / 64, a.R), dim3(64 * nw), 0, s, ev, 0, a, a.x);
  else
    launch_k(k_route<FR, FG, 0>, dim3(a.E / 64, a.R), dim3(64 * nw), 0, s, ev, 0, a, a.x);
  return hipGetLastError();
}

template <int FR>
static hipError_t launch_route_g(int fg, const RouteArgs& a, hipStream_t s, hipEvent_t* ev) {
  switch (fg) {
    case F_Q4: return launch_route_t<FR, F_Q4>(a, s, ev);
    case F_Q8: return launch_route_t<FR, F_Q8>(a, s, ev);
    case F_S4: return launch_route_t<FR, F_S4>(a, s, ev);
    case F_DENSE: return launch_route_t<FR, F_DENSE>(a, s, ev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_route(int fr, int fg, const RouteArgs& a, hipStream_t s, hipEvent_t* ev) {
  switch (fr) {
    case F_Q4: return launch_route_g<F_Q4>(fg, a, s, ev);
    case F_Q8: return launch_route_g<F_Q8>(fg, a, s, ev);
    case F_S4: return launch_route_g<F_S4>(fg, a, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
