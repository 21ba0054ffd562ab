// Router kernel: fp32 logits over the experts and the shared expert's gate
// row, top-k with ties to the lower id, renormalised weights, sigmoid gate.
// ("qwen3_5_moe on native CUDA with 3-bit routed experts #803", Activity,
//  comment "Progress on the 4-bit gate".)
//
// One workgroup per row. Lanes own router rows (experts) exactly as the
// expert kernels own weight rows; the K axis is cut into 256-wide slices,
// each wave summing a fixed residue class of slices in ascending order, and
// the waves of a tile are reduced in LDS in wave order. The gate row is
// one more job whose lanes walk the K axis. The pick runs in wave 0 as k
// rounds of a wave-wide arg-max under the total order
// (NaN, value desc, id asc) built from shuffles.
#include "moe_kernels.h"
#include "moe_launch.h"

namespace moe {

constexpr int RT_WAVES = 16;

template <int FG>
__device__ __forceinline__ float gate_row_part(const uint8_t* codes, const uint8_t* scales,
                                               const half2v* xh, const float* xc, int H, int lane) {
  float part = 0.f;
  const int nch = H / 32;
  for (int c = lane; c < nch; c += 64) {
    float contrib;
    if constexpr (FG == F_DENSE) {
      const uint16_t* w = reinterpret_cast<const uint16_t*>(codes) + 32 * c;
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const half2v xv = xh[16 * c + i];
        a = fmaf(bf16_to_f(w[2 * i]), (float)xv.x, a);
        a = fmaf(bf16_to_f(w[2 * i + 1]), (float)xv.y, a);
      }
      contrib = a;
    } else {
      uint32_t w[8], v[16];
      const uint32_t* src = reinterpret_cast<const uint32_t*>(codes + (uint64_t)c * Fmt<FG>::CB);
#pragma unroll
      for (int i = 0; i < Fmt<FG>::WORDS; ++i) w[i] = src[i];
      unpack_chunk<FG>(w, v);
      const float acc = dot_chunk(v, xh + 16 * c, 0.f);
      const int g = (32 * c) / Fmt<FG>::G;
      float ms, bm;
      if constexpr (Fmt<FG>::AFF) {
        const uint32_t sv = reinterpret_cast<const uint32_t*>(scales)[g];
        const float s = bf16_to_f(sv & 0xFFFFu), b = bf16_to_f(sv >> 16);
        ms = (float)Fmt<FG>::M * s;
        bm = b - ms;
      } else {
        const float s = f16_bits_to_f(reinterpret_cast<const uint16_t*>(scales)[g]);
        ms = (float)Fmt<FG>::M * s;
        bm = -8.0f * s - ms;
      }
      contrib = fmaf(bm, xc[c], ms * acc);
    }
    part += contrib;
  }
  // fixed butterfly over the wave
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  return part;
}

template <int FR, int FG>
__global__ __launch_bounds__(64 * RT_WAVES) void k_route(RouteArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int H = a.H, E = a.E, k = a.k;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  half2v* xh = reinterpret_cast<half2v*>(smem);                 // [H/2]
  float* xc = reinterpret_cast<float*>(xh + H / 2);              // [H/32]
  float* red = xc + H / 32;                                      // [wpt][E]
  float* lg = red + RT_WAVES * E;                                // [E + 1]

  // stage x as fp16 pairs and the per-chunk sums of the fp16 values
  const uint32_t* xr = reinterpret_cast<const uint32_t*>(a.x + (uint64_t)row * H);
  for (int i = tid; i < H / 2; i += blockDim.x) {
    const uint32_t v = xr[i];
    half2v h;
    h.x = (f16)act_to_f((uint16_t)(v & 0xFFFFu), a.act_fp16);
    h.y = (f16)act_to_f((uint16_t)(v >> 16), a.act_fp16);
    xh[i] = h;
  }
  __syncthreads();
  for (int c = tid; c < H / 32; c += blockDim.x) {
    float s = 0.f;
    for (int i = 0; i < 16; ++i) {
      const half2v h = xh[16 * c + i];
      s += (float)h.x;
      s += (float)h.y;
    }
    xc[c] = s;
  }
  __syncthreads();

  // waves 0 .. ntile*wpt-1: tile t = wave / wpt, part q = wave % wpt takes
  // the slices q, q+wpt, ... in ascending order; the last wave: the gate row
  const int ntile = E / 64, nsl = H / KBLK;
  const int wpt = (RT_WAVES - 1) / ntile;
  const int nch = H / 32;
  const uint8_t* rc = a.base + a.r_off;
  const uint8_t* rs = a.base + a.r_soff;
  if (wave < ntile * wpt) {
    const int t = wave / wpt, q = wave % wpt;
    constexpr int GPS = KBLK / Fmt<FR>::G, CPG = Fmt<FR>::G / 32;
    float out = 0.f;
    for (int sl = q; sl < nsl; sl += wpt) {
      uint32_t w[8][Fmt<FR>::WORDS];
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) load_chunk<FR>(rc + chunk_off<FR>(t, sl * 8 + cc, nch), lane, w[cc]);
      const uint8_t* sblk = rs + sblk_off<FR>(t, sl, nsl);
#pragma unroll
      for (int gi = 0; gi < GPS; ++gi) {
        float acc = 0.f, X = 0.f;
#pragma unroll
        for (int cc = 0; cc < CPG; ++cc) {
          const int c = sl * 8 + gi * CPG + cc;
          uint32_t v[16];
          unpack_chunk<FR>(w[gi * CPG + cc], v);
          acc = dot_chunk(v, xh + 16 * c, acc);
          X += xc[c];
        }
        float ms, bm;
        group_coef<FR>(sblk, lane, gi, ms, bm);
        out = fmaf(ms, acc, out);
        out = fmaf(bm, X, out);
      }
    }
    red[q * E + 64 * t + lane] = out;
  } else if (wave == RT_WAVES - 1) {
    const float c = gate_row_part<FG>(a.base + a.g_off, a.base + a.g_soff, xh, xc, H, lane);
    if (lane == 0) lg[E] = c;
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    float s = 0.f;
    for (int q = 0; q < wpt; ++q) s += red[q * E + e];
    if (a.bias) s += a.bias[e];
    lg[e] = s;
  }
  __syncthreads();
  if (a.logits) {
    for (int e = tid; e <= E; e += blockDim.x) a.logits[(uint64_t)row * (E + 1) + e] = lg[e];
  }
  if (wave == 0) {
    float v[4];
    bool taken[4];
    const int ncand = E / 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = i < ncand ? lg[lane + 64 * i] : 0.f;
      taken[i] = i >= ncand;
    }
    float sel_v[8];
    int sel_i[8];
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!taken[i] && pick_better(v[i], lane + 64 * i, bv, bi)) { bv = v[i]; bi = lane + 64 * i; }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (pick_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if ((bi & 63) == lane) {
#pragma unroll
        for (int i = 0; i < 4; ++i) if (bi == lane + 64 * i) taken[i] = true;
      }
      sel_v[j] = bv;
      sel_i[j] = bi;
    }
    if (lane == 0) {
      float ex[8], S = 0.f;
      for (int j = 0; j < k; ++j) {
        ex[j] = expf(sel_v[j] - sel_v[0]);
        S += ex[j];
      }
      for (int j = 0; j < k; ++j) {
        a.ids[(uint64_t)row * k + j] = sel_i[j];
        a.p[(uint64_t)row * k + j] = ex[j] / S;
      }
      a.sg[row] = 1.0f / (1.0f + expf(-lg[E]));
    }
  }
}

size_t route_smem_bytes(int H, int E) {
  return (size_t)(H / 2) * 4 + (size_t)(H / 32) * 4 + (size_t)RT_WAVES * E * 4 + (size_t)(E + 1) * 4;
}

template <int FR, int FG>
static hipError_t launch_route_t(const RouteArgs& a, int rows, hipStream_t s) {
  const size_t smem = route_smem_bytes(a.H, a.E);
  hipLaunchKernelGGL((k_route<FR, FG>), dim3(rows), dim3(64 * RT_WAVES), smem, s, a);
  return hipGetLastError();
}

template <int FR>
static hipError_t launch_route_g(int fg, const RouteArgs& a, int rows, hipStream_t s) {
  switch (fg) {
    case F_Q4: return launch_route_t<FR, F_Q4>(a, rows, s);
    case F_Q8: return launch_route_t<FR, F_Q8>(a, rows, s);
    case F_S4: return launch_route_t<FR, F_S4>(a, rows, s);
    case F_DENSE: return launch_route_t<FR, F_DENSE>(a, rows, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_route(int fr, int fg, const RouteArgs& a, int rows, hipStream_t s) {
  switch (fr) {
    case F_Q4: return launch_route_g<F_Q4>(fg, a, rows, s);
    case F_Q8: return launch_route_g<F_Q8>(fg, a, rows, s);
    case F_S4: return launch_route_g<F_S4>(fg, a, rows, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
