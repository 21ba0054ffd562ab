// Decode path: routed + shared experts for up to 16 independent rows.
//
// Expert-centric: one workgroup per (unique expert of the batch, 64-row tile).
// It streams the tile's packed codes once (coalesced 128-bit loads, lane =
// output row) and applies them to every row that picked the expert. Rows
// sharing an expert share its reads ("Native server: --backend xpu for
// Nemotron on Intel Arc", review comments: each extra row costs about 3.7 ms
// because more distinct experts are read; a gain needs expert reads shared
// across rows).
//
// Each row's arithmetic is fixed: K is cut into 256-wide slices owned by
// fixed waves, chunks and groups are summed in K order, slices are reduced
// in LDS in wave order, and the combine runs the slots in pick order with
// the shared expert last. None of it depends on how many rows share the
// launch, so a row's y is bit-identical alone or in a batch ("Sage-A1.5 ...
// #1329", Limits to agree on: the per-row kernels keep one stream's sum).
//
// Kernels per call: gate/up + SwiGLU -> h (fp32), down -> e (fp32), combine -> y.
#include "moe_kernels.h"
#include "moe_launch.h"

namespace moe {

constexpr int GU_WAVES = 8;   // waves per gate/up workgroup (K slices of 256)
constexpr int DN_WAVES = 2;   // waves per down workgroup
constexpr int NRP = 4;        // rows per pass

// Finds which expert this workgroup serves (unit u: the u-th smallest picked
// id, then the shared expert at u == #unique) and the rows (ascending) that
// picked it with their slot. Returns the expert id, E for the shared expert,
// or -1 when the unit is empty.
__device__ int resolve_unit(const int32_t* ids, int R, int k, int E, int u, int* s_rows,
                            int* s_slots, int* s_nr, uint32_t* s_mask, int* s_expert) {
  const int tid = threadIdx.x;
  if (tid < 8) s_mask[tid] = 0u;
  __syncthreads();
  for (int i = tid; i < R * k; i += blockDim.x) {
    const int id = ids[i];
    if (id >= 0 && id < E) atomicOr(&s_mask[id >> 5], 1u << (id & 31));
  }
  __syncthreads();
  if (tid == 0) {
    int nu = 0;
    for (int w = 0; w < 8; ++w) nu += __popc(s_mask[w]);
    int e = -1;
    if (u < nu) {
      int left = u;
      for (int w = 0; w < 8; ++w) {
        const int c = __popc(s_mask[w]);
        if (left < c) {
          uint32_t m = s_mask[w];
          for (int b = 0; b < left; ++b) m &= m - 1;   // drop the lowest set bits
          e = 32 * w + __ffs(m) - 1;
          break;
        }
        left -= c;
      }
    } else if (u == nu) {
      e = E;
    }
    *s_expert = e;
  }
  __syncthreads();
  const int e = *s_expert;
  if (e < 0) return -1;
  if (tid < 64) {
    int slot = -1;
    if (tid < R) {
      if (e == E) {
        slot = k;
      } else {
        for (int j = 0; j < k; ++j)
          if (ids[tid * k + j] == e) { slot = j; break; }
      }
    }
    const unsigned long long m = __ballot(slot >= 0);
    const int pos = __popcll(m & ((1ull << tid) - 1ull));
    if (slot >= 0) { s_rows[pos] = tid; s_slots[pos] = slot; }
    if (tid == 0) *s_nr = __popcll(m);
  }
  __syncthreads();
  return e;
}

// ------------------------------------------------------------------ gate/up
template <int F>
__device__ void gateup_body(const DecodeArgs& a, const uint8_t* codes, const uint8_t* scales,
                            int t, int n_r, const int* s_rows, const int* s_slots,
                            uint8_t* smem) {
  const int H = a.H, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = H / 32, nkb = H / KBLK;
  half2v* xh = reinterpret_cast<half2v*>(smem);           // [NRP][H/2]
  float* xc = reinterpret_cast<float*>(xh + NRP * (H / 2)); // [NRP][H/32]
  float* red = xc + NRP * (H / 32);                        // [GU_WAVES][NRP][64]
  constexpr int GPS = KBLK / Fmt<F>::G, CPG = Fmt<F>::G / 32;
  for (int r0 = 0; r0 < n_r; r0 += NRP) {
    const int nr = min(NRP, n_r - r0);
    for (int i = tid; i < nr * (H / 2); i += blockDim.x) {
      const int rr = i / (H / 2), ii = i % (H / 2);
      const uint32_t v = reinterpret_cast<const uint32_t*>(a.x + (uint64_t)s_rows[r0 + rr] * H)[ii];
      half2v h;
      h.x = (f16)act_to_f((uint16_t)(v & 0xFFFFu), a.act_fp16);
      h.y = (f16)act_to_f((uint16_t)(v >> 16), a.act_fp16);
      xh[rr * (H / 2) + ii] = h;
    }
    __syncthreads();
    for (int i = tid; i < nr * nch; i += blockDim.x) {
      const int rr = i / nch, c = i % nch;
      const half2v* xr = xh + rr * (H / 2) + 16 * c;
      float s = 0.f;
      for (int q = 0; q < 16; ++q) {
        s += (float)xr[q].x;
        s += (float)xr[q].y;
      }
      xc[rr * nch + c] = s;
    }
    __syncthreads();
    float out[NRP];
#pragma unroll
    for (int rr = 0; rr < NRP; ++rr) out[rr] = 0.f;
    for (int sl = wave; sl < nkb; sl += GU_WAVES) {
      uint32_t w[8][Fmt<F>::WORDS];
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) load_chunk<F>(codes + chunk_off<F>(t, sl * 8 + cc, nch), lane, w[cc]);
      const uint8_t* sblk = scales + sblk_off<F>(t, sl, nkb);
#pragma unroll
      for (int gi = 0; gi < GPS; ++gi) {
        float ms, bm;
        group_coef<F>(sblk, lane, gi, ms, bm);
        float acc[NRP];
#pragma unroll
        for (int rr = 0; rr < NRP; ++rr) acc[rr] = 0.f;
#pragma unroll
        for (int cc = 0; cc < CPG; ++cc) {
          const int c = sl * 8 + gi * CPG + cc;
          uint32_t v[16];
          unpack_chunk<F>(w[gi * CPG + cc], v);
#pragma unroll
          for (int rr = 0; rr < NRP; ++rr)
            if (rr < nr) acc[rr] = dot_chunk(v, xh + rr * (H / 2) + 16 * c, acc[rr]);
        }
#pragma unroll
        for (int rr = 0; rr < NRP; ++rr) {
          if (rr < nr) {
            float X = 0.f;
            for (int cc = 0; cc < CPG; ++cc) X += xc[rr * nch + sl * 8 + gi * CPG + cc];
            out[rr] = fmaf(ms, acc[rr], out[rr]);
            out[rr] = fmaf(bm, X, out[rr]);
          }
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < NRP; ++rr) red[(wave * NRP + rr) * 64 + lane] = out[rr];
    __syncthreads();
    if (tid < NRP * 32) {
      const int rr = tid / 32, j = tid % 32;
      if (rr < nr) {
        float g = 0.f, u = 0.f;
        for (int w2 = 0; w2 < GU_WAVES; ++w2) {
          g += red[(w2 * NRP + rr) * 64 + j];
          u += red[(w2 * NRP + rr) * 64 + 32 + j];
        }
        const int r = s_rows[r0 + rr], slot = s_slots[r0 + rr];
        const uint64_t rs = (uint64_t)r * (a.k + 1) + slot;
        const int col = 32 * t + j;
        a.h_ws[rs * a.Imax + col] = silu_mul(g, u);
        if (a.tap_gu) {
          a.tap_gu[(rs * 2 + 0) * a.Imax + col] = g;
          a.tap_gu[(rs * 2 + 1) * a.Imax + col] = u;
        }
        if (a.tap_h) a.tap_h[rs * a.Imax + col] = silu_mul(g, u);
      }
    }
    __syncthreads();
  }
}

template <int FR, int FS>
__global__ __launch_bounds__(64 * GU_WAVES) void k_decode_gateup(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_rows[16], s_slots[16], s_nr, s_expert;
  __shared__ uint32_t s_mask[8];
  const int e = resolve_unit(a.ids, a.R, a.k, a.E, blockIdx.y, s_rows, s_slots, &s_nr, s_mask,
                             &s_expert);
  if (e < 0) return;
  const int t = blockIdx.x;
  if (e == a.E) {
    if (t >= 2 * a.sh.inter / 64) return;
    const uint8_t* blk = a.base + a.sh.base_off;
    gateup_body<FS>(a, blk + a.sh.gu_codes, blk + a.sh.gu_scales, t, s_nr, s_rows, s_slots, smem);
  } else {
    if (t >= 2 * a.rt.inter / 64) return;
    const uint8_t* blk = a.base + a.rt.base_off + (uint64_t)e * a.rt.stride;
    gateup_body<FR>(a, blk + a.rt.gu_codes, blk + a.rt.gu_scales, t, s_nr, s_rows, s_slots, smem);
  }
}

// --------------------------------------------------------------------- down
template <int F>
__device__ void down_body(const DecodeArgs& a, const uint8_t* codes, const uint8_t* scales, int I,
                          int t, int n_r, const int* s_rows, const int* s_slots, uint8_t* smem) {
  const int H = a.H, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = I / 32, nkb = I / KBLK;
  half2v* hhi = reinterpret_cast<half2v*>(smem);            // [NRP][Imax/2]
  half2v* hlo = hhi + NRP * (a.Imax / 2);                    // [NRP][Imax/2]
  float* hc = reinterpret_cast<float*>(hlo + NRP * (a.Imax / 2));  // [NRP][Imax/32]
  float* red = hc + NRP * (a.Imax / 32);                     // [DN_WAVES][NRP][64]
  const int hs = a.Imax / 2, cs = a.Imax / 32;
  constexpr int GPS = KBLK / Fmt<F>::G, CPG = Fmt<F>::G / 32;
  for (int r0 = 0; r0 < n_r; r0 += NRP) {
    const int nr = min(NRP, n_r - r0);
    for (int i = tid; i < nr * (I / 2); i += blockDim.x) {
      const int rr = i / (I / 2), ii = i % (I / 2);
      const uint64_t rs = (uint64_t)s_rows[r0 + rr] * (a.k + 1) + s_slots[r0 + rr];
      const float2 hv = reinterpret_cast<const float2*>(a.h_ws + rs * a.Imax)[ii];
      half2v hi, lo;
      hi.x = (f16)hv.x;
      hi.y = (f16)hv.y;
      lo.x = (f16)(hv.x - (float)hi.x);
      lo.y = (f16)(hv.y - (float)hi.y);
      hhi[rr * hs + ii] = hi;
      hlo[rr * hs + ii] = lo;
    }
    __syncthreads();
    for (int i = tid; i < nr * nch; i += blockDim.x) {
      const int rr = i / nch, c = i % nch;
      float s = 0.f;
      for (int q = 0; q < 16; ++q) {
        const half2v hi = hhi[rr * hs + 16 * c + q], lo = hlo[rr * hs + 16 * c + q];
        s += (float)hi.x + (float)lo.x;
        s += (float)hi.y + (float)lo.y;
      }
      hc[rr * cs + c] = s;
    }
    __syncthreads();
    float out[NRP];
#pragma unroll
    for (int rr = 0; rr < NRP; ++rr) out[rr] = 0.f;
    for (int sl = wave; sl < nkb; sl += DN_WAVES) {
      uint32_t w[8][Fmt<F>::WORDS];
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) load_chunk<F>(codes + chunk_off<F>(t, sl * 8 + cc, nch), lane, w[cc]);
      const uint8_t* sblk = scales + sblk_off<F>(t, sl, nkb);
#pragma unroll
      for (int gi = 0; gi < GPS; ++gi) {
        float ms, bm;
        group_coef<F>(sblk, lane, gi, ms, bm);
        float acc[NRP];
#pragma unroll
        for (int rr = 0; rr < NRP; ++rr) acc[rr] = 0.f;
#pragma unroll
        for (int cc = 0; cc < CPG; ++cc) {
          const int c = sl * 8 + gi * CPG + cc;
          uint32_t v[16];
          unpack_chunk<F>(w[gi * CPG + cc], v);
#pragma unroll
          for (int rr = 0; rr < NRP; ++rr) {
            if (rr < nr) {
              acc[rr] = dot_chunk(v, hhi + rr * hs + 16 * c, acc[rr]);
              acc[rr] = dot_chunk(v, hlo + rr * hs + 16 * c, acc[rr]);
            }
          }
        }
#pragma unroll
        for (int rr = 0; rr < NRP; ++rr) {
          if (rr < nr) {
            float X = 0.f;
            for (int cc = 0; cc < CPG; ++cc) X += hc[rr * cs + sl * 8 + gi * CPG + cc];
            out[rr] = fmaf(ms, acc[rr], out[rr]);
            out[rr] = fmaf(bm, X, out[rr]);
          }
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < NRP; ++rr) red[(wave * NRP + rr) * 64 + lane] = out[rr];
    __syncthreads();
    for (int i = tid; i < nr * 64; i += blockDim.x) {
      const int rr = i / 64, l = i % 64;
      float s = 0.f;
      for (int w2 = 0; w2 < DN_WAVES; ++w2) s += red[(w2 * NRP + rr) * 64 + l];
      const uint64_t rs = (uint64_t)s_rows[r0 + rr] * (a.k + 1) + s_slots[r0 + rr];
      a.e_ws[rs * H + 64 * t + l] = s;
      if (a.tap_e) a.tap_e[rs * H + 64 * t + l] = s;
    }
    __syncthreads();
  }
}

template <int FR, int FS>
__global__ __launch_bounds__(64 * DN_WAVES) void k_decode_down(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_rows[16], s_slots[16], s_nr, s_expert;
  __shared__ uint32_t s_mask[8];
  const int e = resolve_unit(a.ids, a.R, a.k, a.E, blockIdx.y, s_rows, s_slots, &s_nr, s_mask,
                             &s_expert);
  if (e < 0) return;
  const int t = blockIdx.x;
  if (e == a.E) {
    const uint8_t* blk = a.base + a.sh.base_off;
    down_body<FS>(a, blk + a.sh.dn_codes, blk + a.sh.dn_scales, a.sh.inter, t, s_nr, s_rows,
                  s_slots, smem);
  } else {
    const uint8_t* blk = a.base + a.rt.base_off + (uint64_t)e * a.rt.stride;
    down_body<FR>(a, blk + a.rt.dn_codes, blk + a.rt.dn_scales, a.rt.inter, t, s_nr, s_rows,
                  s_slots, smem);
  }
}

// ------------------------------------------------------------------ combine
__global__ __launch_bounds__(256) void k_decode_combine(DecodeArgs a) {
  const int n = blockIdx.x * 256 + threadIdx.x, r = blockIdx.y;
  if (n >= a.H) return;
  const int k = a.k;
  const float* e = a.e_ws + (uint64_t)r * (k + 1) * a.H + n;
  float acc = 0.f;
  for (int j = 0; j < k; ++j) acc = fmaf(a.p[r * k + j], e[(uint64_t)j * a.H], acc);
  acc = fmaf(a.sg[r], e[(uint64_t)k * a.H], acc);
  a.y[(uint64_t)r * a.H + n] = acc;
}

// ------------------------------------------------------------------ launch
static size_t gu_smem(int H) {
  return (size_t)NRP * (H / 2) * 4 + (size_t)NRP * (H / 32) * 4 + (size_t)GU_WAVES * NRP * 64 * 4;
}
static size_t dn_smem(int Imax) {
  return (size_t)2 * NRP * (Imax / 2) * 4 + (size_t)NRP * (Imax / 32) * 4 +
         (size_t)DN_WAVES * NRP * 64 * 4;
}

template <int FR, int FS>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  const int units = min(a.E, a.R * a.k) + 1;
  const int gu_tiles = 2 * a.Imax / 64;
  hipLaunchKernelGGL((k_decode_gateup<FR, FS>), dim3(gu_tiles, units), dim3(64 * GU_WAVES),
                     gu_smem(a.H), s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((k_decode_down<FR, FS>), dim3(a.H / 64, units), dim3(64 * DN_WAVES),
                     dn_smem(a.Imax), s, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_decode_combine, dim3((a.H + 255) / 256, a.R), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int FR>
static hipError_t launch_decode_s(int fs, const DecodeArgs& a, hipStream_t s) {
  switch (fs) {
    case F_Q4: return launch_decode_t<FR, F_Q4>(a, s);
    case F_Q3: return launch_decode_t<FR, F_Q3>(a, s);
    case F_S4: return launch_decode_t<FR, F_S4>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(int fr, int fs, const DecodeArgs& a, hipStream_t s) {
  switch (fr) {
    case F_Q4: return launch_decode_s<F_Q4>(fs, a, s);
    case F_Q3: return launch_decode_s<F_Q3>(fs, a, s);
    case F_S4: return launch_decode_s<F_S4>(fs, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
