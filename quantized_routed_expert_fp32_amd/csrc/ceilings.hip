// Measured ceilings for the benchmark's context (not part of the hot path):
// the rate of back-to-back v_mfma_f32_32x32x16_f16 on every SIMD, against
// which the published dense fp16 peak can be read. Built into its own
// library (libmoe_ceilings.so) beside libmoe.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

namespace {

// Every wave runs `iters` rounds of NCH independent 32x32x16 MFMA chains
// (enough in flight to keep the matrix pipe busy); the accumulators' sum is
// stored so the work is not removed.
constexpr int NCH = 8;
__global__ __launch_bounds__(256) void k_mfma_loop(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  h8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (lane + i));
    b[i] = (_Float16)(0.002f * (lane - i));
  }
  f16v c[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) c[j] = f16v{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[j][i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

// Times `reps` launches of the MFMA loop (grid `blocks` x 256 threads,
// `iters` rounds per wave) with events on `stream`; returns 0 and writes the
// achieved dense fp16 TFLOP/s, or a hipError_t. out: device buffer of
// blocks * 256 floats (caller-owned).
extern "C" int moe_ceiling_mfma_f16(int blocks, int iters, int reps, float* out, void* stream,
                                    double* tflops) {
  if (blocks <= 0 || iters <= 0 || reps <= 0 || !out || !tflops) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0, e1;
  hipError_t err;
  if ((err = hipEventCreate(&e0)) != hipSuccess) return (int)err;
  if ((err = hipEventCreate(&e1)) != hipSuccess) { hipEventDestroy(e0); return (int)err; }
  hipLaunchKernelGGL(k_mfma_loop, dim3(blocks), dim3(256), 0, s, iters, out);   // warm-up
  hipEventRecord(e0, s);
  for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(k_mfma_loop, dim3(blocks), dim3(256), 0, s, iters, out);
  hipEventRecord(e1, s);
  err = hipEventSynchronize(e1);
  float ms = 0.f;
  if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
  if (err == hipSuccess) err = hipGetLastError();
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  if (err != hipSuccess) return (int)err;
  // 4 waves per block, NCH MFMAs per round, 2 * 32 * 32 * 16 flop each
  const double flop = (double)blocks * 4 * (double)iters * NCH * 2.0 * 32 * 32 * 16 * reps;
  *tflops = flop / (ms * 1e-3) / 1e12;
  return 0;
}
