// Matrix-core rate probe (measurement aid, not part of the attention path).
//
// Every wave of a chip-filling grid (8 waves per CU, two per SIMD) runs eight
// independent accumulation chains of v_mfma_f32_32x32x16_bf16 on operands
// held in registers, so nothing but the matrix cores is exercised. The
// operands are either all zero or fixed pseudo-random bf16 values in [-1, 1)
// that rotate from one MFMA to the next, as streamed K/V tiles do. The part is
// power-limited: random operands draw more power and run at a lower clock
// than zeros, so the random-operand rate is the practical ceiling that the
// attention kernels' MFMA-busy time is compared with.

#include <hip/hip_runtime.h>

#include <string>

#include "branch_attn.h"
#include "plan.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kProbeBlocks = 2048;  // 256 CUs x 8 workgroups, queued
constexpr int kProbeThreads = 256;  // 4 waves

// Uniform in [-1, 1) from a 32-bit integer hash (Wang hash).
__device__ __forceinline__ float hash_unit(uint32_t x) {
  x = (x ^ 61u) ^ (x >> 16);
  x *= 9u;
  x ^= x >> 4;
  x *= 0x27d4eb2du;
  x ^= x >> 15;
  return float(x >> 8) * (2.0f / 16777216.0f) - 1.0f;
}

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters, int random, float *sink) {
  const uint32_t tid = blockIdx.x * kProbeThreads + threadIdx.x;
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[s][e] = __bf16(random ? hash_unit(tid * 64u + s * 16u + e) : 0.f);
      b[s][e] = __bf16(random ? hash_unit(tid * 64u + s * 16u + 8u + e) : 0.f);
    }
  f32x16_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x16_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j + (j >> 2)) & 3], c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += c[j][v];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = s;
}

}  // namespace

extern "C" ba_status ba_probe_mfma(int32_t random_operands, int32_t iters, float *sink,
                                   int64_t sink_len, void *stream, double *tflops) {
  try {
    if (tflops == nullptr || sink == nullptr) return ba::fail(BA_E_INVALID, "sink and tflops are required");
    if (iters < 1 || iters > (1 << 24)) return ba::fail(BA_E_INVALID, "iters must be in 1..2^24");
    const int64_t need = int64_t(kProbeBlocks) * (kProbeThreads / 64);
    if (sink_len < need)
      return ba::fail(BA_E_INVALID, "sink needs " + std::to_string(need) + " floats");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) e = hipEventRecord(e0, s);
    if (e == hipSuccess) {
      hipLaunchKernelGGL(mfma_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, s, int(iters),
                         random_operands ? 1 : 0, sink);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (e != hipSuccess) return ba::fail(BA_E_HIP, std::string("probe: ") + hipGetErrorString(e));
    const double flop = double(kProbeBlocks) * (kProbeThreads / 64) * double(iters) * 8.0 * 32768.0;
    *tflops = ms > 0.f ? flop / (double(ms) * 1e-3) / 1e12 : 0.0;
    return BA_OK;
  } catch (...) {
    return ba::fail(BA_E_INVALID, "unexpected error in ba_probe_mfma");
  }
}
