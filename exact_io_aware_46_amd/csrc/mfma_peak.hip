// Matrix-core throughput probe used by the bench: every wave issues back-to-back,
// independent MFMAs (four accumulator chains) with no memory traffic inside the loop, so
// the launch measures what the matrix units sustain on this part at its current clock and
// power. The attention kernels' rates are reported against this figure beside the spec
// sheet's peak. The roofline's compute ceiling is the platform's peak matrix throughput
// ("FlashAttention学习笔记", amentiraz.github.io, sections 计算限制与内存限制 and Roofline);
// this gives it by measurement.
//
//   kind 0: v_mfma_f32_32x32x16_bf16          32768 FLOP per instruction
//   kind 1: v_mfma_scale_f32_32x32x64_f8f6f4   131072 FLOP per instruction (E4M3, unit scales)
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 4;

template <int KIND>
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* __restrict__ out, int iters) {
  const int lane = (int)threadIdx.x & 63;
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  if constexpr (KIND == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(0.001f * (float)((lane + e) % 7));
      b[e] = (__bf16)(0.001f * (float)((lane * 3 + e) % 5));
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  } else {
    i32x8 a, b;  // E4M3 codes 0x20 .. 0x27 (2^-3 .. 2^-3 * 1.875)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = 0x20202020 + ((lane + e) & 7);
      b[e] = 0x20202020 + ((lane * 3 + e) & 7);
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127,
                                                                 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Matrix instructions per wave per launch: iters * 4. out: device float [workgroups * 256].
// Returns 0, or -1 for bad arguments, or the HIP launch error.
int mfma_peak_launch(int kind, float* out, int workgroups, int iters, void* stream) {
  if (!out || workgroups < 1 || iters < 1 || (kind != 0 && kind != 1)) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(mfma_peak_kernel<0>, dim3(workgroups), dim3(256), 0, s, out, iters);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(workgroups), dim3(256), 0, s, out, iters);
  return (int)hipGetLastError();
}

int mfma_peak_chains() { return kChains; }

}  // extern "C"
