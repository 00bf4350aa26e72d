// Measurement probe: the sustained dense bf16 MFMA rate of the device, the
// ceiling the attention kernels' roofline fraction is read against beside the
// published peak.  Not part of attention.
//
// Every wavefront issues `iters` rounds of four independent
// v_mfma_f32_32x32x16_bf16 chains on register operands (32768 FLOP each, no
// memory traffic); the launch holds two wavefronts per SIMD on every compute
// unit.  Back-to-back accumulation into the same registers needs no wait
// states, and the instructions are volatile, so none is removed.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters) {
  f32x16_t c0 = zero16(), c1 = zero16(), c2 = zero16(), c3 = zero16();
  const u32x4_t a = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 pairs
  const u32x4_t b = a;
  for (int i = 0; i < iters; ++i) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c0) : "v"(a), "v"(b));
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c1) : "v"(a), "v"(b));
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c2) : "v"(a), "v"(b));
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c3) : "v"(a), "v"(b));
  }
  mfma_wait_v(c0, c1, c2, c3);
}

hipError_t launch_mfma_peak(int workgroups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(workgroups), dim3(256), 0, stream, iters);
  return hipGetLastError();
}

}  // namespace fa
