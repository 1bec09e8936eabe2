// A kernel that holds compute units idle for a set time, for measuring the
// grouped GEMMs' tile order under contention: the Domyn page (section
// "Dynamic tile scheduling in SonicMoE") compares the static and the dynamic
// tile order with and without a dummy kernel occupying part of the GPU, the
// way a collective's thread blocks occupy it during training.
//
// Each workgroup is one wave that reserves lds_bytes of LDS (so that a
// GEMM workgroup cannot share its CU) and waits on the fixed-frequency
// real-time counter until the time is up; the wait is bounded by the time
// alone.
#include "internal.h"

namespace moe {

__global__ void __launch_bounds__(64) hold_kernel(uint64_t ticks) {
  extern __shared__ uint32_t reserved[];
  if (threadIdx.x == 0) reserved[0] = 0;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

hipError_t launch_hold(int workgroups, int lds_bytes, int microseconds, hipStream_t s) {
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(hold_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e != hipSuccess) return e;
  const uint64_t ticks = (uint64_t)khz * (uint64_t)microseconds / 1000u;
  hold_kernel<<<(unsigned)workgroups, 64, (size_t)lds_bytes, s>>>(ticks);
  return hipGetLastError();
}

}  // namespace moe
