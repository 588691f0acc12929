// check.hip - the validating kernels of the FA_CHECK=1 mode: scans that raise
// a flag in device memory, which the host reads back after a sync.
//
// The bf16 projection converts the cache to fp16 MFMA operands, exact for
// |x| in [2^-14, 65504]; a bf16 value of magnitude 65536 or more (bits & 0x7fff
// >= 0x4780, which includes inf and NaN) would become inf.  The decode
// kernels skip dims entries outside [0, D), which gives unspecified results.
#include <algorithm>

#include "kernels.hpp"

namespace fa {
namespace {

__global__ __launch_bounds__(256) void clear_flag_kernel(int32_t* flag) {
  if (threadIdx.x == 0) flag[0] = 0;
}

// flag |= 1 when some bf16 element of x [n] has magnitude >= 65536 (or is inf / NaN)
__global__ __launch_bounds__(256) void bf16_range_kernel(const uint16_t* x, int64_t n, int32_t* flag) {
  bool bad = false;
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    bad = bad || (x[i] & 0x7fffu) >= 0x4780u;
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, 1);
}

// flag |= 2 when some entry of dims [n] lies outside [0, D)
__global__ __launch_bounds__(256) void dims_range_kernel(const int32_t* dims, int n, int D, int32_t* flag) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const bool bad = i < n && (dims[i] < 0 || dims[i] >= D);
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, 2);
}

}  // namespace

hipError_t launch_check_clear(int32_t* flag, hipStream_t s) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(64), 0, s, flag);
  return hipGetLastError();
}

hipError_t launch_check_bf16_range(const void* x, int64_t n, int32_t* flag, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(bf16_range_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), n, flag);
  return hipGetLastError();
}

hipError_t launch_check_dims(const int32_t* dims, int n, int D, int32_t* flag, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(dims_range_kernel, dim3((n + 255) / 256), dim3(256), 0, s, dims, n, D, flag);
  return hipGetLastError();
}

}  // namespace fa
