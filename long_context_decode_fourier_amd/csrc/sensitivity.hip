// sensitivity.hip - the two small kernels of fa_dim_sensitivity (skill page
// "fourier-approximated-kv-cache", Step 1: dimension analysis by noise on the
// values).
//
// Noise on dim d of the values changes only dim d of the attention outputs,
// by P noise[:, d] (P the unperturbed probabilities), so the per-dim change
// of every output row is one attention pass with the noise as the values.
// fa_dim_sensitivity runs that pass with the decode kernels (all dims exact,
// identity dims table from iota_dims_kernel) and sens_norm_kernel sums the
// squares per (query head, dim) in a fixed order.
#include "kernels.hpp"

namespace fa {
namespace {

__global__ __launch_bounds__(256) void iota_dims_kernel(int32_t* dims, int hkv, int D) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < hkv * D) dims[i] = i % D;
}

// sq[i][d] = sum over b, then t, of resp[b][t][i][d]^2 (resp [B][nq][hq][D]).
__global__ __launch_bounds__(256) void sens_norm_kernel(const float* resp, float* sq, int B, int nq, int hq,
                                                        int D) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= hq * D) return;
  const int64_t stride = static_cast<int64_t>(hq) * D;
  float acc = 0.0f;
  for (int64_t r = 0; r < static_cast<int64_t>(B) * nq; ++r) {
    const float v = resp[r * stride + i];
    acc = fmaf(v, v, acc);
  }
  sq[i] = acc;
}

}  // namespace

hipError_t launch_iota_dims(int32_t* dims, int hkv, int D, hipStream_t s) {
  const int n = hkv * D;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(iota_dims_kernel, dim3((n + 255) / 256), dim3(256), 0, s, dims, hkv, D);
  return hipGetLastError();
}

hipError_t launch_sens_norm(const float* resp, float* sq, int B, int nq, int hq, int D, hipStream_t s) {
  const int n = hq * D;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(sens_norm_kernel, dim3((n + 255) / 256), dim3(256), 0, s, resp, sq, B, nq, hq, D);
  return hipGetLastError();
}

}  // namespace fa
