// mfma_util.hpp - device helpers shared by the MFMA decode kernels (gfx950):
// operand vector types, the transposed LDS read, 16-lane reductions, bf16
// rounding and the lazy softmax reference.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace mfma {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

// Transposed 4 x 16-bit LDS read: lane 4a+e of each 16-lane group receives
// element e of the 8-byte chunks addressed by lanes a, a+4, a+8, a+12 of its
// group.
__device__ inline short4v lds_read_tr4(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p));
}

// All-reduce over aligned groups of 16 lanes: DPP rotations inside a row.
template <int CTRL> __device__ inline float dpp_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ inline float row16_max(float v) {
  v = fmaxf(v, dpp_ror<0x128>(v));
  v = fmaxf(v, dpp_ror<0x124>(v));
  v = fmaxf(v, dpp_ror<0x122>(v));
  v = fmaxf(v, dpp_ror<0x121>(v));
  return v;
}
__device__ inline float row16_sum(float v) {
  v += dpp_ror<0x128>(v);
  v += dpp_ror<0x124>(v);
  v += dpp_ror<0x122>(v);
  v += dpp_ror<0x121>(v);
  return v;
}
// round-to-nearest-even float -> bf16 bits (finite inputs)
__device__ inline uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
// Softmax reference maximum: moved only when a score exceeds it by more than
// this (probabilities stay below e^8 ~ 3e3, well inside fp16 and bf16 range).
constexpr float kLazyMax = 8.0f;

__device__ inline int add_mod(int x, int d, int M) {
  x += d;
  return x >= M ? x - M : x;
}

}  // namespace mfma
}  // namespace fa
