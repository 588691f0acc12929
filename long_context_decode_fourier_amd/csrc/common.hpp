// common.hpp - shared device/host definitions of libfa (gfx950).
//
// Per-sequence tables travel by value in kernel arguments (the host knows the
// sequence lengths), so no kernel reads a device-side length array.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr int kMaxBatch = 64;

// Basis convention (orthonormal real Fourier basis of period P over the M
// middle positions; P = M unless the descriptor fixes a period P >= M):
// index n has frequency f = (n+1)/2; n = 0 and odd n are cosines, even n >= 2
// sines, of 2 pi f tau / P; scale sqrt(2/P), or 1/sqrt(P) for f = 0 and for
// 2f = P.  Kernels work with the unscaled trig values and apply the scale on
// the coefficient side.
__host__ __device__ inline int basis_freq(int n) { return (n + 1) >> 1; }
__host__ __device__ inline bool basis_is_cos(int n) { return n == 0 || (n & 1); }

// Layout of one sequence b inside the dim-split cache and its work split.
struct SeqTable {
  int32_t len[kMaxBatch];    // L_b
  int32_t mid[kMaxBatch];    // M_b = max(0, L_b - sink - recent)
  int32_t per[kMaxBatch];    // basis period P_b: M_b, or the descriptor's fixed period
  int64_t row0[kMaxBatch];   // Hkv * (L_0 + ... + L_{b-1}): first cache row of b
  int32_t item0[kMaxBatch];  // first work item of sequence b
  int32_t nsplit[kMaxBatch]; // token splits of sequence b
  int32_t chunk[kMaxBatch];  // tokens (or middle positions) per split
};

// Which sequence owns work item `item` (items of sequence b are
// [item0[b], item0[b+1]) ); linear scan, B <= 64.
__device__ inline int seq_of_item(const SeqTable& t, int nseq, int item) {
  int b = 0;
  while (b + 1 < nseq && item >= t.item0[b + 1]) ++b;
  return b;
}

// ------------------------------------------------------------ loads ------
__device__ inline float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
template <typename T> __device__ inline float load_f32(const T* p, int64_t i);
template <> __device__ inline float load_f32<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ inline float load_f32<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// --------------------------------------------------------------- trig ----
// sin/cos of 2*pi*x for x in revolutions, hardware transcendental unit
// (absolute error about 1e-7 on [0, 1)).
__device__ inline float sin_rev(float x) { return __builtin_amdgcn_sinf(x); }
__device__ inline float cos_rev(float x) { return __builtin_amdgcn_cosf(x); }

// Two floats to packed fp16 (round to nearest even).  A vector conversion
// (v_cvt_pk_f16_f32 on gfx950) that the compiler schedules and hazard-checks
// like any other instruction.
typedef float pk_float2 __attribute__((ext_vector_type(2)));
typedef _Float16 pk_half2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_f16(float lo, float hi) {
  const pk_half2 h = __builtin_convertvector((pk_float2){lo, hi}, pk_half2);
  return __builtin_bit_cast(uint32_t, h);
}

// (f * tau) mod M, exact, for f, tau >= 0 (64-bit product).
__device__ inline int phase_mod(int f, int tau, int M) {
  return static_cast<int>((static_cast<uint64_t>(f) * static_cast<uint64_t>(tau)) %
                          static_cast<uint64_t>(M));
}

// Accurate cos and sin of 2*pi*r/M for an integer phase 0 <= r < M, through
// the device math library's sincospi (used where fp32 accuracy matters).  The
// phase is folded to (-M/2, M/2] so the argument of sincospi lies in (-1, 1].
__device__ inline void sincos_phase(int r, int M, float* s, float* c) {
  const int rr = (2 * r > M) ? r - M : r;
  const float x = (2.0f * static_cast<float>(rr)) / static_cast<float>(M);
  sincospif(x, s, c);
}

}  // namespace fa
