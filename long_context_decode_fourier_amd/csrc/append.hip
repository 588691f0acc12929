// append.hip - fa_append: one token appended to every sequence of a compressed
// cache whose basis has a fixed period P.
//
// With a fixed period the coefficients of a middle are a sum of one term per
// token, C[n][c] = sum_tau phi_n(tau) x_tau[c], so a middle that grows by one
// token at tau = M gains the term phi_n(M) x[c] and nothing else changes.
// Per (sequence b, KV head h, matrix K or V):
//  - L_b + 1 <= sink + recent: the new token is retained; its compressible
//    row becomes retained row L_b;
//  - otherwise the token leaving the recent window (retained row `sink`, or
//    the new token itself when recent = 0) enters the middle at tau = M_b:
//    C[n][c] += phi_n(M_b) x[c] for every n < k; the recent rows move down by
//    one and the new token's row becomes the last one.
// Two kernels, in this order on the stream: append_coef_kernel reads the
// leaving row, append_edge_kernel then shifts the retained rows over it.
#include "kernels.hpp"

namespace fa {
namespace {

constexpr int kAppendRows = 64;  // coefficient rows per append_coef block

__device__ inline float elem(const void* p, int esz, int64_t i) {
  return esz == 2 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

// Block (b, h, matrix) x coefficient rows [n0, n0 + 64).
__global__ __launch_bounds__(256) void append_coef_kernel(AppendArgs a) {
  __shared__ float xs[kMaxAppendDc];
  __shared__ float phi[kAppendRows];
  const int bhm = blockIdx.x;
  const int mat = bhm % a.nmat, bh = bhm / a.nmat, b = bh / a.hkv;
  const int E = a.sink + a.recent;
  const int L = a.len[b];
  if (L + 1 <= E) return;  // the new token is retained: no coefficient changes
  const int M = L - E;     // tau of the token entering the middle
  const int n0 = blockIdx.y * kAppendRows;
  const int tid = threadIdx.x;
  // the entering row: retained row `sink` (the first recent token), or the
  // new token when nothing is kept at the end
  for (int c = tid; c < a.dc; c += blockDim.x)
    xs[c] = a.recent > 0 ? elem(a.e[mat], a.esz, (static_cast<int64_t>(bh) * E + a.sink) * a.dc + c)
                         : elem(a.xnew[mat], a.esz, static_cast<int64_t>(bh) * a.dc + c);
  if (tid < kAppendRows) {
    const int n = n0 + tid;
    float v = 0.0f;
    if (n < a.k) {
      const int f = basis_freq(n);
      float s, c;
      sincos_phase(phase_mod(f, M, a.period), a.period, &s, &c);
      const float alpha = (f == 0 || 2 * f == a.period) ? 1.0f / sqrtf(static_cast<float>(a.period))
                                                         : sqrtf(2.0f / static_cast<float>(a.period));
      v = alpha * (basis_is_cos(n) ? c : s);
    }
    phi[tid] = v;
  }
  __syncthreads();
  float* C = a.c[mat] + static_cast<int64_t>(bh) * a.k * a.dc;
  const int nrows = min(kAppendRows, a.k - n0);
  for (int i = tid; i < nrows * a.dc; i += blockDim.x) {
    const int r = i / a.dc, c = i % a.dc;
    float* p = C + static_cast<int64_t>(n0 + r) * a.dc + c;
    *p = fmaf(phi[r], xs[c], *p);
  }
}

// Block (b, h, matrix): the retained rows.  Elements move as 16-bit units
// (a float32 row is twice as many units).
__global__ __launch_bounds__(256) void append_edge_kernel(AppendArgs a) {
  const int bhm = blockIdx.x;
  const int mat = bhm % a.nmat, bh = bhm / a.nmat, b = bh / a.hkv;
  const int E = a.sink + a.recent;
  const int L = a.len[b];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int units = a.dc * a.esz / 2;  // 16-bit units per row
  uint16_t* rows = static_cast<uint16_t*>(a.e[mat]) + static_cast<int64_t>(bh) * E * units;
  const uint16_t* xn = static_cast<const uint16_t*>(a.xnew[mat]) + static_cast<int64_t>(bh) * units;
  int dst_row;
  if (L + 1 <= E) {
    dst_row = L;  // appended after the retained rows
  } else if (a.recent > 0) {
    // rows sink + 1 .. E - 1 move to sink .. E - 2, in increasing order:
    // each round reads its units before any thread writes, and a round only
    // writes units that this or an earlier round has read
    const int64_t first = static_cast<int64_t>(a.sink + 1) * units, last = static_cast<int64_t>(E) * units;
    constexpr int kU = 8;
    for (int64_t r0 = first; r0 < last; r0 += static_cast<int64_t>(kU) * nt) {
      uint16_t v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = r0 + tid + static_cast<int64_t>(u) * nt;
        v[u] = i < last ? rows[i] : 0;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = r0 + tid + static_cast<int64_t>(u) * nt;
        if (i < last) rows[i - units] = v[u];
      }
      __syncthreads();
    }
    dst_row = E - 1;
  } else {
    return;  // nothing retained at the end: the new token went to the middle
  }
  for (int i = tid; i < units; i += nt) rows[static_cast<int64_t>(dst_row) * units + i] = xn[i];
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  const int blocks = a.nseq * a.hkv * a.nmat;
  if (blocks == 0) return hipSuccess;
  if (a.c[0]) {
    hipLaunchKernelGGL(append_coef_kernel, dim3(blocks, (a.k + kAppendRows - 1) / kAppendRows), dim3(256), 0,
                       s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.e[0]) hipLaunchKernelGGL(append_edge_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
