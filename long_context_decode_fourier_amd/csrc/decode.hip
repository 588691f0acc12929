// decode.hip - one decode step over the Fourier-approximated KV cache:
// query-side contraction (decode_prep), the VALU split kernel used for fp32
// caches (decode_split) and the split merge (decode_merge).  The MFMA split
// kernel for 16-bit caches is in decode_mfma.hip.
//
// The pages reconstruct the middle tokens (zero-padded inverse transform) and
// then attend (skill page "fourier-approximated-kv-cache", Step 4).  Here the
// reconstruction is never formed.  For a query row q and its KV head:
//
//   middle token tau:  s = scale q_U . kx[tau] + sum_n a_n b_n(tau),
//                      a_n = scale alpha_n (q_C . ck[n])     (decode_prep)
//   edge token t:      s = scale q . [kx[t], ke[t]]
//   out_U = sum_t p_t vx[t]
//   out_C = sum_{edge t} p_t ve[t] + sum_n W_n alpha_n cv[n],
//           W_n = sum_tau p_tau b_n(tau)
//
// with b_n the unscaled cos/sin of the basis (alpha_n its scale) and p the
// softmax of s over all L tokens.  The sequence is split into token ranges
// (split-L); each split keeps a running max m, sum l, o_U, the edge part of
// o_C and W (online softmax), and decode_merge combines the splits with the
// log-sum-exp weights in a fixed order, applies C_V and scatters the dims.
//
// decode_split (fp32) produces the basis along n by complex rotation
// (e^{i theta_j tau} times e^{i 2 pi tau / M}) and along tau by rotation with
// e^{i 2 pi j / M}; both are re-anchored from exact integer phases through
// sincospi, which keeps fp32 results within 1e-5 of the exact value.
#include <algorithm>

#include "kernels.hpp"

namespace fa {
namespace {

template <typename T> __device__ inline float ld(const void* p, int64_t i) {
  return load_f32<T>(static_cast<const T*>(p), i);
}

// Sum over each aligned group of 16 lanes (DPP rotations inside a row).
__device__ inline float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Scale of basis function n for the basis period per.
__device__ inline float basis_alpha(int n, int per) {
  const int f = basis_freq(n);
  return (f == 0 || 2 * f == per) ? 1.0f / sqrtf(static_cast<float>(per))
                                 : sqrtf(2.0f / static_cast<float>(per));
}

// e^{i 2 pi (j * tau mod per) / per} for any integer tau (negative allowed).
__device__ inline float2 unit_phase(int j, int tau, int per) {
  int64_t r = (static_cast<int64_t>(j) * tau) % per;
  if (r < 0) r += per;
  float s, c;
  sincos_phase(static_cast<int>(r), per, &s, &c);
  return make_float2(c, s);
}

__device__ inline float2 cmul(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}

// Pair-order position -> basis index (-1 for the unused slot and padding).
__device__ inline int pair_pos_to_n(int pos, int k) {
  const int j = pos >> 1;
  const int n = (pos & 1) ? (j == 0 ? -1 : 2 * j) : (j == 0 ? 0 : 2 * j - 1);
  return n < k ? n : -1;
}

// --------------------------------------------------------------- prep ----
// A[b][i][n] = scale * alpha_n * sum_c q[b][i][comp_c] ck[b,h][n][c].  One
// kernel with two kinds of block:
//  - edge blocks (MFMA path, one per (sequence, KV head)): the head's query
//    rows at the exact dims in dims order (bf16, for the split kernel) and
//    the edge split: plain softmax attention of those rows over the retained
//    sink and recent tokens (all dims exact), stored as split nsplit-1;
//  - A blocks (sequence, KV head, kPrepPos coefficient positions).
// Every block issues all of its global loads before it waits for any, and
// the dims permutation of q is applied from LDS, so a block costs one memory
// round trip plus its arithmetic.
constexpr int kPrepPos = 64;       // coefficient positions per A block
constexpr int kPrepThreads = 512;  // threads per prep block (edge blocks: one wave per 16-token or 16-dim block)

// Stage the G query rows of (b, h) (scaled, as fp32) and the dims table in LDS.
// Loads of a round are all issued before the first store.
template <typename T>
__device__ inline void stage_q(const DecodeArgs& a, int b, int h, float* qraw, int* dl, float mul) {
  const int G = a.G, D = a.D, n = G * D, nt = blockDim.x;
  constexpr int kQ = 8;
  for (int i0 = threadIdx.x; i0 < n; i0 += kQ * nt) {
    float v[kQ];
#pragma unroll
    for (int u = 0; u < kQ; ++u) {
      const int e = i0 + u * nt;
      v[u] = (e < n) ? ld<T>(a.q, q_row(a, b, h * G + e / D) * D + e % D) : 0.0f;
    }
    const int dj = (i0 < D) ? a.dims[h * D + i0] : 0;  // first round covers the dims (D <= 256)
#pragma unroll
    for (int u = 0; u < kQ; ++u)
      if (i0 + u * nt < n) qraw[i0 + u * nt] = mul * v[u];
    if (i0 < D) dl[i0] = dj;
  }
}

// A block.  Rows n = [r0, r0 + 64) of ck[b,h] (those the block's positions
// use) are copied to LDS with coalesced loads (row stride dc + 4 floats, so
// the 16-byte reads of 8 consecutive rows hit distinct banks); thread
// (position p = tid % 64, row group tid / 64) then forms the dot products
// of its rows g = tid / 64 + 4 j with q_C broadcast from LDS.
template <typename T, bool VEC>
__device__ __forceinline__ void prep_a_block(const DecodeArgs& a, int b, int h, int chunk, float* sm) {
  const int G = a.G, D = a.D, dc = a.dc, du = a.du;
  const int M = a.seq.mid[b], per = a.seq.per[b];
  const int len = a.mfma ? a.kpp : a.k;
  const int p0 = chunk * kPrepPos;
  // pair order: position p >= 2 uses row p - 1, position 0 row 0
  const int r0 = a.mfma ? max(0, p0 - 1) : p0;
  const int CS = dc + 4;
  float* ckl = sm;                       // [64][CS]
  float* qraw = ckl + kPrepPos * CS;     // [G][D]
  float* qc = qraw + G * D;              // [G][dc]
  int* dl = reinterpret_cast<int*>(qc + G * dc);  // [D]
  const float* src = a.ck + ((static_cast<int64_t>(b) * a.hkv + h) * a.k + r0) * dc;
  const int nrows = max(0, min(kPrepPos, a.k - r0));
  const int tid = threadIdx.x;
  if (VEC) {
    const int dc4 = dc / 4, n4 = nrows * dc4;
    constexpr int kB = kPrepPos * 64 / kPrepThreads;  // float4 loads in flight per thread (dc <= 256)
    float4 v[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int i = tid + u * kPrepThreads;
      v[u] = (i < n4) ? reinterpret_cast<const float4*>(src)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    stage_q<T>(a, b, h, qraw, dl, a.scale);
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int i = tid + u * kPrepThreads;
      if (i < n4) *reinterpret_cast<float4*>(ckl + (i / dc4) * CS + 4 * (i % dc4)) = v[u];
    }
  } else {
    stage_q<T>(a, b, h, qraw, dl, a.scale);
    for (int i = tid; i < nrows * dc; i += kPrepThreads) ckl[(i / dc) * CS + i % dc] = src[i];
  }
  __syncthreads();
  for (int idx = tid; idx < G * dc; idx += kPrepThreads) {
    const int g = idx / dc, c = idx % dc;
    const int d = dl[du + c];
    qc[idx] = (d >= 0 && d < D) ? qraw[g * D + d] : 0.0f;
  }
  __syncthreads();
  const int p = tid & 63, pos = p0 + p;
  if (pos >= len) return;
  const int n = a.mfma ? pair_pos_to_n(pos, a.k) : pos;
  const bool live = n >= 0 && n < a.k && M > 0;
  const float alpha = live ? basis_alpha(n, per) : 0.0f;
  const float* crow = ckl + (live ? n - r0 : 0) * CS;
  for (int g = tid >> 6; g < G; g += kPrepThreads / 64) {
    const float* qg = qc + g * dc;
    float acc0 = 0.0f, acc1 = 0.0f;
    if (live) {
      int c = 0;
      if (VEC) {  // dc % 4 == 0: rows and q_C are 16-byte aligned
        for (; c + 8 <= dc; c += 8) {
          const float4 x0 = *reinterpret_cast<const float4*>(crow + c);
          const float4 x1 = *reinterpret_cast<const float4*>(crow + c + 4);
          const float4 q0 = *reinterpret_cast<const float4*>(qg + c);
          const float4 q1 = *reinterpret_cast<const float4*>(qg + c + 4);
          acc0 = fmaf(q0.x, x0.x, acc0); acc0 = fmaf(q0.y, x0.y, acc0);
          acc0 = fmaf(q0.z, x0.z, acc0); acc0 = fmaf(q0.w, x0.w, acc0);
          acc1 = fmaf(q1.x, x1.x, acc1); acc1 = fmaf(q1.y, x1.y, acc1);
          acc1 = fmaf(q1.z, x1.z, acc1); acc1 = fmaf(q1.w, x1.w, acc1);
        }
      }
      for (; c < dc; ++c) acc0 = fmaf(qg[c], crow[c], acc0);
    }
    const float v = alpha * (acc0 + acc1);
    const int64_t i = static_cast<int64_t>(b) * a.hq + h * G + g;
    if (a.mfma)
      static_cast<_Float16*>(a.A16)[i * a.kpp + pos] = static_cast<_Float16>(v);
    else
      a.A[i * a.kpad + pos] = v;
  }
}

// Edge block (16-bit caches).  The retained rows of K and V (exact dims from
// kx / vx, compressible dims from ke / ve, in dims order) are loaded with
// every load in flight at once; K goes to LDS, V waits in registers and
// takes K's place once the scores are formed.
// smem: rows [E][D + 8] bf16 | q [G][D] fp32 raw | q [G][D] fp32 in dims
// order | probabilities [G][E] fp32 | dims [D] int.
constexpr int kEdgeLoads = 8;  // 8-byte or 16-byte chunks per thread and matrix

// KR: query rows per lane group in the scores and values (1, or 4 when G >= 4).
template <int KR>
__device__ __forceinline__ void prep_edge_block(const DecodeArgs& a, int b, int h, float* sm) {
  const int L = a.seq.len[b], M = a.seq.mid[b];
  const int S = a.sink, E = a.sink + a.recent;
  const int ne = (M > 0) ? E : L;  // retained tokens (all of them without a middle)
  const int D = a.D, du = a.du, dc = a.dc, G = a.G;
  const int ns = a.seq.nsplit[b];
  const int RSD = D + 8;  // halves per LDS row
  uint16_t* rows = reinterpret_cast<uint16_t*>(sm);
  float* qraw = sm + (E * RSD) / 2;
  float* qs = qraw + G * D;
  float* ps = qs + G * D;
  int* dl = reinterpret_cast<int*>(ps + G * E);
  const int tid = threadIdx.x, nt = blockDim.x;
  const int64_t row0 = a.seq.row0[b];
  const uint16_t* kxh = static_cast<const uint16_t*>(a.kx) + (row0 + static_cast<int64_t>(h) * L) * du;
  const uint16_t* vxh = static_cast<const uint16_t*>(a.vx) + (row0 + static_cast<int64_t>(h) * L) * du;
  const uint16_t* keh = static_cast<const uint16_t*>(a.ke) + (static_cast<int64_t>(b) * a.hkv + h) * E * dc;
  const uint16_t* veh = static_cast<const uint16_t*>(a.ve) + (static_cast<int64_t>(b) * a.hkv + h) * E * dc;
  // chunk w of a row: CW halves; exact dims first, then compressible dims
  const bool wide = (du % 8 == 0) && (dc % 8 == 0);
  const int CW = wide ? 8 : 2;
  const int nu = du / CW, nc = dc / CW, per_row = nu + nc;
  const int nchunk = ne * per_row;
  auto chunk_src = [&](const uint16_t* xh, const uint16_t* eh, int i) {
    const int e = i / per_row, w = i % per_row;
    if (w < nu) {
      const int t = (M > 0 && e >= S) ? e + M : e;
      return xh + static_cast<int64_t>(t) * du + w * CW;
    }
    return eh + static_cast<int64_t>(e) * dc + (w - nu) * CW;
  };
  auto chunk_dst = [&](int i) {
    const int e = i / per_row, w = i % per_row;
    return rows + e * RSD + w * CW;
  };
  uint4 kv[kEdgeLoads], vv[kEdgeLoads];
  for (int i0 = 0; i0 < nchunk; i0 += kEdgeLoads * nt) {
    // K and V chunks of this round, all in flight
#pragma unroll
    for (int u = 0; u < kEdgeLoads; ++u) {
      const int i = i0 + tid + u * nt;
      kv[u] = vv[u] = make_uint4(0u, 0u, 0u, 0u);
      if (i < nchunk) {
        if (wide) {
          kv[u] = *reinterpret_cast<const uint4*>(chunk_src(kxh, keh, i));
          vv[u] = *reinterpret_cast<const uint4*>(chunk_src(vxh, veh, i));
        } else {
          kv[u].x = *reinterpret_cast<const uint32_t*>(chunk_src(kxh, keh, i));
          vv[u].x = *reinterpret_cast<const uint32_t*>(chunk_src(vxh, veh, i));
        }
      }
    }
    if (i0 == 0) stage_q<uint16_t>(a, b, h, qraw, dl, a.scale);
    if (i0 + kEdgeLoads * nt >= nchunk) break;  // the last round's V stays in registers
    // more rounds than registers (large heads): V goes through LDS later
#pragma unroll
    for (int u = 0; u < kEdgeLoads; ++u) {
      const int i = i0 + tid + u * nt;
      if (i < nchunk) {
        if (wide) *reinterpret_cast<uint4*>(chunk_dst(i)) = kv[u];
        else *reinterpret_cast<uint32_t*>(chunk_dst(i)) = kv[u].x;
      }
    }
  }
  if (nchunk == 0) stage_q<uint16_t>(a, b, h, qraw, dl, a.scale);
  const int last0 = (nchunk > 0) ? ((nchunk - 1) / (kEdgeLoads * nt)) * (kEdgeLoads * nt) : 0;
#pragma unroll
  for (int u = 0; u < kEdgeLoads; ++u) {
    const int i = last0 + tid + u * nt;
    if (i < nchunk) {
      if (wide) *reinterpret_cast<uint4*>(chunk_dst(i)) = kv[u];
      else *reinterpret_cast<uint32_t*>(chunk_dst(i)) = kv[u].x;
    }
  }
  __syncthreads();
  // q in dims order, scaled; the exact-dim part also as bf16 for the split kernel
  const int du32 = (du + 31) & ~31;
  for (int idx = tid; idx < G * D; idx += nt) {
    const int g = idx / D, j = idx % D;
    const int d = dl[j];
    qs[idx] = (d >= 0 && d < D) ? qraw[g * D + d] : 0.0f;
  }
  for (int idx = tid; idx < G * du32; idx += nt) {
    const int g = idx / du32, j = idx % du32;
    const int64_t i = static_cast<int64_t>(b) * a.hq + h * G + g;
    uint16_t bits = 0;
    if (j < du) {
      const int d = dl[j];
      if (d >= 0 && d < D) bits = static_cast<const uint16_t*>(a.q)[q_row(a, b, h * G + g) * D + d];
    }
    static_cast<uint16_t*>(a.Q16)[i * du32 + j] = bits;
  }
  __syncthreads();
  // scores: a group of 16 lanes per (token e, block of KR rows), 8
  // dims per lane and 128-dim pass (2 dims per lane and pass without 16-byte
  // rows): the K chunk is read once for the block's rows, whose 16 partial
  // dots are then summed with DPP rotations
  const int l16 = tid & 15, grp = tid >> 4, ngrp = nt >> 4;
  const int nrb = (G + KR - 1) / KR;
  const int npair = ne * nrb;
  for (int pr0 = 0; pr0 < npair; pr0 += ngrp) {
    const int pr = pr0 + grp;
    const bool ok = pr < npair;
    const int e = ok ? pr / nrb : 0, g0 = ok ? (pr % nrb) * KR : 0;
    const uint16_t* kr = rows + e * RSD;
    float acc[KR];
#pragma unroll
    for (int r = 0; r < KR; ++r) acc[r] = 0.0f;
    if (wide) {
      for (int d0 = 8 * l16; d0 < D; d0 += 128) {
        const uint4 w = *reinterpret_cast<const uint4*>(kr + d0);
        const float k0 = __uint_as_float(w.x << 16), k1 = __uint_as_float(w.x & 0xFFFF0000u);
        const float k2 = __uint_as_float(w.y << 16), k3 = __uint_as_float(w.y & 0xFFFF0000u);
        const float k4 = __uint_as_float(w.z << 16), k5 = __uint_as_float(w.z & 0xFFFF0000u);
        const float k6 = __uint_as_float(w.w << 16), k7 = __uint_as_float(w.w & 0xFFFF0000u);
#pragma unroll
        for (int r = 0; r < KR; ++r) {
          const float* qg = qs + min(g0 + r, G - 1) * D + d0;
          const float4 qa = *reinterpret_cast<const float4*>(qg);
          const float4 qb = *reinterpret_cast<const float4*>(qg + 4);
          float v = acc[r];
          v = fmaf(qa.x, k0, v); v = fmaf(qa.y, k1, v); v = fmaf(qa.z, k2, v); v = fmaf(qa.w, k3, v);
          v = fmaf(qb.x, k4, v); v = fmaf(qb.y, k5, v); v = fmaf(qb.z, k6, v); v = fmaf(qb.w, k7, v);
          acc[r] = v;
        }
      }
    } else {
      for (int d0 = 2 * l16; d0 < D; d0 += 32) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(kr + d0);
        const float k0 = __uint_as_float(w << 16), k1 = __uint_as_float(w & 0xFFFF0000u);
#pragma unroll
        for (int r = 0; r < KR; ++r) {
          const float* qg = qs + min(g0 + r, G - 1) * D + d0;
          acc[r] = fmaf(qg[1], k1, fmaf(qg[0], k0, acc[r]));
        }
      }
    }
#pragma unroll
    for (int r = 0; r < KR; ++r) acc[r] = row16_sum(acc[r]);
    if (ok && l16 == 0)
#pragma unroll
      for (int r = 0; r < KR; ++r)
        if (g0 + r < G) ps[(g0 + r) * ne + e] = acc[r];
  }
  __syncthreads();
  // V replaces K in LDS (the last round from registers, earlier rounds reloaded)
  for (int i0 = 0; i0 < last0; i0 += nt) {
    const int i = i0 + tid;
    if (wide) *reinterpret_cast<uint4*>(chunk_dst(i)) = *reinterpret_cast<const uint4*>(chunk_src(vxh, veh, i));
    else *reinterpret_cast<uint32_t*>(chunk_dst(i)) = *reinterpret_cast<const uint32_t*>(chunk_src(vxh, veh, i));
  }
#pragma unroll
  for (int u = 0; u < kEdgeLoads; ++u) {
    const int i = last0 + tid + u * nt;
    if (i < nchunk) {
      if (wide) *reinterpret_cast<uint4*>(chunk_dst(i)) = vv[u];
      else *reinterpret_cast<uint32_t*>(chunk_dst(i)) = vv[u].x;
    }
  }
  // softmax of each row: one wave per row
  const int lane = tid & 63, nwv = nt >> 6;
  for (int g = tid >> 6; g < G; g += nwv) {
    float m = -INFINITY;
    for (int e = lane; e < ne; e += 64) m = fmaxf(m, ps[g * ne + e]);
    m = wave_max(m);
    float l = 0.0f;
    for (int e = lane; e < ne; e += 64) {
      const float pe = (m == -INFINITY) ? 0.0f : __expf(ps[g * ne + e] - m);
      ps[g * ne + e] = pe;
      l += pe;
    }
    l = wave_sum(l);
    if (lane == 0) {
      float* P = a.part + (static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(h * G + g) * ns + ns - 1) * a.RS;
      P[0] = m;
      P[1] = l;
    }
  }
  __syncthreads();
  // values: a group of 16 lanes per (8-dim chunk, block of KR rows),
  // tokens split over the lanes (e = lane, lane + 16, ...): each V chunk is
  // read once for the block's rows; the 16 partial sums are added with DPP
  // rotations (a thread per (row, dim) without 16-byte rows)
  float* P0 = a.part + (static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(h * G) * ns + ns - 1) * a.RS + 2;
  const int64_t prs = static_cast<int64_t>(ns) * a.RS;  // partial-row stride of consecutive rows g
  if (wide) {
    const int nch = D / 8, nunit = nch * nrb;
    for (int u0 = 0; u0 < nunit; u0 += ngrp) {
      const int un = u0 + grp;
      const bool ok = un < nunit;
      const int c8 = ok ? un % nch : 0, g0 = ok ? (un / nch) * KR : 0;
      float acc[KR][8];
#pragma unroll
      for (int r = 0; r < KR; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[r][j] = 0.0f;
      for (int e = l16; e < ne; e += 16) {
        const uint4 w = *reinterpret_cast<const uint4*>(rows + e * RSD + 8 * c8);
        const float v0 = __uint_as_float(w.x << 16), v1 = __uint_as_float(w.x & 0xFFFF0000u);
        const float v2 = __uint_as_float(w.y << 16), v3 = __uint_as_float(w.y & 0xFFFF0000u);
        const float v4 = __uint_as_float(w.z << 16), v5 = __uint_as_float(w.z & 0xFFFF0000u);
        const float v6 = __uint_as_float(w.w << 16), v7 = __uint_as_float(w.w & 0xFFFF0000u);
#pragma unroll
        for (int r = 0; r < KR; ++r) {
          const float pe = ps[min(g0 + r, G - 1) * ne + e];
          acc[r][0] = fmaf(pe, v0, acc[r][0]); acc[r][1] = fmaf(pe, v1, acc[r][1]);
          acc[r][2] = fmaf(pe, v2, acc[r][2]); acc[r][3] = fmaf(pe, v3, acc[r][3]);
          acc[r][4] = fmaf(pe, v4, acc[r][4]); acc[r][5] = fmaf(pe, v5, acc[r][5]);
          acc[r][6] = fmaf(pe, v6, acc[r][6]); acc[r][7] = fmaf(pe, v7, acc[r][7]);
        }
      }
#pragma unroll
      for (int r = 0; r < KR; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[r][j] = row16_sum(acc[r][j]);
      if (ok && l16 < 8) {
#pragma unroll
        for (int r = 0; r < KR; ++r) {
          float v = acc[r][0];
#pragma unroll
          for (int j = 1; j < 8; ++j) v = (l16 == j) ? acc[r][j] : v;
          // partial layout [m, l, o_U(du), o_E(dc), W]: dim j of the row sits at 2 + j
          if (g0 + r < G) P0[(g0 + r) * prs + 8 * c8 + l16] = v;
        }
      }
    }
  } else {
    for (int idx = tid; idx < G * D; idx += nt) {
      const int g = idx / D, j = idx % D;
      const float* pg = ps + g * ne;
      float acc = 0.0f;
      for (int e = 0; e < ne; ++e) acc = fmaf(pg[e], bf16_to_f32(rows[e * RSD + j]), acc);
      P0[g * prs + j] = acc;
    }
  }
}

// Edge block on MFMA (16-byte rows, D % 32 == 0, G <= 16): scores
// S = q K^T with v_mfma_f32_16x16x32_bf16 (q and K are bf16, exact products;
// the scale is applied to the fp32 result), values O = P V with
// v_mfma_f32_16x16x16bf16_1k on P split into bf16 hi + lo (about 16 bits of
// p), V read transposed from LDS.  Token blocks of 16 (ne rounded up; the
// padding tokens get a score of -inf and zero V rows).
// smem: rows [E16][D + 8] bf16 | q [G][D] fp32 raw | q [G][D + 8] bf16 in
// dims order | scores / probabilities [G][E16] fp32 | dims [D] int.
typedef __bf16 ebf16x8 __attribute__((ext_vector_type(8)));
typedef short eshort4 __attribute__((ext_vector_type(4)));
typedef float efloat4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) eshort4 elds_short4;

// Transposed 4 x 16-bit LDS read: lane 4c+e of each 16-lane group receives
// element e of the 8-byte chunks addressed by lanes c, c+4, c+8, c+12.
__device__ inline eshort4 edge_tr4(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((elds_short4*)(p));
}
__device__ inline uint16_t edge_bf16_rne(float x) {  // finite inputs
  const uint32_t u = __float_as_uint(x);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__host__ __device__ inline size_t edge_mfma_smem_bytes(int E, int G, int D) {
  const size_t E16 = (static_cast<size_t>(E) + 15) & ~static_cast<size_t>(15);
  const size_t qb = (static_cast<size_t>(G) * (D + 8) + 7) & ~static_cast<size_t>(7);  // halves
  return 2 * E16 * (D + 8) + 4 * static_cast<size_t>(G) * D + 2 * qb + 4 * static_cast<size_t>(G) * E16 + 4 * D;
}

//
// The retained tokens of a (sequence, KV head) are cut into a.edge_split
// parts of whole 16-token blocks; part `part` is split ns - edge_split + part
// of each row (a part past the retained tokens writes an empty split).
__device__ __forceinline__ void prep_edge_block_mfma(const DecodeArgs& a, int b, int h, int part, float* sm) {
  const int L = a.seq.len[b], M = a.seq.mid[b];
  const int S = a.sink, E = a.sink + a.recent;
  const int ne_all = (M > 0) ? E : L;
  const int D = a.D, du = a.du, dc = a.dc, G = a.G;
  const int ns = a.seq.nsplit[b];
  const int E16 = (E + 15) & ~15, RSE = D + 8, QS = D + 8;
  // this part's tokens [e0, e0 + P16) of the retained ones (16-token blocks),
  // ne of them real; local token el is retained token e0 + el
  const int PT = ((E16 / 16 + a.edge_split - 1) / a.edge_split) * 16;
  const int e0 = part * PT;
  const int P16 = max(0, min(E16, e0 + PT) - e0);
  const int ne = max(0, min(ne_all, e0 + P16) - e0);
  const int esp = ns - a.edge_split + part;
  uint16_t* rows = reinterpret_cast<uint16_t*>(sm);
  float* qraw = sm + (E16 * RSE) / 2;
  uint16_t* qb = reinterpret_cast<uint16_t*>(qraw + G * D);
  float* ps = reinterpret_cast<float*>(qb + ((G * QS + 7) & ~7));
  int* dl = reinterpret_cast<int*>(ps + G * E16);
  const int tid = threadIdx.x, nt = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, nwv = nt >> 6, l16 = lane & 15, g4 = lane >> 4;
  const int64_t row0 = a.seq.row0[b];
  const uint16_t* kxh = static_cast<const uint16_t*>(a.kx) + (row0 + static_cast<int64_t>(h) * L) * du;
  const uint16_t* vxh = static_cast<const uint16_t*>(a.vx) + (row0 + static_cast<int64_t>(h) * L) * du;
  const uint16_t* keh = static_cast<const uint16_t*>(a.ke) + (static_cast<int64_t>(b) * a.hkv + h) * E * dc;
  const uint16_t* veh = static_cast<const uint16_t*>(a.ve) + (static_cast<int64_t>(b) * a.hkv + h) * E * dc;
  const int nu = du / 8, per_row = nu + dc / 8;  // 16-byte chunks: exact dims first
  const int nchunk = ne * per_row;
  auto chunk_src = [&](const uint16_t* xh, const uint16_t* eh, int i) {
    const int e = e0 + i / per_row, w = i % per_row;
    if (w < nu) {
      const int t = (M > 0 && e >= S) ? e + M : e;
      return xh + static_cast<int64_t>(t) * du + w * 8;
    }
    return eh + static_cast<int64_t>(e) * dc + (w - nu) * 8;
  };
  auto chunk_dst = [&](int i) { return rows + (i / per_row) * RSE + (i % per_row) * 8; };
  // every load in flight: K to LDS, the last round of V kept in registers
  uint4 kv[kEdgeLoads], vv[kEdgeLoads];
  for (int i0 = 0; i0 < nchunk; i0 += kEdgeLoads * nt) {
#pragma unroll
    for (int u = 0; u < kEdgeLoads; ++u) {
      const int i = i0 + tid + u * nt;
      kv[u] = vv[u] = make_uint4(0u, 0u, 0u, 0u);
      if (i < nchunk) {
        kv[u] = *reinterpret_cast<const uint4*>(chunk_src(kxh, keh, i));
        vv[u] = *reinterpret_cast<const uint4*>(chunk_src(vxh, veh, i));
      }
    }
    if (i0 == 0) stage_q<uint16_t>(a, b, h, qraw, dl, 1.0f);
    if (i0 + kEdgeLoads * nt >= nchunk) break;
#pragma unroll
    for (int u = 0; u < kEdgeLoads; ++u) {
      const int i = i0 + tid + u * nt;
      if (i < nchunk) *reinterpret_cast<uint4*>(chunk_dst(i)) = kv[u];
    }
  }
  if (nchunk == 0) stage_q<uint16_t>(a, b, h, qraw, dl, 1.0f);
  const int last0 = (nchunk > 0) ? ((nchunk - 1) / (kEdgeLoads * nt)) * (kEdgeLoads * nt) : 0;
#pragma unroll
  for (int u = 0; u < kEdgeLoads; ++u) {
    const int i = last0 + tid + u * nt;
    if (i < nchunk) *reinterpret_cast<uint4*>(chunk_dst(i)) = kv[u];
  }
  __syncthreads();
  // q in dims order as bf16 (exact: the raw q values are bf16), and the
  // exact-dim part as the split kernel's operand
  const int du32 = (du + 31) & ~31;
  for (int idx = tid; idx < G * D; idx += nt) {
    const int g = idx / D, j = idx % D;
    const int d = dl[j];
    qb[g * QS + j] = (d >= 0 && d < D) ? static_cast<uint16_t>(__float_as_uint(qraw[g * D + d]) >> 16) : 0;
  }
  for (int idx = tid; part == 0 && idx < G * du32; idx += nt) {
    const int g = idx / du32, j = idx % du32;
    const int64_t i = static_cast<int64_t>(b) * a.hq + h * G + g;
    uint16_t bits = 0;
    if (j < du) {
      const int d = dl[j];
      if (d >= 0 && d < D) bits = static_cast<const uint16_t*>(a.q)[q_row(a, b, h * G + g) * D + d];
    }
    static_cast<uint16_t*>(a.Q16)[i * du32 + j] = bits;
  }
  __syncthreads();
  // scores: wave -> token blocks of 16; lane (l16 = token, g4) -> rows 4 g4 + r
  for (int eb = wave; eb < P16 / 16; eb += nwv) {
    efloat4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kc = 0; kc < D / 32; ++kc) {
      uint4 qa = make_uint4(0u, 0u, 0u, 0u);
      if (l16 < G) qa = *reinterpret_cast<const uint4*>(qb + l16 * QS + kc * 32 + 8 * g4);
      const uint4 kb = *reinterpret_cast<const uint4*>(rows + (eb * 16 + l16) * RSE + kc * 32 + 8 * g4);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(ebf16x8, qa), __builtin_bit_cast(ebf16x8, kb),
                                                    acc, 0, 0, 0);
    }
    const int e = eb * 16 + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * g4 + r;
      if (g < G) ps[g * E16 + e] = (e < ne) ? a.scale * acc[r] : -INFINITY;
    }
  }
  __syncthreads();
  // V replaces K (the last round from registers, earlier rounds reloaded);
  // padding rows [ne, P16) are zero
  for (int i0 = 0; i0 < last0; i0 += nt) {
    const int i = i0 + tid;
    *reinterpret_cast<uint4*>(chunk_dst(i)) = *reinterpret_cast<const uint4*>(chunk_src(vxh, veh, i));
  }
#pragma unroll
  for (int u = 0; u < kEdgeLoads; ++u) {
    const int i = last0 + tid + u * nt;
    if (i < nchunk) *reinterpret_cast<uint4*>(chunk_dst(i)) = vv[u];
  }
  for (int i = tid; i < (P16 - ne) * (D / 8); i += nt)
    *reinterpret_cast<uint4*>(rows + (ne + i / (D / 8)) * RSE + (i % (D / 8)) * 8) = make_uint4(0u, 0u, 0u, 0u);
  // softmax of each row (one wave per row); probabilities of padding tokens are 0
  for (int g = wave; g < G; g += nwv) {
    float m = -INFINITY;
    for (int e = lane; e < ne; e += 64) m = fmaxf(m, ps[g * E16 + e]);
    m = wave_max(m);
    float l = 0.0f;
    for (int e = lane; e < P16; e += 64) {
      const float pe = (e >= ne || m == -INFINITY) ? 0.0f : __expf(ps[g * E16 + e] - m);
      ps[g * E16 + e] = pe;
      l += pe;
    }
    l = wave_sum(l);
    if (lane == 0) {
      float* P = a.part + (static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(h * G + g) * ns + esp) * a.RS;
      P[0] = m;
      P[1] = l;
    }
  }
  __syncthreads();
  // values: wave -> 16-dim blocks; A = P (rows l16, tokens 4 g4 .. +3) as
  // bf16 hi + lo, B = V read transposed (tokens 4 g4 .. +3 of dim l16)
  float* P0 = a.part + (static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(h * G) * ns + esp) * a.RS + 2;
  const int64_t prs = static_cast<int64_t>(ns) * a.RS;
  for (int nb = wave; nb < D / 16; nb += nwv) {
    efloat4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kt = 0; kt < P16 / 16; ++kt) {
      float4 p4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (l16 < G) p4 = *reinterpret_cast<const float4*>(ps + l16 * E16 + kt * 16 + 4 * g4);
      const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
      eshort4 hi4, lo4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint16_t hb = edge_bf16_rne(pv[j]);
        hi4[j] = static_cast<short>(hb);
        lo4[j] = static_cast<short>(edge_bf16_rne(pv[j] - __uint_as_float(static_cast<uint32_t>(hb) << 16)));
      }
      const eshort4 vb = edge_tr4(rows + (kt * 16 + 4 * g4 + (l16 >> 2)) * RSE + nb * 16 + 4 * (l16 & 3));
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi4, vb, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo4, vb, acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * g4 + r;
      // partial layout [m, l, o_U(du), o_E(dc), W]: dim j of the row sits at 2 + j
      if (g < G) P0[g * prs + nb * 16 + l16] = acc[r];
    }
  }
}

// A rows on the MFMA path (dc % 4 == 0, ck 16-byte aligned), as an fp32
// MFMA product per (sequence, KV head): D[g][n] = sum_c qC[g][c] ck[n][c].
// Each wave takes TILES 16-row tiles of ck and runs over the columns in
// groups of 16 NI: lane (r, q) = (lane % 16, lane / 16) holds columns 16 i +
// 4 q .. 16 i + 4 q + 3 of the group for row r as float4 i, so that step (i,
// j) of v_mfma_f32_16x16x4f32 (k index q) sums column 16 i + 4 q + j; q_C
// uses the same column map, read from the block's q rows and dims staged in
// LDS.  NI covers dc in one group up to 128 columns (TILES * NI <= 12 float4
// per lane), so the ck loads and the q / dims loads go out together: one
// memory round trip and one barrier per block.  Coefficient n sits at pair
// position 0 (n = 0) or n + 1; position 1 (the sine of frequency 0) is 0.
constexpr int kPrepF4 = 12;  // float4 of ck in flight per lane
__host__ __device__ constexpr int prep_a_ni(int dc) {
  return dc <= 32 ? 2 : dc <= 64 ? 4 : dc <= 96 ? 6 : 8;
}
__host__ __device__ constexpr int prep_a_tiles(int ni) { return ni >= 8 ? 1 : kPrepF4 / ni / (ni == 2 ? 2 : 1); }
// ck rows per A block
__host__ __device__ inline int prep_a_rows(int dc) { return 16 * prep_a_tiles(prep_a_ni(dc)) * (kPrepThreads / 64); }

__host__ __device__ inline bool prep_a_mfma_ok(const DecodeArgs& a, bool vec) {
  return a.mfma && vec && a.dc % 4 == 0;
}

template <typename T, int NI>
__device__ __forceinline__ void prep_a_mfma(const DecodeArgs& a, int b, int h, int chunk, float* sm) {
  constexpr int TILES = prep_a_tiles(NI);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int G = a.G, D = a.D, dc = a.dc, k = a.k, kpp = a.kpp;
  const int M = a.seq.mid[b], per = a.seq.per[b];
  const int n0 = chunk * (16 * TILES * (kPrepThreads / 64)) + wave * (16 * TILES);
  const float* ckh = a.ck + (static_cast<int64_t>(b) * a.hkv + h) * k * dc;
  float* qraw = sm;                                    // [G][D] scaled q rows
  int* dl = reinterpret_cast<int*>(qraw + G * D);      // [D] dims of KV head h
  auto load_ck = [&](float4 (&ckv)[TILES][NI], int c0) {
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int n = n0 + 16 * t + r16;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int c = c0 + 16 * i + 4 * q4;
        ckv[t][i] = (n < k && c < dc) ? *reinterpret_cast<const float4*>(ckh + static_cast<int64_t>(n) * dc + c)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  float4 ckv[TILES][NI];  // the current column group's tiles
  load_ck(ckv, 0);
  stage_q<T>(a, b, h, qraw, dl, a.scale);
  __syncthreads();
  if (n0 >= kpp) return;  // no barrier follows
  _Float16* A16 = static_cast<_Float16*>(a.A16);
  const int64_t arow0 = static_cast<int64_t>(b) * a.hq + static_cast<int64_t>(h) * G;
  for (int g0 = 0; g0 < G; g0 += 16) {
    const int g = g0 + r16;
    efloat4 acc[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) acc[t] = efloat4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < dc; c0 += 16 * NI) {
      if (c0 > 0 || (g0 > 0 && dc > 16 * NI)) load_ck(ckv, c0);  // else still loaded
      float qc[NI][4];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int c = c0 + 16 * i + 4 * q4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = (c + j < dc) ? dl[a.du + c + j] : -1;
          qc[i][j] = (g < G && d >= 0 && d < D) ? qraw[g * D + d] : 0.0f;
        }
      }
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const float cv4[4] = {ckv[t][i].x, ckv[t][i].y, ckv[t][i].z, ckv[t][i].w};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(qc[i][j], cv4[j], acc[t], 0, 0, 0);
        }
    }
    // lane holds D[g0 + 4 q + r][n0 + 16 t + r16]
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int n = n0 + 16 * t + r16;
      const int pos = (n == 0) ? 0 : n + 1;
      const float alpha = (M > 0 && n < k) ? basis_alpha(n, per) : 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gr = g0 + 4 * q4 + r;
        if (gr >= G) continue;
        _Float16* row = A16 + (arow0 + gr) * kpp;
        if (pos < kpp) row[pos] = static_cast<_Float16>(alpha * acc[t][r]);
        if (n == 0) row[1] = static_cast<_Float16>(0.0f);
      }
    }
  }
}

// Blocks [0, nedge) are edge blocks (MFMA path), the rest A blocks.
template <typename T, bool VEC>
__global__ __launch_bounds__(kPrepThreads) void decode_prep_kernel(DecodeArgs a, int nedge, int chunks) {
  extern __shared__ float smem[];
  int blk = blockIdx.x;
  if (blk < nedge) {
    // edge blocks: (sequence, KV head, part); the VALU edge block takes the
    // retained tokens whole (the planner gives it one part)
    if (a.edge_split) {
      const int bh = blk / a.edge_split, part = blk % a.edge_split;
      if (edge_mfma_ok(a))
        prep_edge_block_mfma(a, bh / a.hkv, bh % a.hkv, part, smem);
      else if (a.G >= 4)
        prep_edge_block<4>(a, bh / a.hkv, bh % a.hkv, smem);
      else
        prep_edge_block<1>(a, bh / a.hkv, bh % a.hkv, smem);
    }
    return;
  }
  blk -= nedge;
  const int bh = blk / chunks, chunk = blk % chunks;
  if (prep_a_mfma_ok(a, VEC)) {
    switch (prep_a_ni(a.dc)) {
      case 2: prep_a_mfma<T, 2>(a, bh / a.hkv, bh % a.hkv, chunk, smem); break;
      case 4: prep_a_mfma<T, 4>(a, bh / a.hkv, bh % a.hkv, chunk, smem); break;
      case 6: prep_a_mfma<T, 6>(a, bh / a.hkv, bh % a.hkv, chunk, smem); break;
      default: prep_a_mfma<T, 8>(a, bh / a.hkv, bh % a.hkv, chunk, smem); break;
    }
  }
  else
    prep_a_block<T, VEC>(a, bh / a.hkv, bh % a.hkv, chunk, smem);
}

// -------------------------------------------------------------- split ----
// VALU kernel: rows <= kDecRows consecutive query heads, tiles of kDecTile
// tokens.  Thread slots own basis pairs j = tid + 256 i (slot 0 = constant).
constexpr int kMaxSlots = 9;  // ceil((4097/2 + 1) / 256)

template <typename T>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int R = kDecRows;
  constexpr int TT = kDecTile;
  extern __shared__ float smem[];
  float* qs = smem;                      // [R][D]
  float* As = qs + R * a.D;              // [R][kpad]
  float* sc = As + R * a.kpad;           // [4][R][TT]
  float* ps = sc + 4 * R * TT;           // [TT][R]
  float* corr = ps + TT * R;             // [R]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int item = blockIdx.x;
  const int b = seq_of_item(a.seq, a.nseq, item);
  const int local = item - a.seq.item0[b];
  const int ns = a.seq.nsplit[b];
  const int rg = local / ns, sp = local % ns;
  const int L = a.seq.len[b], M = a.seq.mid[b], per = a.seq.per[b];
  const int S = a.sink, E = a.sink + a.recent;
  const int t_begin = sp * a.seq.chunk[b];
  const int t_end = min(L, t_begin + a.seq.chunk[b]);
  const int64_t row0 = a.seq.row0[b];
  const bool comp = a.dc > 0;
  const bool has_mid = comp && M > 0;

  int qi[R], kh[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    qi[r] = rg * a.rows + min(r, a.rows - 1);
    kh[r] = qi[r] / a.G;
  }

  // q rows in dim-split order, scaled; A rows.
  for (int idx = tid; idx < R * a.D; idx += blockDim.x) {
    const int r = idx / a.D, j = idx % a.D;
    float v = 0.0f;
    if (r < a.rows) {
      const int d = a.dims[kh[r] * a.D + j];
      if (d >= 0 && d < a.D)
        v = a.scale * ld<T>(a.q, q_row(a, b, qi[r]) * a.D + d);
    }
    qs[idx] = v;
  }
  if (has_mid)
    for (int idx = tid; idx < R * a.kpad; idx += blockDim.x) {
      const int r = idx / a.kpad, n = idx % a.kpad;
      As[idx] = (r < a.rows && n < a.k)
                    ? a.A[(static_cast<int64_t>(b) * a.hq + qi[r]) * a.kpad + n]
                    : 0.0f;
    }

  const int nslots = a.k / 2 + 1;  // slot 0: n = 0; slot j: n = 2j-1, 2j
  const int nown = (nslots > tid) ? (nslots - tid + 255) / 256 : 0;
  const int du4 = (a.du + 3) / 4, dc4 = (a.dc + 3) / 4, sl4 = (nslots + 3) / 4;
  const int part = wave;  // phase A: thread (token lane, part)

  // running softmax state (wave r owns row r)
  float m_run = -INFINITY, l_run = 0.0f;
  float oacc[4], eacc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) oacc[j] = eacc[j] = 0.0f;
  float2 wstep[kMaxSlots];
  float wacc[kMaxSlots][2][R];
#pragma unroll
  for (int i = 0; i < kMaxSlots; ++i) {
    wstep[i] = (has_mid && i < nown) ? unit_phase(tid + 256 * i, 1, per) : make_float2(1.0f, 0.0f);
#pragma unroll
    for (int r = 0; r < R; ++r) wacc[i][0][r] = wacc[i][1][r] = 0.0f;
  }
  __syncthreads();

  for (int tile0 = t_begin; tile0 < t_end; tile0 += TT) {
    // ---------------- phase A: partial scores
    {
      const int t = tile0 + lane;
      float acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.0f;
      if (t < t_end) {
        const int d0 = part * du4, d1 = min(a.du, d0 + du4);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r >= a.rows) break;
          const int64_t base = (row0 + static_cast<int64_t>(kh[r]) * L + t) * a.du;
          // batches of 8 loads in flight (the index is clamped, not branched on)
          for (int dd = d0; dd < d1; dd += 8) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = ld<T>(a.kx, base + min(dd + i, d1 - 1));
#pragma unroll
            for (int i = 0; i < 8; ++i)
              if (dd + i < d1) acc[r] = fmaf(qs[r * a.D + dd + i], v[i], acc[r]);
          }
        }
        if (comp) {
          const bool edge = (M == 0) || t < S || t >= S + M;
          if (edge) {
            const int e = (M == 0 || t < S) ? t : t - M;
            const int c0 = part * dc4, c1 = min(a.dc, c0 + dc4);
#pragma unroll
            for (int r = 0; r < R; ++r) {
              if (r >= a.rows) break;
              const int64_t base = ((static_cast<int64_t>(b) * a.hkv + kh[r]) * E + e) * a.dc;
              for (int cc = c0; cc < c1; cc += 8) {
                float v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = ld<T>(a.ke, base + min(cc + i, c1 - 1));
#pragma unroll
                for (int i = 0; i < 8; ++i)
                  if (cc + i < c1) acc[r] = fmaf(qs[r * a.D + a.du + cc + i], v[i], acc[r]);
              }
            }
          } else {
            const int tau = t - S;
            const int j0 = part * sl4, j1 = min(nslots, j0 + sl4);
            const float2 w = unit_phase(1, tau, per);
            float2 z = make_float2(1.0f, 0.0f);
            for (int j = j0; j < j1; ++j) {
              if (((j - j0) & 31) == 0) z = unit_phase(j, tau, per);
              if (j == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = fmaf(As[r * a.kpad], z.x, acc[r]);
              } else {
                const int n = 2 * j - 1;
                const bool has_sin = n + 1 < a.k;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                  acc[r] = fmaf(As[r * a.kpad + n], z.x, acc[r]);
                  if (has_sin) acc[r] = fmaf(As[r * a.kpad + n + 1], z.y, acc[r]);
                }
              }
              z = cmul(z, w);
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) sc[(part * R + r) * TT + lane] = acc[r];
    }
    __syncthreads();

    // ---------------- phase B: online softmax, wave r owns row r
    if (wave < a.rows) {
      const int r = wave;
      const int t = tile0 + lane;
      const bool valid = t < t_end;
      float s = (sc[(0 * R + r) * TT + lane] + sc[(1 * R + r) * TT + lane]) +
                (sc[(2 * R + r) * TT + lane] + sc[(3 * R + r) * TT + lane]);
      s = valid ? s : -INFINITY;
      const float m_new = fmaxf(m_run, wave_max(s));
      const float c = (m_run == -INFINITY) ? 0.0f : __expf(m_run - m_new);
      const float p = valid ? __expf(s - m_new) : 0.0f;
      l_run = l_run * c + wave_sum(p);
      m_run = m_new;
      ps[lane * R + r] = p;
      if (lane == 0) corr[r] = c;
    } else if (wave < R) {
      ps[lane * R + wave] = 0.0f;
      if (lane == 0) corr[wave] = 1.0f;
    }
    __syncthreads();

    // ---------------- phase C: values
    const int nt = min(TT, t_end - tile0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + 256 * j;
      if (idx >= a.rows * a.du) break;
      const int r = idx / a.du, d = idx % a.du;
      float o = oacc[j] * corr[r];
      const int64_t base = (row0 + static_cast<int64_t>(kh[r]) * L + tile0) * a.du + d;
      // batches of 16 tokens' loads in flight (clamped index, no branch)
      for (int t0 = 0; t0 < nt; t0 += 16) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = ld<T>(a.vx, base + static_cast<int64_t>(min(t0 + i, nt - 1)) * a.du);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (t0 + i < nt) o = fmaf(ps[(t0 + i) * R + r], v[i], o);
      }
      oacc[j] = o;
    }
    if (comp) {
      // only tiles that hold retained tokens read ve
      const bool any_edge = M == 0 || tile0 < S || tile0 + nt > S + M;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = tid + 256 * j;
        if (idx >= a.rows * a.dc) break;
        const int r = idx / a.dc, c = idx % a.dc;
        float o = eacc[j] * corr[r];
        const int64_t base = (static_cast<int64_t>(b) * a.hkv + kh[r]) * E * a.dc + c;
        if (any_edge)
          for (int t0 = 0; t0 < nt; t0 += 16) {
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int t = tile0 + min(t0 + i, nt - 1);
              const bool edge = M == 0 || t < S || t >= S + M;
              const int e = !edge ? 0 : ((M == 0 || t < S) ? t : t - M);
              v[i] = ld<T>(a.ve, base + static_cast<int64_t>(e) * a.dc);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int t = tile0 + t0 + i;
              if (t0 + i < nt && (M == 0 || t < S || t >= S + M)) o = fmaf(ps[(t0 + i) * R + r], v[i], o);
            }
          }
        eacc[j] = o;
      }
    }
    if (has_mid && nown > 0) {
      const int mid_lo = max(0, S - tile0), mid_hi = min(nt, S + M - tile0);
      float2 z[kMaxSlots];
#pragma unroll
      for (int i = 0; i < kMaxSlots; ++i) {
        // anchor at the tile's first middle token (tau >= 0)
        z[i] = (i < nown && mid_lo < mid_hi) ? unit_phase(tid + 256 * i, tile0 + mid_lo - S, per)
                                             : make_float2(0.0f, 0.0f);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          wacc[i][0][r] *= corr[r];
          wacc[i][1][r] *= corr[r];
        }
      }
      for (int tl = mid_lo; tl < mid_hi; ++tl) {
        const float4 p = *reinterpret_cast<const float4*>(&ps[tl * R]);
#pragma unroll
        for (int i = 0; i < kMaxSlots; ++i) {
          if (i < nown) {
            wacc[i][0][0] = fmaf(p.x, z[i].x, wacc[i][0][0]);
            wacc[i][1][0] = fmaf(p.x, z[i].y, wacc[i][1][0]);
            wacc[i][0][1] = fmaf(p.y, z[i].x, wacc[i][0][1]);
            wacc[i][1][1] = fmaf(p.y, z[i].y, wacc[i][1][1]);
            wacc[i][0][2] = fmaf(p.z, z[i].x, wacc[i][0][2]);
            wacc[i][1][2] = fmaf(p.z, z[i].y, wacc[i][1][2]);
            wacc[i][0][3] = fmaf(p.w, z[i].x, wacc[i][0][3]);
            wacc[i][1][3] = fmaf(p.w, z[i].y, wacc[i][1][3]);
            z[i] = cmul(z[i], wstep[i]);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---------------- write partials
  if (wave < a.rows) {
    const int r = wave;
    float* P = a.part + (static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(qi[r]) * ns + sp) * a.RS;
    if (lane == 0) {
      P[0] = m_run;
      P[1] = l_run;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = tid + 256 * j;
    if (idx < a.rows * a.du) {
      const int r = idx / a.du, d = idx % a.du;
      a.part[(static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(qi[r]) * ns + sp) * a.RS + 2 + d] = oacc[j];
    }
    if (idx < a.rows * a.dc) {
      const int r = idx / a.dc, c = idx % a.dc;
      a.part[(static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(qi[r]) * ns + sp) * a.RS + 2 + a.du + c] = eacc[j];
    }
  }
  if (has_mid) {
#pragma unroll
    for (int i = 0; i < kMaxSlots; ++i) {
      if (i >= nown) continue;
      const int j = tid + 256 * i;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r >= a.rows) break;
        float* Wp = a.part + (static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(qi[r]) * ns + sp) * a.RS + 2 + a.du + a.dc;
        if (j == 0) {
          Wp[0] = wacc[i][0][r];
        } else {
          Wp[2 * j - 1] = wacc[i][0][r];
          if (2 * j < a.k) Wp[2 * j] = wacc[i][1][r];
        }
      }
    }
  }
}

// -------------------------------------------------------------- merge ----
// Pass 1 (decode_merge_vec): one block per (query row, 256-wide slice of the
// partial vector [o_U | o_E | W]).  Each block recomputes the log-sum-exp
// weights of the splits, sums its slice over the splits in a fixed order and
// writes o_U / l to out, o_E and alpha * W to the merge buffer (mrg).
// Pass 2 (decode_merge_cv): one block per (sequence, KV head, 32 compressible
// dims) applies C_V to the merged W of the head's query rows and writes those
// dims of out.
constexpr int kMergeRows = 4;
constexpr int kMergeHeld = 2;    // split weights per lane kept in registers
constexpr int kMergeBatch = 32;  // split loads in flight per thread after the first
// FIRST: split loads issued before the weights exist.  64 holds a short
// context's splits in one round but takes about 220 registers (two waves per
// SIMD), so it is used only where the grid is one pass over the chip; larger
// grids issue none early and keep the occupancy (about 80 registers).
constexpr int kMergeFirstDeep = 64;
constexpr int kMergeFirstLean = 0;
constexpr int kMergeDeepBlocks = 512;  // two 256-thread blocks per CU
// Two-pass path: slices of 256 entries that hold any o_U / o_E entry (they
// also sum the W entries among theirs), then blocks of kMergeWSlices slices of
// W entries only.
constexpr int kMergeWSlices = 4;
__host__ __device__ inline int merge_vec_mixed_slices(const DecodeArgs& a) { return (a.du + a.dc + 255) / 256; }
__host__ __device__ inline int merge_vec_slices(const DecodeArgs& a) {
  const int nvec = a.du + a.dc + a.k;
  if (!a.two_pass) return (nvec + 255) / 256;
  const int y0 = merge_vec_mixed_slices(a);
  return y0 + (nvec - 256 * y0 + 256 * kMergeWSlices - 1) / (256 * kMergeWSlices);
}

template <int FIRST>
__global__ __launch_bounds__(256) void decode_merge_vec_kernel(DecodeArgs a) {
  extern __shared__ float smem[];  // [ns] weights
  const int row = blockIdx.x;      // b * hq + i
  const int b = row / a.hq, i = row % a.hq, h = i / a.G;
  const int ns = a.seq.nsplit[b];
  const int M = a.seq.mid[b], per = a.seq.per[b];
  const bool has_mid = a.dc > 0 && M > 0;
  const int nvec = a.du + a.dc + (has_mid ? a.k : 0);
  const int y0 = merge_vec_mixed_slices(a);
  if (a.two_pass && static_cast<int>(blockIdx.y) >= y0) {
    // kMergeWSlices slices of W entries only (entry 256 y0 + 256 (kMergeWSlices
    // (blockIdx.y - y0) + q) + tid for slice q): pass 2 has already scaled each
    // split group's W to the row's maximum, so it needs no split weights: the
    // groups' entries are summed in order, eight loads per slice in flight
    // (clamped indices, groups past the last add 0)
    const int first = 256 * y0 + 256 * kMergeWSlices * (static_cast<int>(blockIdx.y) - y0);
    if (first >= nvec) return;  // uniform per block (rows without middle have no W entries)
    // from here nvec > 256 y0 >= du + dc, so every clamped entry below is a W entry
    const int nsg = (ns - a.edge_split + kMomentWaves - 1) / kMomentWaves;
    const int64_t sgs = static_cast<int64_t>(a.hq) * a.kpad;
    const int e0 = first + threadIdx.x;
    const float* wrow = a.Wp + (static_cast<int64_t>(a.sgcum[b]) * a.hq + i) * a.kpad;
    float v[kMergeWSlices];
#pragma unroll
    for (int q = 0; q < kMergeWSlices; ++q) v[q] = 0.0f;
    for (int sg0 = 0; sg0 < nsg; sg0 += 8) {
      float x[kMergeWSlices][8];
#pragma unroll
      for (int q = 0; q < kMergeWSlices; ++q) {
        const int n = min(e0 + 256 * q, nvec - 1) - a.du - a.dc;  // clamped: past nvec stores nothing
#pragma unroll
        for (int j = 0; j < 8; ++j) x[q][j] = wrow[static_cast<int64_t>(min(sg0 + j, nsg - 1)) * sgs + n];
      }
#pragma unroll
      for (int q = 0; q < kMergeWSlices; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[q] += (sg0 + j < nsg) ? x[q][j] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < kMergeWSlices; ++q) {
      const int e = e0 + 256 * q;
      if (e >= nvec) break;
      const int n = e - a.du - a.dc;
      a.mrg[static_cast<int64_t>(row) * a.MS + a.dc + n] = v[q] * basis_alpha(n, per);
    }
    return;
  }
  const int idx = blockIdx.y * 256 + threadIdx.x;
  if (blockIdx.y * 256 >= nvec) return;  // uniform per block
  const float* P = a.part + (static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(i) * ns) * a.RS;
  // The entry this thread sums (threads past nvec load the last one and
  // store nothing) and the splits that hold it: with edge splits (the last
  // ones), o_E comes from them alone and W from the other splits alone.
  // Neither range is empty where its entry exists.
  const int e = min(idx, nvec - 1);
  int s_lo = 0, s_hi = ns;
  if (a.edge_split && e >= a.du) {
    if (e < a.du + a.dc) s_lo = ns - a.edge_split;
    else s_hi = ns - a.edge_split;
  }
  // two-pass path: W comes from Wp, and the partial rows end after o_E
  const bool wpass = a.two_pass && e >= a.du + a.dc;
  const float* Pi = P + 2 + (wpass ? 0 : e);
  // The entry's first FIRST splits and its output column are loaded in
  // the same round as the (m, l) pairs (clamped indices, no branch around a
  // load), so that the weights and the sum wait on one memory round trip.
  float x0[FIRST > 0 ? FIRST : 1];
#pragma unroll
  for (int j = 0; j < FIRST; ++j) x0[j] = Pi[static_cast<int64_t>(min(s_lo + j, s_hi - 1)) * a.RS];
  const int dd = a.dims[h * a.D + max(0, min(e, a.du - 1))];
  // every wave forms the split weights itself (wave reductions, no block
  // barrier); wave 0 publishes them for the sums below.  The (m, l) pairs of
  // a lane's first kMergeHeld splits are read once (clamped index, no
  // branch); splits beyond 64 kMergeHeld are read again.
  const int lane = threadIdx.x & 63;
  float mh[kMergeHeld], lh[kMergeHeld];
#pragma unroll
  for (int j = 0; j < kMergeHeld; ++j) {
    const int s = lane + 64 * j;
    const int64_t o = static_cast<int64_t>(min(s, ns - 1)) * a.RS;
    mh[j] = P[o];
    lh[j] = P[o + 1];
    if (s >= ns) mh[j] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kMergeHeld; ++j) mx = fmaxf(mx, mh[j]);
  for (int s = lane + 64 * kMergeHeld; s < ns; s += 64) mx = fmaxf(mx, P[static_cast<int64_t>(s) * a.RS]);
  mx = wave_max(mx);
  float lsum = 0.0f;
#pragma unroll
  for (int j = 0; j < kMergeHeld; ++j) {
    const int s = lane + 64 * j;
    const float w = (mh[j] == -INFINITY) ? 0.0f : __expf(mh[j] - mx);
    if (threadIdx.x < 64 && s < ns) smem[s] = w;
    lsum += w * lh[j];
  }
  for (int s = lane + 64 * kMergeHeld; s < ns; s += 64) {
    const float m = P[static_cast<int64_t>(s) * a.RS];
    const float w = (m == -INFINITY) ? 0.0f : __expf(m - mx);
    if (threadIdx.x < 64) smem[s] = w;
    lsum += w * P[static_cast<int64_t>(s) * a.RS + 1];
  }
  const float ltot = wave_sum(lsum), linv = 1.0f / ltot;
  __syncthreads();
  float* mrow = a.mrg + static_cast<int64_t>(row) * a.MS;
  if (blockIdx.y == 0 && threadIdx.x == 0) {
    mrow[a.dc + a.kpad] = linv;
    if (a.lse) a.lse[q_row(a, b, i)] = mx + logf(ltot);
  }
  if (idx >= nvec) return;
  if (wpass) {
    // W relative to the row's maximum over its splits, summed over the split
    // groups in order
    const int n = idx - a.du - a.dc;
    const int nsg = (ns - a.edge_split + kMomentWaves - 1) / kMomentWaves;
    const float* wp = a.Wp + (static_cast<int64_t>(a.sgcum[b]) * a.hq + i) * a.kpad + n;
    const int64_t sgs = static_cast<int64_t>(a.hq) * a.kpad;
    float v = 0.0f;
    for (int sg0 = 0; sg0 < nsg; sg0 += 8) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = wp[static_cast<int64_t>(min(sg0 + j, nsg - 1)) * sgs];
#pragma unroll
      for (int j = 0; j < 8; ++j) v += (sg0 + j < nsg) ? x[j] : 0.0f;
    }
    mrow[a.dc + n] = v * basis_alpha(n, per);
    return;
  }
  // fixed-order sum over the splits s_lo, s_lo + 1, ...: the loads already
  // held (a split past s_hi weighs 0: a multiply, not a branch, so that the
  // compiler keeps the load where it is), then whole batches of kMergeBatch
  // loads in flight, then batches of 16 with a clamped index
  float v = 0.0f;
#pragma unroll
  for (int j = 0; j < FIRST; ++j) {
    const float w = smem[min(s_lo + j, s_hi - 1)] * (s_lo + j < s_hi ? 1.0f : 0.0f);
    v = fmaf(w, x0[j], v);
  }
  int s0 = s_lo + FIRST;
  for (; s0 + kMergeBatch <= s_hi; s0 += kMergeBatch) {
    float x[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) x[j] = Pi[static_cast<int64_t>(s0 + j) * a.RS];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) v = fmaf(smem[s0 + j], x[j], v);
  }
  for (; s0 < s_hi; s0 += 16) {
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = Pi[static_cast<int64_t>(min(s0 + j, s_hi - 1)) * a.RS];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float w = smem[min(s0 + j, s_hi - 1)] * (s0 + j < s_hi ? 1.0f : 0.0f);
      v = fmaf(w, x[j], v);
    }
  }
  if (idx < a.du) {
    if (dd >= 0 && dd < a.D) a.out[q_row(a, b, i) * a.D + dd] = v * linv;
  } else if (idx < a.du + a.dc) {
    mrow[idx - a.du] = v;
  } else {
    const int n = idx - a.du - a.dc;
    mrow[a.dc + n] = v * basis_alpha(n, per);
  }
}

// Pass 2 body: one block per (sequence, KV head, slice of 4 QPB compressible
// dims) computes O_C[g][c] = sum_n (alpha W)[g][n] cv[n][c] for the head's
// query rows, kMergeRows rows at a time.  Thread (column quad cq, n-lane nl)
// reads 4 consecutive columns of the cv rows n = nl + NL j (NL = 256 / QPB
// n-lanes) and the matching (alpha W)[g][n], up to kCvBatch rows of both in
// flight; the NL n-lanes are summed in a fixed order (partial sums over
// groups of lanes, then the partials).  Wide slices (QPB 8: 32 columns, a
// 128-byte run of every cv row per block) read each head's alpha W twice
// instead of eight times; narrow ones (QPB 2) make more blocks for batches of
// few heads.
constexpr int kCvBatch = 16;
constexpr int kCvWideHeads = 128;  // (sequence, KV head) pairs from which slices are 32 columns wide

template <bool VEC, int QPB>
__global__ __launch_bounds__(256) void decode_merge_cv_kernel(DecodeArgs a) {
  constexpr int kCols = 4 * QPB;              // columns of a block
  constexpr int kLanes = 256 / QPB;           // n-lanes
  constexpr int kQ = kMergeRows * kCols;      // (row, column) pairs of a pass
  constexpr int kParts = 256 / kQ;            // partial sums of the lane reduction
  static_assert(kParts >= 1 && kLanes % kParts == 0, "lane groups tile the n-lanes");
  extern __shared__ float smem[];
  const int b = blockIdx.x / a.hkv, h = blockIdx.x % a.hkv;
  const int M = a.seq.mid[b];
  const bool has_mid = a.dc > 0 && M > 0;
  float* red = smem;                         // [kLanes][kQ]
  float* red2 = red + kLanes * kQ;           // [kParts][kQ]
  const int tid = threadIdx.x;
  const int cq = tid % QPB, nl = tid / QPB;
  const int c = blockIdx.y * kCols + 4 * cq;
  const float* cvb = a.cv + (static_cast<int64_t>(b) * a.hkv + h) * a.k * a.dc;
  for (int g0 = 0; g0 < a.G; g0 += kMergeRows) {
    const int ng = min(kMergeRows, a.G - g0);
    const float* wrow = a.mrg + (static_cast<int64_t>(b) * a.hq + h * a.G + g0) * a.MS + a.dc;
    // the epilogue's operands (merged o_E entry, 1/l, output column) are
    // loaded with the pass's first round of loads (clamped, unconditional)
    const int eg = min(tid / kCols, ng - 1);
    const int ecc = min(blockIdx.y * kCols + tid % kCols, a.dc - 1);
    const float* erow = a.mrg + (static_cast<int64_t>(b) * a.hq + h * a.G + g0 + eg) * a.MS;
    const float e_oe = erow[ecc];
    const float e_linv = erow[a.dc + a.kpad];
    const int e_dd = a.dims[h * a.D + a.du + ecc];
    __syncthreads();
    float acc[kMergeRows][4];
#pragma unroll
    for (int g = 0; g < kMergeRows; ++g) acc[g][0] = acc[g][1] = acc[g][2] = acc[g][3] = 0.0f;
    if (has_mid && c < a.dc) {
      for (int n0 = nl; n0 < a.k; n0 += kLanes * kCvBatch) {
        float4 x[kCvBatch];
        float wv[kCvBatch][kMergeRows];
#pragma unroll
        for (int j = 0; j < kCvBatch; ++j) {
          // rows past k (and row slots past ng) read a valid entry (clamped
          // index) and are weighted by 0 below: a multiply, not a select, so
          // that the compiler keeps the load unconditional and its wait counted
          const int n = n0 + kLanes * j;
          const int nc = min(n, a.k - 1);
#pragma unroll
          for (int g = 0; g < kMergeRows; ++g) wv[j][g] = wrow[static_cast<int64_t>(min(g, ng - 1)) * a.MS + nc];
          float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
          if (VEC) {
            v = *reinterpret_cast<const float4*>(cvb + static_cast<int64_t>(nc) * a.dc + c);
          } else if (n < a.k) {
            const float* src = cvb + static_cast<int64_t>(n) * a.dc + c;
            v.x = src[0];
            if (c + 1 < a.dc) v.y = src[1];
            if (c + 2 < a.dc) v.z = src[2];
            if (c + 3 < a.dc) v.w = src[3];
          }
          x[j] = v;
        }
        // every product is taken (rows past k and row slots past ng weigh
        // 0), so no load is left in flight at the loop's back edge and the
        // loop head needs no drain of the loads issued before it; the
        // scheduling barrier keeps all of the batch's loads ahead of its
        // products (interleaved, each row would wait on its own round trip)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kCvBatch; ++j) {
          const int n = n0 + kLanes * j;
#pragma unroll
          for (int g = 0; g < kMergeRows; ++g) {
            const float w = wv[j][g] * ((n < a.k && g < ng) ? 1.0f : 0.0f);
            acc[g][0] = fmaf(w, x[j].x, acc[g][0]);
            acc[g][1] = fmaf(w, x[j].y, acc[g][1]);
            acc[g][2] = fmaf(w, x[j].z, acc[g][2]);
            acc[g][3] = fmaf(w, x[j].w, acc[g][3]);
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < kMergeRows; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[nl * kQ + g * kCols + 4 * cq + e] = acc[g][e];
    __syncthreads();
    {  // kParts partial sums of kLanes / kParts n-lanes each: thread (part, pair)
      const int q = tid % kQ, part = tid / kQ;
      float sum = 0.0f;
      for (int l = 0; l < kLanes / kParts; ++l) sum += red[(part * (kLanes / kParts) + l) * kQ + q];
      red2[part * kQ + q] = sum;
    }
    __syncthreads();
    if (tid < ng * kCols) {
      const int g = tid / kCols, col = tid % kCols;
      const int cc = blockIdx.y * kCols + col;
      if (cc < a.dc) {
        float sum = 0.0f;
        for (int part = 0; part < kParts; ++part) sum += red2[part * kQ + tid];
        const int64_t row = q_row(a, b, h * a.G + g0 + g);
        if (e_dd >= 0 && e_dd < a.D) a.out[row * a.D + e_dd] = (sum + e_oe) * e_linv;
      }
    }
  }
}

// Kernels whose dynamic LDS may pass 64 KB declare their need first.
template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

}  // namespace

size_t decode_prep_a_smem(const DecodeArgs& a) {
  return sizeof(float) * (static_cast<size_t>(kPrepPos) * (a.dc + 4) + static_cast<size_t>(a.G) * a.D +
                          static_cast<size_t>(a.G) * a.dc + a.D);
}
size_t decode_edge_smem(const DecodeArgs& a) {
  const size_t E = static_cast<size_t>(a.sink) + a.recent;  // upper bound of the retained tokens
  const size_t valu = sizeof(uint16_t) * E * (a.D + 8) +
                      sizeof(float) * (2 * static_cast<size_t>(a.G) * a.D + a.G * E + a.D);
  return std::max(valu, edge_mfma_smem_bytes(a.sink + a.recent, a.G, a.D));
}
size_t decode_prep_smem(const DecodeArgs& a) {
  size_t n = a.prep_a ? decode_prep_a_smem(a) : 0;
  if (a.edge_split) n = std::max(n, decode_edge_smem(a));
  return n;
}
size_t decode_split_smem(const DecodeArgs& a) {
  return sizeof(float) * (kDecRows * a.D + kDecRows * a.kpad + 4 * kDecRows * kDecTile +
                          kDecTile * kDecRows + kDecRows);
}
size_t decode_merge_cv_smem(const DecodeArgs& a) {
  (void)a;
  // the larger of the two slice widths: [lanes][pairs] + [parts][pairs]
  constexpr size_t narrow = 128 * (kMergeRows * 8) + 8 * (kMergeRows * 8);
  constexpr size_t wide = 32 * (kMergeRows * 32) + 2 * (kMergeRows * 32);
  return sizeof(float) * (narrow > wide ? narrow : wide);
}

hipError_t launch_decode_prep(const DecodeArgs& a, hipStream_t s) {
  const int nedge = a.mfma ? a.nseq * a.hkv * a.edge_split : 0;
  const bool vec = a.dc % 4 == 0 && (reinterpret_cast<uintptr_t>(a.ck) & 15) == 0;
  const int len = a.mfma ? a.kpp : a.k;
  const int per = prep_a_mfma_ok(a, vec) ? prep_a_rows(a.dc) : kPrepPos;
  const int chunks = a.prep_a ? (len + per - 1) / per : 0;
  const int blocks = nedge + a.nseq * a.hkv * chunks;
  if (blocks == 0) return hipSuccess;
  const size_t sm = decode_prep_smem(a);
  hipError_t e;
#define FA_PREP(T, V)                                                                        \
  do {                                                                                       \
    if ((e = allow_lds(decode_prep_kernel<T, V>, sm)) != hipSuccess) return e;              \
    hipLaunchKernelGGL((decode_prep_kernel<T, V>), dim3(blocks), dim3(kPrepThreads), sm, s, a, nedge, \
                       max(chunks, 1));                                                      \
  } while (0)
  if (a.dtype == 1) {
    if (vec) FA_PREP(uint16_t, true); else FA_PREP(uint16_t, false);
  } else {
    if (vec) FA_PREP(float, true); else FA_PREP(float, false);
  }
#undef FA_PREP
  return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeArgs& a, int nitems, hipStream_t s) {
  if (nitems == 0) return hipSuccess;
  const size_t sm = decode_split_smem(a);
  hipError_t e;
  if (a.dtype == 1) {
    if ((e = allow_lds(decode_split_kernel<uint16_t>, sm)) != hipSuccess) return e;
    hipLaunchKernelGGL(decode_split_kernel<uint16_t>, dim3(nitems), dim3(256), sm, s, a);
  } else {
    if ((e = allow_lds(decode_split_kernel<float>, sm)) != hipSuccess) return e;
    hipLaunchKernelGGL(decode_split_kernel<float>, dim3(nitems), dim3(256), sm, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t s) {
  int max_splits = 1;
  for (int b = 0; b < a.nseq; ++b) max_splits = max(max_splits, a.seq.nsplit[b]);
  const dim3 vgrid(a.nseq * a.hq, merge_vec_slices(a));
  const size_t vsm = sizeof(float) * max_splits;
  hipError_t e;
  if (static_cast<int64_t>(vgrid.x) * vgrid.y <= kMergeDeepBlocks) {
    if ((e = allow_lds(decode_merge_vec_kernel<kMergeFirstDeep>, vsm)) != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_vec_kernel<kMergeFirstDeep>, vgrid, dim3(256), vsm, s, a);
  } else {
    if ((e = allow_lds(decode_merge_vec_kernel<kMergeFirstLean>, vsm)) != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_vec_kernel<kMergeFirstLean>, vgrid, dim3(256), vsm, s, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.dc == 0) return hipSuccess;
  const size_t sm = decode_merge_cv_smem(a);
  const bool vec = a.dc % 4 == 0 && (reinterpret_cast<uintptr_t>(a.cv) & 15) == 0;
  // 32-column slices once the (sequence, KV head) pairs alone fill half the
  // chip; 8-column slices below that
  const bool wide = a.nseq * a.hkv >= kCvWideHeads;
  const dim3 grid(a.nseq * a.hkv, (a.dc + (wide ? 31 : 7)) / (wide ? 32 : 8));
#define FA_MERGE_CV(V, Q)                                                                 \
  do {                                                                                    \
    if ((e = allow_lds(decode_merge_cv_kernel<V, Q>, sm)) != hipSuccess) return e;       \
    hipLaunchKernelGGL((decode_merge_cv_kernel<V, Q>), grid, dim3(256), sm, s, a);       \
  } while (0)
  if (vec) {
    if (wide) FA_MERGE_CV(true, 8); else FA_MERGE_CV(true, 2);
  } else {
    if (wide) FA_MERGE_CV(false, 8); else FA_MERGE_CV(false, 2);
  }
#undef FA_MERGE_CV
  return hipGetLastError();
}

}  // namespace fa
