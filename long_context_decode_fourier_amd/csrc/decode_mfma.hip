// decode_mfma.hip - split-L decode step on MFMA for 16-bit caches.
//
// Same arithmetic as the VALU kernel in decode.hip (scores and values in
// coefficient space, online softmax, partials merged by decode_merge), laid out
// for CDNA4 matrix cores:
//
// * the query rows of a work item (up to 32 query heads that share the
//   sequence, hence its middle length M and its basis) are stacked into the
//   M dimension of v_mfma_f32_16x16x32_f16 / 16x16x16_f16;
// * per tile of T tokens the basis tile phi[t][pos] (unscaled cos/sin, fp16)
//   is generated once into LDS and shared by every row;
// * compressed scores S = A phi^T contract over coefficients: each wave owns a
//   slice of 32-wide coefficient units, keeps its slice of A (scale*alpha*q_C
//   ck, fp16) in registers, reads phi with 16-byte LDS loads, and the four
//   waves' partial scores are summed in LDS;
// * value moments W += P phi contract over tokens: the same LDS tile is read
//   transposed with ds_read_b64_tr_b16, W stays in registers per wave slice;
// * exact dims (and the retained edge rows) are dot products per KV head on
//   VALU with coalesced 16-byte row loads.
//
// Coefficients live in "pair order" inside the kernel: position 2j holds the
// cosine of frequency j (j = 0 is the constant), 2j+1 the sine; position 1 is
// unused.  A is written in that order by decode_prep, W is converted back to
// the basis order when the partials are stored.
#include "kernels.hpp"

namespace fa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

// Transposed 4 x 16-bit LDS read (see kernel header): lane 4a+e of each
// 16-lane group receives element e of the chunks addressed by lanes
// a, a+4, a+8, a+12 of its group.
__device__ inline half4 lds_read_tr4(const _Float16* p) {
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p));
  return __builtin_bit_cast(half4, r);
}

__device__ inline float wmax(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ inline float wsum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int MB, int NW, int MAXU, int T, int RPH>
__global__ __launch_bounds__(64 * NW) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NT = 64 * NW, MR = 16 * MB, NB = T / 16;
  constexpr int SL = (MR * T + NT - 1) / NT;  // softmax (row, token) slots per thread
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int PS = a.kpp + 16;  // LDS row stride in halves; 2*PS = 32 (mod 64) words
  _Float16* phi = reinterpret_cast<_Float16*>(smem);        // [T][PS]
  float* qs = reinterpret_cast<float*>(phi + T * PS);        // [MR][D]
  float* sx = qs + MR * a.D;                                 // [MR][T]
  float* spart = sx + MR * T;                                // [NW][MR][T]
  float* pf = spart + NW * MR * T;                           // [MR][T]
  _Float16* ph = reinterpret_cast<_Float16*>(pf + MR * T);   // [MR][T]
  float* corr = reinterpret_cast<float*>(ph + MR * T);       // [MR]
  int* flag = reinterpret_cast<int*>(corr + MR);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = seq_of_item(a.seq, a.nseq, blockIdx.x);
  const int local = blockIdx.x - a.seq.item0[b];
  const int ns = a.seq.nsplit[b];
  const int rg = local / ns, sp = local % ns;
  const int L = a.seq.len[b], M = a.seq.mid[b];
  const int S = a.sink, E = a.sink + a.recent;
  const int t_begin = sp * a.seq.chunk[b];
  const int t_end = min(L, t_begin + a.seq.chunk[b]);
  const int64_t row0 = a.seq.row0[b];
  const int rows = a.rows;
  const int qi0 = rg * rows;
  const int h0 = qi0 / a.G;
  const int nheads = rows >= a.G ? rows / a.G : 1;
  const int rph = min(rows, a.G);  // query rows per KV head inside the item
  const bool has_mid = a.dc > 0 && M > 0;
  const int du = a.du, dc = a.dc, D = a.D;

  // ---- scaled q rows in dim-split order
  for (int idx = tid; idx < MR * D; idx += NT) {
    const int r = idx / D, j = idx % D;
    float v = 0.0f;
    if (r < rows) {
      const int qi = qi0 + r;
      const int dd = a.dims[(qi / a.G) * D + j];
      if (dd >= 0 && dd < D)
        v = a.scale * bf16_to_f32(static_cast<const uint16_t*>(a.q)[(static_cast<int64_t>(b) * a.hq + qi) * D + dd]);
    }
    qs[idx] = v;
  }

  // ---- this wave's coefficient units and its slice of A (MFMA A operand)
  const int U = a.kpp / 32;
  const int u0 = (U * wave) / NW, nu = (U * (wave + 1)) / NW - u0;
  half8 Areg[MAXU][MB];
#pragma unroll
  for (int u = 0; u < MAXU; ++u)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      half8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0;
      const int row = mb * 16 + (lane & 15);
      if (has_mid && u < nu && row < rows)
        v = *reinterpret_cast<const half8*>(
            static_cast<const _Float16*>(a.A16) +
            (static_cast<int64_t>(b) * a.hq + qi0 + row) * a.kpp + (u0 + u) * 32 + 8 * (lane >> 4));
      Areg[u][mb] = v;
    }
  floatx4 Wacc[MAXU][2][MB];
#pragma unroll
  for (int u = 0; u < MAXU; ++u)
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) Wacc[u][n2][mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // ---- exact-dim value accumulators: thread -> (head, dim pair)
  const int du2 = du / 2, dc2 = dc / 2;
  const int xh = du2 ? tid / du2 : 0, xd = du2 ? tid % du2 : 0;
  const bool xval = du2 > 0 && tid < nheads * du2;
  const int eh = dc2 ? tid / dc2 : 0, ec = dc2 ? tid % dc2 : 0;
  const bool evld = dc2 > 0 && tid < nheads * dc2;
  const int xrb = (rows >= a.G) ? xh * a.G : 0;
  const int erb = (rows >= a.G) ? eh * a.G : 0;
  float oU[RPH][2], oE[RPH][2];
#pragma unroll
  for (int r = 0; r < RPH; ++r) oU[r][0] = oU[r][1] = oE[r][0] = oE[r][1] = 0.0f;

  // ---- softmax slots: thread -> (row, token) for idx = tid and tid + NT
  float m_run[SL], l_run[SL];
#pragma unroll
  for (int j = 0; j < SL; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.0f;
  }

  // ---- basis generation mapping: thread -> (token, run of pair chunks)
  constexpr int kRuns = NT / T;              // runs per token
  const int gt = tid % T, grun = tid / T;
  const int chunks = a.kpp / 8;              // 4 pairs (8 halves) per chunk
  const int cper = (chunks + kRuns - 1) / kRuns;
  const int c_lo = grun * cper, c_hi = min(chunks, c_lo + cper);
  const float invM = has_mid ? 1.0f / static_cast<float>(M) : 0.0f;

  // ---- exact score mapping: thread -> (head, token, part of the dims)
  const int npairs = nheads * T;
  const int tpp = NT / npairs >= 1 ? NT / npairs : 1;  // threads per (head, token)

  __syncthreads();

  for (int tile0 = t_begin; tile0 < t_end; tile0 += T) {
    const int nt = min(T, t_end - tile0);
    // ================= phase 1: basis tile, exact scores
    if (tid == 0) *flag = 0;
    {
      const int t = tile0 + gt;
      const bool mid = has_mid && t < t_end && t >= S && t < S + M;
      _Float16* dst = phi + gt * PS;
      if (!mid) {
        for (int c = c_lo; c < c_hi; ++c) {
          half8 z;
#pragma unroll
          for (int e = 0; e < 8; ++e) z[e] = 0;
          *reinterpret_cast<half8*>(dst + 8 * c) = z;
        }
      } else {
        const int tau = t - S;
        const float c2 = 2.0f * cos_rev(static_cast<float>(tau) * invM);
        // runs of 4 chunks (16 pairs) are seeded from exact phases
        int r0 = phase_mod(4 * c_lo, tau, M);
        const int d16 = phase_mod(16, tau, M);
        for (int c = c_lo; c < c_hi; c += 4) {
          int r1 = r0 + tau % M;
          if (r1 >= M) r1 -= M;
          const float x0 = static_cast<float>(r0) * invM, x1 = static_cast<float>(r1) * invM;
          float cp = cos_rev(x0), sp_ = sin_rev(x0);
          float cc = cos_rev(x1), sc = sin_rev(x1);
          const int cend = min(c + 4, c_hi);
          for (int cc4 = c; cc4 < cend; ++cc4) {
            half8 z;
            z[0] = static_cast<_Float16>(cp);
            z[1] = static_cast<_Float16>(sp_);
            z[2] = static_cast<_Float16>(cc);
            z[3] = static_cast<_Float16>(sc);
            float cn = fmaf(c2, cc, -cp), sn = fmaf(c2, sc, -sp_);
            z[4] = static_cast<_Float16>(cn);
            z[5] = static_cast<_Float16>(sn);
            float cm = fmaf(c2, cn, -cc), sm = fmaf(c2, sn, -sc);
            z[6] = static_cast<_Float16>(cm);
            z[7] = static_cast<_Float16>(sm);
            *reinterpret_cast<half8*>(dst + 8 * cc4) = z;
            cp = fmaf(c2, cm, -cn);
            sp_ = fmaf(c2, sm, -sn);
            cc = fmaf(c2, cp, -cm);
            sc = fmaf(c2, sp_, -sm);
          }
          r0 += d16;
          if (r0 >= M) r0 -= M;
        }
      }
    }
    for (int pr = tid / tpp; pr < npairs; pr += NT / tpp) {
      const int hh = pr / T, tt = pr % T, part = tid % tpp;
      const int t = tile0 + tt;
      const int h = h0 + hh;
      const int rb = (rows >= a.G) ? hh * a.G : 0;
      float acc[RPH];
#pragma unroll
      for (int r = 0; r < RPH; ++r) acc[r] = 0.0f;
      if (t < t_end) {
        const int dper = du / tpp, d0 = part * dper;
        const uint32_t* krow = reinterpret_cast<const uint32_t*>(
            static_cast<const uint16_t*>(a.kx) + (row0 + static_cast<int64_t>(h) * L + t) * du + d0);
        for (int d = 0; d < dper; d += 2) {
          const uint32_t w2 = krow[d >> 1];
          const float k0 = __uint_as_float(w2 << 16), k1 = __uint_as_float(w2 & 0xFFFF0000u);
#pragma unroll
          for (int r = 0; r < RPH; ++r)
            if (r < rph) acc[r] = fmaf(qs[(rb + r) * D + d0 + d], k0, fmaf(qs[(rb + r) * D + d0 + d + 1], k1, acc[r]));
        }
        const bool edge = dc > 0 && (M == 0 || t < S || t >= S + M);
        if (edge) {
          const int e = (M == 0 || t < S) ? t : t - M;
          const int cper_ = dc / tpp, c0 = part * cper_;
          const uint32_t* erow = reinterpret_cast<const uint32_t*>(
              static_cast<const uint16_t*>(a.ke) + ((static_cast<int64_t>(b) * a.hkv + h) * E + e) * dc + c0);
          for (int c = 0; c < cper_; c += 2) {
            const uint32_t w2 = erow[c >> 1];
            const float k0 = __uint_as_float(w2 << 16), k1 = __uint_as_float(w2 & 0xFFFF0000u);
#pragma unroll
            for (int r = 0; r < RPH; ++r)
              if (r < rph)
                acc[r] = fmaf(qs[(rb + r) * D + du + c0 + c], k0, fmaf(qs[(rb + r) * D + du + c0 + c + 1], k1, acc[r]));
          }
        }
      }
#pragma unroll
      for (int r = 0; r < RPH; ++r) acc[r] = wsum(acc[r], tpp);
      if (part == 0)
#pragma unroll
        for (int r = 0; r < RPH; ++r)
          if (r < rph) sx[(rb + r) * T + tt] = (t < t_end) ? acc[r] : -INFINITY;
    }
    __syncthreads();

    // ================= phase 2: compressed score partials (MFMA)
    if (has_mid) {
      floatx4 sacc[MB][NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sacc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < MAXU; ++u) {
        if (u < nu) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const half8 bv = *reinterpret_cast<const half8*>(
                phi + (nb * 16 + (lane & 15)) * PS + (u0 + u) * 32 + 8 * (lane >> 4));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              sacc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Areg[u][mb], bv, sacc[mb][nb], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            spart[(wave * MR + mb * 16 + 4 * (lane >> 4) + r) * T + nb * 16 + (lane & 15)] = sacc[mb][nb][r];
    }
    __syncthreads();

    // ================= phase 3: online softmax over the tile
#pragma unroll
    for (int j = 0; j < SL; ++j) {
      const int idx = tid + NT * j;
      const int row = idx / T, tt = idx % T;  // row >= MR: idle slot
      float s = -INFINITY;
      if (row < rows) {
        s = sx[row * T + tt];
        if (has_mid && s != -INFINITY) {
#pragma unroll
          for (int w = 0; w < NW; ++w) s += spart[(w * MR + row) * T + tt];
        }
      }
      const float m_new = fmaxf(m_run[j], wmax(s, T));
      const float c = (m_new == -INFINITY || m_run[j] == m_new) ? 1.0f : __expf(m_run[j] - m_new);
      const float p = (s == -INFINITY) ? 0.0f : __expf(s - m_new);
      l_run[j] = l_run[j] * c + wsum(p, T);
      m_run[j] = m_new;
      if (row >= MR) continue;
      pf[row * T + tt] = p;
      ph[row * T + tt] = static_cast<_Float16>(p);
      if (tt == 0) {
        corr[row] = c;
        if (c != 1.0f) *flag = 1;
      }
    }
    __syncthreads();

    // ================= phase 4: value moments W (MFMA), exact values (VALU)
    const bool rescale = *flag != 0;
    if (has_mid) {
      if (rescale) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          float cr[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) cr[r] = corr[mb * 16 + 4 * (lane >> 4) + r];
#pragma unroll
          for (int u = 0; u < MAXU; ++u)
#pragma unroll
            for (int n2 = 0; n2 < 2; ++n2)
#pragma unroll
              for (int r = 0; r < 4; ++r) Wacc[u][n2][mb][r] *= cr[r];
        }
      }
      const int g = lane >> 4, s16 = lane & 15;
#pragma unroll
      for (int u = 0; u < MAXU; ++u) {
        if (u < nu) {
#pragma unroll
          for (int n2 = 0; n2 < 2; ++n2) {
            const int nbase = (u0 + u) * 32 + n2 * 16 + 4 * (s16 & 3);
            if constexpr (T == 32) {
              const half4 lo = lds_read_tr4(phi + (8 * g + (s16 >> 2)) * PS + nbase);
              const half4 hi = lds_read_tr4(phi + (8 * g + 4 + (s16 >> 2)) * PS + nbase);
              const half8 bv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) {
                const half8 pv = *reinterpret_cast<const half8*>(ph + (mb * 16 + s16) * T + 8 * g);
                Wacc[u][n2][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pv, bv, Wacc[u][n2][mb], 0, 0, 0);
              }
            } else {
              const half4 bv = lds_read_tr4(phi + (4 * g + (s16 >> 2)) * PS + nbase);
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) {
                const half4 pv = *reinterpret_cast<const half4*>(ph + (mb * 16 + s16) * T + 4 * g);
                Wacc[u][n2][mb] = __builtin_amdgcn_mfma_f32_16x16x16f16(pv, bv, Wacc[u][n2][mb], 0, 0, 0);
              }
            }
          }
        }
      }
    }
    if (xval) {
      const int h = h0 + xh;
      if (rescale)
#pragma unroll
        for (int r = 0; r < RPH; ++r)
          if (r < rph) {
            const float cr = corr[xrb + r];
            oU[r][0] *= cr;
            oU[r][1] *= cr;
          }
      const uint32_t* vcol = reinterpret_cast<const uint32_t*>(
          static_cast<const uint16_t*>(a.vx) + (row0 + static_cast<int64_t>(h) * L + tile0) * du + 2 * xd);
      for (int tt = 0; tt < nt; ++tt) {
        const uint32_t w2 = vcol[static_cast<int64_t>(tt) * du2];
        const float v0 = __uint_as_float(w2 << 16), v1 = __uint_as_float(w2 & 0xFFFF0000u);
#pragma unroll
        for (int r = 0; r < RPH; ++r)
          if (r < rph) {
            const float p = pf[(xrb + r) * T + tt];
            oU[r][0] = fmaf(p, v0, oU[r][0]);
            oU[r][1] = fmaf(p, v1, oU[r][1]);
          }
      }
    }
    if (evld) {
      const int h = h0 + eh;
      if (rescale)
#pragma unroll
        for (int r = 0; r < RPH; ++r)
          if (r < rph) {
            const float cr = corr[erb + r];
            oE[r][0] *= cr;
            oE[r][1] *= cr;
          }
      // edge tokens of this tile: [tile0, S) and [S + M, ...) (all tokens when M = 0)
      const int lo_end = (M == 0) ? tile0 + nt : min(tile0 + nt, S);
      const int hi_beg = (M == 0) ? tile0 + nt : max(tile0, S + M);
      const uint32_t* ecol = reinterpret_cast<const uint32_t*>(
          static_cast<const uint16_t*>(a.ve) + (static_cast<int64_t>(b) * a.hkv + h) * E * dc + 2 * ec);
      for (int t = tile0; t < tile0 + nt; ++t) {
        if (t >= lo_end && t < hi_beg) {
          t = hi_beg - 1;
          continue;
        }
        const int e = (M == 0 || t < S) ? t : t - M;
        const uint32_t w2 = ecol[static_cast<int64_t>(e) * dc2];
        const float v0 = __uint_as_float(w2 << 16), v1 = __uint_as_float(w2 & 0xFFFF0000u);
#pragma unroll
        for (int r = 0; r < RPH; ++r)
          if (r < rph) {
            const float p = pf[(erb + r) * T + (t - tile0)];
            oE[r][0] = fmaf(p, v0, oE[r][0]);
            oE[r][1] = fmaf(p, v1, oE[r][1]);
          }
      }
    }
    __syncthreads();
  }

  // ================= partials
  const int64_t prow = static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(qi0) * ns + sp;
#pragma unroll
  for (int j = 0; j < SL; ++j) {
    const int idx = tid + NT * j;
    const int row = idx / T, tt = idx % T;
    if (tt == 0 && row < rows) {
      float* P = a.part + (prow + static_cast<int64_t>(row) * ns) * a.RS;
      P[0] = m_run[j];
      P[1] = l_run[j];
    }
  }
  if (xval)
#pragma unroll
    for (int r = 0; r < RPH; ++r)
      if (r < rph) {
        float* P = a.part + (prow + static_cast<int64_t>(xrb + r) * ns) * a.RS + 2 + 2 * xd;
        P[0] = oU[r][0];
        P[1] = oU[r][1];
      }
  if (evld)
#pragma unroll
    for (int r = 0; r < RPH; ++r)
      if (r < rph) {
        float* P = a.part + (prow + static_cast<int64_t>(erb + r) * ns) * a.RS + 2 + du + 2 * ec;
        P[0] = oE[r][0];
        P[1] = oE[r][1];
      }
  if (has_mid) {
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
      if (u >= nu) continue;
#pragma unroll
      for (int n2 = 0; n2 < 2; ++n2) {
        const int pos = (u0 + u) * 32 + n2 * 16 + (lane & 15);
        const int j = pos >> 1;
        const int n = (pos & 1) ? (j == 0 ? -1 : 2 * j) : (j == 0 ? 0 : 2 * j - 1);
        if (n < 0 || n >= a.k) continue;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = mb * 16 + 4 * (lane >> 4) + r;
            if (row < rows)
              a.part[(prow + static_cast<int64_t>(row) * ns) * a.RS + 2 + du + dc + n] = Wacc[u][n2][mb][r];
          }
      }
    }
  }
}

template <int MB, int NW, int MAXU, int T, int RPH>
hipError_t launch_one(const DecodeArgs& a, int nitems, size_t smem, hipStream_t s) {
  auto k = decode_mfma_kernel<MB, NW, MAXU, T, RPH>;
  if (smem > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(smem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(nitems), dim3(64 * NW), smem, s, a);
  return hipGetLastError();
}

}  // namespace

// Compiled variants (M blocks, waves, max 32-wide coefficient units per wave,
// tokens per tile), chosen by basis length:
//   k <  512: 16 rows, 4 waves, <= 4 units, 32 tokens
//   k >= 512: 32 rows (<= 1280 positions, 32 tokens) or 16 rows (<= 2304
//             positions, 16 tokens so the basis tile fits LDS), 8 waves.
int decode_mfma_tokens(int kpp) { return kpp <= 1280 ? 32 : 16; }
int decode_mfma_waves(int kpp) { return kpp <= 512 ? 4 : 8; }
int decode_mfma_max_kpp(int mb) { return mb == 1 ? 2304 : 1280; }
int decode_mfma_max_rph(int kpp) { return kpp <= 512 ? 8 : 4; }

size_t decode_mfma_smem(const DecodeArgs& a, int mb) {
  const int T = decode_mfma_tokens(a.kpp), MR = 16 * mb, NW = decode_mfma_waves(a.kpp);
  return static_cast<size_t>(T) * (a.kpp + 16) * 2 +
         sizeof(float) * (MR * a.D + MR * T + NW * MR * T + MR * T) + 2 * MR * T + 4 * MR + 16;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int nitems, hipStream_t s) {
  if (nitems == 0) return hipSuccess;
  const size_t smem = decode_mfma_smem(a, a.mb);
  const int rph = a.rows < a.G ? a.rows : a.G;
  if (a.kpp <= 512) {
    if (a.mb == 1) return launch_one<1, 4, 4, 32, 8>(a, nitems, smem, s);
    return launch_one<2, 4, 4, 32, 8>(a, nitems, smem, s);
  }
  if (rph > 4) return hipErrorInvalidValue;
  if (a.mb == 2) {
    if (a.kpp <= 1280) return launch_one<2, 8, 5, 32, 4>(a, nitems, smem, s);
    return hipErrorInvalidValue;
  }
  if (a.kpp <= 1280) return launch_one<1, 8, 5, 32, 4>(a, nitems, smem, s);
  if (a.kpp <= 2304) return launch_one<1, 8, 9, 16, 4>(a, nitems, smem, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
