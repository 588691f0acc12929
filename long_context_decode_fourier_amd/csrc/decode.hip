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

__device__ inline float basis_alpha(int n, int M) {
  const int f = basis_freq(n);
  return (f == 0 || 2 * f == M) ? 1.0f / sqrtf(static_cast<float>(M))
                                 : sqrtf(2.0f / static_cast<float>(M));
}

// e^{i 2 pi (j * tau mod M) / M} for any integer tau (negative allowed).
__device__ inline float2 unit_phase(int j, int tau, int M) {
  int64_t r = (static_cast<int64_t>(j) * tau) % M;
  if (r < 0) r += M;
  float s, c;
  sincos_phase(static_cast<int>(r), M, &s, &c);
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
// A[b][i][n] = scale * alpha_n * sum_c q[b][i][comp_c] ck[b,h][n][c], one
// block per (sequence, KV head, 32 outputs); 8 threads split the c sum.
// On the MFMA path the first block of each (sequence, KV head) also writes the
// head's query rows at the exact dims in dims order (bf16) and computes the
// edge split: plain softmax attention of those rows over the retained sink and
// recent tokens (all dims exact), stored as split nsplit-1 of each row.
constexpr int kPrepPos = 128;   // coefficient positions per A-part block
constexpr int kPrepPass = 4;    // 64-column passes over the compressible dims (dc <= 256)
constexpr int kPrepRows = 8;    // query rows per pass over q_C

// Edge split of the query rows of (sequence b, KV head h); 16-bit caches.
// The retained rows (exact dims from kx / vx, compressible dims from ke / ve)
// are first copied to LDS with every load of a thread in flight at once, then
// scores, softmax and values run from LDS.
// smem: q of the G rows in dims order, scaled [G][D] fp32 | probabilities
// [G][ne] fp32 | K rows [ne][D] bf16 | V rows [ne][D] bf16.
__device__ void edge_split_attention(const DecodeArgs& a, int b, int h, float* sm) {
  const int L = a.seq.len[b], M = a.seq.mid[b];
  const int S = a.sink, E = a.sink + a.recent;
  const int ne = (M > 0) ? E : L;  // retained tokens (all of them without a middle)
  const int D = a.D, du = a.du, dc = a.dc, G = a.G;
  const int ns = a.seq.nsplit[b];
  const int64_t row0 = a.seq.row0[b];
  float* qs = sm;                                              // [G][D]
  float* ps = qs + G * D;                                      // [G][ne]
  uint16_t* ks = reinterpret_cast<uint16_t*>(ps + G * E);      // [ne][D]
  uint16_t* vs = ks + E * D;                                   // [ne][D]
  const int tid = threadIdx.x, nt = blockDim.x;
  __syncthreads();
  // exact dims: 8-dim chunks (du % 8 == 0 on this path), t = e or e + M
  const int du8 = du / 8, dc2 = dc / 2;
  const uint16_t* kxh = static_cast<const uint16_t*>(a.kx) + (row0 + static_cast<int64_t>(h) * L) * du;
  const uint16_t* vxh = static_cast<const uint16_t*>(a.vx) + (row0 + static_cast<int64_t>(h) * L) * du;
  const uint32_t* keh = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.ke) +
                                                           (static_cast<int64_t>(b) * a.hkv + h) * E * dc);
  const uint32_t* veh = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.ve) +
                                                           (static_cast<int64_t>(b) * a.hkv + h) * E * dc);
  for (int i0 = tid; i0 < ne * du8; i0 += 8 * nt) {
    uint4 kv[8], vv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * nt;
      kv[u] = vv[u] = make_uint4(0u, 0u, 0u, 0u);
      if (i < ne * du8) {
        const int e = i / du8, c8 = i % du8;
        const int t = (M > 0 && e >= S) ? e + M : e;
        kv[u] = *reinterpret_cast<const uint4*>(kxh + static_cast<int64_t>(t) * du + 8 * c8);
        vv[u] = *reinterpret_cast<const uint4*>(vxh + static_cast<int64_t>(t) * du + 8 * c8);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * nt;
      if (i < ne * du8) {
        const int e = i / du8, c8 = i % du8;
        uint32_t* kd = reinterpret_cast<uint32_t*>(ks + e * D + 8 * c8);
        uint32_t* vd = reinterpret_cast<uint32_t*>(vs + e * D + 8 * c8);
        kd[0] = kv[u].x; kd[1] = kv[u].y; kd[2] = kv[u].z; kd[3] = kv[u].w;
        vd[0] = vv[u].x; vd[1] = vv[u].y; vd[2] = vv[u].z; vd[3] = vv[u].w;
      }
    }
  }
  // compressible dims: 2-dim words (dc % 2 == 0 on this path)
  for (int i0 = tid; i0 < ne * dc2; i0 += 8 * nt) {
    uint32_t kw[8], vw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * nt;
      kw[u] = vw[u] = 0u;
      if (i < ne * dc2) {
        kw[u] = keh[i];
        vw[u] = veh[i];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * nt;
      if (i < ne * dc2) {
        const int e = i / dc2, c2 = i % dc2;
        *reinterpret_cast<uint32_t*>(ks + e * D + du + 2 * c2) = kw[u];
        *reinterpret_cast<uint32_t*>(vs + e * D + du + 2 * c2) = vw[u];
      }
    }
  }
  for (int idx = tid; idx < G * D; idx += nt) {
    const int g = idx / D, j = idx % D;
    const int d = a.dims[h * D + j];
    const int64_t i = static_cast<int64_t>(b) * a.hq + h * G + g;
    qs[idx] = (d >= 0 && d < D) ? a.scale * bf16_to_f32(static_cast<const uint16_t*>(a.q)[i * D + d]) : 0.0f;
  }
  __syncthreads();
  // scores: thread -> (token e, row g); D is even
  for (int idx = tid; idx < ne * G; idx += nt) {
    const int e = idx / G, g = idx % G;
    const float* qg = qs + g * D;
    const uint32_t* kr = reinterpret_cast<const uint32_t*>(ks + e * D);
    float s0 = 0.0f, s1 = 0.0f;
    for (int j2 = 0; j2 < D / 2; ++j2) {
      const uint32_t w = kr[j2];
      s0 = fmaf(qg[2 * j2], __uint_as_float(w << 16), s0);
      s1 = fmaf(qg[2 * j2 + 1], __uint_as_float(w & 0xFFFF0000u), s1);
    }
    ps[g * ne + e] = s0 + s1;
  }
  __syncthreads();
  // softmax of each row: one wave per row
  const int lane = tid & 63, nwv = nt >> 6;
  for (int g = tid >> 6; g < G; g += nwv) {
    float m = -INFINITY;
    for (int e = lane; e < ne; e += 64) m = fmaxf(m, ps[g * ne + e]);
    m = wave_max(m);
    float l = 0.0f;
    for (int e = lane; e < ne; e += 64) {
      const float p = (m == -INFINITY) ? 0.0f : __expf(ps[g * ne + e] - m);
      ps[g * ne + e] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) {
      float* P = a.part + (static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(h * G + g) * ns + ns - 1) * a.RS;
      P[0] = m;
      P[1] = l;
    }
  }
  __syncthreads();
  // values: thread -> (row g, dim j: exact dims then compressible dims)
  for (int idx = tid; idx < G * D; idx += nt) {
    const int g = idx / D, j = idx % D;
    const float* pg = ps + g * ne;
    float acc = 0.0f;
    for (int e = 0; e < ne; ++e) acc = fmaf(pg[e], bf16_to_f32(vs[e * D + j]), acc);
    // partial layout [m, l, o_U(du), o_E(dc), W]: dim j of the row sits at 2 + j
    a.part[(static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(h * G + g) * ns + ns - 1) * a.RS + 2 + j] = acc;
  }
}

// A-part: block (b, h, chunk of kPrepPos coefficient positions); each wave
// takes 32 positions, 4 at a time (16 lanes per ck row, 4 columns per lane and
// 64-column pass), with every row load of the wave in flight at once; the 16
// lanes of a row are summed with DPP rotations.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void decode_prep_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  const int bh = blockIdx.x;
  const int b = bh / a.hkv, h = bh % a.hkv;
  const int M = a.seq.mid[b];
  if (a.mfma && blockIdx.y == 0) {
    // MFMA path: this KV head's query rows at the exact dims in dims order
    // (bf16, zero padded to 32), loaded contiguously by the split kernel
    const int du32 = (a.du + 31) & ~31;
    for (int idx = threadIdx.x; idx < a.G * du32; idx += blockDim.x) {
      const int g = idx / du32, j = idx % du32;
      const int64_t i = static_cast<int64_t>(b) * a.hq + h * a.G + g;
      uint16_t bits = 0;
      if (j < a.du) {
        const int d = a.dims[h * a.D + j];
        if (d >= 0 && d < a.D) bits = static_cast<const uint16_t*>(a.q)[i * a.D + d];
      }
      static_cast<uint16_t*>(a.Q16)[i * du32 + j] = bits;
    }
    if (a.edge_split) edge_split_attention(a, b, h, smem);
    return;
  }
  if (!a.prep_a) return;
  float* qc = smem;  // [kPrepRows][dc]
  const int chunk = blockIdx.y - (a.mfma ? 1 : 0);
  const int len = a.mfma ? a.kpp : a.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g4 = lane >> 4;
  const int npass = (a.dc + 63) / 64;
  const float* ckh = a.ck + (static_cast<int64_t>(b) * a.hkv + h) * a.k * a.dc;
  // this lane's ck rows: positions pos0 + 4 s + g4 (s < 8) of its wave
  const int pos0 = chunk * kPrepPos + wave * 32;
  float4 ckv[8][kPrepPass];
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    const int pos = pos0 + 4 * st + g4;
    const int n = (pos >= len) ? -1 : (a.mfma ? pair_pos_to_n(pos, a.k) : pos);
#pragma unroll
    for (int ps = 0; ps < kPrepPass; ++ps) {
      const int c = 64 * ps + 4 * l16;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ps < npass && n >= 0 && M > 0 && c < a.dc) {
        const float* src = ckh + static_cast<int64_t>(n) * a.dc + c;
        if (VEC) {
          v = *reinterpret_cast<const float4*>(src);
        } else {
          v.x = src[0];
          if (c + 1 < a.dc) v.y = src[1];
          if (c + 2 < a.dc) v.z = src[2];
          if (c + 3 < a.dc) v.w = src[3];
        }
      }
      ckv[st][ps] = v;
    }
  }
  for (int g0 = 0; g0 < a.G; g0 += kPrepRows) {
    const int ng = min(kPrepRows, a.G - g0);
    __syncthreads();
    for (int idx = tid; idx < ng * a.dc; idx += blockDim.x) {
      const int g = idx / a.dc, c = idx % a.dc;
      const int d = a.dims[h * a.D + a.du + c];
      const int i = h * a.G + g0 + g;
      qc[g * a.dc + c] = (d >= 0 && d < a.D)
                             ? a.scale * ld<T>(a.q, (static_cast<int64_t>(b) * a.hq + i) * a.D + d)
                             : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int pos = pos0 + 4 * st + g4;
      const int n = (pos >= len) ? -1 : (a.mfma ? pair_pos_to_n(pos, a.k) : pos);
      const float alpha = (n >= 0 && M > 0) ? basis_alpha(n, M) : 0.0f;
#pragma unroll
      for (int g = 0; g < kPrepRows; ++g) {
        if (g >= ng) break;
        float acc = 0.0f;
#pragma unroll
        for (int ps = 0; ps < kPrepPass; ++ps) {
          const int c = 64 * ps + 4 * l16;
          if (ps < npass && c < a.dc) {
            const float* qg = qc + g * a.dc + c;
            acc = fmaf(qg[0], ckv[st][ps].x, acc);
            if (c + 1 < a.dc) acc = fmaf(qg[1], ckv[st][ps].y, acc);
            if (c + 2 < a.dc) acc = fmaf(qg[2], ckv[st][ps].z, acc);
            if (c + 3 < a.dc) acc = fmaf(qg[3], ckv[st][ps].w, acc);
          }
        }
        acc = row16_sum(acc);
        if (l16 == 0 && pos < len) {
          const int64_t i = static_cast<int64_t>(b) * a.hq + h * a.G + g0 + g;
          if (a.mfma)
            static_cast<_Float16*>(a.A16)[i * a.kpp + pos] = static_cast<_Float16>(alpha * acc);
          else
            a.A[i * a.kpad + pos] = alpha * acc;
        }
      }
    }
  }
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
  const int L = a.seq.len[b], M = a.seq.mid[b];
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
        v = a.scale * ld<T>(a.q, (static_cast<int64_t>(b) * a.hq + qi[r]) * a.D + d);
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
    wstep[i] = (has_mid && i < nown) ? unit_phase(tid + 256 * i, 1, M) : make_float2(1.0f, 0.0f);
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
          for (int d = d0; d < d1; ++d) acc[r] = fmaf(qs[r * a.D + d], ld<T>(a.kx, base + d), acc[r]);
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
              for (int c = c0; c < c1; ++c)
                acc[r] = fmaf(qs[r * a.D + a.du + c], ld<T>(a.ke, base + c), acc[r]);
            }
          } else {
            const int tau = t - S;
            const int j0 = part * sl4, j1 = min(nslots, j0 + sl4);
            const float2 w = unit_phase(1, tau, M);
            float2 z = make_float2(1.0f, 0.0f);
            for (int j = j0; j < j1; ++j) {
              if (((j - j0) & 31) == 0) z = unit_phase(j, tau, M);
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
      for (int tl = 0; tl < nt; ++tl) o = fmaf(ps[tl * R + r], ld<T>(a.vx, base + static_cast<int64_t>(tl) * a.du), o);
      oacc[j] = o;
    }
    if (comp) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = tid + 256 * j;
        if (idx >= a.rows * a.dc) break;
        const int r = idx / a.dc, c = idx % a.dc;
        float o = eacc[j] * corr[r];
        const int64_t base = (static_cast<int64_t>(b) * a.hkv + kh[r]) * E * a.dc + c;
        for (int tl = 0; tl < nt; ++tl) {
          const int t = tile0 + tl;
          if (M == 0 || t < S || t >= S + M) {
            const int e = (M == 0 || t < S) ? t : t - M;
            o = fmaf(ps[tl * R + r], ld<T>(a.ve, base + static_cast<int64_t>(e) * a.dc), o);
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
        z[i] = (i < nown && mid_lo < mid_hi) ? unit_phase(tid + 256 * i, tile0 + mid_lo - S, M)
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

__global__ __launch_bounds__(256) void decode_merge_vec_kernel(DecodeArgs a) {
  extern __shared__ float smem[];  // [ns] weights
  __shared__ float red[256];
  const int row = blockIdx.x;      // b * hq + i
  const int b = row / a.hq, i = row % a.hq, h = i / a.G;
  const int ns = a.seq.nsplit[b];
  const int M = a.seq.mid[b];
  const bool has_mid = a.dc > 0 && M > 0;
  const int nvec = a.du + a.dc + (has_mid ? a.k : 0);
  const int idx = blockIdx.y * 256 + threadIdx.x;
  if (blockIdx.y * 256 >= nvec) return;  // uniform per block
  const float* P = a.part + (static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(i) * ns) * a.RS;
  float mx = -INFINITY;
  for (int s = threadIdx.x; s < ns; s += 256) mx = fmaxf(mx, P[static_cast<int64_t>(s) * a.RS]);
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  float lsum = 0.0f;
  for (int s = threadIdx.x; s < ns; s += 256) {
    const float m = P[static_cast<int64_t>(s) * a.RS];
    const float w = (m == -INFINITY) ? 0.0f : __expf(m - mx);
    smem[s] = w;
    lsum += w * P[static_cast<int64_t>(s) * a.RS + 1];
  }
  red[threadIdx.x] = lsum;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const float linv = 1.0f / red[0];
  float* mrow = a.mrg + static_cast<int64_t>(row) * a.MS;
  if (blockIdx.y == 0 && threadIdx.x == 0) mrow[a.dc + a.kpad] = linv;
  if (idx >= nvec) return;
  const float* Pi = P + 2 + idx;
  // splits that hold this entry: with an edge split (the last one), o_E comes
  // from it alone and W from the other splits alone
  int s_lo = 0, s_hi = ns;
  if (a.edge_split && idx >= a.du) {
    if (idx < a.du + a.dc) s_lo = ns - 1;
    else s_hi = ns - 1;
  }
  // fixed-order sum over the splits, 8 loads in flight
  float v = 0.0f;
  for (int s0 = s_lo; s0 < s_hi; s0 += 8) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (s0 + j < s_hi) ? Pi[static_cast<int64_t>(s0 + j) * a.RS] : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < s_hi) v = fmaf(smem[s0 + j], x[j], v);
  }
  if (idx < a.du) {
    const int dd = a.dims[h * a.D + idx];
    if (dd >= 0 && dd < a.D) a.out[static_cast<int64_t>(row) * a.D + dd] = v * linv;
  } else if (idx < a.du + a.dc) {
    mrow[idx - a.du] = v;
  } else {
    const int n = idx - a.du - a.dc;
    mrow[a.dc + n] = v * basis_alpha(n, M);
  }
}

// Pass 2 body: one block per (sequence, KV head, 32-column slice of the
// compressible dims) computes O_C[g][c] = sum_n (alpha W)[g][n] cv[n][c] for
// the head's query rows, kMergeRows rows at a time.  Thread (column quad cq,
// n-lane nl) reads 4 consecutive columns of the cv rows n = nl + 32 j with
// kCvBatch loads in flight; the 32 n-lanes are summed in a fixed order.
constexpr int kCvCols = 32;
constexpr int kCvLanes = 32;
constexpr int kCvBatch = 8;

template <bool VEC>
__global__ __launch_bounds__(256) void decode_merge_cv_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  const int b = blockIdx.x / a.hkv, h = blockIdx.x % a.hkv;
  const int M = a.seq.mid[b];
  const bool has_mid = a.dc > 0 && M > 0;
  float* Wm = smem;                                   // [kMergeRows][kpad]
  float* red = Wm + kMergeRows * a.kpad;              // [kCvLanes][kMergeRows][kCvCols]
  const int tid = threadIdx.x;
  const int cq = tid % (kCvCols / 4), nl = tid / (kCvCols / 4);
  const int c = blockIdx.y * kCvCols + 4 * cq;
  const float* cvb = a.cv + (static_cast<int64_t>(b) * a.hkv + h) * a.k * a.dc;
  for (int g0 = 0; g0 < a.G; g0 += kMergeRows) {
    const int ng = min(kMergeRows, a.G - g0);
    __syncthreads();
    if (has_mid)
      for (int idx = tid; idx < ng * a.k; idx += 256) {
        const int g = idx / a.k, n = idx % a.k;
        const int64_t row = static_cast<int64_t>(b) * a.hq + h * a.G + g0 + g;
        Wm[g * a.kpad + n] = a.mrg[row * a.MS + a.dc + n];
      }
    __syncthreads();
    float acc[kMergeRows][4];
#pragma unroll
    for (int g = 0; g < kMergeRows; ++g) acc[g][0] = acc[g][1] = acc[g][2] = acc[g][3] = 0.0f;
    if (has_mid && c < a.dc) {
      for (int n0 = nl; n0 < a.k; n0 += kCvLanes * kCvBatch) {
        float4 x[kCvBatch];
#pragma unroll
        for (int j = 0; j < kCvBatch; ++j) {
          const int n = n0 + kCvLanes * j;
          float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
          if (n < a.k) {
            const float* src = cvb + static_cast<int64_t>(n) * a.dc + c;
            if (VEC) {
              v = *reinterpret_cast<const float4*>(src);
            } else {
              v.x = src[0];
              if (c + 1 < a.dc) v.y = src[1];
              if (c + 2 < a.dc) v.z = src[2];
              if (c + 3 < a.dc) v.w = src[3];
            }
          }
          x[j] = v;
        }
#pragma unroll
        for (int j = 0; j < kCvBatch; ++j) {
          const int n = n0 + kCvLanes * j;
          if (n >= a.k) break;
#pragma unroll
          for (int g = 0; g < kMergeRows; ++g)
            if (g < ng) {
              const float w = Wm[g * a.kpad + n];
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
      for (int e = 0; e < 4; ++e) red[(nl * kMergeRows + g) * kCvCols + 4 * cq + e] = acc[g][e];
    __syncthreads();
    if (tid < ng * kCvCols) {
      const int g = tid / kCvCols, col = tid % kCvCols;
      const int cc = blockIdx.y * kCvCols + col;
      if (cc < a.dc) {
        float sum = 0.0f;
        for (int q = 0; q < kCvLanes; ++q) sum += red[(q * kMergeRows + g) * kCvCols + col];
        const int64_t row = static_cast<int64_t>(b) * a.hq + h * a.G + g0 + g;
        const float* mrow = a.mrg + row * a.MS;
        const int dd = a.dims[h * a.D + a.du + cc];
        if (dd >= 0 && dd < a.D) a.out[row * a.D + dd] = (sum + mrow[cc]) * mrow[a.dc + a.kpad];
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

size_t decode_prep_smem(const DecodeArgs& a) {
  size_t n = sizeof(float) * kPrepRows * a.dc;
  if (a.edge_split) n = std::max(n, decode_edge_smem(a));
  return n;
}
size_t decode_edge_smem(const DecodeArgs& a) {
  const size_t E = static_cast<size_t>(a.sink) + a.recent;  // upper bound of the retained tokens
  return sizeof(float) * (static_cast<size_t>(a.G) * a.D + a.G * E) + 2 * sizeof(uint16_t) * E * a.D;
}
size_t decode_split_smem(const DecodeArgs& a) {
  return sizeof(float) * (kDecRows * a.D + kDecRows * a.kpad + 4 * kDecRows * kDecTile +
                          kDecTile * kDecRows + kDecRows);
}
size_t decode_merge_cv_smem(const DecodeArgs& a) {
  return sizeof(float) * (kMergeRows * a.kpad + kCvLanes * kMergeRows * kCvCols);
}

hipError_t launch_decode_prep(const DecodeArgs& a, hipStream_t s) {
  if (!a.prep_a && !a.mfma) return hipSuccess;
  const int len = a.mfma ? a.kpp : a.k;
  const int chunks = a.prep_a ? (len + kPrepPos - 1) / kPrepPos : 0;
  dim3 grid(a.nseq * a.hkv, chunks + (a.mfma ? 1 : 0));
  const size_t sm = decode_prep_smem(a);
  const bool vec = a.dc % 4 == 0 && (reinterpret_cast<uintptr_t>(a.ck) & 15) == 0;
  hipError_t e;
#define FA_PREP(T, V)                                                              \
  do {                                                                             \
    if ((e = allow_lds(decode_prep_kernel<T, V>, sm)) != hipSuccess) return e;    \
    hipLaunchKernelGGL((decode_prep_kernel<T, V>), grid, dim3(256), sm, s, a);     \
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
  const int nvec = a.du + a.dc + a.k;
  hipError_t e = allow_lds(decode_merge_vec_kernel, sizeof(float) * max_splits);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_vec_kernel, dim3(a.nseq * a.hq, (nvec + 255) / 256), dim3(256),
                     sizeof(float) * max_splits, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.dc == 0) return hipSuccess;
  const size_t sm = decode_merge_cv_smem(a);
  const dim3 grid(a.nseq * a.hkv, (a.dc + kCvCols - 1) / kCvCols);
  const bool vec = a.dc % 4 == 0 && (reinterpret_cast<uintptr_t>(a.cv) & 15) == 0;
  if (vec) {
    if ((e = allow_lds(decode_merge_cv_kernel<true>, sm)) != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_cv_kernel<true>, grid, dim3(256), sm, s, a);
  } else {
    if ((e = allow_lds(decode_merge_cv_kernel<false>, sm)) != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_cv_kernel<false>, grid, dim3(256), sm, s, a);
  }
  return hipGetLastError();
}

}  // namespace fa
