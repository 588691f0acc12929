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
#include "kernels.hpp"

namespace fa {
namespace {

template <typename T> __device__ inline float ld(const void* p, int64_t i) {
  return load_f32<T>(static_cast<const T*>(p), i);
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
constexpr int kPrepOut = 32;
constexpr int kPrepParts = 8;
constexpr int kPrepRows = 8;

template <typename T>
__global__ __launch_bounds__(256) void decode_prep_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  float* qc = smem;                               // [kPrepRows][dc]
  float* red = smem + kPrepRows * a.dc;           // [kPrepParts][kPrepRows][kPrepOut]
  const int bh = blockIdx.x;
  const int b = bh / a.hkv, h = bh % a.hkv;
  const int M = a.seq.mid[b];
  if (a.mfma && blockIdx.y == 0) {
    // MFMA path: this KV head's query rows in dims order, so that the split
    // kernel loads them contiguously (exact dims bf16, compressible dims fp32)
    const int du32 = (a.du + 31) & ~31;
    const int w = du32 + a.dc;
    for (int idx = threadIdx.x; idx < a.G * w; idx += blockDim.x) {
      const int g = idx / w, j = idx % w;
      const int64_t i = static_cast<int64_t>(b) * a.hq + h * a.G + g;
      if (j < du32) {
        uint16_t bits = 0;
        if (j < a.du) {
          const int d = a.dims[h * a.D + j];
          if (d >= 0 && d < a.D) bits = static_cast<const uint16_t*>(a.q)[i * a.D + d];
        }
        static_cast<uint16_t*>(a.Q16)[i * du32 + j] = bits;
      } else {
        const int c = j - du32;
        const int d = a.dims[h * a.D + a.du + c];
        a.QC[i * a.dc + c] = (d >= 0 && d < a.D) ? a.scale * ld<T>(a.q, i * a.D + d) : 0.0f;
      }
    }
  }
  if (!a.prep_a) return;
  const int o = threadIdx.x % kPrepOut, part = threadIdx.x / kPrepOut;
  const int pos = blockIdx.y * kPrepOut + o;
  const int len = a.mfma ? a.kpp : a.k;
  const int n = (pos >= len) ? -1 : (a.mfma ? pair_pos_to_n(pos, a.k) : pos);
  const int cper = (a.dc + kPrepParts - 1) / kPrepParts;
  const int c0 = part * cper, c1 = min(a.dc, c0 + cper);
  // coefficient loads first: they do not depend on q
  float ckr[32];
  const float* ckrow = a.ck + ((static_cast<int64_t>(b) * a.hkv + h) * a.k + max(n, 0)) * a.dc;
#pragma unroll
  for (int c = 0; c < 32; ++c) ckr[c] = (n >= 0 && M > 0 && c0 + c < c1) ? ckrow[c0 + c] : 0.0f;
  const float alpha = (n >= 0 && M > 0) ? basis_alpha(n, M) : 0.0f;
  for (int g0 = 0; g0 < a.G; g0 += kPrepRows) {
    const int ng = min(kPrepRows, a.G - g0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < ng * a.dc; idx += blockDim.x) {
      const int g = idx / a.dc, c = idx % a.dc;
      const int d = a.dims[h * a.D + a.du + c];
      const int i = h * a.G + g0 + g;
      qc[g * a.dc + c] = (d >= 0 && d < a.D)
                             ? a.scale * ld<T>(a.q, (static_cast<int64_t>(b) * a.hq + i) * a.D + d)
                             : 0.0f;
    }
    __syncthreads();
    float acc[kPrepRows];
#pragma unroll
    for (int g = 0; g < kPrepRows; ++g) acc[g] = 0.0f;
#pragma unroll
    for (int c = 0; c < 32; ++c)
      if (c0 + c < c1)
#pragma unroll
        for (int g = 0; g < kPrepRows; ++g)
          if (g < ng) acc[g] = fmaf(qc[g * a.dc + c0 + c], ckr[c], acc[g]);
#pragma unroll
    for (int g = 0; g < kPrepRows; ++g) red[(part * kPrepRows + g) * kPrepOut + o] = acc[g];
    __syncthreads();
    if (part == 0 && pos < len) {
      for (int g = 0; g < ng; ++g) {
        float s = 0.0f;
#pragma unroll
        for (int p = 0; p < kPrepParts; ++p) s += red[(p * kPrepRows + g) * kPrepOut + o];
        const int64_t i = static_cast<int64_t>(b) * a.hq + h * a.G + g0 + g;
        if (a.mfma)
          static_cast<_Float16*>(a.A16)[i * a.kpp + pos] = static_cast<_Float16>(alpha * s);
        else
          a.A[i * a.kpad + pos] = alpha * s;
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
  // fixed-order sum over the splits, 8 loads in flight
  float v = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += 8) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (s0 + j < ns) ? Pi[static_cast<int64_t>(s0 + j) * a.RS] : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < ns) v = fmaf(smem[s0 + j], x[j], v);
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
  return sizeof(float) * (kPrepRows * a.dc + kPrepParts * kPrepRows * kPrepOut);
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
  const int len = a.prep_a ? (a.mfma ? a.kpp : a.k) : 1;
  dim3 grid(a.nseq * a.hkv, (len + kPrepOut - 1) / kPrepOut);
  if (a.dtype == 1)
    hipLaunchKernelGGL(decode_prep_kernel<uint16_t>, grid, dim3(256), decode_prep_smem(a), s, a);
  else
    hipLaunchKernelGGL(decode_prep_kernel<float>, grid, dim3(256), decode_prep_smem(a), s, a);
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
