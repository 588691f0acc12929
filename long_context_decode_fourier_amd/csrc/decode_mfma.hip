// decode_mfma.hip - split-L decode step on MFMA for 16-bit caches.
//
// Same arithmetic as the VALU kernel in decode.hip (scores and values in
// coefficient space, online softmax, partials merged by decode_merge), laid out
// for CDNA4 matrix cores.  A work item is (sequence, group of up to 32
// consecutive query heads, token range); its query rows are stacked into the
// 16-row M blocks of the MFMA.  Per tile of T tokens:
//
// * the basis tile phi[t][pos] (unscaled cos/sin, fp16) is generated once into
//   LDS and shared by every row (three-term recurrence along the frequency
//   index, seeded from exact integer phases every 16 frequencies);
// * compressed scores  S_c = A phi^T  (fp16 MFMA over coefficients): each wave
//   owns a slice of 32-wide coefficient units and keeps its slice of A
//   (scale * alpha * q_C ck, written by decode_prep) in registers; the waves'
//   partial scores are summed in LDS;
// * exact scores  S_x = q_U kx^T  (bf16 MFMA over the exact dims) per KV head
//   with q_U held in registers and kx staged in LDS;
// * value moments  W += P phi  (fp16 MFMA over tokens, phi read transposed
//   with ds_read_b64_tr_b16) and exact values  o_U += P vx  (bf16 MFMA, vx read
//   transposed; P is split into a bf16 head and a bf16 remainder so the
//   product keeps ~16 bits of P);
// * kx / vx rows of the next tile are loaded (16-byte loads) while the current
//   tile computes, then staged through LDS;
// * the retained edge rows (ke / ve; at most a few tiles per sequence) take a
//   VALU path with batched loads.
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
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

// Transposed 4 x 16-bit LDS read: lane 4a+e of each 16-lane group receives
// element e of the 8-byte chunks addressed by lanes a, a+4, a+8, a+12 of its
// group.
__device__ inline short4v lds_read_tr4(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p));
}

__device__ inline float wmax(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ inline float wsum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// All-reduce over aligned groups of W = 16 or 32 lanes: DPP rotations inside
// each 16-lane row, then one swizzle (xor 16) across the two rows of a
// 32-lane half.
template <int CTRL> __device__ inline float dpp_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ inline float swz_xor16(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
template <int W> __device__ inline float group_max(float v) {
  static_assert(W == 16 || W == 32, "group width");
  v = fmaxf(v, dpp_ror<0x128>(v));
  v = fmaxf(v, dpp_ror<0x124>(v));
  v = fmaxf(v, dpp_ror<0x122>(v));
  v = fmaxf(v, dpp_ror<0x121>(v));
  if constexpr (W == 32) v = fmaxf(v, swz_xor16(v));
  return v;
}
template <int W> __device__ inline float group_sum(float v) {
  static_assert(W == 16 || W == 32, "group width");
  v += dpp_ror<0x128>(v);
  v += dpp_ror<0x124>(v);
  v += dpp_ror<0x122>(v);
  v += dpp_ror<0x121>(v);
  if constexpr (W == 32) v += swz_xor16(v);
  return v;
}
__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// round-to-nearest-even float -> bf16 bits (finite inputs)
__device__ inline uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// MB: 16-row blocks; NW: waves; MAXU: max 32-wide coefficient units per wave;
// T: tokens per tile (16 or 32); PF: 16-byte kx (and vx) chunks staged per
// thread per tile; XPW: max (KV head, 16-dim block) exact-value tiles per
// wave; RPH: max query rows per KV head (edge-row VALU path).
template <int MB, int NW, int MAXU, int T, int PF, int XPW, int RPH>
__global__ __launch_bounds__(64 * NW) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NT = 64 * NW, MR = 16 * MB, NB = T / 16;
  constexpr int SL = (MR * T + NT - 1) / NT;  // softmax (row, token) slots per thread
  constexpr int KCM = 2;                      // max 32-dim chunks of the exact dims
  constexpr int kNoChunk = 1 << 29;           // staging slot without a chunk
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
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
  const int du32 = (du + 31) & ~31;
  const int KC = du32 / 32;        // exact-dim chunks (<= KCM)
  const int DUS = du32 + 8;        // LDS row stride of staged kx / vx (halves)
  const int PS = a.kpp + 16;       // LDS row stride of the basis tile (halves)

  _Float16* phi = reinterpret_cast<_Float16*>(smem);             // [T][PS]
  uint16_t* kxs = reinterpret_cast<uint16_t*>(phi + T * PS);     // [nheads][T][DUS]
  uint16_t* vxs = kxs + nheads * T * DUS;                         // [nheads][T][DUS]
  float* sx = reinterpret_cast<float*>(vxs + nheads * T * DUS);   // [MR][T]
  float* sedge = sx + MR * T;                                     // [MR][T]
  float* spart = sedge + MR * T;                                  // [NW][MR][T]
  float* pf = spart + NW * MR * T;                                // [MR][T]
  _Float16* ph = reinterpret_cast<_Float16*>(pf + MR * T);        // [MR][T]
  uint16_t* pbh = reinterpret_cast<uint16_t*>(ph + MR * T);       // [MR][T]
  uint16_t* pbl = pbh + MR * T;                                   // [MR][T]
  float* qcs = reinterpret_cast<float*>(pbl + MR * T);            // [MR][dc] (edge rows)
  float* corr = qcs + MR * dc;                                    // [MR]
  int* flag = reinterpret_cast<int*>(corr + MR);

  // ---- zero the staging rows once: columns [du, DUS) stay zero (finite operands)
  for (int i = tid; i < 2 * nheads * T * DUS; i += NT) kxs[i] = 0;

  // ---- kx / vx staging: thread -> 16-byte chunks c = tid + NT*i of the tile;
  //      the chunk -> (KV head, token, 8 dims) map is the same for every tile
  const int du8 = du / 8;
  const int nchunk = nheads * T * du8;
  int64_t st_src[PF];  // element offset of the chunk in the tile starting at t_begin
  int st_tt[PF];       // token within the tile (kNoChunk: no chunk)
  int st_lds[PF];      // LDS offset (halves) in kxs / vxs
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int c = tid + NT * i;
    st_tt[i] = kNoChunk;
    st_src[i] = 0;
    st_lds[i] = 0;
    if (du8 > 0 && c < nchunk) {
      const int row = c / du8, c8 = c % du8;  // row = hh * T + tt
      const int hh = row / T, tt = row % T;
      st_tt[i] = tt;
      st_src[i] = (row0 + static_cast<int64_t>(h0 + hh) * L + t_begin + tt) * du + 8 * c8;
      st_lds[i] = row * DUS + 8 * c8;
    }
  }
  uint4 pk[PF], pv[PF];
  auto prefetch = [&](int tile) {
    const int64_t shift = static_cast<int64_t>(tile - t_begin) * du;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      uint4 vk = make_uint4(0u, 0u, 0u, 0u), vv = vk;
      if (tile + st_tt[i] < t_end) {
        vk = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.kx) + st_src[i] + shift);
        vv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.vx) + st_src[i] + shift);
      }
      pk[i] = vk;
      pv[i] = vv;
    }
  };
  if (du8 > 0) prefetch(t_begin);

  // ---- q operands (permuted by decode_prep): exact dims as bf16 MFMA A
  //      operand per 32-dim chunk, compressible dims (scaled fp32) in LDS for
  //      the edge rows
  bf16x8 Qreg[KCM][MB];
#pragma unroll
  for (int kc = 0; kc < KCM; ++kc)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = mb * 16 + l16;
      uint4 bits = make_uint4(0u, 0u, 0u, 0u);
      if (row < rows && kc < KC)
        bits = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.Q16) +
                                               (static_cast<int64_t>(b) * a.hq + qi0 + row) * du32 +
                                               32 * kc + 8 * g4);
      Qreg[kc][mb] = __builtin_bit_cast(bf16x8, bits);
    }
  {
    const float* qsrc = a.QC + (static_cast<int64_t>(b) * a.hq + qi0) * dc;
#pragma unroll 4
    for (int idx = tid; idx < MR * dc; idx += NT) qcs[idx] = (idx < rows * dc) ? qsrc[idx] : 0.0f;
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
      const int row = mb * 16 + l16;
      if (has_mid && u < nu && row < rows)
        v = *reinterpret_cast<const half8*>(
            static_cast<const _Float16*>(a.A16) +
            (static_cast<int64_t>(b) * a.hq + qi0 + row) * a.kpp + (u0 + u) * 32 + 8 * g4);
      Areg[u][mb] = v;
    }
  floatx4 Wacc[MAXU][2][MB];
#pragma unroll
  for (int u = 0; u < MAXU; ++u)
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) Wacc[u][n2][mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // ---- exact-value tiles of this wave: (KV head, 16-dim block) pairs
  const int ndb = du32 / 16;
  floatx4 Uacc[XPW];
#pragma unroll
  for (int x = 0; x < XPW; ++x) Uacc[x] = floatx4{0.f, 0.f, 0.f, 0.f};

  // ---- edge-row value accumulators (VALU): thread -> (head, comp-dim pair)
  const int dc2 = dc / 2;
  const int eh = dc2 ? tid / dc2 : 0, ec = dc2 ? tid % dc2 : 0;
  const bool evld = dc2 > 0 && tid < nheads * dc2;
  const int erb = (rows >= a.G) ? eh * a.G : 0;
  float oE[RPH][2];
#pragma unroll
  for (int r = 0; r < RPH; ++r) oE[r][0] = oE[r][1] = 0.0f;

  // ---- softmax slots: thread -> (row, token) for idx = tid + NT*j
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
  // integer phases of this thread's token (tau = t - sink, taken mod M):
  // tau itself, 4 c_lo tau (first pair of its run) and 16 tau (run step),
  // advanced by T tokens per tile
  int ph_tau = 0, ph_r0 = 0, ph_d16 = 0, inc_tau = 0, inc_r0 = 0, inc_d16 = 0;
  if (has_mid) {
    int tau0 = (t_begin + gt - S) % M;
    if (tau0 < 0) tau0 += M;
    ph_tau = tau0;
    ph_r0 = phase_mod(4 * c_lo, tau0, M);
    ph_d16 = phase_mod(16, tau0, M);
    inc_tau = T % M;
    inc_r0 = phase_mod(4 * c_lo, T, M);
    inc_d16 = phase_mod(16, T, M);
  }

  // ---- edge-score mapping: thread -> (head, token, part of the comp dims)
  const int npairs = nheads * T;
  const int tpp = NT / npairs >= 1 ? NT / npairs : 1;

  __syncthreads();  // staging rows zeroed, qcs ready

  for (int tile0 = t_begin; tile0 < t_end; tile0 += T) {
    const int nt = min(T, t_end - tile0);
    const bool tile_edge = dc > 0 && (M == 0 || tile0 < S || tile0 + nt > S + M);
    // ================= phase 1: stage this tile, prefetch the next, basis tile
    if (tid == 0) *flag = 0;
    if (du8 > 0) {
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        if (st_tt[i] != kNoChunk) {
          *reinterpret_cast<uint4*>(kxs + st_lds[i]) = pk[i];
          *reinterpret_cast<uint4*>(vxs + st_lds[i]) = pv[i];
        }
      }
      if (tile0 + T < t_end) prefetch(tile0 + T);
    }
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
        const int tau = ph_tau;  // t - sink (a middle token: 0 <= t - sink < M)
        const float c2 = 2.0f * cos_rev(static_cast<float>(tau) * invM);
        // runs of 4 chunks (16 pairs) are seeded from exact phases
        int r0 = ph_r0;
        const int d16 = ph_d16;
        for (int c = c_lo; c < c_hi; c += 4) {
          int r1 = r0 + tau;
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
            const float cn = fmaf(c2, cc, -cp), sn = fmaf(c2, sc, -sp_);
            z[4] = static_cast<_Float16>(cn);
            z[5] = static_cast<_Float16>(sn);
            const float cm = fmaf(c2, cn, -cc), sm = fmaf(c2, sn, -sc);
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
      if (has_mid) {
        ph_tau += inc_tau;
        if (ph_tau >= M) ph_tau -= M;
        ph_r0 += inc_r0;
        if (ph_r0 >= M) ph_r0 -= M;
        ph_d16 += inc_d16;
        if (ph_d16 >= M) ph_d16 -= M;
      }
    }
    if (tile_edge) {
      // compressible part of the exact scores of the retained edge rows
      for (int pr = tid / tpp; pr < npairs; pr += NT / tpp) {
        const int hh = pr / T, tt = pr % T, part = tid % tpp;
        const int t = tile0 + tt;
        const int rb = (rows >= a.G) ? hh * a.G : 0;
        float acc[RPH];
#pragma unroll
        for (int r = 0; r < RPH; ++r) acc[r] = 0.0f;
        if (t < t_end && (M == 0 || t < S || t >= S + M)) {
          const int e = (M == 0 || t < S) ? t : t - M;
          const int cper_ = dc / tpp, c0 = part * cper_;
          const uint32_t* erow = reinterpret_cast<const uint32_t*>(
              static_cast<const uint16_t*>(a.ke) + ((static_cast<int64_t>(b) * a.hkv + h0 + hh) * E + e) * dc + c0);
          for (int cb = 0; 2 * cb < cper_; cb += 8) {  // batches of 8 independent loads
            uint32_t ew[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) ew[c] = (2 * (cb + c) < cper_) ? erow[cb + c] : 0u;
#pragma unroll
            for (int c = 0; c < 8; ++c)
              if (2 * (cb + c) < cper_)
#pragma unroll
                for (int r = 0; r < RPH; ++r)
                  if (r < rph) {
                    const int cc = c0 + 2 * (cb + c);
                    acc[r] = fmaf(qcs[(rb + r) * dc + cc], lo_bf16(ew[c]),
                                  fmaf(qcs[(rb + r) * dc + cc + 1], hi_bf16(ew[c]), acc[r]));
                  }
          }
        }
#pragma unroll
        for (int r = 0; r < RPH; ++r) acc[r] = wsum(acc[r], tpp);
        if (part == 0)
#pragma unroll
          for (int r = 0; r < RPH; ++r)
            if (r < rph) sedge[(rb + r) * T + tt] = acc[r];
      }
    }
    __syncthreads();

    // ================= phase 2: compressed score partials, exact scores (MFMA)
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
                phi + (nb * 16 + l16) * PS + (u0 + u) * 32 + 8 * g4);
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
            spart[(wave * MR + mb * 16 + 4 * g4 + r) * T + nb * 16 + l16] = sacc[mb][nb][r];
    }
    for (int p = wave; p < nheads * NB; p += NW) {
      const int hh = p / NB, nb = p % NB;
      const int rb = (rows >= a.G) ? hh * a.G : 0;
      const int mb = rb >> 4;
      floatx4 s = floatx4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = kxs + (hh * T + nb * 16 + l16) * DUS + 8 * g4;
#pragma unroll
      for (int kc = 0; kc < KCM; ++kc) {
        if (kc < KC) {
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(krow + 32 * kc);
          bf16x8 av = Qreg[kc][0];
          if (MB > 1 && mb == 1) av = Qreg[kc][MB - 1];
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, s, 0, 0, 0);
        }
      }
      const int tt = nb * 16 + l16;
      const bool valid = tile0 + tt < t_end;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mb * 16 + 4 * g4 + r;
        if (row >= rb && row < rb + rph) sx[row * T + tt] = valid ? a.scale * s[r] : -INFINITY;
      }
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
        if (s != -INFINITY) {
          if (tile_edge) s += sedge[row * T + tt];
          if (has_mid) {
#pragma unroll
            for (int w = 0; w < NW; ++w) s += spart[(w * MR + row) * T + tt];
          }
        }
      }
      const float m_new = fmaxf(m_run[j], group_max<T>(s));
      const float c = (m_new == -INFINITY || m_run[j] == m_new) ? 1.0f : __expf(m_run[j] - m_new);
      const float p = (s == -INFINITY) ? 0.0f : __expf(s - m_new);
      l_run[j] = l_run[j] * c + group_sum<T>(p);
      m_run[j] = m_new;
      if (row >= MR) continue;
      pf[row * T + tt] = p;
      ph[row * T + tt] = static_cast<_Float16>(p);
      const uint16_t hb = bf16_rne(p);
      pbh[row * T + tt] = hb;
      pbl[row * T + tt] = bf16_rne(p - __uint_as_float(static_cast<uint32_t>(hb) << 16));
      if (tt == 0) {
        corr[row] = c;
        if (c != 1.0f) *flag = 1;
      }
    }
    __syncthreads();

    // ================= phase 4: value moments W, exact values (MFMA)
    const bool rescale = *flag != 0;
    if (rescale) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float cr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) cr[r] = corr[mb * 16 + 4 * g4 + r];
        if (has_mid) {
#pragma unroll
          for (int u = 0; u < MAXU; ++u)
#pragma unroll
            for (int n2 = 0; n2 < 2; ++n2)
#pragma unroll
              for (int r = 0; r < 4; ++r) Wacc[u][n2][mb][r] *= cr[r];
        }
#pragma unroll
        for (int x = 0; x < XPW; ++x) {
          const int p = wave + NW * x;
          const int rb = (rows >= a.G) ? (p / max(ndb, 1)) * a.G : 0;
          if ((rb >> 4) == mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) Uacc[x][r] *= cr[r];
        }
      }
    }
    if (has_mid) {
#pragma unroll
      for (int u = 0; u < MAXU; ++u) {
        if (u < nu) {
#pragma unroll
          for (int n2 = 0; n2 < 2; ++n2) {
            const int nbase = (u0 + u) * 32 + n2 * 16 + 4 * (l16 & 3);
            if constexpr (T == 32) {
              const short4v lo = lds_read_tr4(phi + (8 * g4 + (l16 >> 2)) * PS + nbase);
              const short4v hi = lds_read_tr4(phi + (8 * g4 + 4 + (l16 >> 2)) * PS + nbase);
              const half8 bv = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) {
                const half8 pv8 = *reinterpret_cast<const half8*>(ph + (mb * 16 + l16) * T + 8 * g4);
                Wacc[u][n2][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pv8, bv, Wacc[u][n2][mb], 0, 0, 0);
              }
            } else {
              const half4 bv = __builtin_bit_cast(half4, lds_read_tr4(phi + (4 * g4 + (l16 >> 2)) * PS + nbase));
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) {
                const half4 pv4 = *reinterpret_cast<const half4*>(ph + (mb * 16 + l16) * T + 4 * g4);
                Wacc[u][n2][mb] = __builtin_amdgcn_mfma_f32_16x16x16f16(pv4, bv, Wacc[u][n2][mb], 0, 0, 0);
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int x = 0; x < XPW; ++x) {
      const int p = wave + NW * x;
      if (ndb == 0 || p >= nheads * ndb) continue;
      const int hh = p / ndb, db = p % ndb;
      const int rb = (rows >= a.G) ? hh * a.G : 0;
      const int mb = rb >> 4;
      const uint16_t* vbase = vxs + hh * T * DUS + db * 16 + 4 * (l16 & 3);
      if constexpr (T == 32) {
        const short4v lo = lds_read_tr4(vbase + (8 * g4 + (l16 >> 2)) * DUS);
        const short4v hi = lds_read_tr4(vbase + (8 * g4 + 4 + (l16 >> 2)) * DUS);
        const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8 ph8 = *reinterpret_cast<const bf16x8*>(pbh + (mb * 16 + l16) * T + 8 * g4);
        const bf16x8 pl8 = *reinterpret_cast<const bf16x8*>(pbl + (mb * 16 + l16) * T + 8 * g4);
        Uacc[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph8, bv, Uacc[x], 0, 0, 0);
        Uacc[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl8, bv, Uacc[x], 0, 0, 0);
      } else {
        const short4v bv = lds_read_tr4(vbase + (4 * g4 + (l16 >> 2)) * DUS);
        const short4v ph4 = *reinterpret_cast<const short4v*>(pbh + (mb * 16 + l16) * T + 4 * g4);
        const short4v pl4 = *reinterpret_cast<const short4v*>(pbl + (mb * 16 + l16) * T + 4 * g4);
        Uacc[x] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph4, bv, Uacc[x], 0, 0, 0);
        Uacc[x] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl4, bv, Uacc[x], 0, 0, 0);
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
      if (tile_edge) {
        // edge tokens of this tile: [tile0, mid_lo) and [mid_hi, tile0 + nt)
        const int mid_lo = (M == 0) ? tile0 + nt : max(tile0, min(tile0 + nt, S));
        const int mid_hi = (M == 0) ? tile0 + nt : max(mid_lo, min(tile0 + nt, S + M));
        const uint32_t* ecol = reinterpret_cast<const uint32_t*>(
            static_cast<const uint16_t*>(a.ve) + (static_cast<int64_t>(b) * a.hkv + h) * E * dc + 2 * ec);
        for (int seg = 0; seg < 2; ++seg) {
          const int lo = seg == 0 ? tile0 : mid_hi, hi = seg == 0 ? mid_lo : tile0 + nt;
          for (int t0 = lo; t0 < hi; t0 += 8) {  // batches of 8 independent loads
            uint32_t w8[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const int t = t0 + q;
              const int e = (M == 0 || t < S) ? t : t - M;
              w8[q] = (t < hi) ? ecol[static_cast<int64_t>(e) * dc2] : 0u;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              if (t0 + q >= hi) break;
              const float v0 = lo_bf16(w8[q]), v1 = hi_bf16(w8[q]);
#pragma unroll
              for (int r = 0; r < RPH; ++r)
                if (r < rph) {
                  const float p = pf[(erb + r) * T + (t0 + q - tile0)];
                  oE[r][0] = fmaf(p, v0, oE[r][0]);
                  oE[r][1] = fmaf(p, v1, oE[r][1]);
                }
            }
          }
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
#pragma unroll
  for (int x = 0; x < XPW; ++x) {
    const int p = wave + NW * x;
    if (ndb == 0 || p >= nheads * ndb) continue;
    const int hh = p / ndb, db = p % ndb;
    const int rb = (rows >= a.G) ? hh * a.G : 0;
    const int mb = rb >> 4;
    const int d = db * 16 + l16;
    if (d >= du) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mb * 16 + 4 * g4 + r;
      if (row >= rb && row < rb + rph)
        a.part[(prow + static_cast<int64_t>(row) * ns) * a.RS + 2 + d] = Uacc[x][r];
    }
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
        const int pos = (u0 + u) * 32 + n2 * 16 + l16;
        const int j = pos >> 1;
        const int n = (pos & 1) ? (j == 0 ? -1 : 2 * j) : (j == 0 ? 0 : 2 * j - 1);
        if (n < 0 || n >= a.k) continue;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = mb * 16 + 4 * g4 + r;
            if (row < rows)
              a.part[(prow + static_cast<int64_t>(row) * ns) * a.RS + 2 + du + dc + n] = Wacc[u][n2][mb][r];
          }
      }
    }
  }
}

template <int MB, int NW, int MAXU, int T, int PF, int XPW, int RPH>
hipError_t launch_one(const DecodeArgs& a, int nitems, size_t smem, hipStream_t s) {
  auto k = decode_mfma_kernel<MB, NW, MAXU, T, PF, XPW, RPH>;
  if (smem > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(smem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(nitems), dim3(64 * NW), smem, s, a);
  return hipGetLastError();
}

// Compiled variants, chosen by row blocks and basis length (pair-order
// positions kpp): short bases take 4 waves, long ones 8 waves so that each
// wave's slice of A and W stays in registers.
constexpr MfmaVariant kVariants[] = {
    // mb nw maxu  t pf xpw rph kpp_min kpp_max
    {1, 4, 4, 32, 4, 4, 8, 0, 512},
    {2, 4, 4, 32, 4, 8, 8, 0, 512},
    {2, 8, 5, 32, 2, 4, 4, 513, 1280},
    {1, 8, 5, 32, 2, 4, 4, 513, 1280},
    {1, 8, 9, 16, 1, 4, 4, 1281, 2304},
};

}  // namespace

const MfmaVariant* decode_mfma_pick(int kpp, int mb) {
  for (const MfmaVariant& v : kVariants)
    if (v.mb == mb && kpp >= v.kpp_min && kpp <= v.kpp_max) return &v;
  return nullptr;
}

size_t decode_mfma_smem(const DecodeArgs& a, const MfmaVariant& v, int nheads) {
  const int T = v.t, MR = 16 * v.mb;
  const int dus = ((a.du + 31) & ~31) + 8;
  return static_cast<size_t>(T) * (a.kpp + 16) * 2 + 2 * static_cast<size_t>(2 * nheads * T * dus) +
         sizeof(float) * (MR * T * 2 + v.nw * MR * T + MR * T) + 2 * MR * T * 3 +
         sizeof(float) * (MR * a.dc + MR) + 16;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int nitems, hipStream_t s) {
  if (nitems == 0) return hipSuccess;
  const MfmaVariant* v = decode_mfma_pick(a.kpp, a.mb);
  if (!v) return hipErrorInvalidValue;
  const int nheads = a.rows >= a.G ? a.rows / a.G : 1;
  const size_t smem = decode_mfma_smem(a, *v, nheads);
  switch (v - kVariants) {
    case 0: return launch_one<1, 4, 4, 32, 4, 4, 8>(a, nitems, smem, s);
    case 1: return launch_one<2, 4, 4, 32, 4, 8, 8>(a, nitems, smem, s);
    case 2: return launch_one<2, 8, 5, 32, 2, 4, 4>(a, nitems, smem, s);
    case 3: return launch_one<1, 8, 5, 32, 2, 4, 4>(a, nitems, smem, s);
    case 4: return launch_one<1, 8, 9, 16, 1, 4, 4>(a, nitems, smem, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
