// decode_two_pass.hip - the long-context decode step in two passes over the
// middle tokens, for 16-bit caches on MFMA.
//
// The factored decode (scores a . phi(tau) + q_U . kx, values o_U = P vx and
// W = P phi, then o_C = (alpha W) cv) needs, per query row, both the k-vector
// a (as the score operand) and the k-vector W (an accumulator).  Held together
// in registers they limit an item to 16 stacked query rows, so the basis of a
// token is generated once per 16 rows, and the W product needs the basis in a
// second register layout, which costs an LDS round trip of the whole basis
// tile.  Two passes separate them:
//
// Pass 1, decode_score_kernel: item = (sequence, row group of up to 32 query
//   rows, range of middle tokens), 16-token tiles.  [A] each wave generates
//   its slice of the basis tile as the score MFMA's operand (lane = token, 8
//   consecutive pair-order positions) and multiplies it by its slice of A;
//   exact-dim scores run on bf16 MFMA with kx loaded straight into the operand
//   layout.  [B] the partial scores are summed and the online softmax runs
//   with a lazy reference (moved only when a score exceeds it by more than
//   kLazyMax).  [C] exact values o_U += P vx on bf16 MFMA (P as a bf16 head and
//   remainder, vx staged in LDS and read transposed).  The probabilities go to
//   HBM as fp16 (P16, 2 bytes per row and token, a few percent of the bytes
//   read) with the reference of each 16-token tile (msub); the split's
//   (m, l, o_U) go to the partials.
//
// Pass 2, decode_moment_kernel: item = (sequence, row group, group of 4
//   consecutive pass-1 splits, slice of frequency groups of 16).  Wave w takes
//   split 4 sg + w whole, with no barrier until the end, in blocks of 64
//   tokens, in a frame that rotates with the block: with
//   U_j[f] = sum_t P[tau_j + t] e^{i theta_f t} (t < 64) the moment of the
//   split is W[f] = sum_j e^{i theta_f tau_j} U_j[f], that is
//   W = e^{i theta_f tau_last} V with V_j = U_j + e^{-i theta_f 64} V_{j-1}
//   (exact integer phase for tau_last).  V comes from the second-order
//   recurrence s_j = U_j + 2 cos(theta_f 64) s_{j-1} - s_{j-2} on the cosine
//   and sine parts, V_j = s_j - e^{i theta_f 64} s_{j-1}: one FMA per
//   accumulator and block, where the frame rotation of V took four per pair;
//   the recurrence restarts from its output every 16 blocks, which bounds the
//   growth of its states.  The table e^{i theta_f t} of the lane's 16
//   frequencies and 64 offsets is the same for every block, so it is
//   generated once per item (negated) and held in registers as the B operand
//   of v_mfma_f32_16x16x32_f16 (cosines and sines as two 16-column blocks; the
//   MFMA subtracts U straight from the state s_{j-2}).  The P
//   operand is loaded from P16 (the 4 waves of a split group and the slices
//   of a split group read the same P, which stays in L2).  Each wave's W is
//   relative to its split's reference; scaled by exp(m_split - m_row) (the
//   row's maximum over all its splits), the waves' W are summed in a fixed
//   order and written to Wp.  Tiles of pass 1 whose reference moved later in
//   their split (rare with the lazy reference) have their P rescaled on load.
//
// decode_merge then combines (m, l, o_U, o_E) over the splits and sums Wp over
// the split groups; decode_merge_cv applies (alpha W) cv.
#include <type_traits>

#include "kernels.hpp"
#include "mfma_util.hpp"

namespace fa {
namespace {

// P16 layout (per sequence, a.ngroups * MB 16-row blocks of mpad tokens): block
// g * MB + mb holds query rows g * rows + 16 mb + s (s < 16) of row group g, in
// 32-token chunks of 1 KB, each in the A-operand order of
// v_mfma_f32_16x16x32_f16 (lane s + 16 q holds tokens 8 q .. 8 q + 7 of row s),
// so that pass 2 loads a chunk with one contiguous 16-byte load per lane.
__device__ inline int64_t p16_index(int blk16, int slot, int tau, int mpad) {
  return (static_cast<int64_t>(blk16) * (mpad / 32) + (tau >> 5)) * 512 + 8 * (slot + 16 * ((tau & 31) >> 3)) +
         (tau & 7);
}

using namespace mfma;

// LDS of pass 1: vx staging (double buffer), partial scores of each wave,
// exact scores, P as bf16 head and remainder, per-row rescale factors.
struct ScoreLds {
  int dus;
  int vxs, spart, sx, pbh, pbl, corr, total;
};
__host__ __device__ inline ScoreLds score_lds(int mb, int nw, int nheads, int du) {
  const int T = kMfmaTile, MR = 16 * mb, TP = kMfmaTile + 4;
  const int du32 = (du + 31) & ~31;
  ScoreLds o;
  int off = 0;
  auto take = [&off](int bytes) {
    const int r = off;
    off += (bytes + 15) & ~15;
    return r;
  };
  o.dus = du32 + 16;
  o.vxs = take(du32 ? 2 * nheads * T * o.dus * 2 : 0);
  o.spart = take(nw * MR * TP * 4);
  o.sx = take(MR * TP * 4);
  o.pbh = take(MR * TP * 2);
  o.pbl = take(MR * TP * 2);
  o.corr = take(MR * 4);
  o.total = off;
  return o;
}

// ============================================================== pass 1 ====
// MB: 16-row blocks; NW: waves; MAXU: max 32-wide coefficient units per wave;
// PF: 16-byte vx chunks staged per thread per tile; XP: max (KV head, row
// block) units per wave (exact scores); XU: max (unit, 16-dim block) exact
// value tiles per wave; KCM: max 32-dim chunks of the exact dims; DEPTH:
// tiles of kx / vx loads in flight (1 or 2 register sets).
template <int MB, int NW, int MAXU, int PF, int XP, int XU, int KCM, int DEPTH>
__global__ __launch_bounds__(64 * NW) void decode_score_kernel(DecodeArgs a) {
  constexpr int T = kMfmaTile, TP = kMfmaTile + 4;
  constexpr int NT = 64 * NW, MR = 16 * MB;
  constexpr int kNoChunk = 1 << 29;  // staging slot without a chunk
  static_assert(MR * T <= NT, "one softmax slot per thread");
  static_assert((NW & (NW - 1)) == 0, "power-of-two wave count (partial-score tree)");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g4 = lane >> 4, l16 = lane & 15;
  const int b = seq_of_item(a.seq, a.nseq, blockIdx.x);
  const int local = blockIdx.x - a.seq.item0[b];
  const int ns = a.seq.nsplit[b];
  const int nsm = ns - a.edge_split;  // middle splits (the edge splits come last)
  const int rg = local / nsm, sp = local % nsm;
  const int L = a.seq.len[b], M = a.seq.mid[b], per = a.seq.per[b];
  const int S = a.sink;
  const int t_begin = S + sp * a.seq.chunk[b];
  const int t_end = min(S + M, t_begin + a.seq.chunk[b]);
  const int64_t row0 = a.seq.row0[b];
  const int rows = a.rows;
  const int qi0 = rg * rows;
  const int h0 = qi0 / a.G;
  const int nheads = rows >= a.G ? rows / a.G : 1;
  const int rph = min(rows, a.G);  // query rows per KV head inside the item
  // (KV head, 16-row block) units of the exact-dim work: head u >> bsh, block u & bsh
  const int bph = MB > 1 ? (rph + 15) >> 4 : 1;
  const int bsh = bph - 1;
  const int nunit = nheads * bph;
  const int du = a.du;
  const int du32 = (du + 31) & ~31;
  const int KC = du32 / 32;  // exact-dim chunks (<= KCM)
  const int ndb = du32 / 16;
  const int mpad = (M + kMomentTile - 1) & ~(kMomentTile - 1);

  const ScoreLds lo = score_lds(MB, NW, nheads, du);
  const int DUS = lo.dus;
  uint16_t* vxs = reinterpret_cast<uint16_t*>(smem + lo.vxs);   // [2][nheads][T][DUS]
  float* spart = reinterpret_cast<float*>(smem + lo.spart);     // [NW][MR][TP]
  float* sx = reinterpret_cast<float*>(smem + lo.sx);           // [MR][TP]
  uint16_t* pbh = reinterpret_cast<uint16_t*>(smem + lo.pbh);   // [MR][TP]
  uint16_t* pbl = reinterpret_cast<uint16_t*>(smem + lo.pbl);   // [MR][TP]
  float* corr = reinterpret_cast<float*>(smem + lo.corr);       // [MR]

  // ---- vx staging: thread -> 16-byte chunks c = tid + NT*i of a tile
  const int du8 = du / 8;
  const int nchunk = nheads * T * du8;
  int64_t st_src[PF];
  int st_tt[PF];
  int st_lds[PF];
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
  // Loads of a tile are unconditional (clamped to the last token of the
  // range, the last unit and the last 8 exact dims), so that the waits for
  // them are counted, never a drain; two register sets alternate between
  // even and odd tiles, so two tiles of loads are in flight.
  // tile j's loads sit in set j % DEPTH (native vectors: plain loads and
  // stores, which keep the sets in registers)
  u32x4 kset[DEPTH][XP][KCM], vset[DEPTH][PF];
  int st_ld[PF];  // token of the slot's chunk for the loads (0 for an empty slot)
#pragma unroll
  for (int i = 0; i < PF; ++i) st_ld[i] = st_tt[i] == kNoChunk ? 0 : st_tt[i];
  auto prefetch_v = [&](int tile, auto set_c) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_c)::value;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int64_t shift = static_cast<int64_t>(min(tile + st_ld[i], t_end - 1) - t_begin - st_ld[i]) * du;
      vset[SET][i] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.vx) + st_src[i] + shift);
    }
  };
  auto stage_v = [&](int buf, auto set_c) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_c)::value;
    uint16_t* dst = vxs + buf * nheads * T * DUS;
#pragma unroll
    for (int i = 0; i < PF; ++i)
      if (st_tt[i] != kNoChunk) *reinterpret_cast<u32x4*>(dst + st_lds[i]) = vset[SET][i];
  };

  // ---- kx as the B operand of the exact-score MFMA, loaded from HBM:
  //      lane -> (token l16, dims 32 kc + 8 g4 .. +7) of unit wave + NW x
  int64_t kx_src[XP];
#pragma unroll
  for (int x = 0; x < XP; ++x)
    kx_src[x] = (row0 + static_cast<int64_t>(h0 + (min(wave + NW * x, nunit - 1) >> bsh)) * L + t_begin) * du;
  auto prefetch_k = [&](int tile, auto set_c) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_c)::value;
    const int64_t tok = min(tile + l16, t_end - 1) - t_begin;
#pragma unroll
    for (int x = 0; x < XP; ++x)
#pragma unroll
      for (int kc = 0; kc < KCM; ++kc) {
        // lanes past the exact dims read the last 8 (finite bf16 values) and
        // meet the zero padding of q there, so they add nothing
        const int d0 = min(32 * min(kc, KC - 1) + 8 * g4, du - 8);
        kset[SET][x][kc] =
            *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.kx) + kx_src[x] + tok * du + d0);
      }
  };
  using kSet0 = std::integral_constant<int, 0>;
  using kSet1 = std::integral_constant<int, 1>;
  if (du8 > 0) {
    prefetch_k(t_begin, kSet0());
    prefetch_v(t_begin, kSet0());
  }

  // ---- q at the exact dims (permuted by decode_prep): bf16 A operand
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
  // ---- this wave's coefficient units and its slice of A (fp16 A operand);
  //      none without compressible dims (the compressed partials are then 0)
  const int U = a.dc > 0 ? a.kpp / 32 : 0;
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
      if (u < nu && row < rows)
        v = *reinterpret_cast<const half8*>(
            static_cast<const _Float16*>(a.A16) +
            (static_cast<int64_t>(b) * a.hq + qi0 + row) * a.kpp + (u0 + u) * 32 + 8 * g4);
      Areg[u][mb] = v;
    }
  floatx4 Uacc[XU];
#pragma unroll
  for (int x = 0; x < XU; ++x) Uacc[x] = floatx4{0.f, 0.f, 0.f, 0.f};

  // ---- softmax slot: thread -> (row, token)
  const int s_row = tid / T, s_tt = tid % T;
  float m_run = -INFINITY, l_run = 0.0f;
  // probability and reference outputs of this slot's row
  const int orow = qi0 + min(s_row, rows - 1);
  // the slot's row in the P16 layout (token offsets added per tile)
  _Float16* p_out = static_cast<_Float16*>(a.P16) + static_cast<int64_t>(a.ngroups) * MB * 16 * a.pcum[b] +
                    p16_index(rg * MB + min(s_row, MR - 1) / 16, s_row % 16, 0, mpad);
  float* m_out = a.msub + a.hq * (a.pcum[b] / 16) + static_cast<int64_t>(orow) * (mpad / 16) + (t_begin - S) / 16;

  // ---- basis generator: lane -> token l16 of the tile and frequencies
  //      16 u + 4 g4 + j (j < 4) of its wave's units; integer phases (mod per)
  //      of tau, 16 tau and f0 tau for the lane's token, advanced per tile
  const float inv_per = 1.0f / static_cast<float>(per);
  const int f0 = 16 * u0 + 4 * g4;
  int ph_tau, ph_16, ph_f0;
  {
    const int tau0 = t_begin + l16 - S;  // < M + 16 <= 2^30 + 16
    ph_tau = tau0 % per;
    ph_16 = phase_mod(16, tau0, per);
    ph_f0 = phase_mod(f0, tau0, per);
  }
  const int inc_tau = T % per;
  const int inc_16 = phase_mod(16, T, per);
  const int inc_f0 = phase_mod(f0, T, per);

  // [A] compressed score partials of tile tile0 -> spart
  auto scores_a = [&](int tile0) {
    const bool mid = tile0 + l16 < t_end;
    const float x0 = static_cast<float>(ph_f0) * inv_per;
    const float x1 = static_cast<float>(ph_tau) * inv_per;
    const float x16 = static_cast<float>(ph_16) * inv_per;
    // a lane whose token is past the range seeds zeros: all its values are 0
    const float c0 = mid ? cos_rev(x0) : 0.0f, s0 = mid ? sin_rev(x0) : 0.0f;
    const float c1 = cos_rev(x1), s1 = sin_rev(x1);
    const float c16 = cos_rev(x16), s16 = sin_rev(x16);
    const float tc1 = 2.0f * c1, tc16 = 2.0f * c16;
    float ca[4], sa[4], cb[4], sb[4];
    ca[0] = c0;
    sa[0] = s0;
    ca[1] = fmaf(c0, c1, -s0 * s1);
    sa[1] = fmaf(s0, c1, c0 * s1);
    ca[2] = fmaf(tc1, ca[1], -ca[0]);
    sa[2] = fmaf(tc1, sa[1], -sa[0]);
    ca[3] = fmaf(tc1, ca[2], -ca[1]);
    sa[3] = fmaf(tc1, sa[2], -sa[1]);
#pragma unroll
    for (int j = 0; j < 4; ++j) cb[j] = sb[j] = 0.0f;
    floatx4 sacc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) sacc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
      if (u < nu) {
        if (u == 1) {  // unit u0+1: rotate by 16 frequencies
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            cb[j] = fmaf(ca[j], c16, -sa[j] * s16);
            sb[j] = fmaf(sa[j], c16, ca[j] * s16);
          }
        } else if (u > 1) {  // three-term recurrence, step 16 frequencies
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (u & 1) {
              cb[j] = fmaf(tc16, ca[j], -cb[j]);
              sb[j] = fmaf(tc16, sa[j], -sb[j]);
            } else {
              ca[j] = fmaf(tc16, cb[j], -ca[j]);
              sa[j] = fmaf(tc16, sb[j], -sa[j]);
            }
          }
        }
        const float* zc = (u & 1) ? cb : ca;
        const float* zs = (u & 1) ? sb : sa;
        const uint4 bits = make_uint4(pack_f16(zc[0], zs[0]), pack_f16(zc[1], zs[1]),
                                      pack_f16(zc[2], zs[2]), pack_f16(zc[3], zs[3]));
        const half8 bv = __builtin_bit_cast(half8, bits);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Areg[u][mb], bv, sacc[mb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) spart[(wave * MR + mb * 16 + 4 * g4 + r) * TP + l16] = sacc[mb][r];
    ph_tau = add_mod(ph_tau, inc_tau, per);
    ph_16 = add_mod(ph_16, inc_16, per);
    ph_f0 = add_mod(ph_f0, inc_f0, per);
  };

  // exact-dim scores of tile tile0 from the kx operands kr
  auto exact_a = [&](int tile0, auto set_c) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_c)::value;
    if (du8 > 0) {
#pragma unroll
      for (int x = 0; x < XP; ++x) {
        const int un = wave + NW * x;
        if (un < nunit) {
          const int rb = (rows >= a.G) ? (un >> bsh) * a.G : 0;
          const int mb = (rb >> 4) + (un & bsh);
          floatx4 s = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < KCM; ++kc)
            if (kc < KC) {
              const bf16x8 av = (MB > 1 && mb == 1) ? Qreg[kc][MB - 1] : Qreg[kc][0];
              s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, kset[SET][x][kc]), s, 0, 0, 0);
            }
          const bool valid = tile0 + l16 < t_end;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = mb * 16 + 4 * g4 + r;
            if (row >= rb && row < rb + rph) sx[row * TP + l16] = valid ? a.scale * s[r] : -INFINITY;
          }
        }
      }
    } else {
      for (int idx = tid; idx < MR * T; idx += NT) {
        const int row = idx / T, tt = idx % T;
        sx[row * TP + tt] = (tile0 + tt < t_end) ? 0.0f : -INFINITY;
      }
    }
  };

  // [B] online softmax over the tile; P to LDS (bf16 head + remainder) and,
  // as fp16, to P16 with the tile's reference in msub
  auto phase_b = [&](int tile0) {
    if (s_row < MR) {
      float s = -INFINITY;
      if (s_row < rows) {
        s = sx[s_row * TP + s_tt];
        float pw[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) pw[w] = spart[(w * MR + s_row) * TP + s_tt];
#pragma unroll
        for (int h = NW / 2; h >= 1; h /= 2)
#pragma unroll
          for (int w = 0; w < h; ++w) pw[w] += pw[w + h];
        s += pw[0];
      }
      float c = 1.0f;
      if (__any(s > m_run + kLazyMax)) {
        const float m_tile = row16_max(s);
        if (m_tile > m_run + kLazyMax) {
          c = (m_run == -INFINITY) ? 0.0f : __expf(m_run - m_tile);
          m_run = m_tile;
          l_run *= c;
        }
      }
      const float p = (s == -INFINITY) ? 0.0f : __expf(s - m_run);
      l_run += p;
      const int o = s_row * TP + s_tt;
      const uint16_t hb = bf16_rne(p);
      pbh[o] = hb;
      pbl[o] = bf16_rne(p - __uint_as_float(static_cast<uint32_t>(hb) << 16));
      if (s_tt == 0) corr[s_row] = c;
      if (s_row < rows && a.dc > 0) {  // pass 2's input (no pass 2 without compressible dims)
        const int off = tile0 - t_begin;
        const int tau = tile0 - S + s_tt;
        p_out[((tau >> 5) << 9) + (((tau >> 3) & 3) << 7) + (tau & 7)] = static_cast<_Float16>(p);
        if (s_tt == 0) m_out[off / T] = m_run;
      }
    }
  };

  // [C] rescale o_U of the rows whose reference moved, then o_U += P vx
  auto rescale = [&]() {
    float cr[MB][4];
    bool any = false;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        cr[mb][r] = corr[mb * 16 + 4 * g4 + r];
        any = any || cr[mb][r] != 1.0f;
      }
    if (__any(any)) {
#pragma unroll
      for (int x = 0; x < XU; ++x) {
        const int q = wave + NW * x;
        const int qu = q / max(ndb, 1);
        const int rb = (rows >= a.G) ? (qu >> bsh) * a.G : 0;
        const int mbx = (rb >> 4) + (qu & bsh);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          if (mbx == mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) Uacc[x][r] *= cr[mb][r];
      }
    }
  };
  auto values_u = [&](int buf) {
    const uint16_t* vbuf = vxs + buf * nheads * T * DUS;
#pragma unroll
    for (int x = 0; x < XU; ++x) {
      const int q = wave + NW * x;
      if (ndb == 0 || q >= nunit * ndb) continue;
      const int hh = (q / ndb) >> bsh, db = q % ndb;
      const int rb = (rows >= a.G) ? hh * a.G : 0;
      const int mb = (rb >> 4) + ((q / ndb) & bsh);
      const uint16_t* vbase = vbuf + hh * T * DUS + db * 16 + 4 * (l16 & 3);
      const short4v bv = lds_read_tr4(vbase + (4 * g4 + (l16 >> 2)) * DUS);
      const short4v ph4 = *reinterpret_cast<const short4v*>(pbh + (mb * 16 + l16) * TP + 4 * g4);
      const short4v pl4 = *reinterpret_cast<const short4v*>(pbl + (mb * 16 + l16) * TP + 4 * g4);
      Uacc[x] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph4, bv, Uacc[x], 0, 0, 0);
      Uacc[x] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl4, bv, Uacc[x], 0, 0, 0);
    }
  };

  // ---- pipeline: [A](0) | { [B](i) | [C](i) with [A](i+1) } ...
  // Tile j's loads sit in set j % DEPTH and are issued DEPTH tiles ahead of
  // their use (clamped to the last tile near the end).  Every prologue load
  // completes here, so that no wait inside the loop (for A, q or the first
  // tile) also waits for the loop's own prefetches.
  __builtin_amdgcn_s_waitcnt(0);
  const int ntiles = (t_end - t_begin + T - 1) / T;
  const int last_tile = t_begin + max(ntiles - 1, 0) * T;
  auto prefetch = [&](int tile, auto set_c) __attribute__((always_inline)) {
    if (du8 > 0) {
      prefetch_k(min(tile, last_tile), set_c);
      prefetch_v(min(tile, last_tile), set_c);
    }
  };
  if constexpr (DEPTH > 1) prefetch(t_begin + T, kSet1());
  if (du8 > 0) stage_v(0, kSet0());
  exact_a(t_begin, kSet0());
  prefetch(t_begin + DEPTH * T, kSet0());
  scores_a(t_begin);
  __syncthreads();
  // one iteration: finish tile i, prepare tile i + 1 (from set set_c, a
  // compile-time index), and refill that set with tile i + 1 + DEPTH
  auto step = [&](int i, auto set_c) __attribute__((always_inline)) {
    const int tile0 = t_begin + i * T;
    phase_b(tile0);
    __syncthreads();
    rescale();
    if (du8 > 0) stage_v((i + 1) & 1, set_c);
    values_u(i & 1);
    exact_a(tile0 + T, set_c);
    prefetch(tile0 + (1 + DEPTH) * T, set_c);
    scores_a(tile0 + T);
    __syncthreads();
  };
  if constexpr (DEPTH > 1) {
    // both halves in every iteration and a separate last odd step
    int i = 0;
    for (; i + 2 < ntiles; i += 2) {
      step(i, kSet1());
      step(i + 1, kSet0());
    }
    if (i + 1 < ntiles) step(i, kSet1());
  } else {
    for (int i = 0; i + 1 < ntiles; ++i) step(i, kSet0());
  }
  if (ntiles > 0) {
    phase_b(t_begin + (ntiles - 1) * T);
    __syncthreads();
    rescale();
    values_u((ntiles - 1) & 1);
  }

  // ================= partials: m, l, o_U
  const int64_t prow = static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(qi0) * ns + sp;
  if (s_row < MR) {
    const float l_row = row16_sum(l_run);
    if (s_row < rows && s_tt == 0) {
      float* P = a.part + (prow + static_cast<int64_t>(s_row) * ns) * a.RS;
      P[0] = m_run;
      P[1] = l_row;
    }
  }
#pragma unroll
  for (int x = 0; x < XU; ++x) {
    const int q = wave + NW * x;
    if (ndb == 0 || q >= nunit * ndb) continue;
    const int hh = (q / ndb) >> bsh, db = q % ndb;
    const int rb = (rows >= a.G) ? hh * a.G : 0;
    const int mb = (rb >> 4) + ((q / ndb) & bsh);
    const int d = db * 16 + l16;
    if (d >= du) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mb * 16 + 4 * g4 + r;
      if (row >= rb && row < rb + rph)
        a.part[(prow + static_cast<int64_t>(row) * ns) * a.RS + 2 + d] = Uacc[x][r];
    }
  }
}

template <int MB, int MAXU, int PF, int XP, int XU, int KCM, int DEPTH>
hipError_t launch_score_one(const DecodeArgs& a, int nitems, size_t smem, hipStream_t s) {
  auto k = decode_score_kernel<MB, 8, MAXU, PF, XP, XU, KCM, DEPTH>;
  if (smem > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(smem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(nitems), dim3(512), smem, s, a);
  return hipGetLastError();
}

// Compiled pass-1 variants; the first that fits is taken.
constexpr ScoreVariant kScoreVariants[] = {
    // mb maxu pf xp xu kcm kpp_max (variants 0-1: two tiles of loads in flight,
    // the others one)
    {2, 5, 2, 1, 4, 2, 1280},   // 32 rows of up to 8 KV heads, exact dims <= 64
    {2, 9, 2, 1, 4, 2, 2304},
    {2, 5, 4, 1, 8, 4, 1280},   // exact dims <= 128
    {2, 9, 4, 1, 8, 4, 2304},
    {1, 9, 4, 1, 8, 4, 2304},   // 8 or 16 rows of up to 8 KV heads, exact dims <= 128
    {1, 17, 4, 1, 8, 4, 4352},  // k up to 4351
};

// ============================================================== pass 2 ====
constexpr int kMomentRun = 16;  // 64-token blocks between restarts of the moment recurrence
// MB: 16-row blocks; NGW: max frequency groups (of 16) per item.  Two
// blocks per CU, as the planner's rounds assume: the bound keeps the kernel
// within 256 registers (two waves per SIMD); with NGW = 3 both state sets of
// the moment recurrence, the table and two sets of P fit in them.
template <int MB, int NGW>
__global__ __launch_bounds__(64 * kMomentWaves, 2) void decode_moment_kernel(DecodeArgs a) {
  constexpr int NW = kMomentWaves, MR = 16 * MB, TT = kMomentTile;
  constexpr int TB = 64;  // tokens per block of the rotating frame
  extern __shared__ __attribute__((aligned(16))) float red[];  // [NW][NGW][2][MR][16], then mg[MR]
  float* mg = red + NW * NGW * 2 * MR * 16;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  // XCD-aware order: consecutive items (the slices of one split group) run on
  // the same XCD, whose L2 then serves their common P
  const int per = (a.nitems2 + 7) / 8;
  const int item = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (item >= a.nitems2) return;  // whole block
  int b = 0;
  while (b + 1 < a.nseq && item >= a.item2_0[b + 1]) ++b;
  const int local = item - a.item2_0[b];
  const int ns = a.seq.nsplit[b];
  const int nsm = ns - a.edge_split;
  const int nsg = (nsm + NW - 1) / NW;
  const int sigma = local % a.nslices;
  const int rem = local / a.nslices;
  const int sg = rem % nsg, rg = rem / nsg;
  const int M = a.seq.mid[b], period = a.seq.per[b], chunk = a.seq.chunk[b];
  const int mpad = (M + TT - 1) & ~(TT - 1);
  const int m16 = (M + 15) & ~15;
  const int rows = a.rows, qi0 = rg * rows;
  const int gbeg = (a.ngr * sigma) / a.nslices;
  const int ng = (a.ngr * (sigma + 1)) / a.nslices - gbeg;  // <= NGW
  const int sidx = sg * NW + wave;  // this wave's pass-1 split
  const bool active = sidx < nsm;
  const int64_t prow = static_cast<int64_t>(a.prow0[b]) + static_cast<int64_t>(qi0) * ns;

  // The prologue's loads go out together and the basis table is generated
  // while they are in flight: the row maxima, this wave's split references,
  // the first tile references (whether any moved) and the first block's P.

  // maximum of every row over all its splits (the merge uses the same):
  // 64 * NW / MR threads per row, each with its splits' loads all in flight
  // before the first use (row and split indices clamped, so that every thread
  // loads), then a reduction over the row's lanes
  constexpr int TPR = 64 * NW / MR;  // threads per row (a power of two <= 64)
  constexpr int kLoads = 8;
  const int mrow = tid / TPR, mpart = tid % TPR;
  const float* mpr = a.part + (prow + static_cast<int64_t>(min(mrow, rows - 1)) * ns) * a.RS;
  float mv[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) mv[u] = mpr[static_cast<int64_t>(min(mpart + TPR * u, ns - 1)) * a.RS];
  // this wave's split: its final reference of the lane's output rows (C layout)
  float mfC[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = min(mb * 16 + 4 * g4 + r, rows - 1);
      mfC[mb][r] = a.part[(prow + static_cast<int64_t>(row) * ns + min(sidx, nsm - 1)) * a.RS];
    }

  // the two states of the moments' recurrence in the rotating frame (sets V
  // and S, whose roles alternate between blocks), then (in place in V) the
  // split's W; zero for a wave without a split
  floatx4 Vc[NGW][MB], Vs[NGW][MB], Sc[NGW][MB], Ss[NGW][MB];
#pragma unroll
  for (int j = 0; j < NGW; ++j)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      Vc[j][mb] = Vs[j][mb] = Sc[j][mb] = Ss[j][mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // the split's tokens and P operand (set and used by active waves only):
  // lane (row mb*16 + l16, tokens block + 32 kp + 8 g4 .. +7), one contiguous
  // KB per (16-row block, 32 tokens); rows past the group (never stored) are
  // zeroed after the load, blocks past the split read its last block (never
  // used)
  const int tau_beg = sidx * chunk, tau_end = min(M, tau_beg + chunk);
  const int nblk = (tau_end - tau_beg + TB - 1) / TB;
  const _Float16* pbase =
      static_cast<const _Float16*>(a.P16) + static_cast<int64_t>(a.ngroups) * MB * 16 * a.pcum[b];
  const float* mbase = a.msub + a.hq * (a.pcum[b] / 16);
  int64_t poff[MB], moff[MB];
  bool row_ok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = qi0 + min(mb * 16 + l16, rows - 1);
    poff[mb] = p16_index(rg * MB + mb, l16, tau_beg + 8 * g4, mpad);
    moff[mb] = static_cast<int64_t>(r) * (mpad / 16);
    row_ok[mb] = mb * 16 + l16 < rows;
  }
  // the split's final reference of the lane's P rows (A layout), the
  // reference of the split's first tile, and block 0's P (three register sets
  // of P rotate between blocks below; block 0 is in pa)
  float mfA[MB], mfirst[MB];
  uint4 pa[MB][2], pb[MB][2], pq[MB][2];
  if (active) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = min(mb * 16 + l16, rows - 1);
      mfA[mb] = a.part[(prow + static_cast<int64_t>(r) * ns + sidx) * a.RS];
      mfirst[mb] = mbase[moff[mb] + tau_beg / 16];
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) pa[mb][kp] = *reinterpret_cast<const uint4*>(pbase + poff[mb] + kp * 512);
    }
  }

  // Fixed basis table of the lane's frequencies f = 16 (gbeg + j) + l16 at
  // the block offsets t = 32 kp + 8 g4 + e (the B operand layout), fp16 and
  // negated (the MFMAs subtract U from a state), and e^{i theta_f TB}, the
  // frame's turn from one block to the next
  const float inv_period = 1.0f / static_cast<float>(period);
  half8 Ec[NGW][2], Es[NGW][2];
  float rc[NGW], rs[NGW], c2[NGW];
  if (active) {
#pragma unroll
    for (int j = 0; j < NGW; ++j) {
      if (j >= ng) break;  // uniform: groups past the item's are never used
      // integer phases f t mod period: f < 2^13 and t < 64 keep every product in
      // 32 bits; consecutive offsets add f mod period
      const int f = 16 * (gbeg + j) + l16;
      const int fm = f % period;
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        int ph = (f * (32 * kp + 8 * g4)) % period;
        uint32_t pc[4], ps[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float x0 = static_cast<float>(ph) * inv_period;
          ph = add_mod(ph, fm, period);
          const float x1 = static_cast<float>(ph) * inv_period;
          ph = add_mod(ph, fm, period);
          pc[e2] = pack_f16(-cos_rev(x0), -cos_rev(x1));
          ps[e2] = pack_f16(-sin_rev(x0), -sin_rev(x1));
        }
        Ec[j][kp] = __builtin_bit_cast(half8, make_uint4(pc[0], pc[1], pc[2], pc[3]));
        Es[j][kp] = __builtin_bit_cast(half8, make_uint4(ps[0], ps[1], ps[2], ps[3]));
      }
      const float xr = static_cast<float>((f * TB) % period) * inv_period;
      rc[j] = cos_rev(xr);
      rs[j] = sin_rev(xr);
      c2[j] = 2.0f * rc[j];
    }
  }

  // the row maxima (splits past the first kLoads per thread in further rounds)
  {
    float m = -INFINITY;
    if (mrow < rows) {
#pragma unroll
      for (int u = 0; u < kLoads; ++u) m = fmaxf(m, mv[u]);
      for (int j0 = mpart + TPR * kLoads; j0 < ns; j0 += TPR * kLoads) {
        float v[kLoads];
#pragma unroll
        for (int u = 0; u < kLoads; ++u) v[u] = mpr[static_cast<int64_t>(min(j0 + TPR * u, ns - 1)) * a.RS];
#pragma unroll
        for (int u = 0; u < kLoads; ++u) m = fmaxf(m, v[u]);
      }
    }
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (mpart == 0) mg[mrow] = m;
  }
  __syncthreads();

  if (active) {
    // References only grow inside a pass-1 split, so a row whose first tile
    // already has the split's final reference kept it throughout: when that
    // holds for every row of the wave, no tile needs rescaling and the
    // per-tile references are not read at all
    bool moved_any;
    {
      bool mv_any = false;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) mv_any = mv_any || mfirst[mb] != mfA[mb];
      moved_any = __any(mv_any);
    }
    // the references of the lane's 16-token tiles of block t (a split whose
    // reference moved) and block t's P operand
    auto load_m = [&](float (&mn)[MB][2], int t) {
      const int tt = min(t, nblk - 1) * TB;
      if (moved_any) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) {
            const int tau = tau_beg + tt + 32 * kp + 8 * g4;
            mn[mb][kp] = mbase[moff[mb] + min(tau, m16 - 16) / 16];
          }
      }
    };
    auto load_p = [&](uint4 (&pn)[MB][2], int t) {
      const int tt = min(t, nblk - 1) * TB;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
          pn[mb][kp] = *reinterpret_cast<const uint4*>(pbase + poff[mb] + (tt / 32 + kp) * 512);
    };
    // Block t of the split: U_t = sum_{i < TB} P[tau_t + i] e^{i theta_f i}
    // (complex per row and frequency; cosine and sine parts), and the frame
    // sum V_t = U_t + e^{-i theta_f TB} V_{t-1} through the second-order
    // recurrence s_t = U_t + 2 cos(theta_f TB) s_{t-1} - s_{t-2} on each real
    // part (s_{-1} = s_{-2} = 0), whose output is V_t = s_t - e^{i theta_f TB}
    // s_{t-1}: one FMA per accumulator per block instead of a complex
    // rotation.  D holds s_{t-2} and becomes s_t; O holds s_{t-1}.
    auto block = [&](int t, const uint4 (&pc)[MB][2], floatx4 (&Dc)[NGW][MB], floatx4 (&Ds)[NGW][MB],
                     const floatx4 (&Oc)[NGW][MB], const floatx4 (&Os)[NGW][MB]) {
      const int tau0 = tau_beg + t * TB;
      half8 P[MB][2];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) P[mb][kp] = __builtin_bit_cast(half8, pc[mb][kp]);
      // rows past the group hold no probabilities
      if (rows < MR) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int kp = 0; kp < 2; ++kp)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (!row_ok[mb]) P[mb][kp][e] = 0;
      }
      // tokens past the last written 16-token tile hold no probabilities
      if (tau0 + TB > m16) {
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
          if (tau0 + 32 * kp + 8 * g4 >= m16)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
              for (int e = 0; e < 8; ++e) P[mb][kp][e] = 0;
      }
      // 16-token tiles whose reference moved later in their split: rescale
      // (their references read here, when needed: rare with the lazy reference)
      if (moved_any) {
        float ms[MB][2];
        load_m(ms, t);
        float fs[MB][2];
        bool moved = false;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) {
            fs[mb][kp] = 1.0f;
            if (tau0 + 32 * kp + 8 * g4 < m16 && ms[mb][kp] != mfA[mb]) {
              fs[mb][kp] = __expf(ms[mb][kp] - mfA[mb]);
              moved = true;
            }
          }
        if (__any(moved)) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int kp = 0; kp < 2; ++kp)
#pragma unroll
              for (int e = 0; e < 8; ++e)
                P[mb][kp][e] = static_cast<_Float16>(static_cast<float>(P[mb][kp][e]) * fs[mb][kp]);
        }
      }
#pragma unroll
      for (int j = 0; j < NGW; ++j) {
        if (j < ng) {
          // D = s_{t-2} - U_t (the table is negated)
#pragma unroll
          for (int kp = 0; kp < 2; ++kp)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              Dc[j][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P[mb][kp], Ec[j][kp], Dc[j][mb], 0, 0, 0);
              Ds[j][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P[mb][kp], Es[j][kp], Ds[j][mb], 0, 0, 0);
            }
          // s_t = 2 cos(theta_f TB) s_{t-1} - D
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              Dc[j][mb][r] = fmaf(c2[j], Oc[j][mb][r], -Dc[j][mb][r]);
              Ds[j][mb][r] = fmaf(c2[j], Os[j][mb][r], -Ds[j][mb][r]);
            }
        }
      }
    };
    // Out = L - e^{i theta_f TB} Q, the recurrence's output from its latest
    // state L and the one before, Q (elementwise, so Out may be L or Q)
    auto output = [&](const floatx4 (&Lc)[NGW][MB], const floatx4 (&Ls)[NGW][MB], const floatx4 (&Qc)[NGW][MB],
                      const floatx4 (&Qs)[NGW][MB], floatx4 (&Oc)[NGW][MB], floatx4 (&Os)[NGW][MB]) {
#pragma unroll
      for (int j = 0; j < NGW; ++j) {
        if (j >= ng) break;  // uniform
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float lc = Lc[j][mb][r], ls = Ls[j][mb][r], qc = Qc[j][mb][r], qs = Qs[j][mb][r];
            Oc[j][mb][r] = fmaf(rs[j], qs, fmaf(-rc[j], qc, lc));
            Os[j][mb][r] = fmaf(-rs[j], qc, fmaf(-rc[j], qs, ls));
          }
      }
    };
    // even blocks take s_t into V, odd blocks into S; every kMomentRun blocks
    // (after an odd block) the recurrence restarts from its output (S <- V_t,
    // V <- 0), which bounds the growth of its states (for theta_f TB near 0
    // or pi they grow with the square of the blocks since the start)
    // after an odd block t (S holds s_t): restart every kMomentRun blocks
    auto restart = [&](int t) {
      if (t + 1 < nblk && (t + 1) % kMomentRun == 0) {  // uniform
        output(Sc, Ss, Vc, Vs, Sc, Ss);
#pragma unroll
        for (int j = 0; j < NGW; ++j)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) Vc[j][mb] = Vs[j][mb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    };
    // P two blocks ahead in three register sets (block t in set t % 3; block
    // 0's is in pa already), six blocks per round so that the sets and the
    // state roles come back to their places
    load_p(pb, 1);
    for (int t = 0; t < nblk; t += 6) {
      load_p(pq, t + 2);
      block(t, pa, Vc, Vs, Sc, Ss);
      if (t + 1 >= nblk) break;  // uniform
      load_p(pa, t + 3);
      block(t + 1, pb, Sc, Ss, Vc, Vs);
      restart(t + 1);
      if (t + 2 >= nblk) break;
      load_p(pb, t + 4);
      block(t + 2, pq, Vc, Vs, Sc, Ss);
      if (t + 3 >= nblk) break;
      load_p(pq, t + 5);
      block(t + 3, pa, Sc, Ss, Vc, Vs);
      restart(t + 3);
      if (t + 4 >= nblk) break;
      load_p(pa, t + 6);
      block(t + 4, pb, Vc, Vs, Sc, Ss);
      if (t + 5 >= nblk) break;
      load_p(pb, t + 7);
      block(t + 5, pq, Sc, Ss, Vc, Vs);
      restart(t + 5);
    }
    // V_last into V
    if (nblk & 1)
      output(Vc, Vs, Sc, Ss, Vc, Vs);
    else
      output(Sc, Ss, Vc, Vs, Vc, Vs);
    // back to absolute phases: W = e^{i theta_f tau_last} V (in place),
    // tau_last the start of the last block (exact integer phase)
    const int tau_last = tau_beg + (nblk - 1) * TB;
#pragma unroll
    for (int j = 0; j < NGW; ++j) {
      if (j >= ng) break;  // uniform: the other groups stay zero
      const int f = 16 * (gbeg + j) + l16;
      const float x = static_cast<float>(phase_mod(f, tau_last, period)) * inv_period;
      const float cb = cos_rev(x), sb = sin_rev(x);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float vc = Vc[j][mb][r], vs = Vs[j][mb][r];
          Vc[j][mb][r] = fmaf(vc, cb, -vs * sb);
          Vs[j][mb][r] = fmaf(vc, sb, vs * cb);
        }
    }
    // relative to the row's maximum: W *= exp(m_split - m_row)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mb * 16 + 4 * g4 + r;
        const float f = row < rows ? __expf(mfC[mb][r] - mg[row]) : 0.0f;
#pragma unroll
        for (int j = 0; j < NGW; ++j) {
          Vc[j][mb][r] *= f;
          Vs[j][mb][r] *= f;
        }
      }
  }
  // the waves' W, summed in wave order
#pragma unroll
  for (int j = 0; j < NGW; ++j)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mb * 16 + 4 * g4 + r;
        red[(((wave * NGW + j) * 2 + 0) * MR + row) * 16 + l16] = Vc[j][mb][r];
        red[(((wave * NGW + j) * 2 + 1) * MR + row) * 16 + l16] = Vs[j][mb][r];
      }
  __syncthreads();
  // thread -> (row tid / 16 + 16 i, frequency lane tid % 16), over the groups
  // and cosines / sines (no index division)
  float* wout = a.Wp + (static_cast<int64_t>(a.sgcum[b] + sg) * a.hq + qi0) * a.kpad;
  const int fl = tid % 16;
  for (int row = tid / 16; row < rows; row += 64 * NW / 16)
    for (int j = 0; j < ng; ++j)
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) v += red[(((w * NGW + j) * 2 + cs) * MR + row) * 16 + fl];
        const int f = 16 * (gbeg + j) + fl;
        const int n = cs ? 2 * f : (f == 0 ? 0 : 2 * f - 1);
        if (n < a.k && !(cs && f == 0)) wout[static_cast<int64_t>(row) * a.kpad + n] = v;
      }
}

template <int MB, int NGW>
hipError_t launch_moment_one(const DecodeArgs& a, hipStream_t s) {
  auto k = decode_moment_kernel<MB, NGW>;
  const size_t smem = decode_moment_smem(MB, NGW);
  if (smem > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(smem));
    if (e != hipSuccess) return e;
  }
  // whole rounds of 8 blocks: the XCD-aware block -> item map is a bijection
  // of [0, 8 * ceil(items / 8)); blocks mapped past the last item return
  const int blocks = (a.nitems2 + 7) / 8 * 8;
  hipLaunchKernelGGL(k, dim3(blocks), dim3(64 * kMomentWaves), smem, s, a);
  return hipGetLastError();
}

}  // namespace

const ScoreVariant* decode_score_pick(int kpp, int mb, int nheads, int nunit, int du) {
  const int du32 = (du + 31) / 32 * 32;
  for (const ScoreVariant& v : kScoreVariants) {
    if (v.mb != mb || kpp > v.kpp_max || du32 > 32 * v.kcm) continue;
    const int U = kpp / 32;
    if ((U + 7) / 8 > v.maxu) continue;
    if (nunit > v.xp * 8 || nunit * (du32 / 16) > v.xu * 8 || nheads * kMfmaTile * (du / 8) > v.pf * 512)
      continue;
    return &v;
  }
  return nullptr;
}

size_t decode_score_smem(int mb, int nheads, int du) {
  return static_cast<size_t>(score_lds(mb, 8, nheads, du).total);
}

hipError_t launch_decode_score(const DecodeArgs& a, int nitems, hipStream_t s) {
  if (nitems == 0) return hipSuccess;
  const int nheads = a.rows >= a.G ? a.rows / a.G : 1;
  const int nunit = nheads * ((std::min(a.rows, a.G) + 15) / 16);
  const ScoreVariant* v = decode_score_pick(a.dc > 0 ? a.kpp : 0, a.mb, nheads, nunit, a.du);
  if (!v) return hipErrorInvalidValue;
  const size_t smem = decode_score_smem(a.mb, nheads, a.du);
  switch (v - kScoreVariants) {
    case 0: return launch_score_one<2, 5, 2, 1, 4, 2, 2>(a, nitems, smem, s);
    case 1: return launch_score_one<2, 9, 2, 1, 4, 2, 2>(a, nitems, smem, s);
    case 2: return launch_score_one<2, 5, 4, 1, 8, 4, 1>(a, nitems, smem, s);
    case 3: return launch_score_one<2, 9, 4, 1, 8, 4, 1>(a, nitems, smem, s);
    case 4: return launch_score_one<1, 9, 4, 1, 8, 4, 1>(a, nitems, smem, s);
    case 5: return launch_score_one<1, 17, 4, 1, 8, 4, 1>(a, nitems, smem, s);
  }
  return hipErrorInvalidValue;
}

int decode_moment_max_groups(int mb) { return mb > 1 ? 3 : 3; }

size_t decode_moment_smem(int mb, int ngw) {
  return sizeof(float) * (static_cast<size_t>(kMomentWaves) * ngw * 2 * 16 * mb * 16 + 16 * mb);
}

hipError_t launch_decode_moment(const DecodeArgs& a, hipStream_t s) {
  if (a.nitems2 == 0) return hipSuccess;
  if (a.mb > 1) return launch_moment_one<2, 3>(a, s);
  return launch_moment_one<1, 3>(a, s);
}

}  // namespace fa
