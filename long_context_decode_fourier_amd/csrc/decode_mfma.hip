// decode_mfma.hip - split-L decode step on MFMA for 16-bit caches.
//
// Same arithmetic as the VALU kernel in decode.hip (scores and values in
// coefficient space, online softmax, partials merged by decode_merge), laid out
// for CDNA4 matrix cores.  A work item is (sequence, group of up to 32
// consecutive query heads, range of middle tokens); its query rows are stacked
// into the 16-row M blocks of the MFMA.  Tiles hold 16 tokens.  The retained
// sink and recent tokens form one more split of every row, computed by
// decode_prep, so this kernel sees middle tokens only.
//
// Per tile:
//
// [A] basis and scores.  Every wave owns a slice of 32-wide coefficient units
//     and generates its slice of the basis tile directly as the MFMA operand
//     (lane = token, 8 consecutive pair-order positions = 4 frequencies): each
//     lane seeds e^{i f x}, e^{i x} and e^{i 16 x} from exact integer phases
//     (phases advance by 16 tokens per tile, so nothing drifts), builds its 4
//     frequencies by rotation and recurrence, and steps 16 frequencies per unit
//     with the three-term recurrence.  The wave's compressed score partials
//     S_c = A phi^T (fp16 MFMA, A = scale alpha q_C ck in registers) go to LDS,
//     and its basis slice is written to a wave-private LDS slice for [C].
//     Exact-dim scores q_U kx^T run on bf16 MFMA with kx loaded from HBM
//     straight into the operand layout (no LDS).
// [B] online softmax over the tile (one thread per row and token).  A row's
//     reference maximum moves only when a score exceeds it by more than
//     kLazyMax, so probabilities stay below e^kLazyMax (exact in value: m and
//     l share the reference) and the accumulators are rarely rescaled; the
//     sum l is kept per lane and reduced once at the end.  P goes to LDS as
//     fp16 (for W) and as a bf16 head plus remainder (for the exact values).
// [C] value moments W += P phi (fp16 MFMA, the wave's basis slice read back
//     transposed with ds_read_b64_tr_b16) and exact values o_U += P vx (bf16
//     MFMA, vx staged in a double-buffered LDS tile and read transposed).
//
// Two barriers per tile: after [A] and after [B].  The loop is rotated so that
// [C] of one tile and [A] of the next share a segment: the W and o_U MFMAs of
// tile i overlap the basis generation of tile i+1.
//
// Coefficients live in "pair order" inside the kernel: position 2j holds the
// cosine of frequency j (j = 0 is the constant), 2j+1 the sine; position 1 is
// unused (its basis value sin(0) is 0).  A is written in that order by
// decode_prep, W is converted back to the basis order when the partials are
// stored.
#include <type_traits>

#include "kernels.hpp"
#include "mfma_util.hpp"

namespace fa {
namespace {

using namespace mfma;

// MB: 16-row blocks; NW: waves; MAXU: max 32-wide coefficient units per wave;
// PF: 16-byte vx chunks staged per thread per tile; XP: max KV heads per wave
// (exact scores); XU: max (KV head, 16-dim block) exact-value tiles per wave.
template <int MB, int NW, int MAXU, int PF, int XP, int XU>
__global__ __launch_bounds__(64 * NW) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int T = kMfmaTile, TP = kMfmaTile + 4;
  constexpr int NT = 64 * NW, MR = 16 * MB;
  constexpr int KCM = 2;             // max 32-dim chunks of the exact dims
  constexpr int kNoChunk = 1 << 29;  // staging slot without a chunk
  static_assert(MR * T <= NT, "one softmax slot per thread");
  static_assert((NW & (NW - 1)) == 0, "power-of-two wave count (partial-score tree)");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g4 = lane >> 4, l16 = lane & 15;
  const int b = seq_of_item(a.seq, a.nseq, blockIdx.x);
  const int local = blockIdx.x - a.seq.item0[b];
  const int ns = a.seq.nsplit[b];  // middle splits + the edge split
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
  // 16-row blocks per KV head: 1 when a head's rows sit inside one block, 2
  // when one head's rows fill an item of more than 16 rows.  The exact-dim
  // work is cut into (KV head, row block) units u: head u / bph, block u % bph.
  const int bph = MB > 1 ? (rph + 15) >> 4 : 1;  // compile-time 1 for one-block items
  const int bsh = bph - 1;  // log2(bph): unit u is head u >> bsh, block u & bsh
  const int nunit = nheads * bph;
  const bool has_mid = a.dc > 0;  // items exist only for sequences with middle tokens
  const int du = a.du, dc = a.dc;
  const int du32 = (du + 31) & ~31;
  const int KC = du32 / 32;  // exact-dim chunks (<= KCM)
  const int ndb = du32 / 16;

  const MfmaLds lo = mfma_lds(MB, NW, a.kpp, nheads, du, dc);
  const int PS = lo.ps, DUS = lo.dus;
  _Float16* phi = reinterpret_cast<_Float16*>(smem + lo.phi);   // [T][PS]
  uint16_t* vxs = reinterpret_cast<uint16_t*>(smem + lo.vxs);   // [2][nheads][T][DUS]
  float* spart = reinterpret_cast<float*>(smem + lo.spart);     // [NW][MR][TP]
  float* sx = reinterpret_cast<float*>(smem + lo.sx);           // [MR][TP]
  _Float16* ph = reinterpret_cast<_Float16*>(smem + lo.ph);     // [MR][TP]
  uint16_t* pbh = reinterpret_cast<uint16_t*>(smem + lo.pbh);   // [MR][TP]
  uint16_t* pbl = reinterpret_cast<uint16_t*>(smem + lo.pbl);   // [MR][TP]
  float* corr = reinterpret_cast<float*>(smem + lo.corr);       // [MR]

  // ---- vx staging: thread -> 16-byte chunks c = tid + NT*i of a tile; the
  //      chunk -> (KV head, token, 8 dims) map is the same for every tile
  const int du8 = du / 8;
  const int nchunk = nheads * T * du8;
  int64_t st_src[PF];  // element offset of the chunk in the tile starting at t_begin
  int st_tt[PF];       // token within the tile (kNoChunk: no chunk)
  int st_lds[PF];      // LDS offset (elements) inside one vxs buffer
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
  uint4 pv[PF];
  auto prefetch_v = [&](int tile) {
    const int64_t shift = static_cast<int64_t>(tile - t_begin) * du;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (tile + st_tt[i] < t_end)
        v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.vx) + st_src[i] + shift);
      pv[i] = v;
    }
  };
  auto stage_v = [&](int buf) {
    uint16_t* dst = vxs + buf * nheads * T * DUS;
#pragma unroll
    for (int i = 0; i < PF; ++i)
      if (st_tt[i] != kNoChunk) *reinterpret_cast<uint4*>(dst + st_lds[i]) = pv[i];
  };

  // ---- kx as the B operand of the exact-score MFMA, loaded from HBM:
  //      lane -> (token l16, dims 32 kc + 8 g4 .. +7) of KV head wave + NW x
  int64_t kx_src[XP];
  uint4 kreg[XP][KCM];
#pragma unroll
  for (int x = 0; x < XP; ++x)
    kx_src[x] = (row0 + static_cast<int64_t>(h0 + ((wave + NW * x) >> bsh)) * L + t_begin + l16) * du + 8 * g4;
  auto prefetch_k = [&](int tile) {
    const int64_t shift = static_cast<int64_t>(tile - t_begin) * du;
    const bool tok_ok = tile + l16 < t_end;
#pragma unroll
    for (int x = 0; x < XP; ++x)
#pragma unroll
      for (int kc = 0; kc < KCM; ++kc) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (tok_ok && wave + NW * x < nunit && kc < KC && 32 * kc + 8 * g4 < du)
          v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.kx) + kx_src[x] + shift + 32 * kc);
        kreg[x][kc] = v;
      }
  };
  if (du8 > 0) {
    prefetch_k(t_begin);
    prefetch_v(t_begin);
  }

  // ---- q at the exact dims (permuted by decode_prep): bf16 MFMA A operand
  //      per 32-dim chunk
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
  floatx4 Uacc[XU];
#pragma unroll
  for (int x = 0; x < XU; ++x) Uacc[x] = floatx4{0.f, 0.f, 0.f, 0.f};

  // ---- softmax slot: thread -> (row, token); threads beyond MR * T idle
  const int s_row = tid / T, s_tt = tid % T;
  float m_run = -INFINITY, l_run = 0.0f;

  // ---- basis generator: lane -> token l16 of the tile and frequencies
  //      16 u + 4 g4 + j (j < 4) of its wave's units.  Integer phases (mod per)
  //      of tau, 16 tau and f0 tau (f0 = 16 u0 + 4 g4) for this lane's token,
  //      advanced by 16 tokens per tile.
  const float inv_per = has_mid ? 1.0f / static_cast<float>(per) : 0.0f;
  const int f0 = 16 * u0 + 4 * g4;
  int ph_tau = 0, ph_16 = 0, ph_f0 = 0, inc_tau = 0, inc_16 = 0, inc_f0 = 0;
  if (has_mid) {
    int tau0 = (t_begin + l16 - S) % per;
    if (tau0 < 0) tau0 += per;
    ph_tau = tau0;
    ph_16 = phase_mod(16, tau0, per);
    ph_f0 = phase_mod(f0, tau0, per);
    inc_tau = T % per;
    inc_16 = phase_mod(16, T, per);
    inc_f0 = phase_mod(f0, T, per);
  }

  // ============================================ [C] value moments + [A] basis
  // One pass over this wave's units does, per unit, the value-moment MFMAs of
  // the previous tile (do_w: W += P phi, phi read back transposed) and then
  // the basis, score MFMA and LDS store of tile tile0 (do_a).  The transposed
  // reads of a unit precede its stores in program order, so one basis buffer
  // serves both tiles, and the basis VALU work of one tile interleaves with
  // the MFMA and LDS work of the other.
  // do_w / do_a are compile-time flags (std::integral_constant), so that the
  // unit loop holds no branch on them
  auto fused = [&](auto do_w_c, auto do_a_c, int tile0) {
    constexpr bool do_w = decltype(do_w_c)::value;
    constexpr bool do_a = decltype(do_a_c)::value;
    if (has_mid) {
      half4 pv4[MB];
      if (do_w) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) pv4[mb] = *reinterpret_cast<const half4*>(ph + (mb * 16 + l16) * TP + 4 * g4);
      }
      const bool mid = do_a && tile0 + l16 < t_end;
      // seeds of this lane's token: e^{i f0 x}, e^{i x}, e^{i 16 x}, x = 2 pi tau / per
      const float x0 = static_cast<float>(ph_f0) * inv_per;
      const float x1 = static_cast<float>(ph_tau) * inv_per;
      const float x16 = static_cast<float>(ph_16) * inv_per;
      // a lane whose token is not a middle token seeds zeros: all its values are 0
      const float c0 = mid ? cos_rev(x0) : 0.0f, s0 = mid ? sin_rev(x0) : 0.0f;
      const float c1 = cos_rev(x1), s1 = sin_rev(x1);
      const float c16 = cos_rev(x16), s16 = sin_rev(x16);
      const float tc1 = 2.0f * c1, tc16 = 2.0f * c16;
      // two register sets alternate between even and odd units
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
      _Float16* dst = phi + l16 * PS + u0 * 32 + 8 * g4;
      // W operands of the previous tile, read one unit ahead so that the LDS
      // latency overlaps a unit's basis arithmetic (a unit's slot is
      // overwritten only after its reads; the read past the last unit repeats
      // the last unit, which keeps it unconditional)
      const _Float16* wsrc = phi + (4 * g4 + (l16 >> 2)) * PS + u0 * 32 + 4 * (l16 & 3);
      half4 bw[2][2];
      if (do_w) {
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2) bw[0][n2] = __builtin_bit_cast(half4, lds_read_tr4(wsrc + n2 * 16));
      }
#pragma unroll
      for (int u = 0; u < MAXU; ++u) {
        if (u < nu) {
          if (do_w) {
#pragma unroll
            for (int n2 = 0; n2 < 2; ++n2)
#pragma unroll
              for (int mb = 0; mb < MB; ++mb)
                Wacc[u][n2][mb] = __builtin_amdgcn_mfma_f32_16x16x16f16(pv4[mb], bw[u & 1][n2], Wacc[u][n2][mb], 0, 0, 0);
            if (u + 1 < MAXU) {
              const int un = min(u + 1, nu - 1);
#pragma unroll
              for (int n2 = 0; n2 < 2; ++n2)
                bw[(u + 1) & 1][n2] = __builtin_bit_cast(half4, lds_read_tr4(wsrc + un * 32 + n2 * 16));
            }
          }
          if (!do_a) continue;
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
          *reinterpret_cast<uint4*>(dst + 32 * u) = bits;
        }
      }
      if (do_a) {
        // this wave's partial scores: lane -> token l16, rows 4 g4 + r
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) spart[(wave * MR + mb * 16 + 4 * g4 + r) * TP + l16] = sacc[mb][r];
        ph_tau = add_mod(ph_tau, inc_tau, per);
        ph_16 = add_mod(ph_16, inc_16, per);
        ph_f0 = add_mod(ph_f0, inc_f0, per);
      }
    }
  };

  // exact-dim scores of tile tile0 (kx prefetched one segment earlier), then
  // the loads of the next tile: issued first in their segment, so that the
  // MFMA and load latencies overlap the long basis pass
  auto exact_a = [&](int tile0) {
    // exact-dim scores of this wave's KV heads
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
              s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, kreg[x][kc]), s, 0, 0, 0);
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
      // no exact dims: every row's exact part is 0 (or -inf past the end)
      for (int idx = tid; idx < MR * T; idx += NT) {
        const int row = idx / T, tt = idx % T;
        sx[row * TP + tt] = (tile0 + tt < t_end) ? 0.0f : -INFINITY;
      }
    }
    // next tile's kx and vx: issued last, so that no wait above covers them
    if (du8 > 0 && tile0 + T < t_end) {
      prefetch_k(tile0 + T);
      prefetch_v(tile0 + T);
    }
  };

  // =================================================================== [B]
  auto phase_b = [&]() {
    if (s_row < MR) {  // whole waves (MR * T is a multiple of 64)
      float s = -INFINITY;
      if (s_row < rows) {
        // all reads issued before the first use; the partials of a token past
        // the end are 0, so its -inf exact score passes through the sum
        const float e = sx[s_row * TP + s_tt];
        s = e;
        if (has_mid) {
          float pw[NW];
#pragma unroll
          for (int w = 0; w < NW; ++w) pw[w] = spart[(w * MR + s_row) * TP + s_tt];
#pragma unroll
          for (int h = NW / 2; h >= 1; h /= 2)
#pragma unroll
            for (int w = 0; w < h; ++w) pw[w] += pw[w + h];
          s += pw[0];
        }
      }
      float c = 1.0f;
      if (__any(s > m_run + kLazyMax)) {  // some row of this wave moves its reference
        const float m_tile = row16_max(s);
        if (m_tile > m_run + kLazyMax) {
          c = (m_run == -INFINITY) ? 0.0f : __expf(m_run - m_tile);
          m_run = m_tile;
          l_run *= c;
        }
      }
      const float p = (s == -INFINITY) ? 0.0f : __expf(s - m_run);
      l_run += p;  // this lane's share of the row sum
      const int o = s_row * TP + s_tt;
      ph[o] = static_cast<_Float16>(p);
      const uint16_t hb = bf16_rne(p);
      pbh[o] = hb;
      pbl[o] = bf16_rne(p - __uint_as_float(static_cast<uint32_t>(hb) << 16));
      if (s_tt == 0) corr[s_row] = c;
    }
  };

  // =================================================================== [C]
  // rescale the running sums of the rows whose reference moved (wave-uniform test)
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
      for (int mb = 0; mb < MB; ++mb) {
        if (has_mid) {
#pragma unroll
          for (int u = 0; u < MAXU; ++u)
#pragma unroll
            for (int n2 = 0; n2 < 2; ++n2)
#pragma unroll
              for (int r = 0; r < 4; ++r) Wacc[u][n2][mb][r] *= cr[mb][r];
        }
#pragma unroll
        for (int x = 0; x < XU; ++x) {
          const int q = wave + NW * x;
          const int qu = q / max(ndb, 1);  // (KV head, row block) unit
          const int rb = (rows >= a.G) ? (qu >> bsh) * a.G : 0;
          if ((rb >> 4) + (qu & bsh) == mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) Uacc[x][r] *= cr[mb][r];
        }
      }
    }
  };
  // exact values o_U += P vx of the tile staged in vxs[buf]
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

  // ---- pipeline: [A](0) | { [B](i) | [C](i) fused with [A](i+1) } ...
  // Every prologue load completes here, so that no wait inside the loop (for
  // A, q or the first tile) also waits for the loop's own prefetches.
  __builtin_amdgcn_s_waitcnt(0);
  const int ntiles = (t_end - t_begin + T - 1) / T;
  if (du8 > 0) stage_v(0);
  using kOn = std::integral_constant<bool, true>;
  using kOff = std::integral_constant<bool, false>;
  exact_a(t_begin);
  fused(kOff(), kOn(), t_begin);
  __syncthreads();
  // tiles 0 .. ntiles-2 also prepare the next tile; the last one only
  // finishes its own
  for (int i = 0; i + 1 < ntiles; ++i) {
    const int tile0 = t_begin + i * T;
    phase_b();
    __syncthreads();
    rescale();
    if (du8 > 0) stage_v((i + 1) & 1);
    values_u(i & 1);
    exact_a(tile0 + T);
    fused(kOn(), kOn(), tile0 + T);
    __syncthreads();
  }
  if (ntiles > 0) {
    phase_b();
    __syncthreads();
    rescale();
    values_u((ntiles - 1) & 1);
    fused(kOn(), kOff(), 0);
    __syncthreads();
  }

  // ================= partials
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

template <int MB, int NW, int MAXU, int PF, int XP, int XU>
hipError_t launch_one(const DecodeArgs& a, int nitems, size_t smem, hipStream_t s) {
  auto k = decode_mfma_kernel<MB, NW, MAXU, PF, XP, XU>;
  if (smem > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(smem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(nitems), dim3(64 * NW), smem, s, a);
  return hipGetLastError();
}

// Compiled variants, chosen by row blocks, basis length (pair-order
// positions kpp) and the item's KV heads: each wave's slice of A and W stays
// in registers.  The first variant that fits is taken, so leaner variants
// (fewer staging and exact-dim slots) come first.
constexpr MfmaVariant kVariants[] = {
    // mb nw maxu pf xp xu kpp_min kpp_max
    {1, 8, 2, 2, 1, 4, 0, 512},  // up to 8 KV heads of <= 64 exact dims
    {1, 8, 2, 4, 2, 8, 0, 512},
    {2, 8, 2, 2, 1, 4, 0, 512},
    {2, 8, 5, 1, 1, 2, 513, 1280},
    {1, 8, 5, 2, 2, 4, 513, 1280},
    {1, 8, 9, 1, 1, 2, 1281, 2304},
};

}  // namespace

// LDS carve-up shared by the kernel and the host-side size check.
__host__ __device__ MfmaLds mfma_lds(int mb, int nw, int kpp, int nheads, int du, int dc) {
  const int T = kMfmaTile, MR = 16 * mb, TP = kMfmaTile + 4;
  const int du32 = (du + 31) & ~31;
  MfmaLds o;
  int off = 0;
  auto take = [&off](int bytes) {
    const int r = off;
    off += (bytes + 15) & ~15;
    return r;
  };
  // basis-tile row stride = 80 (mod 128) halves = 8 (mod 32) dwords: the
  // 16-byte stores of 16 rows x 4 column chunks and the transposed 8-byte
  // reads of 4 rows x 4 chunks spread evenly over the LDS banks (strides of
  // 48, 80 and 112 mod 128 measure alike; 0 and 32 mod 128 conflict)
  o.ps = kpp + ((80 - kpp % 128) + 128) % 128;
  o.dus = du32 + 16;
  o.phi = take(T * o.ps * 2);
  o.vxs = take(du32 ? 2 * nheads * T * o.dus * 2 : 0);
  o.spart = take(nw * MR * TP * 4);
  o.sx = take(MR * TP * 4);
  o.ph = take(MR * TP * 2);
  o.pbh = take(MR * TP * 2);
  o.pbl = take(MR * TP * 2);
  o.corr = take(MR * 4);
  o.total = off;
  return o;
}

// The item's exact dims fit the variant's per-wave slots: KV heads for the
// exact scores, (KV head, 16-dim block) tiles for the exact values, 16-byte
// vx chunks staged per thread.
bool decode_mfma_fits(const MfmaVariant& v, int nheads, int nunit, int du) {
  const int du32 = (du + 31) / 32 * 32, nt = 64 * v.nw;
  return nunit <= v.xp * v.nw && nunit * (du32 / 16) <= v.xu * v.nw &&
         nheads * kMfmaTile * (du / 8) <= v.pf * nt;
}

const MfmaVariant* decode_mfma_pick(int kpp, int mb, int nheads, int nunit, int du) {
  for (const MfmaVariant& v : kVariants)
    if (v.mb == mb && kpp >= v.kpp_min && kpp <= v.kpp_max && decode_mfma_fits(v, nheads, nunit, du))
      return &v;
  return nullptr;
}

size_t decode_mfma_smem(const DecodeArgs& a, const MfmaVariant& v, int nheads) {
  return static_cast<size_t>(mfma_lds(v.mb, v.nw, a.kpp, nheads, a.du, a.dc).total);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int nitems, hipStream_t s) {
  if (nitems == 0) return hipSuccess;
  const int nheads = a.rows >= a.G ? a.rows / a.G : 1;
  const int nunit = nheads * ((std::min(a.rows, a.G) + 15) / 16);
  const MfmaVariant* v = decode_mfma_pick(a.kpp, a.mb, nheads, nunit, a.du);
  if (!v) return hipErrorInvalidValue;
  const size_t smem = decode_mfma_smem(a, *v, nheads);
  switch (v - kVariants) {
    case 0: return launch_one<1, 8, 2, 2, 1, 4>(a, nitems, smem, s);
    case 1: return launch_one<1, 8, 2, 4, 2, 8>(a, nitems, smem, s);
    case 2: return launch_one<2, 8, 2, 2, 1, 4>(a, nitems, smem, s);
    case 3: return launch_one<2, 8, 5, 1, 1, 2>(a, nitems, smem, s);
    case 4: return launch_one<1, 8, 5, 2, 2, 4>(a, nitems, smem, s);
    case 5: return launch_one<1, 8, 9, 1, 1, 2>(a, nitems, smem, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
