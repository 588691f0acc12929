// project.hip - prefill projection of the compressible dims of the middle
// tokens onto the real Fourier basis (skill page "fourier-approximated-kv-cache",
// Step 2; arXiv 2506.11886 abstract: projection onto orthogonal Fourier bases).
//
//   C[n][col] = sum_{tau < M} phi_n(tau) X[sink + tau][col]
//
// is a dense contraction over tau: per sequence, [k x M] basis times [M x cols]
// cache rows.  16-bit inputs run it on MFMA (v_mfma_f32_32x32x16_f16): the
// basis operand is generated in registers (never read from memory), the cache
// tile is staged through LDS, transposed so that each lane reads its 8
// consecutive positions with one 16-byte load.  Operands are fp16: bf16 inputs
// convert to fp16 exactly for |x| in [2^-14, 65504], and the unscaled cos/sin
// values in [-1, 1] keep 11 significant bits (bf16 would keep 8, which costs
// an order of magnitude in coefficient accuracy).  Accumulation is fp32.
// Two tilings: 256 x 128 tiles of 4-wave blocks, two per CU, for large
// contractions (project_f16_kernel: each wave owns 64 coefficient rows of all
// 128 columns, so every basis row is generated once per block) and tall
// 512 x 64 tiles for a small k (project_tall_kernel); long sequences are split
// over positions and the partial tiles summed in a fixed order by
// project_reduce_kernel.
//
// Basis values along a lane's run of 32 consecutive positions come from the
// three-term recurrence y(t+1) = 2 cos(theta) y(t) - y(t-1), seeded with two
// exact values from the integer phase (f*tau mod M) and the hardware sin unit;
// the run length bounds the recurrence's error growth (about 3e-5 absolute,
// a tenth of the fp16 rounding of the operand).
//
// fp32 inputs take a VALU kernel with correctly rounded phases (sincospi per
// value) and compensated summation, which keeps coefficients within 1e-5.
#include <algorithm>
#include <type_traits>

#include "kernels.hpp"

namespace fa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kLdsStride = kProjTT + 8;  // halves per LDS column (padding spreads banks)

struct ProjItem {
  int b, ktile, ctile, t_begin, t_end, M, per;  // M middle positions, per the basis period
  int slot;  // partial-tile slot: item0[b] + (ktile * nctiles + ctile) * nsplit + split
};

// XCD-aware schedule.  Blocks are dispatched round-robin over the 8 XCDs
// (block p runs on XCD p % 8), each with its own L2.  Items are numbered so
// that the coefficient tiles reading the same cache slice (same column tile
// and token range) are consecutive, and consecutive items go to the same XCD:
// block p takes item (p % 8) * per + p / 8.  Returns false for the few padding
// blocks of the last round.
constexpr int kXcds = 8;
__device__ inline bool proj_item(const ProjArgs& a, int nitems, int block, ProjItem* out) {
  const int per = (nitems + kXcds - 1) / kXcds;
  const int item = (block % kXcds) * per + block / kXcds;
  if (item >= nitems) return false;
  ProjItem it;
  it.b = seq_of_item(a.seq, a.nseq, item);
  const int local = item - a.seq.item0[it.b];
  const int ns = a.seq.nsplit[it.b];
  it.ktile = local % a.nktiles;                 // fastest: coefficient tiles of one slice
  const int group = local / a.nktiles;          // (column tile, split)
  it.ctile = group / ns;
  const int sp = group % ns;
  it.M = a.seq.mid[it.b];
  it.per = a.seq.per[it.b];
  it.t_begin = sp * a.seq.chunk[it.b];
  it.t_end = min(it.M, it.t_begin + a.seq.chunk[it.b]);
  it.slot = a.seq.item0[it.b] + (it.ktile * a.nctiles + it.ctile) * ns + sp;
  *out = it;
  return true;
}

// Wave grid WR x WC; each wave owns RB x CB blocks of 32 x 32 outputs.
//
// Cache tile staging: thread (cg, tg) loads 4 consecutive columns (8 bytes)
// of 8 consecutive positions, converts bf16 -> fp16 and packs each column's 8
// positions into one 16-byte LDS store.  LDS holds column-major blocks of 8
// positions with a 144-byte column stride; the block index is XOR-swizzled
// with (col >> 3) & 7, which keeps the stores (8 lanes, 8 column groups) and
// the MFMA operand reads (8 lanes, 8 consecutive columns) on distinct 16-byte
// bank slots.  The tile is double-buffered: the next step's loads are issued
// before the MFMA loop of the current step and stored to the other buffer
// after it, so one barrier per step suffices.
__device__ inline int xt_off(int col, int tblock) {
  return col * kLdsStride + ((tblock ^ ((col >> 3) & 7)) << 3);
}

template <int WR, int WC, int RB, int CB>
__global__ __launch_bounds__(64 * WR * WC, 2) void project_f16_kernel(ProjArgs a) {
  constexpr int kThreads = 64 * WR * WC;
  constexpr int TK = WR * RB * 32;
  constexpr int TN = WC * CB * 32;
  constexpr int kColGroups = TN / 4;
  constexpr int kPosGroups = kThreads / kColGroups;
  constexpr int NPG = kProjTT / (8 * kPosGroups);  // 8-position groups per thread
  static_assert(NPG >= 1 && NPG * kPosGroups * 8 == kProjTT, "the loader threads cover the step");

  __shared__ __attribute__((aligned(16))) _Float16 xts[2][TN * kLdsStride];

  ProjItem it;
  if (!proj_item(a, a.nitems, blockIdx.x, &it)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave / WC, wc = wave % WC;
  // a wave whose coefficient rows all lie past k (the padding of the last
  // k-tile) only loads and converts the cache tile
  const bool active = it.ktile * TK + wr * (RB * 32) < a.k;
  const int M = it.M, per = it.per;
  const int L = a.seq.len[it.b];
  const int64_t row0 = a.seq.row0[it.b];

  // ---- loader: 4 consecutive columns x NPG groups of 8 positions per thread
  //      (groups tg, tg + kPosGroups, ...)
  const int cg = tid % kColGroups, tg = tid / kColGroups;
  const int col0 = it.ctile * TN + cg * 4;
  const bool col_ok = col0 < a.ncols;  // Dc % 4 == 0: the 4 columns share (mat, h)
  const uint16_t* xbase = static_cast<const uint16_t*>(a.x[0]);
  if (col_ok) {
    const int blk = col0 / a.dc, c0 = col0 % a.dc;
    const int mat = blk / a.hkv, h = blk % a.hkv;
    xbase = static_cast<const uint16_t*>(mat ? a.x[1] : a.x[0]) +
            (row0 + static_cast<int64_t>(h) * L + a.sink) * a.dc + c0;
  }
  uint2 raw[NPG][8];

  // ---- basis generator state, one coefficient row per lane and row block
  const float inv_per = 1.0f / static_cast<float>(per);
  float c2[RB], off[RB];
  int fr[RB], ph[RB], d64[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int n = it.ktile * TK + wr * (RB * 32) + rb * 32 + (lane & 31);
    const int ne = min(n, a.k - 1);
    const int f = basis_freq(ne) % per;
    float s, c;
    sincos_phase(f, per, &s, &c);
    c2[rb] = 2.0f * c;
    off[rb] = basis_is_cos(ne) ? 0.25f : 0.0f;  // cos(2 pi x) = sin(2 pi (x + 1/4))
    fr[rb] = f;
    ph[rb] = phase_mod(f, it.t_begin + 32 * (lane >> 5), per);
    d64[rb] = phase_mod(f, kProjTT, per);
  }

  floatx16 acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.0f;

  auto load_raw = [&](int step) {
#pragma unroll
    for (int j = 0; j < NPG; ++j) {
      const int p0 = step + (tg + kPosGroups * j) * 8;
      const uint16_t* src = xbase + static_cast<int64_t>(p0) * a.dc;
      if (col_ok && step + kProjTT <= it.t_end) {  // full step: no per-position test
#pragma unroll
        for (int i = 0; i < 8; ++i) raw[j][i] = *reinterpret_cast<const uint2*>(src + static_cast<int64_t>(i) * a.dc);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          raw[j][i] = (col_ok && p0 + i < it.t_end)
                          ? *reinterpret_cast<const uint2*>(src + static_cast<int64_t>(i) * a.dc)
                          : make_uint2(0u, 0u);
      }
    }
  };
  auto store_raw = [&](_Float16* xt) {
    // bf16 -> fp32 -> fp16 (exact for |x| in [2^-14, 65504]), one column of 8
    // positions per 16-byte store
#pragma unroll
    for (int j = 0; j < NPG; ++j) {
      uint4 c[4];
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const uint2 r0 = raw[j][i], r1 = raw[j][i + 1];
        const float a0 = __uint_as_float(r0.x << 16), a1 = __uint_as_float(r1.x << 16);
        const float b0 = __uint_as_float(r0.x & 0xFFFF0000u), b1 = __uint_as_float(r1.x & 0xFFFF0000u);
        const float c0 = __uint_as_float(r0.y << 16), c1 = __uint_as_float(r1.y << 16);
        const float d0 = __uint_as_float(r0.y & 0xFFFF0000u), d1 = __uint_as_float(r1.y & 0xFFFF0000u);
        (&c[0].x)[i / 2] = pack_f16(a0, a1);
        (&c[1].x)[i / 2] = pack_f16(b0, b1);
        (&c[2].x)[i / 2] = pack_f16(c0, c1);
        (&c[3].x)[i / 2] = pack_f16(d0, d1);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint4*>(&xt[xt_off(cg * 4 + q, tg + kPosGroups * j)]) = c[q];
    }
  };

  load_raw(it.t_begin);
  store_raw(xts[0]);
  __syncthreads();
  int buf = 0;
  for (int step = it.t_begin; step < it.t_end; step += kProjTT) {
    const bool more = step + kProjTT < it.t_end;
    if (more) load_raw(step + kProjTT);
    const _Float16* xt = xts[buf];
    auto read_b = [&](int s, half8* bv) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        bv[cb] = *reinterpret_cast<const half8*>(
            &xt[xt_off(wc * (CB * 32) + cb * 32 + (lane & 31), 4 * (lane >> 5) + s)]);
    };
    // basis operand of sub-step s (16 positions): lane -> coefficient row,
    // 8 consecutive positions (lane half h covers positions 32 h + 8 s ..
    // +7 of the step, so its 4 sub-steps are one run of 32 positions, seeded
    // from exact phases at sub-step 0 and continued by the recurrence)
    float yp[RB], yc[RB];
    auto gen_a = [&](int s, half8* av) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float v[8];
        if (s == 0) {
          const int r0 = ph[rb];
          int r1 = r0 + fr[rb];
          if (r1 >= per) r1 -= per;
          v[0] = sin_rev(fmaf(static_cast<float>(r0), inv_per, off[rb]));
          v[1] = sin_rev(fmaf(static_cast<float>(r1), inv_per, off[rb]));
#pragma unroll
          for (int e = 2; e < 8; ++e) v[e] = fmaf(c2[rb], v[e - 1], -v[e - 2]);
        } else {
          v[0] = fmaf(c2[rb], yc[rb], -yp[rb]);
          v[1] = fmaf(c2[rb], v[0], -yc[rb]);
#pragma unroll
          for (int e = 2; e < 8; ++e) v[e] = fmaf(c2[rb], v[e - 1], -v[e - 2]);
        }
        yp[rb] = v[6];
        yc[rb] = v[7];
        const uint4 bits = make_uint4(pack_f16(v[0], v[1]), pack_f16(v[2], v[3]),
                                      pack_f16(v[4], v[5]), pack_f16(v[6], v[7]));
        av[rb] = __builtin_bit_cast(half8, bits);
      }
    };
    // software pipeline over the 4 sub-steps: the operands of sub-step s+1
    // (LDS reads, basis VALU) are produced while sub-step s's MFMAs run
    if (active) {
      half8 bcur[CB], bnxt[CB], acur[RB], anxt[RB];
      read_b(0, bcur);
      gen_a(0, acur);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s < 3) {
          read_b(s + 1, bnxt);
          gen_a(s + 1, anxt);
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(acur[rb], bcur[cb], acc[rb][cb], 0, 0, 0);
        if (s < 3) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) bcur[cb] = bnxt[cb];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) acur[rb] = anxt[rb];
        }
      }
    }
    // the next step's tile goes to the other buffer (last read in the
    // previous step, before its barrier) after this step's MFMAs, so that its
    // loads have the whole step to arrive; after the last step the store
    // repeats data nobody reads.  The raw rows pass through an empty asm
    // statement here, which keeps their conversion (and the wait for their
    // loads) at the end of the step: hoisted into the early sub-steps, it
    // would wait for loads issued moments before.
#pragma unroll
    for (int j = 0; j < NPG; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(raw[j][i].x), "+v"(raw[j][i].y));
    store_raw(xts[buf ^ 1]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      ph[rb] += d64[rb];
      if (ph[rb] >= per) ph[rb] -= per;
    }
    __syncthreads();
    buf ^= 1;
  }

  if (a.direct) {
    // single split: scale by the basis normalisation and scatter to ck / cv
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = it.ktile * TK + wr * (RB * 32) + rb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = it.ctile * TN + wc * (CB * 32) + cb * 32 + (lane & 31);
          if (n < a.k && col < a.ncols) {
            const int f = basis_freq(n);
            const float alpha = (f == 0 || 2 * f == per) ? 1.0f / sqrtf(static_cast<float>(per))
                                                       : sqrtf(2.0f / static_cast<float>(per));
            const int blk = col / a.dc, c = col % a.dc, mat = blk / a.hkv, h = blk % a.hkv;
            (mat ? a.out[1] : a.out[0])[((static_cast<int64_t>(it.b) * a.hkv + h) * a.k + n) * a.dc + c] = alpha * acc[rb][cb][r];
          }
        }
    return;
  }
  float* P = a.partial + static_cast<int64_t>(it.slot) * TK * TN;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int nl = wr * (RB * 32) + rb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int cl = wc * (CB * 32) + cb * 32 + (lane & 31);
        if (it.ktile * TK + nl < a.k) P[nl * TN + cl] = acc[rb][cb][r];  // the reduce reads rows < k only
      }
}

// Tall tiles for few coefficients: the 8 waves of a block are stacked along
// the coefficient rows (wave w owns rows 64 w .. 64 w + 63 of a 512-row tile)
// and share one cache tile of 64 columns, so each cache value is loaded and
// converted once per block and each basis row is generated by one wave.  A
// block per CU; to keep enough bytes in flight for HBM, the cache rows are
// prefetched D steps ahead into registers.  Every load is unconditional (a
// position past the item's end reads the last valid row and is zeroed when it
// is staged), so the waits for a step count the loads of the later steps
// instead of draining them.
//
// Loader: thread (cg = tid % 16, pp = tid / 16) owns columns 4 cg .. 4 cg + 3
// at positions 2 pp and 2 pp + 1 of a step and stores each column's pair as
// one 4-byte word of the column-major LDS layout of project_f16_kernel.
constexpr int kTallWaves = 8;
constexpr int kTallTN = 64;

template <int RB, int D>
__global__ __launch_bounds__(64 * kTallWaves, 2) void project_tall_kernel(ProjArgs a) {
  constexpr int CB = kTallTN / 32;
  constexpr int TK = kTallWaves * RB * 32;
  static_assert((kTallTN / 4) * (kProjTT / 2) == 64 * kTallWaves, "one column quad x position pair per thread");
  static_assert(D == 2 || D == 4, "the unrolled step loop keeps slots and LDS buffer parity static");

  __shared__ __attribute__((aligned(16))) _Float16 xts[2][kTallTN * kLdsStride];

  ProjItem it;
  if (!proj_item(a, a.nitems, blockIdx.x, &it)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool active = it.ktile * TK + wave * (RB * 32) < a.k;
  const int M = it.M, per = it.per;
  const int L = a.seq.len[it.b];
  const int64_t row0 = a.seq.row0[it.b];

  // ---- loader (a column past ncols reads column 0 and is zeroed)
  const int cg = tid & 15, pp = tid >> 4;
  const int col0 = it.ctile * kTallTN + cg * 4;
  const bool col_ok = col0 < a.ncols;
  const int colc = col_ok ? col0 : 0;
  const int blk = colc / a.dc, c0 = colc % a.dc;
  const int mat = blk / a.hkv, h = blk % a.hkv;
  const uint16_t* xb = static_cast<const uint16_t*>(mat ? a.x[1] : a.x[0]) +
                       (row0 + static_cast<int64_t>(h) * L + a.sink) * a.dc + c0;
  const int last = it.t_end - 1;
  uint2 raw[D][2];
  auto load = [&](int i, uint2 (&r)[2]) {
    const int q = it.t_begin + i * kProjTT + 2 * pp;
    r[0] = *reinterpret_cast<const uint2*>(xb + static_cast<int64_t>(min(q, last)) * a.dc);
    r[1] = *reinterpret_cast<const uint2*>(xb + static_cast<int64_t>(min(q + 1, last)) * a.dc);
  };
  // bf16 -> fp32 -> fp16 (exact for |x| in [2^-14, 65504]); positions past
  // the item's end (and columns past ncols) become zeros
  auto stage = [&](int i, const uint2 (&r)[2], _Float16* xt) {
    const int q = it.t_begin + i * kProjTT + 2 * pp;
    const uint32_t m0 = (col_ok && q <= last) ? 0xFFFFFFFFu : 0u;
    const uint32_t m1 = (col_ok && q + 1 <= last) ? 0xFFFFFFFFu : 0u;
    const uint32_t ax = r[0].x & m0, ay = r[0].y & m0, bx = r[1].x & m1, by = r[1].y & m1;
    uint32_t w[4];
    w[0] = pack_f16(__uint_as_float(ax << 16), __uint_as_float(bx << 16));
    w[1] = pack_f16(__uint_as_float(ax & 0xFFFF0000u), __uint_as_float(bx & 0xFFFF0000u));
    w[2] = pack_f16(__uint_as_float(ay << 16), __uint_as_float(by << 16));
    w[3] = pack_f16(__uint_as_float(ay & 0xFFFF0000u), __uint_as_float(by & 0xFFFF0000u));
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      *reinterpret_cast<uint32_t*>(&xt[xt_off(cg * 4 + qq, pp >> 2) + 2 * (pp & 3)]) = w[qq];
  };

  // ---- basis generator state, one coefficient row per lane and row block
  const float inv_per = 1.0f / static_cast<float>(per);
  float c2[RB], off[RB];
  int fr[RB], ph[RB], d64[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int n = it.ktile * TK + wave * (RB * 32) + rb * 32 + (lane & 31);
    const int ne = min(n, a.k - 1);
    const int f = basis_freq(ne) % per;
    float sn, cs;
    sincos_phase(f, per, &sn, &cs);
    c2[rb] = 2.0f * cs;
    off[rb] = basis_is_cos(ne) ? 0.25f : 0.0f;
    fr[rb] = f;
    ph[rb] = phase_mod(f, it.t_begin + 32 * (lane >> 5), per);
    d64[rb] = phase_mod(f, kProjTT, per);
  }
  floatx16 acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.0f;

  // basis operand of sub-step s (same runs as project_f16_kernel: seeded at
  // s = 0 from the exact phases of the step, continued by the recurrence)
  float yp[RB], yc[RB];
  auto gen_a = [&](int s, half8* av) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float v[8];
      if (s == 0) {
        const int r0 = ph[rb];
        int r1 = r0 + fr[rb];
        if (r1 >= per) r1 -= per;
        v[0] = sin_rev(fmaf(static_cast<float>(r0), inv_per, off[rb]));
        v[1] = sin_rev(fmaf(static_cast<float>(r1), inv_per, off[rb]));
#pragma unroll
        for (int e = 2; e < 8; ++e) v[e] = fmaf(c2[rb], v[e - 1], -v[e - 2]);
      } else {
        v[0] = fmaf(c2[rb], yc[rb], -yp[rb]);
        v[1] = fmaf(c2[rb], v[0], -yc[rb]);
#pragma unroll
        for (int e = 2; e < 8; ++e) v[e] = fmaf(c2[rb], v[e - 1], -v[e - 2]);
      }
      yp[rb] = v[6];
      yc[rb] = v[7];
      const uint4 bits = make_uint4(pack_f16(v[0], v[1]), pack_f16(v[2], v[3]),
                                    pack_f16(v[4], v[5]), pack_f16(v[6], v[7]));
      av[rb] = __builtin_bit_cast(half8, bits);
    }
  };

  // one step of MFMAs on the staged tile xt (the sub-step pipeline of
  // project_f16_kernel), then the basis phases move on by one step
  auto compute = [&](const _Float16* xt) {
    auto read_b = [&](int s, half8* bv) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        bv[cb] = *reinterpret_cast<const half8*>(&xt[xt_off(cb * 32 + (lane & 31), 4 * (lane >> 5) + s)]);
    };
    if (active) {
      half8 bcur[CB], bnxt[CB], acur[RB], anxt[RB];
      read_b(0, bcur);
      gen_a(0, acur);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s < 3) {
          read_b(s + 1, bnxt);
          gen_a(s + 1, anxt);
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(acur[rb], bcur[cb], acc[rb][cb], 0, 0, 0);
        if (s < 3) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) bcur[cb] = bnxt[cb];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) acur[rb] = anxt[rb];
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      ph[rb] += d64[rb];
      if (ph[rb] >= per) ph[rb] -= per;
    }
  };

  // Step i's rows sit in raw[i % D] from D steps before they are staged;
  // step i is staged into buffer i & 1 one step before its MFMAs, and its
  // slot is refilled with step i + D at once.  Stages and loads past the last
  // step touch only valid rows and a buffer nobody reads.
  const int nsteps = (it.t_end - it.t_begin + kProjTT - 1) / kProjTT;
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, raw[d]);
  stage(0, raw[0], xts[0]);
  load(D, raw[0]);
  __syncthreads();
  // (whole rounds of D steps first: a loop with an early exit would merge
  // its exit path into the loop head and make every wait there a full drain)
  auto step = [&](int i, auto dc) {
    constexpr int d = decltype(dc)::value;
    compute(xts[d & 1]);
    stage(i + 1, raw[(d + 1) % D], xts[(d + 1) & 1]);
    load(i + 1 + D, raw[(d + 1) % D]);
    __syncthreads();
  };
  int i0 = 0;
  for (; i0 + D <= nsteps; i0 += D) {
    step(i0, std::integral_constant<int, 0>());
    step(i0 + 1, std::integral_constant<int, 1>());
    if constexpr (D > 2) {
      step(i0 + 2, std::integral_constant<int, 2>());
      step(i0 + 3, std::integral_constant<int, 3>());
    }
  }
  if (i0 < nsteps) step(i0, std::integral_constant<int, 0>());
  if (i0 + 1 < nsteps) step(i0 + 1, std::integral_constant<int, 1>());
  if constexpr (D > 2) {
    if (i0 + 2 < nsteps) step(i0 + 2, std::integral_constant<int, 2>());
  }

  if (a.direct) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = it.ktile * TK + wave * (RB * 32) + rb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = it.ctile * kTallTN + cb * 32 + (lane & 31);
          if (n < a.k && col < a.ncols) {
            const int f = basis_freq(n);
            const float alpha = (f == 0 || 2 * f == per) ? 1.0f / sqrtf(static_cast<float>(per))
                                                       : sqrtf(2.0f / static_cast<float>(per));
            const int cblk = col / a.dc, c = col % a.dc, cmat = cblk / a.hkv, ch = cblk % a.hkv;
            (cmat ? a.out[1] : a.out[0])[((static_cast<int64_t>(it.b) * a.hkv + ch) * a.k + n) * a.dc + c] =
                alpha * acc[rb][cb][r];
          }
        }
    return;
  }
  float* P = a.partial + static_cast<int64_t>(it.slot) * TK * kTallTN;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int nl = wave * (RB * 32) + rb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int cl = cb * 32 + (lane & 31);
        if (it.ktile * TK + nl < a.k) P[nl * kTallTN + cl] = acc[rb][cb][r];
      }
}

// Retained rows (sink, then recent; all rows when L <= sink + recent) of
// kc (vc), copied to ke (ve) in 16-, 8- or 4-byte words: grid-stride over
// (sequence, matrix, KV head, retained row, word).
__device__ inline void edge_copy(const EdgeArgs& a, int64_t first, int64_t stride) {
  const int E = a.sink + a.recent;
  const int nbytes = a.dc * a.elem_bytes;
  const int wsz = (nbytes % 16 == 0) ? 16 : ((nbytes % 8 == 0) ? 8 : 4);
  const int nw = nbytes / wsz;
  const int64_t per_seq = static_cast<int64_t>(a.nmat) * a.hkv * E * nw;
  const int64_t total = per_seq * a.nseq;
  for (int64_t g = first; g < total; g += stride) {
    const int b = static_cast<int>(g / per_seq);
    int64_t r = g - b * per_seq;
    const int w = static_cast<int>(r % nw);
    r /= nw;
    const int e = static_cast<int>(r % E);
    r /= E;
    const int h = static_cast<int>(r % a.hkv);
    const int mat = static_cast<int>(r / a.hkv);
    const int L = a.seq.len[b];
    int t;
    if (L <= E) {
      if (e >= L) continue;
      t = e;
    } else {
      t = (e < a.sink) ? e : L - E + e;
    }
    const char* src = static_cast<const char*>(a.x[mat]) +
                      (a.seq.row0[b] + static_cast<int64_t>(h) * L + t) * nbytes + w * wsz;
    char* dst = static_cast<char*>(a.e[mat]) +
                ((static_cast<int64_t>(b) * a.hkv + h) * E + e) * nbytes + w * wsz;
    if (wsz == 16)
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    else if (wsz == 8)
      *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
    else
      *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
  }
}

// Fixed-order sum of the split partials of each tile element, scaled by the
// basis normalisation, scattered to ck / cv.  Block (chunk, tile, sequence)
// covers 256 / (tn / 4) rows of a tile, one thread per 4 consecutive columns
// (tn / 4 divides 256).  Sequences without middle get zeros.
__global__ __launch_bounds__(256) void project_reduce_kernel(ProjArgs a, EdgeArgs ea) {
  const int tn4 = a.tn / 4, rows = 256 / tn4;
  const int b = blockIdx.z, tile = blockIdx.y;
  const int nl = blockIdx.x * rows + static_cast<int>(threadIdx.x) / tn4;
  const int q4 = static_cast<int>(threadIdx.x) % tn4;
  const int kt = tile / a.nctiles, ct = tile % a.nctiles;
  const int n = kt * a.tk + nl;
  const int col0 = ct * a.tn + 4 * q4;
  if (nl < a.tk && n < a.k && col0 < a.ncols) {
    const int ns = a.seq.nsplit[b];
    const float* P = a.partial + (static_cast<int64_t>(a.seq.item0[b] + tile * ns) * a.tk + nl) * a.tn + 4 * q4;
    const int64_t stride = static_cast<int64_t>(a.tk) * a.tn;
    // splits in ascending order, kReduceBatch loads in flight (clamped index,
    // no branch around a load, so the waits count instead of draining)
    constexpr int kReduceBatch = 8;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp0 = 0; sp0 < ns; sp0 += kReduceBatch) {
      float4 v[kReduceBatch];
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j) v[j] = *reinterpret_cast<const float4*>(P + min(sp0 + j, ns - 1) * stride);
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j)
        if (sp0 + j < ns) {
          sum.x += v[j].x;
          sum.y += v[j].y;
          sum.z += v[j].z;
          sum.w += v[j].w;
        }
    }
    const int M = a.seq.mid[b], per = a.seq.per[b];
    float alpha = 0.0f;
    if (M > 0) {
      const int f = basis_freq(n);
      alpha = (f == 0 || 2 * f == per) ? 1.0f / sqrtf(static_cast<float>(per))
                                     : sqrtf(2.0f / static_cast<float>(per));
    }
    // Dc % 4 == 0: the 4 columns share (matrix, KV head) and are 16-byte aligned
    const int blk = col0 / a.dc, c = col0 % a.dc, mat = blk / a.hkv, h = blk % a.hkv;
    float* o = (mat ? a.out[1] : a.out[0]) + ((static_cast<int64_t>(b) * a.hkv + h) * a.k + n) * a.dc + c;
    *reinterpret_cast<float4*>(o) = make_float4(alpha * sum.x, alpha * sum.y, alpha * sum.z, alpha * sum.w);
  }
  // the retained rows ride along (no launch of their own)
  if (ea.nmat > 0) {
    const int64_t flat = (static_cast<int64_t>(blockIdx.z) * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    edge_copy(ea, flat * blockDim.x + threadIdx.x,
              static_cast<int64_t>(gridDim.x) * gridDim.y * gridDim.z * blockDim.x);
  }
}

// fp32 inputs: one block per (sequence, matrix, KV head, kF32Coefs
// coefficients); few per block, so that small problems still spread over many
// CUs.  The middle positions are walked in chunks of kF32Chunk: the chunk's
// basis values are computed once into LDS (exact integer phase, sincospi) and
// shared by the 32 column lanes; each thread (column lane, position lane of
// 8) prefetches its 8 cache values of the next chunk while the current one is
// summed, with Kahan compensation; the 8 position lanes are added in a fixed
// tree.
constexpr int kF32Coefs = 4;
constexpr int kF32Chunk = 64;
static_assert(kF32Coefs * kF32Chunk == 256, "one basis value per thread and chunk");

__global__ __launch_bounds__(256) void project_f32_kernel(ProjArgs a) {
  __shared__ float phis[kF32Coefs][kF32Chunk];
  __shared__ float red[8][kF32Coefs][32];
  const int ntile = (a.k + kF32Coefs - 1) / kF32Coefs;
  int g = blockIdx.x;
  const int nt = g % ntile;
  g /= ntile;
  const int h = g % a.hkv;
  g /= a.hkv;
  const int mat = g % a.nmat, b = g / a.nmat;
  const int M = a.seq.mid[b], per = a.seq.per[b], L = a.seq.len[b];
  const int cl = threadIdx.x & 31, tl = threadIdx.x >> 5;
  const float* X = static_cast<const float*>(a.x[mat]) +
                   (a.seq.row0[b] + static_cast<int64_t>(h) * L + a.sink) * a.dc;
  float* out = a.out[mat] + (static_cast<int64_t>(b) * a.hkv + h) * a.k * a.dc;
  // this thread's basis value of each chunk: coefficient bn, position bt
  const int bn = min(nt * kF32Coefs + static_cast<int>(threadIdx.x) / kF32Chunk, a.k - 1);
  const int bt = static_cast<int>(threadIdx.x) % kF32Chunk;
  const int bf = M > 0 ? basis_freq(bn) % per : 0;
  const bool bcos = basis_is_cos(bn);
  for (int c0 = 0; c0 < a.dc; c0 += 32) {
    const int c = c0 + cl;
    const bool col_ok = c < a.dc;
    const float* xc = X + (col_ok ? c : 0);
    float sum[kF32Coefs], comp[kF32Coefs];
#pragma unroll
    for (int i = 0; i < kF32Coefs; ++i) sum[i] = comp[i] = 0.0f;
    // positions p0 + tl + 8 i of a chunk; reads past the middle are clamped
    // to its last row (and weighted by a zero basis value)
    float xv[8], xn[8];
    auto load_x = [&](int p0, float* dst) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[i] = xc[static_cast<int64_t>(min(p0 + tl + 8 * i, M - 1)) * a.dc];
    };
    if (M > 0) load_x(0, xv);
    for (int p0 = 0; p0 < M; p0 += kF32Chunk) {
      {
        const int tau = p0 + bt;
        float sn = 0.0f, cs = 0.0f;
        if (tau < M) sincos_phase(phase_mod(bf, tau, per), per, &sn, &cs);
        phis[threadIdx.x / kF32Chunk][bt] = bcos ? cs : sn;
      }
      if (p0 + kF32Chunk < M) load_x(p0 + kF32Chunk, xn);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = col_ok ? xv[i] : 0.0f;
#pragma unroll
        for (int j = 0; j < kF32Coefs; ++j) {
          const float term = x * phis[j][tl + 8 * i] - comp[j];
          const float t = sum[j] + term;
          comp[j] = (t - sum[j]) - term;
          sum[j] = t;
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[i] = xn[i];
    }
#pragma unroll
    for (int i = 0; i < kF32Coefs; ++i) red[tl][i][cl] = sum[i];
    __syncthreads();
    if (tl == 0 && col_ok) {
#pragma unroll
      for (int i = 0; i < kF32Coefs; ++i) {
        const int n = nt * kF32Coefs + i;
        const float s01 = red[0][i][cl] + red[1][i][cl], s23 = red[2][i][cl] + red[3][i][cl];
        const float s45 = red[4][i][cl] + red[5][i][cl], s67 = red[6][i][cl] + red[7][i][cl];
        const float total = (s01 + s23) + (s45 + s67);
        if (n < a.k) {
          float alpha = 0.0f;
          if (M > 0) {
            const int f = basis_freq(n);
            alpha = (f == 0 || 2 * f == per) ? 1.0f / sqrtf(static_cast<float>(per))
                                           : sqrtf(2.0f / static_cast<float>(per));
          }
          out[static_cast<int64_t>(n) * a.dc + c] = alpha * total;
        }
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void edge_gather_kernel(EdgeArgs a) {
  edge_copy(a, static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x,
            static_cast<int64_t>(gridDim.x) * blockDim.x);
}

int64_t edge_words(const EdgeArgs& a) {
  const int nbytes = a.dc * a.elem_bytes;
  const int wsz = (nbytes % 16 == 0) ? 16 : ((nbytes % 8 == 0) ? 8 : 4);
  return static_cast<int64_t>(a.nseq) * a.nmat * a.hkv * (a.sink + a.recent) * (nbytes / wsz);
}

}  // namespace

// Tile configurations of the 16-bit path: 256 x 128 tiles of 4-wave blocks for
// large contractions, 512 x 64 tall tiles of 8-wave blocks otherwise.
hipError_t launch_project_f16(const ProjArgs& a, int nitems, hipStream_t s) {
  if (nitems == 0) return hipSuccess;
  const int blocks = (nitems + kXcds - 1) / kXcds * kXcds;
  if (a.tk == 256 && a.tn == 128)
    hipLaunchKernelGGL((project_f16_kernel<4, 1, 2, 4>), dim3(blocks), dim3(256), 0, s, a);
  else if (a.tk == kTallWaves * 64 && a.tn == kTallTN)
    hipLaunchKernelGGL((project_tall_kernel<2, 4>), dim3(blocks), dim3(64 * kTallWaves), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_project_reduce(const ProjArgs& a, const EdgeArgs& ea, hipStream_t s) {
  if (a.direct) return hipSuccess;
  const int tn4 = a.tn / 4;
  if (tn4 <= 0 || 256 % tn4 != 0) return hipErrorInvalidValue;
  const int rows = 256 / tn4;
  const int tiles = a.nktiles * a.nctiles;
  if (a.nseq <= 0 || tiles <= 0) return hipSuccess;
  const dim3 grid((a.tk + rows - 1) / rows, tiles, a.nseq);
  hipLaunchKernelGGL(project_reduce_kernel, grid, dim3(256), 0, s, a, ea);
  return hipGetLastError();
}

hipError_t launch_project_f32(const ProjArgs& a, hipStream_t s) {
  const int ntile = (a.k + kF32Coefs - 1) / kF32Coefs;
  const int blocks = a.nseq * a.nmat * a.hkv * ntile;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(project_f32_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_edge_gather(const EdgeArgs& a, hipStream_t s) {
  const int64_t words = edge_words(a);
  if (words == 0) return hipSuccess;
  const int blocks = static_cast<int>(std::min<int64_t>((words + 255) / 256, 8 * 2048));
  hipLaunchKernelGGL(edge_gather_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
