// kernels.hpp - argument blocks and launchers of libfa's HIP kernels.
//
// The host API (fa_api.cpp) validates, plans the work split and fills these
// blocks; the launchers enqueue kernels on the caller's stream.
#pragma once

#include "common.hpp"

namespace fa {

// ------------------------------------------------------------ projection --
// Projection of the middle rows of kc / vc onto the first k basis functions.
// Columns are numbered mat-major: col = (mat * Hkv + h) * Dc + c.
constexpr int kProjTT = 64;   // middle positions per pipeline step (16-bit path)

struct ProjArgs {
  const void* x[2];  // kc / vc (element type from dtype); x[m] for mat index m
  float* out[2];     // ck / cv
  int nmat;          // matrices present (1 or 2)
  int hkv, dc, k, sink;
  int ncols;         // nmat * hkv * dc
  int tk, tn;        // tile: coefficient rows x columns (16-bit path)
  int nktiles, nctiles;
  int nseq;
  int nitems;        // work items (16-bit path)
  float* partial;    // [items][tk][tn] (16-bit path, when not direct)
  int direct;        // every sequence has one split: the kernel writes ck / cv
  SeqTable seq;      // item0/nsplit: items = tiles * nsplit; chunk = positions per split
};

// Supported tiles (tk x tn): 256 x 128 (4-wave blocks) and 512 x 64 (tall).
hipError_t launch_project_f16(const ProjArgs& a, int nitems, hipStream_t s);
hipError_t launch_project_f32(const ProjArgs& a, hipStream_t s);

// Gather of the sink/recent rows of kc (vc) into ke (ve).
struct EdgeArgs {
  const void* x[2];
  void* e[2];
  int nmat, hkv, dc, sink, recent, nseq, elem_bytes;
  SeqTable seq;
};
hipError_t launch_edge_gather(const EdgeArgs& a, hipStream_t s);
// Split-partial reduction of the 16-bit path; with ea.nmat > 0 it also copies
// the retained rows (then no separate gather is launched).
hipError_t launch_project_reduce(const ProjArgs& a, const EdgeArgs& ea, hipStream_t s);

// ---------------------------------------------------------------- append --
// One token appended to each sequence of a fixed-period cache (fa_append).
constexpr int kMaxAppendDc = 256;
struct AppendArgs {
  const void* xnew[2];     // new token's compressible rows [B*Hkv][Dc] (K, V)
  float* c[2];             // ck, cv [B*Hkv][k][Dc] (nullptr: no sequence gets a middle)
  void* e[2];              // ke, ve [B*Hkv][sink+recent][Dc] (nullptr: nothing retained)
  int nmat, hkv, dc, k, sink, recent, esz, nseq, period;
  int32_t len[kMaxBatch];  // lengths before the append
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);

// ------------------------------------------------------- FA_CHECK mode --
// A flag word in device memory: cleared, then or-ed by the scans (1: a bf16
// cache value of magnitude >= 65536, inf or NaN; 2: a dims entry outside [0, D)).
hipError_t launch_check_clear(int32_t* flag, hipStream_t s);
hipError_t launch_check_bf16_range(const void* x, int64_t n, int32_t* flag, hipStream_t s);
hipError_t launch_check_dims(const int32_t* dims, int n, int D, int32_t* flag, hipStream_t s);

// ---------------------------------------------------- dimension analysis --
// Identity dims table [hkv][D], and sq[i][d] = sum_{b,t} resp[b][t][i][d]^2.
hipError_t launch_iota_dims(int32_t* dims, int hkv, int D, hipStream_t s);
hipError_t launch_sens_norm(const float* resp, float* sq, int B, int nq, int hq, int D, hipStream_t s);

// ---------------------------------------------------------------- decode --
constexpr int kDecRows = 4;    // query rows per work item (VALU path)
constexpr int kDecTile = 64;   // tokens per tile (VALU path)

// A work item covers `rows` consecutive query heads of one sequence (query
// head i reads KV head i / G) and one token range of it.
struct DecodeArgs {
  int dtype;                   // 0 f32, 1 bf16
  const void* q;
  const void* kx;
  const void* vx;
  const void* ke;
  const void* ve;
  const float* ck;
  const float* cv;
  const int32_t* dims;
  float* out;
  float* A;      // VALU path: [B][Hq][kpad] fp32, basis order
  void* A16;     // MFMA path: [B][Hq][kpp] fp16, pair order
  void* Q16;     // MFMA path: [B][Hq][du32] bf16, q at the exact dims (dims order, zero pad)
  int prep_a;    // decode_prep computes A (Dc > 0 and some sequence has middle tokens)
  float* part;   // partials [prow][RS]: m, l, o_U[du], o_E[dc], W[kpad]
  float* mrg;    // merged rows [B*Hq][MS]: o_E[dc], alpha*W[kpad], 1/l
  int nseq, hq, hkv, G, D, du, dc, k, kpad, kpp, sink, recent;
  int mfma;      // 1: decode_mfma kernel, 0: VALU kernel
  int edge_split;  // > 0: the last edge_split splits of every row hold the
                   //    sink/recent tokens (decode_prep, one part each); the
                   //    other splits cover middle tokens only
  int mb;        // MFMA path: 16-row blocks per item
  int rows;      // query rows per work item
  int ngroups;   // row groups per sequence (Hq / rows)
  int RS;        // floats per partial row: 2 + du + dc + kpad
  int MS;        // floats per merged row: dc + kpad + 1
  float scale;
  int nq;        // queries per sequence in this pass; hq and G count nq * (query heads)
  int nq_total;  // queries per sequence in q / out / lse (passes of nq cover q0 ..)
  int q0;        // first query of this pass
  float* lse;    // optional [B][nq][Hq]: log sum_t exp(s_t) of each query row
  SeqTable seq;  // item0 / nsplit (splits per row, edge split included) / chunk
  int32_t prow0[kMaxBatch];  // first partial row of sequence b: sum Hq * nsplit
  // Two-pass path (two_pass = 1; MFMA only): decode_score writes each middle
  // split's probabilities and references, decode_moment forms W from them.
  //   P16  fp16 [b][row i < hq][tau < mpad_b]: p of middle token tau relative
  //        to the reference of its 16-token tile (mpad_b = M_b rounded up to 128);
  //   msub fp32 [b][row][mpad_b / 16]: that reference, per 16-token tile;
  //   Wp   fp32 [b][sg][row][kpad]: W of sequence b over its middle splits
  //        4 sg .. 4 sg + 3, relative to the row's maximum over all its splits,
  //        in basis order (without the basis scale).
  int two_pass;
  void* P16;
  float* msub;
  float* Wp;
  int nitems2;    // decode_moment items: (sequence, row group, split group, frequency slice)
  int nslices;    // frequency slices per (sequence, row group, split group)
  int ngr;        // frequency groups of 16 (frequencies 0 .. k/2)
  int64_t pcum[kMaxBatch];   // sum of mpad over sequences before b
  int32_t sgcum[kMaxBatch];  // sum of split groups over sequences before b
  int32_t item2_0[kMaxBatch];  // first decode_moment item of sequence b
};

// Rows of the kernels are "virtual" query heads: with nq queries per
// sequence in a pass, KV head h owns rows h*G .. h*G + G-1 (G = nq * Hq/Hkv),
// row h*G + t*(G/nq) + g being query q0 + t of query head h*(G/nq) + g.  q,
// out and lse are laid out [B][nq_total][Hq]; this gives the (b, row) entry's
// index in them.
__host__ __device__ inline int64_t q_row(const DecodeArgs& a, int b, int i) {
  if (a.nq_total == 1) return static_cast<int64_t>(b) * a.hq + i;
  const int gu = a.G / a.nq;  // query heads per KV head
  const int h = i / a.G, r = i % a.G;
  return (static_cast<int64_t>(b) * a.nq_total + a.q0 + r / gu) * (a.hq / a.nq) + h * gu + r % gu;
}

// The sink/recent split runs on MFMA for 16-byte rows, whole 32-dim chunks
// and at most 16 query rows per KV head; there its retained tokens are cut
// into up to kEdgeParts parts (prep blocks) of whole 16-token blocks, else it
// is one part.  Short parts shorten the prep kernel's slowest blocks; each
// part adds a split to the merge.
constexpr int kEdgeParts = 6;
__host__ __device__ inline bool edge_mfma_ok(const DecodeArgs& a) {
  return a.du % 8 == 0 && a.dc % 8 == 0 && a.D % 32 == 0 && a.G <= 16;
}
// The parts are also capped so that the edge blocks of all (sequence, KV
// head) pairs fit one block per CU: past that, more parts only queue behind
// each other.
constexpr int kEdgeBlocksMax = 256;
inline int edge_parts(const DecodeArgs& a) {
  if (!edge_mfma_ok(a)) return 1;
  const int blocks16 = (a.sink + a.recent + 15) / 16;
  int parts = blocks16 < kEdgeParts ? blocks16 : kEdgeParts;
  const int heads = a.nseq * a.hkv;
  if (heads > 0 && parts > kEdgeBlocksMax / heads) parts = kEdgeBlocksMax / heads;
  return parts > 1 ? parts : 1;
}

hipError_t launch_decode_prep(const DecodeArgs& a, hipStream_t s);
size_t decode_edge_smem(const DecodeArgs& a);  // LDS of the edge split (decode_prep)
size_t decode_prep_smem(const DecodeArgs& a);  // LDS of decode_prep
hipError_t launch_decode_split(const DecodeArgs& a, int nitems, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, int nitems, hipStream_t s);
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t s);
// Two-pass path: pass 1 (scores, softmax, exact values; writes P16 / msub and
// the (m, l, o_U) partials) and pass 2 (W = P phi into Wp).
constexpr int kMomentTile = 128;   // tokens per pass-2 step of one wave
constexpr int kMomentWaves = 4;    // pass-1 splits per split group (one wave each)
struct ScoreVariant {
  int mb, maxu, pf, xp, xu, kcm, kpp_max;
};
const ScoreVariant* decode_score_pick(int kpp, int mb, int nheads, int nunit, int du);
size_t decode_score_smem(int mb, int nheads, int du);
hipError_t launch_decode_score(const DecodeArgs& a, int nitems, hipStream_t s);
int decode_moment_max_groups(int mb);  // frequency groups per item of the compiled variants
size_t decode_moment_smem(int mb, int ngw);
hipError_t launch_decode_moment(const DecodeArgs& a, hipStream_t s);
// MFMA decode kernel: tokens per tile, compiled variants and LDS carve-up.
constexpr int kMfmaTile = 16;
struct MfmaVariant {
  int mb;       // 16-row blocks
  int nw;       // waves per workgroup
  int maxu;     // max 32-wide coefficient units per wave
  int pf;       // 16-byte vx chunks staged per thread per tile
  int xp;       // max KV heads per wave (exact scores)
  int xu;       // max (KV head, 16-dim block) exact-value tiles per wave
  int kpp_min, kpp_max;
};
struct MfmaLds {
  int ps, dus;  // row strides (halves) of the basis tile and the staged vx rows
  int phi, vxs, spart, sx, ph, pbh, pbl, corr, total;  // byte offsets
};
__host__ __device__ MfmaLds mfma_lds(int mb, int nw, int kpp, int nheads, int du, int dc);
// nheads: KV heads of an item; nunit: its (KV head, 16-row block) units
const MfmaVariant* decode_mfma_pick(int kpp, int mb, int nheads, int nunit, int du);
bool decode_mfma_fits(const MfmaVariant& v, int nheads, int nunit, int du);
size_t decode_mfma_smem(const DecodeArgs& a, const MfmaVariant& v, int nheads);

}  // namespace fa
