/*
 * fa.h - C ABI of libfa: Fourier-approximated KV-cache attention on MI355X.
 *
 * The method (arXiv 2506.11886, "Beyond Homogeneous Attention: Memory-Efficient
 * LLMs via Fourier-Approximated KV Cache", abstract; skill page
 * "fourier-approximated-kv-cache", Core concept and Steps 2-4): for each KV head
 * a set of "compressible" head dims is chosen; along the sequence, the first
 * `sink` tokens and the last `recent` tokens are kept exactly; the
 * M = L - sink - recent tokens between them (the middle) keep only k << M
 * coefficients per compressible dim, their projection onto an orthonormal real
 * Fourier basis over the M middle positions.  The other dims are kept exactly
 * for every token.
 *
 * Basis (tau = 0 .. M-1 counts middle tokens, n = 0 .. k-1):
 *   phi_0(tau)      = 1/sqrt(M)
 *   phi_{2j-1}(tau) = a_j cos(2 pi j tau / M)
 *   phi_{2j}(tau)   = a_j sin(2 pi j tau / M)
 *   a_j = sqrt(2/M), or 1/sqrt(M) for the Nyquist cosine (2j = M).
 *
 * ----------------------------------------------------------------------------
 * Cache layout ("dim-split" cache).  For KV head h, dims[h] (int32, D entries)
 * lists the exact dims ascending, then the compressible dims ascending; Du =
 * D - Dc.  Tensors are row-major, dtype = desc.dtype unless noted:
 *
 *   kx, vx  [rows, Du]   exact dims of every token;
 *   kc, vc  [rows, Dc]   compressible dims of every token (input of fa_project);
 *       row of (sequence b, KV head h, token t) = Hkv*off_b + h*L_b + t,
 *       off_b = L_0 + ... + L_{b-1}.  Column j of kx is dim dims[h][j],
 *       column c of kc is dim dims[h][Du + c].
 *   ke, ve  [B*Hkv, sink+recent, Dc]  compressible dims of the retained rows of
 *       block b*Hkv+h: the sink tokens, then the recent tokens.  When
 *       L_b <= sink+recent the block holds all L_b tokens in order and the rest
 *       of its rows are ignored.
 *   ck, cv  [B*Hkv, k, Dc]  float32 Fourier coefficients of the middle rows.
 *   q       [B, Hq, D]   queries, natural dim order.
 *   out     [B, Hq, D]   float32 attention outputs, natural dim order.
 *
 * Query head i reads KV head i / (Hq/Hkv).
 *
 * ----------------------------------------------------------------------------
 * Ownership and streams.  The caller owns every buffer, including the
 * workspace (size from the *_workspace_size queries, alignment 256 bytes).
 * The library allocates no memory, copies nothing between host and device and
 * never synchronises: calls enqueue kernels on `stream` (a hipStream_t; NULL is
 * the default stream) and return.  Outputs must not overlap inputs.  Calls that
 * share a workspace must be ordered on one stream.
 *
 * Errors.  Arguments are validated on the host before any HIP call; a failed
 * check returns its code and enqueues nothing.  A failing kernel launch returns
 * FA_ERR_HIP.  fa_last_error() gives a text for the last failure on the calling
 * thread.  Device arrays are not read by the host: entries of `dims` outside
 * [0, D) are skipped by the kernels (no fault) and give unspecified results.
 *
 * Check mode.  With the environment variable FA_CHECK=1 (read at every call),
 * fa_project (bf16) first scans kc / vc for values its fp16 operands cannot
 * hold (magnitude >= 65536, inf, NaN) and fa_decode / fa_attend scan
 * desc.dims for entries outside [0, D); the call then synchronises its stream,
 * reads the result and returns FA_ERR_SHAPE (with a text) before any other
 * kernel runs.  The workspace queries add one 256-byte slot for the flag in
 * this mode.  It is the one mode in which a call copies to the host and waits.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL                        */
  FA_ERR_SHAPE = 2,     /* sizes out of range or inconsistent                */
  FA_ERR_DTYPE = 3,     /* unknown dtype                                     */
  FA_ERR_WORKSPACE = 4, /* workspace missing, too small or misaligned        */
  FA_ERR_HIP = 5,       /* the HIP runtime reported an error                 */
  FA_ERR_ALIAS = 6      /* an output overlaps an input or another output     */
} fa_status_t;

typedef enum {
  FA_F32 = 0, /* float32 q, K, V                                             */
  FA_BF16 = 1 /* bfloat16 q, K, V (coefficients and outputs stay float32)    */
} fa_dtype_t;

#define FA_MAX_BATCH 64

typedef struct {
  int32_t dtype;       /* fa_dtype_t                                          */
  int32_t batch;       /* B, 1 .. FA_MAX_BATCH                                */
  int32_t n_q_heads;   /* Hq, a positive multiple of n_kv_heads               */
  int32_t n_kv_heads;  /* Hkv >= 1                                            */
  int32_t head_dim;    /* D, 1 .. 256                                         */
  int32_t n_comp_dims; /* Dc, 0 .. D                                          */
  int32_t sink;        /* tokens kept exactly at the start, >= 0              */
  int32_t recent;      /* tokens kept exactly at the end, >= 0                */
  int32_t n_coef;      /* k >= 1; k <= M_b for every b with M_b > 0           */
  int32_t period;      /* basis period P: 0 = each sequence's M_b (default);  */
                       /* > 0: a fixed P with M_b <= P and k <= P (fa_append) */
  const int32_t *seq_len; /* HOST array [B], L_b >= 1                         */
  const int32_t *dims;    /* DEVICE array [Hkv][D] (fa_decode only)           */
} fa_desc_t;

/* Workspace bytes fa_project needs for `desc` (0 is possible). */
fa_status_t fa_project_workspace_size(const fa_desc_t *desc, size_t *bytes);

/*
 * fa_project: prefill compression.  For every sequence b with M_b > 0 and
 * KV head h:  ck[b*Hkv+h][n][c] = sum_tau phi_n(tau) * kc[row(b,h,sink+tau)][c]
 * (and cv from vc), the projection of the middle rows onto the first k basis
 * functions (skill page, Step 2; arXiv 2506.11886 abstract).  Blocks of
 * sequences with M_b = 0 are set to zero.  When ke (ve) is not NULL the
 * retained sink/recent rows of kc (vc) are also gathered into it (skill page,
 * Step 3).  Either matrix may be skipped: pass kc = ck = ke = NULL (or the V
 * trio).  With n_comp_dims = 0 the call does nothing and every pointer may be
 * NULL.  The 16-bit path needs n_comp_dims % 4 == 0 and 8-byte aligned kc/vc;
 * it computes in fp16 operands, so |kc|, |vc| must stay below 65504 (FA_CHECK=1
 * rejects larger values, see Check mode above).
 * desc.dims is not used.
 */
fa_status_t fa_project(const fa_desc_t *desc, const void *kc, const void *vc,
                       float *ck, float *cv, void *ke, void *ve,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes fa_decode needs for `desc`. */
fa_status_t fa_decode_workspace_size(const fa_desc_t *desc, size_t *bytes);

/*
 * fa_decode: one decode step.  For sequence b and query head i (KV head
 * g = i / (Hq/Hkv)) over the cache in which the middle rows' compressible dims
 * are the Fourier reconstruction sum_n phi_n(tau) ck[n][c] (skill page, Step 4):
 *   s_t = scale * q[b][i] . K~[t],   p = softmax_t(s),
 *   out[b][i] = sum_t p_t V~[t]      for t = 0 .. L_b-1.
 * The reconstruction is never formed: compressed scores are
 * (scale q_C ck^T) . phi(tau) and compressed values are (sum_tau p phi(tau)) cv.
 * Required pointers: q, out, desc.dims; kx and vx when Du > 0; ke and ve when
 * Dc > 0 and sink + recent > 0; ck and cv when Dc > 0 and some sequence has
 * middle tokens (others may be NULL, FA_ERR_NULL otherwise).
 * bf16 caches need 16-byte aligned kx, vx, ke, ve.
 */
fa_status_t fa_decode(const fa_desc_t *desc, const void *q, const void *kx,
                      const void *vx, const void *ke, const void *ve,
                      const float *ck, const float *cv, float scale, float *out,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes fa_attend needs for `desc` and `n_query`. */
fa_status_t fa_attend_workspace_size(const fa_desc_t *desc, int32_t n_query, size_t *bytes);

/*
 * fa_attend: n_query queries per sequence, each attending to the whole cache
 * exactly as fa_decode's query does (no mask between the queries).  This is
 * attention over the compressed cache during prefill as well as decode (skill
 * page, Architecture overview and Practical guidance: the kernel serves the
 * memory-bound attention of both phases): a chunk of new tokens attends to the
 * cached past through this call, and to itself through ordinary causal
 * attention; the two parts combine with their log-sum-exp values.
 *   q    [B, n_query, Hq, D]   queries (desc.dtype), natural dim order;
 *   out  [B, n_query, Hq, D]   float32;
 *   lse  [B, n_query, Hq]      float32 log sum_t exp(s_t), the natural log of
 *                              the softmax denominator in the units of s
 *                              (scale included), or NULL.
 * Query t of head i reads KV head i / (Hq/Hkv).  The queries run in passes
 * over the cache: one pass takes as many queries as the prep kernel's LDS
 * holds for a KV head's rows on the single query's kernel path (96 query rows
 * per KV head at D = 128, Dc = 64, i.e. 24 queries of a 4-head group), and the
 * G * (queries of the pass) rows of a KV head share that pass; more queries
 * take more passes, in order, on `stream`.  n_query is 1 .. 1024 and a
 * sequence has at most 65536 query rows (n_query * Hq; this bounds
 * fa_decode's Hq too); FA_ERR_SHAPE otherwise.  Everything else
 * (required pointers, alignment, errors) is as for fa_decode, which is
 * fa_attend with n_query = 1 and lse = NULL.
 */
fa_status_t fa_attend(const fa_desc_t *desc, int32_t n_query, const void *q,
                      const void *kx, const void *vx, const void *ke,
                      const void *ve, const float *ck, const float *cv,
                      float scale, float *out, float *lse, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * fa_attend_plan: how fa_attend (fa_decode for n_query = 1) would run `desc`,
 * host only (nothing is enqueued, device arrays are not read):
 *   path     0: VALU kernels (fp32 caches and shapes the MFMA kernels do not
 *               take), 1: one MFMA pass over the middle tokens, 2: two MFMA
 *               passes (scores and exact values, then the value moments W);
 *   rows     query rows stacked per work item;
 *   items    work items of the main kernel (per pass over the cache);
 *   items2   work items of the second MFMA pass (path 2), else 0;
 *   passes   passes over the cache (queries per pass bounded by LDS);
 *   queries_per_pass  queries of a full pass.
 * Errors as for fa_attend_workspace_size.
 */
typedef struct {
  int32_t path, rows, items, items2, passes, queries_per_pass;
} fa_plan_t;
fa_status_t fa_attend_plan(const fa_desc_t *desc, int32_t n_query, fa_plan_t *plan);

/*
 * fa_append: one token appended to every sequence (streaming decode).  The
 * pages name a translation-invariant transform (skill page, Architecture
 * overview; Step 2) but give no rule for a middle that grows; the reading
 * taken here is a fixed basis period P = desc.period > 0 (fa_project and
 * fa_decode use the same P), under which the coefficients of a middle are a
 * sum of one term per token.  desc describes the cache BEFORE the append
 * (seq_len = L_b); afterwards the caller describes it with L_b + 1.  For each
 * sequence b and KV head h, K and V alike:
 *   - L_b + 1 <= sink + recent: the new token is retained: its compressible
 *     row becomes retained row L_b of ke / ve;
 *   - otherwise the token that leaves the recent window (retained row `sink`,
 *     or the new token itself when recent = 0) enters the middle at tau =
 *     M_b = L_b - sink - recent:  ck[n][c] += phi_n(M_b) * x[c]  for n < k
 *     (the ck of fa_project for L_b tokens becomes the ck of fa_project for
 *     L_b + 1 tokens, to rounding); the recent rows of ke / ve move down by
 *     one and the new token's row becomes the last.
 * k_new, v_new: [B][Hkv][Dc] compressible dims of the new token (dims order
 * of the cache, desc.dtype).  ck, cv, ke, ve are updated in place.  kx / vx
 * are the caller's: with the packed row layout the new token's exact dims go
 * into the caller's own layout for L_b + 1.  Required: k_new and v_new; ke
 * and ve when sink + recent > 0; ck and cv when some sequence has middle
 * tokens after the append (others may be NULL).  With n_comp_dims = 0 the
 * call does nothing.  Errors: desc.period = 0 or a middle that would exceed
 * the period is FA_ERR_SHAPE; overlapping buffers FA_ERR_ALIAS.  No workspace;
 * two small kernels on `stream`, so calls on one stream are ordered.
 */
fa_status_t fa_append(const fa_desc_t *desc, const void *k_new, const void *v_new,
                      float *ck, float *cv, void *ke, void *ve, void *stream);

/* Workspace bytes fa_dim_sensitivity needs for `desc` and `n_query`. */
fa_status_t fa_dim_sensitivity_workspace_size(const fa_desc_t *desc, int32_t n_query, size_t *bytes);

/*
 * fa_dim_sensitivity: the dimension analysis of the skill page (Step 1;
 * Architecture overview, dimension analysis stage), over the uncompressed
 * cache.  Dim d is perturbed by adding noise[row][d] to dim d of the values of
 * every token; the score of dim d is the change of the attention outputs.
 * Adding noise to one dim of V changes only that dim of the outputs, by
 * sum_t p_t noise[t][d] (p the unperturbed probabilities), so
 *   sq[i][d] = sum over sequences b and queries t of
 *              ( sum_tau p_{b,t,i}(tau) noise[row(b, i/G, tau)][d] )^2,
 * the squared change for query head i; the pages' score of dim d is
 * sqrt(sum_i sq[i][d]) (small: dim d can be compressed).
 * q     [B, n_query, Hq, D]  queries (natural dim order; [B, Hq, D] for 1);
 * k     [rows, D]            keys of every token, natural dim order, rows
 *                            packed as kx (row(b, h, t) = Hkv*off_b + h*L_b + t);
 * noise [rows, D]            the perturbations (the pages draw N(0, 0.1^2)),
 *                            same layout and dtype as k;
 * sq    [Hq, D] float32.
 * Every query attends to all L_b tokens.  desc.n_comp_dims, n_coef, period,
 * sink, recent and dims are not used (the analysis precedes the dim split).
 * The values themselves do not enter.  Runs the decode kernels on all-exact
 * dims (noise as the values, an identity dims table in the workspace), then a
 * fixed-order sum of squares.  Errors as fa_attend; sq must not overlap an
 * input or the workspace (FA_ERR_ALIAS).
 */
fa_status_t fa_dim_sensitivity(const fa_desc_t *desc, int32_t n_query, const void *q,
                               const void *k, const void *noise, float scale, float *sq,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa_coef_budget: the number of real coefficients that spans the same space as
 * the first floor(fraction * M) bins of the middle's real FFT, which is how the
 * skill page (Step 3) sizes its coefficient budget (fraction 0.3 of the middle
 * length, kept as frequency bins, Step 2).  The constant bin gives one real
 * coefficient and every further bin a cosine and a sine, so
 *   k = 2 * floor(fraction * M) - 1,   clamped to [1, M]
 * (floor of the double product, as the pages' int() of a float).  Host only;
 * M < 1 or a fraction outside [0, 1] (or NaN) returns 0.
 */
int32_t fa_coef_budget(int32_t M, double fraction);

/*
 * fa_cache_bytes: memory of the KV cache described by `desc`, before and after
 * compression (the pages report the KV-cache reduction; skill page, Practical
 * guidance and References):
 *   *full:       K and V of every token, all D dims, at desc.dtype;
 *   *compressed: kx and vx (exact dims of every token), the compressible dims
 *                of the retained rows (min(L_b, sink+recent) per sequence and
 *                KV head, as in ke / ve) and, for every sequence with middle
 *                tokens, ck and cv (k float32 values per compressible dim).
 * The compression ratio is 1 - compressed / full.  Host only; desc.dims is not
 * used.  Either output pointer may be NULL.
 */
fa_status_t fa_cache_bytes(const fa_desc_t *desc, uint64_t *full, uint64_t *compressed);

/* Static text for a status code. */
const char *fa_status_string(fa_status_t status);

/* Text of the last failure on the calling thread ("" if none). */
const char *fa_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t fa_version(void);

/*
 * fa_decode_noalloc: fa_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The workspace is a static device
 * array inside the library, FA_NOALLOC_SCRATCH_MIB MiB per GPU, held by every
 * GPU the library runs on until the process ends; its device address is
 * looked up once per device (hipGetSymbolAddress) on the first call made with
 * that device current.  The call allocates nothing and runs the same kernels
 * as fa_decode on that array, so its results are fa_decode's.  A shape whose
 * fa_decode_workspace_size exceeds the array returns FA_ERR_WORKSPACE (with a
 * text in fa_last_error) and enqueues nothing.  Every call on one GPU shares
 * the one array: calls that may overlap on a GPU (several host threads, or
 * several streams without ordering between them) race and must not be made;
 * calls ordered on one stream are fine.  Arguments, outputs and errors are
 * otherwise those of fa_decode.
 */
#define FA_NOALLOC_SCRATCH_MIB 256
fa_status_t fa_decode_noalloc(const fa_desc_t *desc, const void *q, const void *kx,
                              const void *vx, const void *ke, const void *ve,
                              const float *ck, const float *cv, float scale, float *out,
                              void *stream);

/*
 * fa_time_main_kernel: measurement hook.  With two events given (hipEvent_t
 * handles, created by the caller), every later fa_project / fa_decode /
 * fa_attend call made by the calling thread records `before` on its stream
 * right before its dominant kernel and `after` right after it, so that the
 * caller can time that kernel alone with hipEventElapsedTime: the projection
 * kernel of fa_project (not its reduce or gather), the main split kernel of
 * fa_decode, and of fa_attend's first pass.  NULL, NULL turns it off (the
 * default).  Only one of the two NULL is FA_ERR_NULL.  The library keeps the
 * handles (thread-local), not the events: the caller keeps them alive while
 * the hook is on.
 */
fa_status_t fa_time_main_kernel(void *before, void *after);

#ifdef __cplusplus
}
#endif
#endif /* FA_H */
