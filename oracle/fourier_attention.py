"""CPU oracle for Fourier-approximated KV-cache decode (float64, numpy).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it, and it
shares no code with the GPU library: it is a plain, slow restatement of what the
method computes, written so that each step can be checked by eye against the
pages that describe the method.

Sources (cited by title and section; no text is quoted):

* [SKILL] the skill page "fourier-approximated-kv-cache" (agent-skills.jp,
  "Beyond homogeneous attention: memory-efficient LLMs via a Fourier-approximated
  KV cache"), sections Core concept, Architecture overview, Step 2 (Fourier-basis
  compression), Step 3 (selective token retention), Step 4 (reconstruction during
  decoding).
* [ABSTRACT] "Beyond Homogeneous Attention: Memory-Efficient LLMs via
  Fourier-Approximated KV Cache", arXiv 2506.11886, English abstract (as printed
  on the shd-paper.top and fugumt.com pages).

What the method computes, restated:

1. Segmentation [SKILL Step 3]: the first ``sink`` tokens and the last
   ``recent`` tokens stay exact; the ``M = L - sink - recent`` tokens between
   them are the "middle".  With ``L <= sink + recent`` there is no middle and
   every token stays exact (each token once).
2. Dim split [SKILL Core concept, Step 3; ABSTRACT]: a per-head set of
   compressible dims; the other dims stay exact for every token.
3. Projection [SKILL Step 2; ABSTRACT]: each compressible dim's time series over
   the middle tokens is projected onto ``k`` orthonormal Fourier basis functions
   (``fourier_basis``).  The pages show a complex ``rfft`` truncated to its first
   bins; the real orthonormal basis below spans the same space as the first
   ``(k+1)/2`` rfft bins for odd ``k`` (pinned in the tests through numpy's
   rfft/irfft).
4. Reconstruction [SKILL Step 4]: the middle compressible entries are replaced by
   ``Phi @ C`` (the real-basis form of zero-padding the kept bins and inverting).
5. Decode: standard softmax attention of the query over the cache in which the
   middle compressible entries are the reconstruction.
6. Streaming append (a reading; the pages name a translation-invariant
   transform in the Architecture overview but give no update rule): with a
   fixed basis period P (``fourier_basis(..., period=P)``) the coefficients of
   a middle are a sum of one term per token, so the token that leaves the
   recent window when a new token arrives adds its term (``append``).
7. Dimension analysis [SKILL Step 1]: noise added to one dim of the values at a
   time, and the norm of the change of the attention output, per dim
   (``dim_sensitivity``); low scores mark dims that can be compressed.

Readings where the pages are silent (each is listed in the design notes too):
basis order is the constant term, then (cos, sin) pairs of ascending frequency;
orthonormal scaling ``sqrt(2/M)``, with ``1/sqrt(M)`` for the constant and the
Nyquist cosine; tau = 0 is the first middle token; query head i reads KV head
``i // (Hq/Hkv)``.

Parity pins for every function here live in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------- step 1 -----

def segment(L: int, sink: int, recent: int):
    """Return (first middle token, M) for a sequence of length L [SKILL Step 3].

    The middle is tokens [sink, L - recent).  When L <= sink + recent the
    sequence has no middle (M = 0) and all L tokens are kept exactly.
    """
    M = max(0, L - sink - recent)
    return sink, M


# --------------------------------------------------------------- step 3 -----

def fourier_basis(M: int, k: int, period: int = 0) -> np.ndarray:
    """Orthonormal real Fourier basis Phi [M, k]: Phi[tau, n] = phi_n(tau).

    phi_0 is the constant; basis index n >= 1 has frequency f = ceil(n/2); odd n
    is the cosine and even n the sine of 2 pi f tau / P.  Scale sqrt(2/P), or
    1/sqrt(P) for the constant and for the Nyquist cosine (2f = P).  The phase
    f*tau is reduced mod P in integer arithmetic before the trig call.
    [ABSTRACT: orthogonal Fourier bases; SKILL Step 2.]

    P is the period: the middle length M itself (``period`` 0, the pages'
    transform of the middle), or a fixed P >= M, the basis of a window of P
    positions of which the first M are filled (a reading for streaming
    appends, under which appending a token adds one term; the pages give no
    update rule).  The columns are orthonormal over [0, P).
    """
    P = M if period == 0 else period
    if not (1 <= k <= P) or not (0 <= M <= P):
        raise ValueError("need 1 <= k <= P and M <= P (k=%d, M=%d, P=%d)" % (k, M, P))
    tau = np.arange(M, dtype=np.int64)
    n = np.arange(k, dtype=np.int64)
    f = (n + 1) // 2
    r = np.outer(tau, f) % P
    angle = 2.0 * np.pi * r / P
    use_cos = (n == 0) | (n % 2 == 1)
    phi = np.where(use_cos[None, :], np.cos(angle), np.sin(angle))
    scale = np.where((f == 0) | (2 * f == P), 1.0 / np.sqrt(P), np.sqrt(2.0 / P))
    return phi * scale[None, :]


# The last basis built, reused while (M, k, period) repeat (the K and V blocks
# and the KV heads of one sequence share it).  A memo only: it changes no
# value.  The key holds the basis function itself, so a replaced
# fourier_basis (the tests' planted mistakes) is never answered from an
# earlier function's result.
_BASIS_MEMO = {}


def _basis(M: int, k: int, period: int = 0) -> np.ndarray:
    key = (fourier_basis, M, k, period)
    if key not in _BASIS_MEMO:
        _BASIS_MEMO.clear()
        _BASIS_MEMO[key] = fourier_basis(M, k, period)
    return _BASIS_MEMO[key]


def project(x_mid: np.ndarray, k: int, period: int = 0) -> np.ndarray:
    """Fourier coefficients C [k, c] = Phi^T x_mid of middle rows x_mid [M, c].

    [SKILL Step 2: project the middle tokens onto k << M basis functions.]
    """
    x_mid = np.asarray(x_mid, dtype=np.float64)
    Phi = _basis(x_mid.shape[0], k, period)
    return Phi.T @ x_mid


def coef_budget(M: int, fraction: float = 0.3) -> int:
    """Real coefficients for the pages' coefficient budget [SKILL Step 3]: the
    first ``int(fraction * M)`` bins of the middle's rfft are kept (Step 2).
    Bin 0 is the constant (one real coefficient); each further bin below the
    Nyquist frequency has a cosine and a sine.  Clamped to [1, M]."""
    bins = int(fraction * M)
    real = 0
    for j in range(bins):
        real += 1 if (j == 0 or 2 * j == M) else 2
    return max(1, min(M, real))


# --------------------------------------------------------------- step 4 -----

def reconstruct(coef: np.ndarray, M: int, period: int = 0) -> np.ndarray:
    """Approximate middle rows [M, c] = Phi @ coef  [SKILL Step 4]."""
    coef = np.asarray(coef, dtype=np.float64)
    return _basis(M, coef.shape[0], period) @ coef


def approximate_cache(X: np.ndarray, comp_dims, coef, sink: int, recent: int, period: int = 0):
    """The cache as decode sees it: X [L, D] with the middle rows' compressible
    dims replaced by their reconstruction from ``coef`` [k, len(comp_dims)].

    Sink rows, recent rows and the exact dims are untouched [SKILL Step 3].
    """
    X = np.array(X, dtype=np.float64, copy=True)
    start, M = segment(X.shape[0], sink, recent)
    comp_dims = np.asarray(comp_dims, dtype=np.int64)
    if M > 0 and comp_dims.size > 0:
        X[start:start + M][:, comp_dims] = reconstruct(coef, M, period)
    return X


# --------------------------------------------------------------- step 5 -----

def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                      return_probs: bool = False):
    """out[i] = sum_t p_it V[t], p_i = softmax_t(scale * q[i] . K[t])."""
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    s = scale * (q @ np.asarray(K, dtype=np.float64).T)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=1, keepdims=True)
    out = p @ np.asarray(V, dtype=np.float64)
    return (out, p) if return_probs else out


def decode(q_rows, K, V, comp_dims, ck, cv, sink: int, recent: int, scale: float, period: int = 0):
    """One decode step of the query rows q_rows [G, D] that share one KV head.

    K, V: [L, D] in natural dim order (their middle compressible entries are not
    used: those come from the coefficients ck, cv [k, Dc]).  Reconstruct, then
    attend [SKILL Step 4, then standard attention].
    """
    Kt = approximate_cache(K, comp_dims, ck, sink, recent, period)
    Vt = approximate_cache(V, comp_dims, cv, sink, recent, period)
    return softmax_attention(q_rows, Kt, Vt, scale)


# ------------------------------------------------------ several queries ----

def softmax_attention_lse(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """(out, lse): softmax attention outputs of the query rows q and, per row,
    lse_i = log sum_t exp(s_it) with s_it = scale * q[i] . K[t] (natural log,
    in the units of s), taken through the row maximum so it cannot overflow."""
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    s = scale * (q @ np.asarray(K, dtype=np.float64).T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    out = (e / z) @ np.asarray(V, dtype=np.float64)
    return out, (m + np.log(z))[:, 0]


def attend(q_rows, K, V, comp_dims, ck, cv, sink: int, recent: int, scale: float, period: int = 0):
    """Several queries of one KV head over the compressed cache.

    Every row of q_rows [n, D] attends to all L cached tokens, with no mask
    between the rows: the attention the pages' kernel serves in prefill as well
    as in decode [SKILL Architecture overview, Practical guidance].  Returns
    (out [n, D], lse [n]); the lse lets a caller combine this attention with
    attention over tokens that are not in the cache (a prefill chunk's own).
    """
    Kt = approximate_cache(K, comp_dims, ck, sink, recent, period)
    Vt = approximate_cache(V, comp_dims, cv, sink, recent, period)
    return softmax_attention_lse(q_rows, Kt, Vt, scale)


# ------------------------------------------------------ streaming append --

def retained(X: np.ndarray, sink: int, recent: int) -> np.ndarray:
    """The rows a sequence keeps exactly, in token order [SKILL Step 3]: all L
    rows when there is no middle, else the first ``sink`` and the last
    ``recent`` rows."""
    X = np.asarray(X)
    start, M = segment(X.shape[0], sink, recent)
    if M == 0:
        return X.copy()
    return np.concatenate([X[:start], X[start + M:]], axis=0)


def append(coef: np.ndarray, kept: np.ndarray, x_new: np.ndarray, L: int, sink: int,
           recent: int, period: int):
    """One token appended to a compressed sequence of length L, under the
    fixed-period reading (``fourier_basis`` with ``period`` P > 0; the pages
    give no update rule for a growing middle).

    ``coef`` [k, c] are the middle's coefficients, ``kept`` [min(L, sink +
    recent), c] the retained rows in token order, ``x_new`` [c] the new token's
    row.  The new token is the last recent token; the token that leaves the
    recent window (the first recent one, or the new token itself when
    ``recent`` is 0) becomes middle position tau = M and adds its term
    phi_n(M) x to every coefficient.  Returns (coef, kept) of length L + 1.
    """
    coef = np.array(coef, dtype=np.float64, copy=True)
    kept = np.asarray(kept, dtype=np.float64)
    x_new = np.asarray(x_new, dtype=np.float64)
    _, M = segment(L, sink, recent)
    _, M1 = segment(L + 1, sink, recent)
    if M1 == M:  # still no middle: the new token is kept
        return coef, np.concatenate([kept, x_new[None, :]], axis=0)
    # the middle grows by one position, tau = M
    if recent > 0:
        leaving = kept[sink]
        kept = np.concatenate([kept[:sink], kept[sink + 1:], x_new[None, :]], axis=0)
    else:
        leaving = x_new
    phi_M = fourier_basis(M + 1, coef.shape[0], period)[M]
    return coef + np.outer(phi_M, leaving), kept


# ------------------------------------------------------ dimension analysis --

def dim_sensitivity(q_rows, K, V, noise, scale: float) -> np.ndarray:
    """Per-dim sensitivity of one head's attention output to noise on the
    values [SKILL Step 1, Architecture overview (dimension analysis stage)]:
    for each dim d, the values get ``noise[:, d]`` added to their dim d only,
    attention runs again, and the score is the Frobenius norm of the change of
    the outputs of the query rows ``q_rows`` [n, D] over the cache K, V
    [L, D].  ``noise`` [L, D] holds the pages' N(0, 0.1^2) draws, one column
    per perturbed dim, passed in.  Every query row attends to every token (the
    module's mask is not given; decode and ``attend`` use none).  Returns the
    squared norms [D] (the pages' score is their square root, summed over the
    heads and rows a caller aggregates before the root)."""
    q_rows = np.atleast_2d(np.asarray(q_rows, dtype=np.float64))
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    noise = np.asarray(noise, dtype=np.float64)
    base = softmax_attention(q_rows, K, V, scale)
    out = np.zeros(V.shape[1])
    for d in range(V.shape[1]):
        Vn = V.copy()
        Vn[:, d] += noise[:, d]
        diff = softmax_attention(q_rows, K, Vn, scale) - base
        out[d] = float((diff * diff).sum())
    return out


def exact_attention(q_rows, K, V, scale: float):
    """Uncompressed attention (context only: the approximation error)."""
    return softmax_attention(q_rows, K, V, scale)
