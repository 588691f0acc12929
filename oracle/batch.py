"""Batched drivers of the oracle over a whole workload (CPU, float64).

TEST INFRASTRUCTURE (see ``oracle/fourier_attention.py``).  These loops only
walk the (sequence, KV head) blocks of a workload and call the per-head oracle;
they add no arithmetic.  The workload object is duck-typed (``cfg``, ``lens``,
``natural_kv``, ``comp_dims``, ``q``, ``f64``); nothing from the GPU library is
imported.

Query head i of a sequence reads KV head ``i // (Hq / Hkv)`` (a reading: the
pages do not discuss grouped heads).
"""
from __future__ import annotations

import numpy as np

from . import fourier_attention as fa


def _period(c):
    """The workload's basis period: 0 (each sequence's own M) or a fixed P."""
    return getattr(c, "period", 0)


def _pkw(c):
    p = _period(c)
    return {"period": p} if p else {}


def project_block(w, b: int, h: int):
    """(C_K, C_V) [k, Dc] of sequence b, KV head h; zeros when M = 0."""
    c = w.cfg
    K, V = w.natural_kv(b, h)
    start, M = fa.segment(K.shape[0], c.sink, c.recent)
    cd = w.comp_dims(h)
    if M == 0:
        z = np.zeros((c.n_coef, c.n_comp))
        return z, z.copy()
    return (fa.project(K[start:start + M][:, cd], c.n_coef, **_pkw(c)),
            fa.project(V[start:start + M][:, cd], c.n_coef, **_pkw(c)))


def project_all(w):
    """Coefficients for every block, in the library's [B*Hkv, k, Dc] layout."""
    c = w.cfg
    ck = np.zeros((c.batch * c.n_kv_heads, c.n_coef, c.n_comp))
    cv = np.zeros_like(ck)
    for b in range(c.batch):
        for h in range(c.n_kv_heads):
            ck[b * c.n_kv_heads + h], cv[b * c.n_kv_heads + h] = project_block(w, b, h)
    return ck, cv


def decode_block(w, ck_blk, cv_blk, scale: float, b: int, h: int, heads=None):
    """Outputs [len(heads), D] for the query heads of KV head h in sequence b.

    ``heads`` defaults to all G query heads that read KV head h.
    """
    c = w.cfg
    G = c.n_q_heads // c.n_kv_heads
    if heads is None:
        heads = list(range(h * G, (h + 1) * G))
    K, V = w.natural_kv(b, h)
    q = w.f64(w.q[b, heads])
    return fa.decode(q, K, V, w.comp_dims(h), ck_blk, cv_blk,
                     c.sink, c.recent, scale, **_pkw(c))


def decode_all(w, ck, cv, scale: float):
    """out [B, Hq, D] for every query row, given coefficients [B*Hkv, k, Dc]."""
    c = w.cfg
    G = c.n_q_heads // c.n_kv_heads
    out = np.zeros((c.batch, c.n_q_heads, c.head_dim))
    for b in range(c.batch):
        for h in range(c.n_kv_heads):
            i = b * c.n_kv_heads + h
            out[b, h * G:(h + 1) * G] = decode_block(w, ck[i], cv[i], scale, b, h)
    return out


def attend_all(w, ck, cv, scale: float):
    """(out [B, nq, Hq, D], lse [B, nq, Hq]) for a workload with nq queries per
    sequence (``w.q`` [B, nq, Hq, D], or [B, Hq, D] when nq = 1): the nq * G
    query rows of KV head h are attended in one call of the per-head oracle."""
    c = w.cfg
    G = c.n_q_heads // c.n_kv_heads
    q4 = w.q if w.q.ndim == 4 else w.q[:, None]
    nq = q4.shape[1]
    out = np.zeros((c.batch, nq, c.n_q_heads, c.head_dim))
    lse = np.zeros((c.batch, nq, c.n_q_heads))
    for b in range(c.batch):
        for h in range(c.n_kv_heads):
            i = b * c.n_kv_heads + h
            K, V = w.natural_kv(b, h)
            q = w.f64(q4[b, :, h * G:(h + 1) * G]).reshape(nq * G, c.head_dim)
            o, l = fa.attend(q, K, V, w.comp_dims(h), ck[i], cv[i], c.sink, c.recent, scale,
                             **_pkw(c))
            out[b, :, h * G:(h + 1) * G] = o.reshape(nq, G, c.head_dim)
            lse[b, :, h * G:(h + 1) * G] = l.reshape(nq, G)
    return out, lse


def append_all(w, ck, cv, ke, ve, k_new, v_new):
    """One appended token per sequence (``fa.append`` on every (sequence, KV
    head) block, K and V), for a workload with a fixed basis period.

    ck, cv [B*Hkv, k, Dc] and ke, ve [B*Hkv, S+R, Dc] (retained rows in token
    order, rows past min(L_b, S+R) unused) describe the cache at lengths
    ``w.lens``; k_new, v_new [B, Hkv, Dc] are the new token's compressible
    rows.  Returns the four arrays for lengths ``w.lens + 1``."""
    c = w.cfg
    ck, cv = np.array(ck, dtype=np.float64), np.array(cv, dtype=np.float64)
    ke, ve = np.array(ke, dtype=np.float64), np.array(ve, dtype=np.float64)
    for b in range(c.batch):
        L = int(w.lens[b])
        n = min(L, c.sink + c.recent)
        for h in range(c.n_kv_heads):
            i = b * c.n_kv_heads + h
            for C, E, x in ((ck, ke, k_new), (cv, ve, v_new)):
                C[i], kept = fa.append(C[i], E[i][:n], np.asarray(x[b, h], dtype=np.float64), L,
                                       c.sink, c.recent, _period(c))
                E[i][:kept.shape[0]] = kept
    return ck, cv, ke, ve


def dim_sensitivity_all(w, noise, scale: float):
    """Squared per-dim sensitivities [Hq, D] of a workload [SKILL Step 1]:
    entry (i, d) sums, over the sequences and the n_query queries, the squared
    change of query head i's outputs when ``noise[:, d]`` (``noise`` [rows, D],
    natural dim order, packed like the cache rows) is added to dim d of its
    KV head's values.  The pages' score of dim d is sqrt(sum_i entry (i, d))."""
    c = w.cfg
    G = c.n_q_heads // c.n_kv_heads
    q4 = w.q if w.q.ndim == 4 else w.q[:, None]
    out = np.zeros((c.n_q_heads, c.head_dim))
    for b in range(c.batch):
        for h in range(c.n_kv_heads):
            K, V = w.natural_kv(b, h)
            eps = w.natural_rows(noise, b, h)
            for i in range(h * G, (h + 1) * G):
                q = w.f64(q4[b, :, i])
                out[i] += fa.dim_sensitivity(q, K, V, eps, scale)
    return out


def cache_bytes(w):
    """(uncompressed, compressed) bytes of the workload's KV cache: K and V in
    full (the sizes of the natural [L, D] arrays), versus the exact dims of
    every token, the compressible dims of the retained rows and the float32
    coefficients of every (sequence, KV head) with a middle [SKILL Step 3]."""
    c = w.cfg
    esz = np.dtype(w.storage_dtype).itemsize
    full = comp = 0
    for b in range(c.batch):
        for h in range(c.n_kv_heads):
            K, V = w.natural_kv(b, h)
            full += (K.size + V.size) * esz
            comp += 2 * K.shape[0] * c.n_exact * esz  # kx, vx: exact dims of every token
            start, M = fa.segment(K.shape[0], c.sink, c.recent)
            kept = K.shape[0] - M
            comp += 2 * kept * c.n_comp * esz
            if M > 0 and c.n_comp > 0:
                comp += 2 * c.n_coef * c.n_comp * 4
    return full, comp
