"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin checks the oracle against one of: numpy's FFT (a library routine the
pages' own code uses), closed forms, invariants of orthonormal projections and
of softmax attention, PyTorch's CPU attention (a library routine), the pages'
printed defaults (tests/golden/pages_facts.json) and brute force with
pure-Python loops on tiny inputs.  ``test_mutants_are_caught`` plants plausible
mistakes in the oracle (on the CPU) and checks that some pin fails for each.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import fourier_attention as fa
from oracle import batch as ob
from long_context_decode_fourier_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


# ------------------------------------------------------------------ pins ----
# Each pin takes the oracle module (possibly mutated) and raises on failure.

def pin_orthonormal(o):
    """P-1: Phi^T Phi = I_k (the pages call the bases orthogonal; the abstract)."""
    for M, k in [(1, 1), (2, 2), (3, 3), (7, 7), (8, 8), (8, 5), (416, 33),
                 (416, 416), (1000, 201)]:
        P = o.fourier_basis(M, k)
        assert P.shape == (M, k)
        err = np.abs(P.T @ P - np.eye(k)).max()
        assert err < 1e-12, (M, k, err)


def pin_rfft(o):
    """P-2: coefficients equal scaled real/imag parts of numpy.fft.rfft."""
    rng = _rng(1)
    for M in (5, 8, 13, 416):
        x = rng.standard_normal(M)
        X = np.fft.rfft(x)
        c = o.project(x[:, None], M)[:, 0]
        assert abs(c[0] - X[0].real / math.sqrt(M)) < 1e-12
        for j in range(1, (M + 1) // 2):
            assert abs(c[2 * j - 1] - math.sqrt(2.0 / M) * X[j].real) < 1e-12
            assert abs(c[2 * j] + math.sqrt(2.0 / M) * X[j].imag) < 1e-12
        if M % 2 == 0:
            assert abs(c[M - 1] - X[M // 2].real / math.sqrt(M)) < 1e-12


def pin_irfft_lowpass(o):
    """P-3: the pages' reconstruction (keep the first bins of rfft, zero-pad,
    irfft with n = M; skill page Steps 2 and 4) equals reconstruct(project(x))
    for k = 2P + 1 real coefficients <-> P + 1 kept bins."""
    rng = _rng(2)
    for M, P in [(9, 2), (16, 3), (416, 16), (4000, 200), (7, 3)]:
        k = 2 * P + 1
        x = rng.standard_normal((M, 3))
        X = np.fft.rfft(x, axis=0)
        kept = np.zeros_like(X)
        kept[:P + 1] = X[:P + 1]
        ref = np.fft.irfft(kept, n=M, axis=0)
        got = o.reconstruct(o.project(x, k), M)
        assert np.abs(got - ref).max() < 1e-12, (M, P)


def pin_parseval_bessel(o):
    """P-4: k = M reconstructs exactly and keeps the energy (Parseval); k < M
    loses energy (Bessel) and leaves a residual orthogonal to every basis fn."""
    rng = _rng(3)
    for M in (6, 7, 64, 415):
        x = rng.standard_normal((M, 2))
        c = o.project(x, M)
        assert np.abs(o.reconstruct(c, M) - x).max() < 1e-11
        assert abs((c ** 2).sum() - (x ** 2).sum()) < 1e-9 * (x ** 2).sum()
        k = max(1, M // 3)
        ck = o.project(x, k)
        assert (ck ** 2).sum() <= (x ** 2).sum() + 1e-12
        resid = x - o.reconstruct(ck, M)
        assert np.abs(o.fourier_basis(M, k).T @ resid).max() < 1e-10


def pin_closed_form(o):
    """P-5: A sin(2 pi j tau / M + ph) has exactly two non-zero coefficients,
    A sqrt(M/2) sin(ph) on the cosine and A sqrt(M/2) cos(ph) on the sine of
    frequency j; a constant c has only c sqrt(M) on the constant term."""
    M, k = 48, 21
    tau = np.arange(M)
    for j, A, ph in [(1, 1.0, 0.3), (4, -2.5, 2.0), (10, 0.7, -1.1)]:
        x = A * np.sin(2 * np.pi * j * tau / M + ph)
        c = o.project(x[:, None], k)[:, 0]
        want = np.zeros(k)
        want[2 * j - 1] = A * math.sqrt(M / 2) * math.sin(ph)
        want[2 * j] = A * math.sqrt(M / 2) * math.cos(ph)
        assert np.abs(c - want).max() < 1e-12, j
    c = o.project(np.full((M, 1), 3.0), k)[:, 0]
    want = np.zeros(k)
    want[0] = 3.0 * math.sqrt(M)
    assert np.abs(c - want).max() < 1e-12


def pin_golden_basis(o):
    """Hand-derived basis values for M = 4 (tests/golden/basis_m4.json)."""
    with open(os.path.join(GOLDEN, "basis_m4.json")) as f:
        g = json.load(f)
    P = o.fourier_basis(g["M"], g["k"])
    assert np.abs(P - np.array(g["phi"])).max() < 1e-15


def pin_segment(o):
    """Segmentation follows the pages' Step 3 slicing: initial = the first 32
    tokens, recent = the last 64, middle in between; no middle when the
    sequence is not longer than both (tests/golden/pages_facts.json)."""
    with open(os.path.join(GOLDEN, "pages_facts.json")) as f:
        facts = json.load(f)
    S, R = facts["preserve_initial"], facts["preserve_recent"]
    for L in (512, 4096, 97, 96, 50, 1):
        toks = list(range(L))
        start, M = o.segment(L, S, R)
        if L > S + R:
            middle = toks[S:L - R]
            assert (start, M) == (middle[0], len(middle)), L
        else:
            assert M == 0, L


def _tiny_case(seed, L=8, D=4, Dc=2, S=1, R=1, k=3, G=2):
    rng = _rng(seed)
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    q = rng.standard_normal((G, D))
    comp = np.array(sorted(rng.permutation(D)[:Dc]), dtype=np.int64)
    return K, V, q, comp, S, R, k


def _brute_force(K, V, q, comp, S, R, k, scale):
    """Pure-Python loops: basis, projection, reconstruction, attention."""
    L, D = len(K), len(K[0])
    M = max(0, L - S - R)
    Kt = [list(map(float, row)) for row in K]
    Vt = [list(map(float, row)) for row in V]
    if M > 0:
        def phi(n, t):
            f = (n + 1) // 2
            r = (f * t) % M
            a = 1.0 / math.sqrt(M) if (f == 0 or 2 * f == M) else math.sqrt(2.0 / M)
            trig = math.cos if (n == 0 or n % 2 == 1) else math.sin
            return a * trig(2.0 * math.pi * r / M)
        for X, Xt in ((K, Kt), (V, Vt)):
            for d in comp:
                coef = [sum(phi(n, t) * float(X[S + t][d]) for t in range(M))
                        for n in range(k)]
                for t in range(M):
                    Xt[S + t][d] = sum(phi(n, t) * coef[n] for n in range(k))
    outs = []
    for qi in q:
        s = [scale * sum(float(qi[d]) * Kt[t][d] for d in range(D)) for t in range(L)]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        z = sum(e)
        outs.append([sum(e[t] * Vt[t][d] for t in range(L)) / z for d in range(D)])
    return np.array(outs)


def _oracle_decode(o, K, V, q, comp, S, R, k, scale):
    start, M = o.segment(len(K), S, R)
    if M > 0:
        ck = o.project(K[start:start + M][:, comp], k)
        cv = o.project(V[start:start + M][:, comp], k)
    else:
        ck = cv = np.zeros((k, len(comp)))
    return o.decode(q, K, V, comp, ck, cv, S, R, scale)


def pin_brute_force(o):
    """P-8: the whole pipeline against pure-Python loops on tiny inputs."""
    cases = [dict(), dict(L=7, k=5), dict(L=6, D=3, Dc=3, k=4), dict(L=2),
             dict(L=8, S=2, R=2, k=4, G=3), dict(L=5, Dc=0, k=1)]
    for i, kw in enumerate(cases):
        K, V, q, comp, S, R, k = _tiny_case(10 + i, **kw)
        scale = 0.7
        want = _brute_force(K, V, q, comp, S, R, k, scale)
        got = _oracle_decode(o, K, V, q, comp, S, R, k, scale)
        assert np.abs(got - want).max() < 1e-12, (i, kw)


def _sdpa(q, K, V, scale):
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q)[None, None], t(K)[None, None], t(V)[None, None], scale=scale)
    return out[0, 0].numpy()


def pin_reduces_to_attention(o):
    """P-6: k = M, no compressible dims, or L <= S + R leave the cache exact,
    so decode equals PyTorch's CPU scaled-dot-product attention."""
    rng = _rng(5)
    for L, D, Dc, S, R, kfull in [(40, 8, 4, 3, 5, True), (40, 8, 0, 3, 5, False),
                                  (8, 8, 4, 3, 5, False), (200, 16, 7, 32, 64, True)]:
        K = rng.standard_normal((L, D))
        V = rng.standard_normal((L, D))
        q = rng.standard_normal((3, D))
        comp = np.sort(rng.permutation(D)[:Dc]).astype(np.int64)
        start, M = o.segment(L, S, R)
        k = M if (kfull and M > 0) else 1
        got = _oracle_decode(o, K, V, q, comp, S, R, k, 0.3)
        assert np.abs(got - _sdpa(q, K, V, 0.3)).max() < 1e-12, (L, Dc)


def pin_factored(o):
    """P-7: scores scale*(q_U.k_U + a.phi(tau)) with a = q_C C_K^T, and values
    o_U + W C_V with W = sum_tau p phi(tau): the factored form the GPU computes
    equals reconstruct-then-attend."""
    rng = _rng(6)
    L, D, Dc, S, R, k, G = 300, 16, 10, 32, 64, 37, 3
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    q = rng.standard_normal((G, D))
    comp = np.sort(rng.permutation(D)[:Dc])
    exact = np.setdiff1d(np.arange(D), comp)
    start, M = o.segment(L, S, R)
    ck = o.project(K[start:start + M][:, comp], k)
    cv = o.project(V[start:start + M][:, comp], k)
    got = o.decode(q, K, V, comp, ck, cv, S, R, 0.25)
    # factored form, written independently here
    P = o.fourier_basis(M, k)
    mid = np.zeros(L, bool)
    mid[start:start + M] = True
    s = 0.25 * (q @ K.T)
    s[:, mid] = 0.25 * (q[:, exact] @ K[mid][:, exact].T) + (0.25 * q[:, comp] @ ck.T) @ P.T
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    out = np.zeros((G, D))
    out[:, exact] = p @ V[:, exact]
    W = p[:, mid] @ P
    out[:, comp] = p[:, ~mid] @ V[~mid][:, comp] + W @ cv
    assert np.abs(got - out).max() < 1e-12


def pin_softmax_invariants(o):
    """P-9: probabilities sum to 1, outputs lie in the convex hull of V's rows,
    equal scores average V, and one dominant score selects its row."""
    rng = _rng(7)
    K = rng.standard_normal((50, 6))
    V = rng.standard_normal((50, 6))
    q = rng.standard_normal((4, 6))
    out, p = o.softmax_attention(q, K, V, 0.5, return_probs=True)
    assert np.abs(p.sum(1) - 1).max() < 1e-14
    assert (out <= V.max(0) + 1e-12).all() and (out >= V.min(0) - 1e-12).all()
    flat = o.softmax_attention(np.zeros((1, 6)), K, V, 0.5)
    assert np.abs(flat[0] - V.mean(0)).max() < 1e-13
    Kd = K.copy()
    Kd[17] = 1e3 * q[0]
    dom = o.softmax_attention(q[:1], Kd, V, 1.0)
    assert np.abs(dom[0] - V[17]).max() < 1e-12


def pin_gqa_stacking(o):
    """P-10: a GQA workload's batched oracle equals separate single-head calls
    with query head i reading KV head i // G, and decode of stacked query rows
    equals one call per row."""
    cfg = wl.custom(dtype="f32", batch=2, n_q_heads=6, n_kv_heads=2, head_dim=8,
                    n_comp=3, n_coef=5, sink=2, recent=3, mask="seeded", seed=9)
    w = wl.make(cfg, lens=[20, 13])
    ck, cv = ob.project_all(w)
    out = ob.decode_all(w, ck, cv, 0.4)
    for b in range(2):
        for i in range(6):
            h = i // 3
            K, V = w.natural_kv(b, h)
            q = w.f64(w.q[b, i])[None]
            single = o.decode(q, K, V, w.comp_dims(h), ck[b * 2 + h], cv[b * 2 + h],
                              2, 3, 0.4)
            assert np.abs(out[b, i] - single[0]).max() < 1e-13


def _brute_force_lse(K, V, q, comp, S, R, k, scale):
    """Pure-Python log sum_t exp(s_t) per query row over the reconstructed keys
    (the reconstruction of _brute_force, then math.log of a plain sum)."""
    L, D = len(K), len(K[0])
    M = max(0, L - S - R)
    Kt = [list(map(float, row)) for row in K]
    if M > 0:
        def phi(n, t):
            f = (n + 1) // 2
            r = (f * t) % M
            a = 1.0 / math.sqrt(M) if (f == 0 or 2 * f == M) else math.sqrt(2.0 / M)
            trig = math.cos if (n == 0 or n % 2 == 1) else math.sin
            return a * trig(2.0 * math.pi * r / M)
        for d in comp:
            coef = [sum(phi(n, t) * float(K[S + t][d]) for t in range(M)) for n in range(k)]
            for t in range(M):
                Kt[S + t][d] = sum(phi(n, t) * coef[n] for n in range(k))
    return np.array([math.log(sum(math.exp(scale * sum(float(qi[d]) * Kt[t][d] for d in range(D)))
                                  for t in range(L))) for qi in q])


def _oracle_attend(o, K, V, q, comp, S, R, k, scale):
    start, M = o.segment(len(K), S, R)
    if M > 0:
        ck = o.project(K[start:start + M][:, comp], k)
        cv = o.project(V[start:start + M][:, comp], k)
    else:
        ck = cv = np.zeros((k, len(comp)))
    return o.attend(q, K, V, comp, ck, cv, S, R, scale)


def pin_attend_brute_force(o):
    """Several queries of one KV head: outputs equal one decode per query row
    and the pure-Python loops; lse equals a pure-Python log of the plain sum of
    exp(s_t) over the reconstructed keys."""
    cases = [dict(G=5), dict(L=7, k=5, G=3), dict(L=2, G=4), dict(L=8, S=2, R=2, k=4, G=6)]
    for i, kw in enumerate(cases):
        K, V, q, comp, S, R, k = _tiny_case(30 + i, **kw)
        out, lse = _oracle_attend(o, K, V, q, comp, S, R, k, 0.6)
        assert np.abs(out - _brute_force(K, V, q, comp, S, R, k, 0.6)).max() < 1e-12, (i, kw)
        assert np.abs(lse - _brute_force_lse(K, V, q, comp, S, R, k, 0.6)).max() < 1e-12, (i, kw)
        for r in range(len(q)):
            one = _oracle_decode(o, K, V, q[r:r + 1], comp, S, R, k, 0.6)
            assert np.abs(out[r] - one[0]).max() < 1e-13


def pin_lse_closed_form(o):
    """lse in closed form: zero keys give s = 0, so lse = log L; keys all equal
    to kappa give s = scale q . kappa for every token, so lse = that + log L."""
    rng = _rng(11)
    L, D = 37, 6
    V = rng.standard_normal((L, D))
    q = rng.standard_normal((3, D))
    _, lse0 = o.softmax_attention_lse(q, np.zeros((L, D)), V, 0.9)
    assert np.abs(lse0 - math.log(L)).max() < 1e-13
    kappa = rng.standard_normal(D)
    _, lse1 = o.softmax_attention_lse(q, np.tile(kappa, (L, 1)), V, 0.9)
    assert np.abs(lse1 - (0.9 * q @ kappa + math.log(L))).max() < 1e-12


def pin_lse_merge(o):
    """What the lse is for: attention over the cache and over further tokens
    (a prefill chunk's own) combine into attention over their union, with
    weights exp(lse_part - lse_union) and lse_union = logaddexp of the parts.
    Checked against PyTorch's CPU attention over the concatenated keys."""
    rng = _rng(12)
    L, D, Dc, S, R, k = 120, 8, 5, 4, 6, 110
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    q = rng.standard_normal((4, D))
    comp = np.sort(rng.permutation(D)[:Dc])
    Kn = rng.standard_normal((9, D))
    Vn = rng.standard_normal((9, D))
    start, M = o.segment(L, S, R)
    out1, lse1 = o.attend(q, K, V, comp, o.project(K[start:start + M][:, comp], k),
                          o.project(V[start:start + M][:, comp], k), S, R, 0.5)
    out2, lse2 = o.softmax_attention_lse(q, Kn, Vn, 0.5)
    lse = np.logaddexp(lse1, lse2)
    merged = np.exp(lse1 - lse)[:, None] * out1 + np.exp(lse2 - lse)[:, None] * out2
    Kt = o.approximate_cache(K, comp, o.project(K[start:start + M][:, comp], k), S, R)
    Vt = o.approximate_cache(V, comp, o.project(V[start:start + M][:, comp], k), S, R)
    want = _sdpa(q, np.vstack([Kt, Kn]), np.vstack([Vt, Vn]), 0.5)
    assert np.abs(merged - want).max() < 1e-12
    s = 0.5 * q @ np.vstack([Kt, Kn]).T
    assert np.abs(lse - np.log(np.exp(s).sum(1))).max() < 1e-12


def pin_coef_budget(o):
    """The pages' budget keeps the first int(fraction * M) rfft bins [SKILL
    Steps 2-3]; coef_budget must give the k whose projector Phi_k Phi_k^T is
    exactly that low-pass (numpy's irfft of the zero-padded bins), for the
    pages' fraction 0.3 (tests/golden/pages_facts.json) and for fractions that
    reach the Nyquist bin and the whole spectrum."""
    with open(os.path.join(GOLDEN, "pages_facts.json")) as f:
        frac0 = json.load(f)["example_coefficient_fraction"]
    rng = _rng(13)
    for M in (4, 7, 8, 10, 33, 416, 1000):
        x = rng.standard_normal(M)
        for frac in (frac0, 0.55, 0.7, 1.0):
            bins = int(frac * M)
            if bins < 1:
                continue
            X = np.fft.rfft(x)
            X[bins:] = 0
            low = np.fft.irfft(X, n=M)
            k = o.coef_budget(M, frac)
            P = o.fourier_basis(M, k)
            assert np.abs(P @ (P.T @ x) - low).max() < 1e-12, (M, frac, k)
    assert o.coef_budget(3, 0.3) == 1  # no bin kept: the constant at least


def pin_cache_bytes(o):
    """Cache sizes on a worked example: one f32 head, L = 100, D = 4 (2
    compressible), sink = recent = 1, k = 3: full 2*100*4*4 = 3200 bytes;
    compressed = exact dims 2*100*2*4 + retained rows 2*2*2*4 + coefficients
    2*3*2*4 = 1680 bytes; a second sequence of 2 tokens has no middle and
    keeps both rows (2*2*4*4 = 64 bytes either way)."""
    cfg = wl.custom(dtype="f32", batch=2, n_q_heads=1, n_kv_heads=1, head_dim=4, n_comp=2,
                    n_coef=3, sink=1, recent=1, mask="low", seed=14)
    w = wl.make(cfg, lens=[100, 2])
    assert ob.cache_bytes(w) == (3200 + 64, 1680 + 64)


def pin_fixed_period_basis(o):
    """A fixed period P reduces to the pinned basis: the first M rows of the
    period-P basis (M <= P), for odd and even P (the Nyquist cosine); P = M is
    the plain basis."""
    for M, k, P in [(5, 3, 12), (7, 7, 8), (1, 4, 4), (9, 9, 9), (10, 6, 15)]:
        np.testing.assert_allclose(o.fourier_basis(M, k, P), o.fourier_basis(P, k)[:M], atol=1e-14)
    np.testing.assert_allclose(o.fourier_basis(6, 4, 6), o.fourier_basis(6, 4), atol=1e-14)


def pin_fixed_period_complete(o):
    """With k = P the period-P basis is complete over its window: the middle
    rows come back exactly from their coefficients (the window's unfilled
    positions act as zeros)."""
    x = _rng(31).standard_normal((9, 3))
    for P in (9, 12, 13):
        c = o.project(x, P, period=P)
        np.testing.assert_allclose(o.reconstruct(c, 9, period=P), x, atol=1e-12)
        # and the energy is kept (Parseval over the window)
        np.testing.assert_allclose((c * c).sum(0), (x * x).sum(0), rtol=1e-12)


def _stream(o, X, L0, S, R, k, P):
    """Compress X[:L0], then append X[L0], X[L0+1], ... one at a time."""
    start, M = o.segment(L0, S, R)
    coef = o.project(X[start:start + M], k, period=P)
    kept = o.retained(X[:L0], S, R)
    for L in range(L0, X.shape[0]):
        coef, kept = o.append(coef, kept, X[L], L, S, R, P)
    return coef, kept


def pin_append_equals_project(o):
    """Appending token by token gives what compressing the longer sequence at
    once gives: the same retained rows and (to rounding) the same coefficients,
    across the step where the sequence first gets a middle, with and without
    sink and recent tokens."""
    X = _rng(32).standard_normal((40, 3))
    for S, R, L0, k, P in [(2, 3, 1, 5, 48), (2, 3, 6, 7, 40), (0, 4, 2, 3, 37),
                           (3, 0, 3, 6, 50), (0, 0, 1, 4, 41), (2, 3, 20, 9, 64)]:
        coef, kept = _stream(o, X, L0, S, R, k, P)
        start, M = o.segment(40, S, R)
        np.testing.assert_allclose(coef, o.project(X[start:start + M], k, period=P), atol=1e-12)
        np.testing.assert_array_equal(kept, o.retained(X, S, R))


def pin_append_brute_force(o):
    """Pure-Python loops: the coefficients of a streamed sequence are
    sum_tau phi_n(tau) x[S + tau] with the period-P cos/sin written out."""
    X = _rng(33).standard_normal((14, 2))
    S, R, k, P = 2, 3, 5, 16
    coef, kept = _stream(o, X, 1, S, R, k, P)
    M = 14 - S - R
    for n in range(k):
        f = (n + 1) // 2
        a = 1 / math.sqrt(P) if (f == 0 or 2 * f == P) else math.sqrt(2 / P)
        for c in range(2):
            want = 0.0
            for tau in range(M):
                ang = 2 * math.pi * f * tau / P
                want += a * (math.cos(ang) if (n == 0 or n % 2 == 1) else math.sin(ang)) * X[S + tau, c]
            assert abs(coef[n, c] - want) < 1e-12, (n, c)
    assert kept.shape == (S + R, 2)
    assert np.array_equal(kept[:S], X[:S]) and np.array_equal(kept[S:], X[14 - R:])


def pin_sensitivity_linear(o):
    """Noise on one dim of the values changes only that dim of the outputs, by
    the attention probabilities applied to the noise (linearity of attention
    in V): the score of dim d is |P noise[:, d]|^2 with P the softmax of the
    unperturbed scores, whatever V holds."""
    rng = _rng(41)
    L, D, n = 30, 6, 4
    K, V, q = rng.standard_normal((L, D)), rng.standard_normal((L, D)), rng.standard_normal((n, D))
    eps = 0.1 * rng.standard_normal((L, D))
    got = o.dim_sensitivity(q, K, V, eps, 0.4)
    s = 0.4 * q @ K.T
    P = np.exp(s - s.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    np.testing.assert_allclose(got, ((P @ eps) ** 2).sum(0), rtol=1e-9, atol=1e-15)
    # V does not enter; a dim without noise scores 0
    eps2 = eps.copy()
    eps2[:, 2] = 0.0
    got2 = o.dim_sensitivity(q, K, 5.0 * V + 1.0, eps2, 0.4)
    np.testing.assert_allclose(np.delete(got2, 2), np.delete(got, 2), rtol=1e-9, atol=1e-15)
    assert abs(got2[2]) < 1e-24


def pin_sensitivity_uniform(o):
    """Zero queries attend uniformly: each row's change in dim d is the mean
    noise of dim d over the L tokens, so the score is n * mean^2."""
    rng = _rng(42)
    L, D, n = 17, 5, 3
    eps = 0.1 * rng.standard_normal((L, D))
    got = o.dim_sensitivity(np.zeros((n, D)), rng.standard_normal((L, D)), rng.standard_normal((L, D)), eps, 1.0)
    np.testing.assert_allclose(got, n * eps.mean(0) ** 2, rtol=1e-9, atol=1e-18)


def pin_sensitivity_brute_force(o):
    """Pure-Python loops: perturb dim d of V, rerun attention, sum the squared
    changes of every output entry."""
    rng = _rng(43)
    L, D, n, scale = 5, 3, 2, 0.7
    K, V, q = rng.standard_normal((L, D)), rng.standard_normal((L, D)), rng.standard_normal((n, D))
    eps = 0.1 * rng.standard_normal((L, D))

    def attn(Vm):
        out = []
        for i in range(n):
            sc = [scale * sum(q[i][j] * K[t][j] for j in range(D)) for t in range(L)]
            m = max(sc)
            e = [math.exp(x - m) for x in sc]
            z = sum(e)
            out.append([sum(e[t] / z * Vm[t][j] for t in range(L)) for j in range(D)])
        return out

    base = attn(V.tolist())
    got = o.dim_sensitivity(q, K, V, eps, scale)
    for d in range(D):
        Vn = V.tolist()
        for t in range(L):
            Vn[t][d] += eps[t][d]
        pert = attn(Vn)
        want = sum((pert[i][j] - base[i][j]) ** 2 for i in range(n) for j in range(D))
        assert abs(got[d] - want) < 1e-12 * max(1.0, want), (d, got[d], want)


PINS = [pin_orthonormal, pin_rfft, pin_irfft_lowpass, pin_parseval_bessel,
        pin_closed_form, pin_golden_basis, pin_segment, pin_brute_force,
        pin_reduces_to_attention, pin_factored, pin_softmax_invariants,
        pin_gqa_stacking, pin_attend_brute_force, pin_lse_closed_form, pin_lse_merge,
        pin_coef_budget, pin_cache_bytes, pin_fixed_period_basis, pin_fixed_period_complete,
        pin_append_equals_project, pin_append_brute_force, pin_sensitivity_linear,
        pin_sensitivity_uniform, pin_sensitivity_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(fa)


# --------------------------------------------------------------- mutants ----
# Plausible mistakes planted in the oracle (CPU only).  Each must fail a pin.

def _basis_variant(**mut):
    def basis(M, k, period=0):
        P = M if (period == 0 or mut.get("period_ignored")) else period
        if not (1 <= k <= P) or M > P:
            raise ValueError
        tau = np.arange(M, dtype=np.int64) + mut.get("tau_shift", 0)
        n = np.arange(k)
        f = n // 2 if mut.get("freq_off") else (n + 1) // 2
        ang = 2 * np.pi * (np.outer(tau, f) % P) / P
        use_cos = (n == 0) | (n % 2 == 1)
        if mut.get("swap"):
            use_cos = (n == 0) | ((n % 2 == 0) & (n > 0))
        sin = -np.sin(ang) if mut.get("neg_sin") else np.sin(ang)
        phi = np.where(use_cos[None], np.cos(ang), sin)
        a = np.where((f == 0) | (2 * f == P), 1 / np.sqrt(P), np.sqrt(2 / P))
        if mut.get("nyquist"):
            a = np.where(f == 0, 1 / np.sqrt(P), np.sqrt(2 / P))
        if mut.get("no_scale"):
            a = np.ones_like(a)
        if mut.get("period_scale_m"):  # angle over P but the scale of M
            a = np.where((f == 0) | (2 * f == M), 1 / np.sqrt(max(M, 1)), np.sqrt(2 / max(M, 1)))
        return phi * a[None]
    return basis


def _append_variant(**mut):
    def append(coef, kept, x_new, L, sink, recent, period):
        coef = np.array(coef, dtype=np.float64, copy=True)
        kept = np.asarray(kept, dtype=np.float64)
        _, M = fa.segment(L, sink, recent)
        _, M1 = fa.segment(L + 1, sink, recent)
        if M1 == M:
            return coef, np.concatenate([kept, x_new[None, :]], axis=0)
        if recent > 0:
            leaving = kept[-1] if mut.get("last_recent") else kept[sink]
            if mut.get("wrong_end"):  # drops the newest recent row instead of the oldest
                kept = np.concatenate([kept[:-1], x_new[None, :]], axis=0)
            else:
                kept = np.concatenate([kept[:sink], kept[sink + 1:], x_new[None, :]], axis=0)
        else:
            leaving = np.zeros_like(x_new) if mut.get("r0_dropped") else x_new
        tau = M + 1 if mut.get("next_phase") else M
        phi = fa.fourier_basis(tau + 1, coef.shape[0], period)[tau]
        return coef + np.outer(phi, leaving), kept
    return append


def _decode_no_scale(q_rows, K, V, comp_dims, ck, cv, sink, recent, scale, period=0):
    Kt = fa.approximate_cache(K, comp_dims, ck, sink, recent, period)
    Vt = fa.approximate_cache(V, comp_dims, cv, sink, recent, period)
    return fa.softmax_attention(q_rows, Kt, Vt, 1.0)


def _decode_values_exact(q_rows, K, V, comp_dims, ck, cv, sink, recent, scale, period=0):
    Kt = fa.approximate_cache(K, comp_dims, ck, sink, recent, period)
    return fa.softmax_attention(q_rows, Kt, V, scale)


def _segment_off_by_one(L, sink, recent):
    return sink + 1, max(0, L - sink - recent)


def _segment_keeps_recent_short(L, sink, recent):
    return sink, max(0, L - sink)


def _approx_wrong_dims(X, comp_dims, coef, sink, recent, period=0):
    X = np.array(X, dtype=np.float64, copy=True)
    start, M = fa.segment(X.shape[0], sink, recent)
    cd = np.sort(np.asarray(comp_dims))[::-1]  # dims permuted vs the coefficients
    if M > 0 and cd.size > 0:
        X[start:start + M][:, cd] = fa.reconstruct(coef, M, period)
    return X


def _softmax_transposed_v(q, K, V, scale, return_probs=False):
    q = np.atleast_2d(q)
    s = scale * (q @ K.T)
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    out = p @ V[::-1]
    return (out, p) if return_probs else out


def _lse_log2(q, K, V, scale):
    out, lse = _ORIG_LSE(q, K, V, scale)
    return out, lse / math.log(2.0)


def _lse_no_max(q, K, V, scale):
    out, lse = _ORIG_LSE(q, K, V, scale)
    s = scale * (np.atleast_2d(q) @ np.asarray(K).T)
    return out, lse - s.max(1)


def _attend_values_exact(q_rows, K, V, comp_dims, ck, cv, sink, recent, scale, period=0):
    Kt = fa.approximate_cache(K, comp_dims, ck, sink, recent, period)
    return fa.softmax_attention_lse(q_rows, Kt, V, scale)


_ORIG_LSE = fa.softmax_attention_lse


def _budget_plus_one_pair(M, fraction=0.3):
    return min(M, 2 * int(fraction * M) + 1)

def _sens_variant(**mut):
    def dim_sensitivity(q_rows, K, V, noise, scale):
        q_rows = np.atleast_2d(np.asarray(q_rows, dtype=np.float64))
        K, V, noise = (np.asarray(x, dtype=np.float64) for x in (K, V, noise))
        base = fa.softmax_attention(q_rows, K, V, scale)
        out = np.zeros(V.shape[1])
        for d in range(V.shape[1]):
            Vn, Kn = V.copy(), K.copy()
            if mut.get("all_dims"):
                Vn += noise
            elif mut.get("keys"):
                Kn[:, d] += noise[:, d]
            else:
                Vn[:, d] += noise[:, d]
            col = (d + 1) % V.shape[1] if mut.get("wrong_column") else d
            if mut.get("wrong_column"):
                Vn = V.copy()
                Vn[:, d] += noise[:, col]
            diff = fa.softmax_attention(q_rows, Kn, Vn, scale) - base
            out[d] = float(np.sqrt((diff * diff).sum())) if mut.get("root") else float((diff * diff).sum())
        return out
    return dim_sensitivity


MUTANTS = {
    "sin_cos_swapped": ("fourier_basis", _basis_variant(swap=True)),
    "sin_sign": ("fourier_basis", _basis_variant(neg_sin=True)),
    "freq_off_by_one": ("fourier_basis", _basis_variant(freq_off=True)),
    "nyquist_scale": ("fourier_basis", _basis_variant(nyquist=True)),
    "no_normalisation": ("fourier_basis", _basis_variant(no_scale=True)),
    "phase_origin": ("fourier_basis", _basis_variant(tau_shift=1)),
    "decode_no_scale": ("decode", _decode_no_scale),
    "values_not_reconstructed": ("decode", _decode_values_exact),
    "segment_off_by_one": ("segment", _segment_off_by_one),
    "segment_drops_recent": ("segment", _segment_keeps_recent_short),
    "comp_dims_permuted": ("approximate_cache", _approx_wrong_dims),
    "value_rows_reversed": ("softmax_attention", _softmax_transposed_v),
    "lse_log2": ("softmax_attention_lse", _lse_log2),
    "lse_without_max": ("softmax_attention_lse", _lse_no_max),
    "attend_values_not_reconstructed": ("attend", _attend_values_exact),
    "budget_one_pair_too_many": ("coef_budget", _budget_plus_one_pair),
    "period_ignored": ("fourier_basis", _basis_variant(period_ignored=True)),
    "period_scale_of_middle": ("fourier_basis", _basis_variant(period_scale_m=True)),
    "append_last_recent_leaves": ("append", _append_variant(last_recent=True)),
    "append_window_shifted_at_wrong_end": ("append", _append_variant(wrong_end=True)),
    "append_no_recent_drops_token": ("append", _append_variant(r0_dropped=True)),
    "append_phase_one_ahead": ("append", _append_variant(next_phase=True)),
    "sensitivity_noise_on_every_dim": ("dim_sensitivity", _sens_variant(all_dims=True)),
    "sensitivity_noise_on_keys": ("dim_sensitivity", _sens_variant(keys=True)),
    "sensitivity_noise_column_shifted": ("dim_sensitivity", _sens_variant(wrong_column=True)),
    "sensitivity_norm_not_squared": ("dim_sensitivity", _sens_variant(root=True)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(fa, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin(fa)
        except AssertionError:  # a wrong value; other exceptions do not count
            failed.append(pin.__name__)
        except Exception:  # noqa: BLE001
            pass
    assert failed, "mutant %s passed every pin" % name


def test_k_greater_than_m_rejected():
    with pytest.raises(ValueError):
        fa.fourier_basis(4, 5)
    with pytest.raises(ValueError):
        fa.fourier_basis(4, 0)
