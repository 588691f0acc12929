"""Pins of the oracle's batched drivers (oracle/batch.py).

The drivers only walk the (sequence, KV head) blocks of a workload and call
the per-head oracle, whose arithmetic is pinned in test_oracle.py.  What can go
wrong in them is placement: which rows form a block, which block index a
(sequence, KV head) pair gets, which KV head a query head reads, how the
n_query * G query rows of a KV head are ordered, and the zero coefficients of
a sequence without middle tokens.  Each pin rebuilds the blocks here from the
raw cache arrays with the documented row formula (row of sequence b, KV head h,
token t = Hkv * (L_0 + ... + L_{b-1}) + h * L_b + t; exact dims listed first in
dims[h]) and compares the drivers with one call of the pinned per-head oracle
per block or per query row.  ``test_batch_mutants_are_caught`` plants plausible
placement mistakes in the drivers (on the CPU) and checks that a pin fails for
each.
"""
import numpy as np
import pytest

from long_context_decode_fourier_amd import workloads as wl
from oracle import batch as ob
from oracle import fourier_attention as fa

SCALE = 0.35


def _workload(n_query=1):
    # ragged lengths with one sequence shorter than sink + recent (no middle),
    # three query heads per KV head
    cfg = wl.custom(name="batch_pin", dtype="f32", batch=3, n_q_heads=6, n_kv_heads=2,
                    head_dim=8, n_comp=3, n_coef=5, sink=3, recent=4, mask="seeded",
                    seed=21 + n_query, n_query=n_query)
    return wl.make(cfg, lens=[40, 6, 23])


def _rows(w, X, b, h):
    """Rows of (sequence b, KV head h) of a dim-split array, by the row formula."""
    c = w.cfg
    off = int(np.sum(w.lens[:b]))
    r0 = c.n_kv_heads * off + h * int(w.lens[b])
    return X[r0:r0 + int(w.lens[b])]


def _natural(w, b, h):
    """(K, V) [L, D] float64 of block (b, h), natural dim order, rebuilt here."""
    c = w.cfg
    L = int(w.lens[b])
    exact, comp = w.dims[h, :c.n_exact], w.dims[h, c.n_exact:]
    out = []
    for Xx, Xc in ((w.kx, w.kc), (w.vx, w.vc)):
        A = np.full((L, c.head_dim), np.nan)
        A[:, exact] = _rows(w, Xx, b, h).astype(np.float64)
        A[:, comp] = _rows(w, Xc, b, h).astype(np.float64)
        assert np.isfinite(A).all()
        out.append(A)
    return out


def _coefs(w):
    """Coefficients [B*Hkv, k, Dc] from fa.project of each block's middle rows."""
    c = w.cfg
    ck = np.full((c.batch * c.n_kv_heads, c.n_coef, c.n_comp), np.nan)
    cv = np.full_like(ck, np.nan)
    for b in range(c.batch):
        for h in range(c.n_kv_heads):
            L = int(w.lens[b])
            M = L - c.sink - c.recent
            for X, C in ((w.kc, ck), (w.vc, cv)):
                if M > 0:
                    mid = _rows(w, X, b, h)[c.sink:c.sink + M].astype(np.float64)
                    C[b * c.n_kv_heads + h] = fa.project(mid, c.n_coef)
                else:
                    C[b * c.n_kv_heads + h] = 0.0
    return ck, cv


def pin_project_blocks(o):
    """project_all / project_block: block b*Hkv + h holds the projection of the
    middle rows of (b, h), K and V in that order; a sequence without middle
    tokens gets zero coefficients."""
    w = _workload()
    c = w.cfg
    want_k, want_v = _coefs(w)
    got_k, got_v = o.project_all(w)
    assert got_k.shape == want_k.shape and got_v.shape == want_v.shape
    assert np.abs(got_k - want_k).max() < 1e-12
    assert np.abs(got_v - want_v).max() < 1e-12
    assert not got_k[1 * c.n_kv_heads:2 * c.n_kv_heads].any()  # sequence 1: L = 6 <= 3 + 4
    for b in range(c.batch):
        for h in range(c.n_kv_heads):
            bk, bv = o.project_block(w, b, h)
            i = b * c.n_kv_heads + h
            assert np.abs(bk - want_k[i]).max() < 1e-12 and np.abs(bv - want_v[i]).max() < 1e-12


def pin_decode_rows(o):
    """decode_all / decode_block: query head i of sequence b equals one call of
    fa.decode for that row alone, over KV head i // G and block b*Hkv + h."""
    w = _workload()
    c = w.cfg
    G = c.n_q_heads // c.n_kv_heads
    ck, cv = _coefs(w)
    got = o.decode_all(w, ck, cv, SCALE)
    assert got.shape == (c.batch, c.n_q_heads, c.head_dim)
    for b in range(c.batch):
        for i in range(c.n_q_heads):
            h = i // G
            K, V = _natural(w, b, h)
            q = w.q[b, i].astype(np.float64)[None]
            want = fa.decode(q, K, V, w.dims[h, c.n_exact:], ck[b * c.n_kv_heads + h],
                             cv[b * c.n_kv_heads + h], c.sink, c.recent, SCALE)[0]
            assert np.abs(got[b, i] - want).max() < 1e-12, (b, i)
    # a subset of a KV head's query heads, in the order asked for
    b, h = 2, 1
    sub = o.decode_block(w, ck[b * c.n_kv_heads + h], cv[b * c.n_kv_heads + h], SCALE, b, h,
                         heads=[5, 3])
    assert np.abs(sub - got[b, [5, 3]]).max() < 1e-12


def pin_attend_rows(o):
    """attend_all: query t of head i of sequence b (q [B, nq, Hq, D]) equals one
    call of fa.attend for that row alone, outputs and log-sum-exp; with one
    query per sequence (q [B, Hq, D]) the result is fa.decode's."""
    for nq in (3, 1):
        w = _workload(nq)
        c = w.cfg
        G = c.n_q_heads // c.n_kv_heads
        ck, cv = _coefs(w)
        out, lse = o.attend_all(w, ck, cv, SCALE)
        assert out.shape == (c.batch, nq, c.n_q_heads, c.head_dim)
        assert lse.shape == (c.batch, nq, c.n_q_heads)
        q4 = w.q if w.q.ndim == 4 else w.q[:, None]
        for b in range(c.batch):
            for t in range(nq):
                for i in range(c.n_q_heads):
                    h = i // G
                    K, V = _natural(w, b, h)
                    blk = b * c.n_kv_heads + h
                    o_want, l_want = fa.attend(q4[b, t, i].astype(np.float64)[None], K, V,
                                               w.dims[h, c.n_exact:], ck[blk], cv[blk],
                                               c.sink, c.recent, SCALE)
                    assert np.abs(out[b, t, i] - o_want[0]).max() < 1e-12, (nq, b, t, i)
                    assert abs(lse[b, t, i] - l_want[0]) < 1e-12, (nq, b, t, i)
        if nq == 1:
            assert np.abs(out[:, 0] - o.decode_all(w, ck, cv, SCALE)).max() < 1e-12


def _period_workload():
    # fixed basis period 48 (every middle of the lengths + 1 fits); sequence 1
    # gets its first middle token on the append (L = 7 = sink + recent), and
    # sequence 3 stays without one (L = 5)
    cfg = wl.custom(name="batch_append", dtype="f32", batch=4, n_q_heads=6, n_kv_heads=2,
                    head_dim=8, n_comp=3, n_coef=5, sink=3, recent=4, mask="seeded", seed=29,
                    period=48)
    return wl.make(cfg, lens=[41, 8, 23, 6])


def _kept_rows(w, X, b, h):
    """Retained rows of block (b, h) in token order, padded to sink + recent."""
    c = w.cfg
    rows = _rows(w, X, b, h).astype(np.float64)
    L = rows.shape[0]
    out = np.zeros((c.sink + c.recent, rows.shape[1]))
    kept = rows if L <= c.sink + c.recent else np.concatenate([rows[:c.sink], rows[L - c.recent:]])
    out[:kept.shape[0]] = kept
    return out


def pin_append_blocks(o):
    """append_all: each (sequence, KV head) block, K and V, takes its own new
    row; the result equals the coefficients (fixed period) and retained rows
    of the longer cache, built here block by block.  project_all passes the
    workload's period to the per-block projection."""
    w1 = _period_workload()
    c = w1.cfg
    w0 = w1.truncated(w1.lens - 1)
    P = c.period
    nb = c.batch * c.n_kv_heads

    def state(w):
        ck = np.zeros((nb, c.n_coef, c.n_comp))
        cv = np.zeros_like(ck)
        ke = np.zeros((nb, c.sink + c.recent, c.n_comp))
        ve = np.zeros_like(ke)
        for b in range(c.batch):
            M = max(0, int(w.lens[b]) - c.sink - c.recent)
            for h in range(c.n_kv_heads):
                i = b * c.n_kv_heads + h
                for X, C, E in ((w.kc, ck, ke), (w.vc, cv, ve)):
                    if M > 0:
                        C[i] = fa.project(_rows(w, X, b, h)[c.sink:c.sink + M].astype(np.float64),
                                          c.n_coef, period=P)
                    E[i] = _kept_rows(w, X, b, h)
        return ck, cv, ke, ve

    ck0, cv0, ke0, ve0 = state(w0)
    k_new = np.zeros((c.batch, c.n_kv_heads, c.n_comp))
    v_new = np.zeros_like(k_new)
    for b in range(c.batch):
        for h in range(c.n_kv_heads):
            k_new[b, h] = _rows(w1, w1.kc, b, h)[-1]
            v_new[b, h] = _rows(w1, w1.vc, b, h)[-1]
    got = o.append_all(w0, ck0, cv0, ke0, ve0, k_new, v_new)
    want = state(w1)
    for g, x in zip(got, want):
        assert g.shape == x.shape and np.abs(g - x).max() < 1e-12
    for b in (0, 2):  # middles longer than k
        for h in range(c.n_kv_heads):
            bk, bv = o.project_block(w1, b, h)
            i = b * c.n_kv_heads + h
            assert np.abs(bk - want[0][i]).max() < 1e-12 and np.abs(bv - want[1][i]).max() < 1e-12
    pk, pv = o.project_all(w1)
    assert np.abs(pk - want[0]).max() < 1e-12 and np.abs(pv - want[1]).max() < 1e-12


def pin_sensitivity_rows(o):
    """dim_sensitivity_all: entry (i, d) sums fa.dim_sensitivity of query head
    i's rows (every query of every sequence) over KV head i // G's cache and
    its noise rows, rebuilt here by the row formula."""
    for nq in (1, 3):
        w = _workload(nq)
        c = w.cfg
        G = c.n_q_heads // c.n_kv_heads
        rng = np.random.Generator(np.random.PCG64(5))
        noise = 0.1 * rng.standard_normal((int(c.n_kv_heads * w.lens.sum()), c.head_dim))
        got = o.dim_sensitivity_all(w, noise, SCALE)
        assert got.shape == (c.n_q_heads, c.head_dim)
        q4 = w.q if w.q.ndim == 4 else w.q[:, None]
        want = np.zeros_like(got)
        for b in range(c.batch):
            for i in range(c.n_q_heads):
                h = i // G
                K, V = _natural(w, b, h)
                eps = _rows(w, noise, b, h)
                want[i] += fa.dim_sensitivity(q4[b, :, i].astype(np.float64), K, V, eps, SCALE)
        assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())


PINS = [pin_project_blocks, pin_decode_rows, pin_attend_rows, pin_append_blocks, pin_sensitivity_rows]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(ob)


# --------------------------------------------------------------- mutants ----
# Placement mistakes planted in the drivers (CPU only).  Each must fail a pin.

_ORIG_PROJECT_BLOCK = ob.project_block
_ORIG_DECODE_BLOCK = ob.decode_block


def _project_all_index_swapped(w):
    c = w.cfg
    ck = np.zeros((c.batch * c.n_kv_heads, c.n_coef, c.n_comp))
    cv = np.zeros_like(ck)
    for b in range(c.batch):
        for h in range(c.n_kv_heads):
            ck[h * c.batch + b], cv[h * c.batch + b] = _ORIG_PROJECT_BLOCK(w, b, h)
    return ck, cv


def _project_block_kv_swapped(w, b, h):
    k, v = _ORIG_PROJECT_BLOCK(w, b, h)
    return v, k


def _project_block_empty_ones(w, b, h):
    c = w.cfg
    if int(w.lens[b]) <= c.sink + c.recent:
        z = np.ones((c.n_coef, c.n_comp))
        return z, z.copy()
    return _ORIG_PROJECT_BLOCK(w, b, h)


def _decode_block_next_head(w, ck_blk, cv_blk, scale, b, h, heads=None):
    # query heads of KV head h read the cache rows of the next KV head
    c = w.cfg
    G = c.n_q_heads // c.n_kv_heads
    if heads is None:
        heads = list(range(h * G, (h + 1) * G))
    K, V = w.natural_kv(b, (h + 1) % c.n_kv_heads)
    return fa.decode(w.f64(w.q[b, heads]), K, V, w.comp_dims(h), ck_blk, cv_blk,
                     c.sink, c.recent, scale)


def _decode_all_modulo_map(w, ck, cv, scale):
    # query head i -> KV head i % Hkv instead of i // G
    c = w.cfg
    out = np.zeros((c.batch, c.n_q_heads, c.head_dim))
    for b in range(c.batch):
        for i in range(c.n_q_heads):
            h = i % c.n_kv_heads
            out[b, i] = _ORIG_DECODE_BLOCK(w, ck[b * c.n_kv_heads + h], cv[b * c.n_kv_heads + h],
                                           scale, b, h, heads=[i])[0]
    return out


def _attend_all_rows_transposed(w, ck, cv, scale):
    # the (query, head) rows of a KV head stacked head-major, unstacked query-major
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
            q = w.f64(q4[b, :, h * G:(h + 1) * G]).transpose(1, 0, 2).reshape(nq * G, c.head_dim)
            o, l = fa.attend(q, K, V, w.comp_dims(h), ck[i], cv[i], c.sink, c.recent, scale)
            out[b, :, h * G:(h + 1) * G] = o.reshape(nq, G, c.head_dim)
            lse[b, :, h * G:(h + 1) * G] = l.reshape(nq, G)
    return out, lse


_ORIG_ATTEND_ALL = ob.attend_all


def _attend_all_lse_shifted(w, ck, cv, scale):
    out, lse = _ORIG_ATTEND_ALL(w, ck, cv, scale)
    return out, np.roll(lse, 1, axis=2)


_ORIG_APPEND_ALL = ob.append_all


def _append_all_kv_rows_swapped(w, ck, cv, ke, ve, k_new, v_new):
    return _ORIG_APPEND_ALL(w, ck, cv, ke, ve, v_new, k_new)


def _append_all_head_rows_rolled(w, ck, cv, ke, ve, k_new, v_new):
    return _ORIG_APPEND_ALL(w, ck, cv, ke, ve, np.roll(k_new, 1, axis=1), np.roll(v_new, 1, axis=1))


def _project_block_period_dropped(w, b, h):
    c = w.cfg
    K, V = w.natural_kv(b, h)
    start, M = fa.segment(K.shape[0], c.sink, c.recent)
    cd = w.comp_dims(h)
    if M == 0:
        z = np.zeros((c.n_coef, c.n_comp))
        return z, z.copy()
    return (fa.project(K[start:start + M][:, cd], c.n_coef),
            fa.project(V[start:start + M][:, cd], c.n_coef))


_ORIG_SENS_ALL = ob.dim_sensitivity_all


def _sens_all_noise_of_other_block(w, noise, scale):
    return _ORIG_SENS_ALL(w, np.roll(noise, 7, axis=0), scale)


def _sens_all_heads_reversed(w, noise, scale):
    return _ORIG_SENS_ALL(w, noise, scale)[::-1]


BATCH_MUTANTS = {
    "sensitivity_noise_rows_shifted": ("dim_sensitivity_all", _sens_all_noise_of_other_block),
    "sensitivity_query_heads_reversed": ("dim_sensitivity_all", _sens_all_heads_reversed),
    "append_all_k_v_rows_swapped": ("append_all", _append_all_kv_rows_swapped),
    "append_all_new_rows_of_other_head": ("append_all", _append_all_head_rows_rolled),
    "project_block_period_dropped": ("project_block", _project_block_period_dropped),
    "project_all_block_index_swapped": ("project_all", _project_all_index_swapped),
    "project_block_k_v_swapped": ("project_block", _project_block_kv_swapped),
    "project_block_no_middle_not_zero": ("project_block", _project_block_empty_ones),
    "decode_block_reads_next_kv_head": ("decode_block", _decode_block_next_head),
    "decode_all_head_map_modulo": ("decode_all", _decode_all_modulo_map),
    "attend_all_rows_transposed": ("attend_all", _attend_all_rows_transposed),
    "attend_all_lse_shifted": ("attend_all", _attend_all_lse_shifted),
}


@pytest.mark.parametrize("name", sorted(BATCH_MUTANTS))
def test_batch_mutants_are_caught(name, monkeypatch):
    attr, fn = BATCH_MUTANTS[name]
    monkeypatch.setattr(ob, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin(ob)
        except AssertionError:  # a wrong value; other exceptions do not count
            failed.append(pin.__name__)
        except Exception:  # noqa: BLE001
            pass
    assert failed, "mutant %s passed every pin" % name
