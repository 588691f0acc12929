"""C-ABI checks that need no GPU: the library loads, exports every function
include/fa.h declares, and host validation returns its status codes before any
HIP call (so these run on a machine without a GPU)."""
import ctypes
import os
import re

import pytest

from long_context_decode_fourier_amd import binding as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fb.LIB_PATH),
                                reason="libfa.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert {"fa_project", "fa_decode", "fa_project_workspace_size",
            "fa_decode_workspace_size", "fa_status_string", "fa_last_error",
            "fa_version"} <= set(names)
    L = ctypes.CDLL(fb.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert fb.lib().fa_version() >= 100


def test_status_strings():
    for code in range(7):
        assert fb.lib().fa_status_string(code)


def _desc(**kw):
    base = dict(dtype=fb.BF16, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                n_comp_dims=64, n_coef=33, seq_len=[4096, 1000])
    base.update(kw)
    return fb.Desc(**base)


def _size(fn, d):
    n = ctypes.c_size_t(0)
    st = fn(ctypes.byref(d.c), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 3),
    (dict(batch=0, seq_len=[]), 2),
    (dict(batch=65, seq_len=[100] * 65), 2),
    (dict(n_q_heads=7), 2),
    (dict(n_kv_heads=0), 2),
    (dict(head_dim=0), 2),
    (dict(head_dim=512), 2),
    (dict(n_comp_dims=129), 2),
    (dict(n_comp_dims=-1), 2),
    (dict(n_coef=0), 2),
    (dict(n_coef=4098), 2),
    (dict(seq_len=[4096, 0]), 2),
    (dict(seq_len=[4096, 120]), 2),   # 24 middle tokens < 33 coefficients
    (dict(sink=-1), 2),
    (dict(period=-1), 2),
    (dict(period=3000), 2),          # sequence 0's middle (4000) exceeds the period
    (dict(period=4000, n_coef=4001), 2),  # k past the period
])
def test_invalid_desc(kw, code):
    d = _desc(**kw)
    for fn in (fb.lib().fa_project_workspace_size, fb.lib().fa_decode_workspace_size):
        st, _ = _size(fn, d)
        assert st == code, (kw, st, fb.lib().fa_last_error())
        assert fb.lib().fa_last_error()


def test_workspace_sizes_and_short_sequences():
    d = _desc()
    st, n = _size(fb.lib().fa_decode_workspace_size, d)
    assert st == 0 and n > 0 and n % 256 == 0
    st, n = _size(fb.lib().fa_project_workspace_size, d)
    assert st == 0 and n % 256 == 0
    # sequences not longer than sink + recent have no middle: any k is accepted
    st, _ = _size(fb.lib().fa_decode_workspace_size, _desc(seq_len=[96, 50], n_coef=4000))
    assert st == 0
    # no compressible dims: k is not checked against the middle length
    st, _ = _size(fb.lib().fa_decode_workspace_size, _desc(n_comp_dims=0, seq_len=[100, 100]))
    assert st == 0


def test_fixed_period_accepts_k_past_the_middle():
    # with a fixed period, k is bounded by the period, not by each middle
    st, _ = _size(fb.lib().fa_decode_workspace_size, _desc(period=5000, n_coef=2049, seq_len=[4096, 200]))
    assert st == 0, fb.lib().fa_last_error()
    st, _ = _size(fb.lib().fa_project_workspace_size, _desc(period=5000, n_coef=2049, seq_len=[4096, 200]))
    assert st == 0, fb.lib().fa_last_error()


GB = 1 << 30  # fake device addresses, 1 GiB apart; every call below fails validation


def _call_decode(d, q=1, kx=2, vx=3, ke=4, ve=5, ck=6, cv=7, out=8, ws=9 * GB, nws=1 << 30):
    P = lambda v: ctypes.c_void_p(v * GB if 0 < v < 64 else v)
    return fb.lib().fa_decode(ctypes.byref(d.c), P(q), P(kx), P(vx), P(ke), P(ve), P(ck), P(cv),
                              ctypes.c_float(0.1), P(out), P(ws), nws, None)


def test_decode_host_errors_without_gpu():
    dims_holder = type("T", (), {"data_ptr": lambda self: 10 * GB})()
    d = _desc(dims=dims_holder)
    assert _call_decode(d, q=0) == 1
    assert _call_decode(d, out=0) == 1
    assert _call_decode(d, kx=0) == 1
    assert _call_decode(d, ke=0) == 1
    assert _call_decode(d, ck=0) == 1
    assert _call_decode(d, ws=0) == 4
    assert _call_decode(d, nws=16) == 4
    assert _call_decode(d, ws=9 * GB + 8) == 4          # misaligned workspace
    assert _call_decode(d, out=1 * GB + 64) == 6         # out inside q
    assert _call_decode(d, ws=3 * GB + 256) == 6         # workspace inside vx
    assert _call_decode(_desc()) == 1                    # desc.dims missing


def test_project_host_errors_without_gpu():
    d = _desc()
    P = lambda v: ctypes.c_void_p(v)
    f = fb.lib().fa_project
    base = 1 << 40
    # nothing to project
    assert f(ctypes.byref(d.c), P(0), P(0), P(0), P(0), P(0), P(0), P(0), 0, None) == 1
    # kc without ck
    assert f(ctypes.byref(d.c), P(base), P(0), P(0), P(0), P(0), P(0), P(0), 0, None) == 1
    # ck overlapping kc
    assert f(ctypes.byref(d.c), P(base), P(0), P(base + 64), P(0), P(0), P(0), P(0), 0, None) == 6
    # misaligned kc (bf16 path needs 16-byte rows)
    assert f(ctypes.byref(d.c), P(base + 2), P(0), P(base * 2), P(0), P(0), P(0),
             P(base * 3), 1 << 30, None) == 2
    # workspace too small: one long sequence over few tiles always splits the
    # middle, so this plan needs a workspace (checked before the call)
    dl = _desc(batch=1, n_q_heads=1, n_kv_heads=1, seq_len=[131136])
    assert _size(fb.lib().fa_project_workspace_size, dl)[1] > 16
    assert f(ctypes.byref(dl.c), P(base), P(0), P(base * 2), P(0), P(0), P(0), P(base * 3),
             16, None) == 4
    # bf16 projection needs Dc % 4 == 0
    d10 = _desc(n_comp_dims=10)
    assert f(ctypes.byref(d10.c), P(base), P(0), P(base * 2), P(0), P(0), P(0), P(base * 3),
             1 << 30, None) == 2


def _attend_size(d, nq):
    n = ctypes.c_size_t(0)
    st = fb.lib().fa_attend_workspace_size(ctypes.byref(d.c), nq, ctypes.byref(n))
    return st, n.value


def test_attend_workspace_and_limits():
    d = _desc()
    # one query per sequence is fa_decode
    assert _attend_size(d, 1) == _size(fb.lib().fa_decode_workspace_size, d)
    st4, n4 = _attend_size(d, 4)
    assert st4 == 0 and n4 > _attend_size(d, 1)[1] and n4 % 256 == 0
    assert _attend_size(d, 0)[0] == 2
    assert _attend_size(d, 1025)[0] == 2
    big = _desc(n_q_heads=1 << 15, n_kv_heads=1 << 14)  # 2^15 heads x 4 queries: too many rows
    assert _attend_size(big, 4)[0] == 2 and "query rows" in fb.lib().fa_last_error().decode()
    # more query rows than one pass over the cache holds run as several passes
    # that share one workspace: 64 and 1024 queries need no more than one pass
    st64, n64 = _attend_size(d, 64)
    st1k, n1k = _attend_size(d, 1024)
    assert st64 == 0 and st1k == 0 and n1k == n64


def _call_attend(d, nq, q=1, out=8, lse=0, ws=9 * GB, nws=1 << 30):
    P = lambda v: ctypes.c_void_p(v * GB if 0 < v < 64 else v)
    return fb.lib().fa_attend(ctypes.byref(d.c), nq, P(q), P(2), P(3), P(4), P(5), P(6), P(7),
                              ctypes.c_float(0.1), P(out), P(lse), P(ws), nws, None)


def test_attend_host_errors_without_gpu():
    dims_holder = type("T", (), {"data_ptr": lambda self: 10 * GB})()
    d = _desc(dims=dims_holder)
    assert _call_attend(d, 0) == 2
    assert _call_attend(d, 2, q=0) == 1
    assert _call_attend(d, 2, lse=8 * GB + 64) == 6      # lse inside out
    assert _call_attend(d, 2, lse=1 * GB + 64) == 6      # lse inside q
    assert _call_attend(d, 2, lse=9 * GB + 256) == 6     # lse inside the workspace
    assert _call_attend(d, 2, nws=16) == 4


def test_coef_budget_matches_oracle():
    from oracle import fourier_attention as fa
    for M in list(range(1, 70)) + [416, 4000, 32672, 131040]:
        for frac in (0.0, 0.1, 0.3, 0.5, 0.55, 0.7, 1.0):
            assert fb.coef_budget(M, frac) == fa.coef_budget(M, frac), (M, frac)
    assert fb.coef_budget(0, 0.3) == 0 and fb.coef_budget(10, 1.5) == 0
    assert fb.coef_budget(10, float("nan")) == 0


def test_cache_bytes_matches_oracle():
    from long_context_decode_fourier_amd import workloads as wl
    from oracle import batch as ob
    cases = [(wl.custom(dtype="bf16", batch=3, n_q_heads=4, n_kv_heads=2, head_dim=16, n_comp=6,
                        n_coef=9, seed=1), [300, 50, 105]),
             (wl.custom(dtype="f32", batch=1, n_q_heads=2, n_kv_heads=2, head_dim=8, n_comp=0,
                        n_coef=1, seed=2), [40]),
             (wl.CONFIGS["llama2_7b_layer"], None)]
    for cfg, lens in cases:
        w = wl.make(cfg, lens=lens)
        d = fb.Desc.from_workload(w)
        assert fb.cache_bytes(d) == ob.cache_bytes(w), cfg.name


def test_decode_noalloc_rejects_oversized_without_gpu():
    """fa_decode_noalloc refuses a shape whose workspace exceeds its static
    scratch array, before any HIP call."""
    dims_holder = type("T", (), {"data_ptr": lambda self: 10 * GB})()
    d = _desc(batch=64, n_q_heads=256, n_kv_heads=8, n_coef=4097, seq_len=[1 << 20] * 64,
              dims=dims_holder)
    st, need = _size(fb.lib().fa_decode_workspace_size, d)
    assert st == 0 and need > fb.NOALLOC_SCRATCH_BYTES
    P = lambda v: ctypes.c_void_p(v * GB)
    st = fb.lib().fa_decode_noalloc(ctypes.byref(d.c), P(1), P(2), P(3), P(4), P(5), P(6), P(7),
                                    ctypes.c_float(0.1), P(8), None)
    assert st == 4
    assert "static scratch" in fb.lib().fa_last_error().decode()
    # invalid shapes report their own code first
    assert fb.lib().fa_decode_noalloc(ctypes.byref(_desc(n_coef=0).c), P(1), P(2), P(3), P(4), P(5),
                                      P(6), P(7), ctypes.c_float(0.1), P(8), None) == 2


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    import re as _re
    mib = int(_re.search(r"#define FA_NOALLOC_SCRATCH_MIB (\d+)", text).group(1))
    assert fb.NOALLOC_SCRATCH_BYTES == mib << 20


def _call_append(d, kn=1, vn=2, ck=3, cv=4, ke=5, ve=6):
    P = lambda v: ctypes.c_void_p(v * GB if 0 < v < 64 else v)
    return fb.lib().fa_append(ctypes.byref(d.c), P(kn), P(vn), P(ck), P(cv), P(ke), P(ve), None)


def test_append_host_errors_without_gpu():
    # the basis must have a fixed period
    assert _call_append(_desc()) == 2
    assert "period" in fb.lib().fa_last_error().decode()
    d = _desc(period=4500)
    # a middle that would pass the period: 4500 - 4000 = 500 more tokens fit, then no more
    assert _call_append(_desc(period=4000, seq_len=[4096, 1000])) == 2
    assert _call_append(d, kn=0) == 1
    assert _call_append(d, ve=0) == 1
    assert _call_append(d, cv=0) == 1
    assert _call_append(d, ck=1) == 6                     # ck overlaps k_new
    assert _call_append(d, ke=3) == 6                     # ke overlaps ck
    # no compressible dims: nothing to do, every pointer may be NULL
    assert _call_append(_desc(period=4500, n_comp_dims=0), 0, 0, 0, 0, 0, 0) == 0


def test_dim_sensitivity_host_errors_without_gpu():
    d = _desc(n_coef=5000, period=0)  # k and the dim split are ignored by the analysis
    n = ctypes.c_size_t(0)
    assert fb.lib().fa_dim_sensitivity_workspace_size(ctypes.byref(d.c), 4, ctypes.byref(n)) == 0, \
        fb.lib().fa_last_error()
    assert n.value > 0 and n.value % 256 == 0
    assert fb.lib().fa_dim_sensitivity_workspace_size(ctypes.byref(d.c), 0, ctypes.byref(n)) == 2
    P = lambda v: ctypes.c_void_p(v * GB if 0 < v < 64 else v)
    f = fb.lib().fa_dim_sensitivity
    args = lambda q=1, k=2, nz=3, sq=4, ws=5, nws=1 << 40: (ctypes.byref(d.c), 4, P(q), P(k), P(nz),
                                                            ctypes.c_float(0.1), P(sq), P(ws), nws, None)
    assert f(*args(q=0)) == 1
    assert f(*args(nz=0)) == 1
    assert f(*args(sq=0)) == 1
    assert f(*args(ws=0)) == 4
    assert f(*args(nws=64)) == 4
    assert f(*args(sq=2)) == 6  # sq inside k
    assert f(*args(sq=5)) == 6  # sq inside the workspace


def test_check_mode_adds_a_flag_slot(monkeypatch):
    d = _desc()
    st, n0 = _size(fb.lib().fa_decode_workspace_size, d)
    st2, p0 = _size(fb.lib().fa_project_workspace_size, d)
    assert st == 0 and st2 == 0
    monkeypatch.setenv("FA_CHECK", "1")
    st, n1 = _size(fb.lib().fa_decode_workspace_size, d)
    st2, p1 = _size(fb.lib().fa_project_workspace_size, d)
    assert st == 0 and st2 == 0
    assert n1 == (n0 + 255) // 256 * 256 + 256 and p1 == (p0 + 255) // 256 * 256 + 256
    monkeypatch.setenv("FA_CHECK", "0")
    assert _size(fb.lib().fa_decode_workspace_size, d)[1] == n0
