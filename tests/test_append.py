"""GPU parity of fa_append (streaming decode with a fixed basis period).

A cache is compressed at lengths L_b - a (fa_project), then the last a tokens
of each sequence are appended one call at a time (fa_append).  The result must
match the oracle's projection of the longer cache (the fixed-period reading
makes the two the same to rounding, pinned in tests/test_oracle.py): the
retained rows bit for bit, the coefficients to the projection's bars (fp32
max-abs 1e-5, bf16 relative L2 1e-3 per block), and a decode step over the
appended cache to the decode bars.  The cases cover sequences that stay
without a middle, that get their first middle token, and long ones; caches
without sink or recent tokens; fp32 and bf16.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from long_context_decode_fourier_amd import workloads as wl  # noqa: E402
from oracle import batch as ob  # noqa: E402

from test_parity import Run, _check_coefs, _check_out, _edges_ok, poisoned_workspace  # noqa: E402

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_decode_fourier_amd import binding
    binding.lib()
    return binding


# name: (config fields, final lengths, tokens appended one call at a time)
CASES = {
    # sink 32 / recent 64: a sequence that stays short (40 -> 43), one that gets
    # its first middle token on the way (94 -> 99), long ones
    "bf16_mixed": (dict(dtype="bf16", batch=4, n_q_heads=8, n_kv_heads=2, head_dim=128, n_comp=64,
                        n_coef=129, period=4096), [43, 99, 3000, 1777], 5),
    "f32_mixed": (dict(dtype="f32", batch=3, n_q_heads=4, n_kv_heads=2, head_dim=16, n_comp=8,
                       n_coef=9, period=700), [40, 99, 600], 4),
    # no recent window: the new token itself enters the middle
    "bf16_no_recent": (dict(dtype="bf16", batch=2, n_q_heads=4, n_kv_heads=4, head_dim=64, n_comp=32,
                            n_coef=33, sink=8, recent=0, period=1500), [1200, 10], 3),
    # no sink: the first recent token is retained row 0
    "bf16_no_sink": (dict(dtype="bf16", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64, n_comp=32,
                          n_coef=65, sink=0, recent=24, period=2100), [2000, 30], 3),
    # a long two-pass-sized middle and k past the one-pass limit
    "bf16_long": (dict(dtype="bf16", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, n_comp=64,
                       n_coef=2401, period=12000), [9003], 2),
}


def _new_rows(w1, lens, which):
    """[B, Hkv, Dc] compressible rows of token lens[b] of each block of w1."""
    c = w1.cfg
    X = w1.kc if which == "k" else w1.vc
    out = np.zeros((c.batch, c.n_kv_heads, c.n_comp), dtype=X.dtype)
    for b in range(c.batch):
        for h in range(c.n_kv_heads):
            out[b, h] = w1.block(X, b, h)[int(lens[b])]
    return out


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_matches_projection_of_longer_cache(fb, name):
    kw, lens, n_app = CASES[name]
    cfg = wl.custom(name=name, seed=400 + sorted(CASES).index(name), **kw)
    _say("case %s final lens=%s appends %d period %d" % (name, lens, n_app, cfg.period))
    w1 = wl.make(cfg, lens=lens)
    lens0 = w1.lens - n_app
    run = Run(fb, w1.truncated(lens0))
    run.project()
    # the appended state lives in run's ck / cv / ke / ve
    for a in range(n_app):
        cur = lens0 + a
        desc = fb.Desc(fb.BF16 if cfg.dtype == "bf16" else fb.F32, cfg.batch, cfg.n_q_heads,
                       cfg.n_kv_heads, cfg.head_dim, cfg.n_comp, cfg.n_coef, [int(x) for x in cur],
                       sink=cfg.sink, recent=cfg.recent, period=cfg.period)
        kn = fb.to_device(_new_rows(w1, cur, "k"))
        vn = fb.to_device(_new_rows(w1, cur, "v"))
        fb.append(desc, kn, vn, run.ck, run.cv, run.ke, run.ve)
    torch.cuda.synchronize()
    # retained rows: bit for bit those of the longer cache
    full = Run(fb, w1)
    full.ke, full.ve, full.ck, full.cv = run.ke, run.ve, run.ck, run.cv
    _edges_ok(full)
    # coefficients: the oracle's projection of the longer cache
    ck_o, cv_o = ob.project_all(w1)
    got_k = run.ck.cpu().numpy().astype(np.float64)
    got_v = run.cv.cpu().numpy().astype(np.float64)
    _check_coefs(w1, got_k, got_v, ck_o, cv_o)
    # a decode step over the appended cache
    want = ob.decode_all(w1, ck_o, cv_o, full.scale)
    _check_out(w1, full.decode(), want, "decode after append")


def test_append_then_project_agree_on_gpu(fb):
    """fa_append of one token and fa_project of the longer cache, both on the
    GPU, agree to the coefficient bar (independent of the oracle)."""
    kw, lens, _ = CASES["bf16_mixed"]
    cfg = wl.custom(name="gpu_pair", seed=450, **kw)
    w1 = wl.make(cfg, lens=lens)
    lens0 = w1.lens - 1
    run = Run(fb, w1.truncated(lens0))
    run.project()
    desc0 = fb.Desc.from_workload(w1.truncated(lens0))
    fb.append(desc0, fb.to_device(_new_rows(w1, lens0, "k")), fb.to_device(_new_rows(w1, lens0, "v")),
              run.ck, run.cv, run.ke, run.ve)
    full = Run(fb, w1)
    ck1, cv1 = full.project()
    _check_coefs(w1, run.ck.cpu().numpy().astype(np.float64), run.cv.cpu().numpy().astype(np.float64),
                 ck1, cv1)
    assert torch.equal(run.ke, full.ke) and torch.equal(run.ve, full.ve)
