"""GPU parity of fa_attend (several queries per sequence over the compressed
cache) against the CPU oracle's ``attend``, through the C ABI.

Bars: outputs as for decode (fp32 inputs: max-abs <= 1e-5; bf16 inputs:
max-abs <= 3e-3); the log-sum-exp of each row to the same bars (it is a
weighted mean of the scores' errors, so it shares the outputs' error budget).
Each case runs end to end (GPU coefficients against oracle coefficients) and in
isolation (both sides fed the oracle's coefficients rounded to fp32).  The
cases cover 1, 3, 4, 8, 16, 40 and 300 queries, GQA groups of 1, 2 and 4 (3 to
600 query rows per KV head: the MFMA and the VALU edge blocks, and queries run
as several passes over the cache), a sequence without middle tokens, fp32
inputs, and sampled blocks of the LLaMA-3-8B-shaped batch with four queries
per sequence.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from long_context_decode_fourier_amd import workloads as wl  # noqa: E402
from oracle import batch as ob  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 3e-3}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_decode_fourier_amd import binding
    binding.lib()  # raises if libfa.so is missing: no fallback
    return binding


class AttendRun:
    def __init__(self, fb, w):
        self.fb, self.w, c = fb, w, w.cfg
        self.c = c
        self.dims = torch.from_numpy(w.dims).cuda()
        self.desc = fb.Desc.from_workload(w, self.dims)
        self.kc, self.vc = fb.to_device(w.kc), fb.to_device(w.vc)
        self.q = fb.to_device(w.q)
        self.kx = fb.to_device(w.kx) if w.kx is not None and w.kx.size else None
        self.vx = fb.to_device(w.vx) if w.vx is not None and w.vx.size else None
        nblk = c.batch * c.n_kv_heads
        self.ck = torch.full((nblk, c.n_coef, c.n_comp), float("nan"), device="cuda")
        self.cv = torch.full_like(self.ck, float("nan"))
        E = c.sink + c.recent
        self.ke = torch.zeros((nblk, E, c.n_comp), dtype=self.kc.dtype, device="cuda")
        self.ve = torch.zeros_like(self.ke)
        self.scale = 1.0 / np.sqrt(c.head_dim)
        ws = self.fb.workspace(self.fb.project_workspace_size(self.desc))
        ws.fill_(0xFF)  # NaN everywhere: reads of unwritten workspace show up
        self.fb.project(self.desc, self.kc, self.vc, self.ck, self.cv, self.ke, self.ve, ws)
        torch.cuda.synchronize()

    def attend(self, ck=None, cv=None, nq=None):
        c = self.c
        nq = c.n_query if nq is None else nq
        ck = self.ck if ck is None else torch.from_numpy(np.asarray(ck, np.float32)).cuda()
        cv = self.cv if cv is None else torch.from_numpy(np.asarray(cv, np.float32)).cuda()
        out = torch.full((c.batch, nq, c.n_q_heads, c.head_dim), float("nan"), device="cuda")
        lse = torch.full((c.batch, nq, c.n_q_heads), float("nan"), device="cuda")
        ws = self.fb.workspace(self.fb.attend_workspace_size(self.desc, nq))
        ws.fill_(0xFF)  # NaN everywhere: reads of unwritten workspace show up
        self.fb.attend(self.desc, nq, self.q, self.kx, self.vx, self.ke, self.ve, ck, cv,
                       self.scale, out, lse, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(w, got, want, what):
    (go, gl), (wo, wlse) = got, want
    eo, el = np.abs(go - wo).max(), np.abs(gl - wlse).max()
    _say("  %s: out max-abs %.2e, lse max-abs %.2e" % (what, eo, el))
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    assert eo <= TOL[w.cfg.dtype] and el <= TOL[w.cfg.dtype]


CASES = {
    "bf16_g4_q3_ragged": (dict(dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                               n_comp=64, n_coef=129, n_query=3), [700, 333]),
    "bf16_g1_q8": (dict(dtype="bf16", batch=1, n_q_heads=4, n_kv_heads=4, head_dim=128,
                        n_comp=64, n_coef=65, n_query=8), [1500]),
    "bf16_g4_q4_many_tiles": (dict(dtype="bf16", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
                                   n_comp=96, n_coef=257, n_query=4), [3000]),
    "bf16_g4_q16_short": (dict(dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                               n_comp=64, n_coef=33, n_query=16), [90, 260]),
    "f32_q4": (dict(dtype="f32", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64, n_comp=32,
                    n_coef=33, n_query=4), [512, 200]),
    # more queries than one pass over the cache holds: 40 queries of a 4-head
    # group (160 rows per KV head) run as passes of 24 and 16 queries; 300 fp32
    # queries of a 2-head group as passes of up to 195
    "bf16_g4_q40_passes": (dict(dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                n_comp=64, n_coef=97, n_query=40), [1300, 600]),
    "f32_g2_q300_passes": (dict(dtype="f32", batch=1, n_q_heads=4, n_kv_heads=2, head_dim=64,
                                n_comp=32, n_coef=17, n_query=300), [230]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_attend_small(fb, name):
    kw, lens = CASES[name]
    cfg = wl.custom(name=name, seed=300 + sorted(CASES).index(name), **kw)
    _say("case %s lens=%s n_query=%d" % (name, lens, cfg.n_query))
    w = wl.make(cfg, lens=lens)
    run = AttendRun(fb, w)
    ck_o, cv_o = ob.project_all(w)
    _check(w, run.attend(), ob.attend_all(w, ck_o, cv_o, run.scale), "end-to-end")
    ck32, cv32 = ck_o.astype(np.float32), cv_o.astype(np.float32)
    want = ob.attend_all(w, ck32.astype(np.float64), cv32.astype(np.float64), run.scale)
    _check(w, run.attend(ck32, cv32), want, "isolated")


def test_attend_one_query_is_decode(fb):
    """n_query = 1: the same kernels as fa_decode, bit for bit, plus the lse."""
    _say("case attend n_query=1 vs decode")
    cfg = wl.custom(name="q1", dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                    n_comp=64, n_coef=201, seed=321)
    w = wl.make(cfg, lens=[2500, 1111])
    run = AttendRun(fb, w)
    out = torch.full((2, 8, 128), float("nan"), device="cuda")
    fb.decode(run.desc, run.q, run.kx, run.vx, run.ke, run.ve, run.ck, run.cv, run.scale, out)
    torch.cuda.synchronize()
    got_o, got_l = run.attend(nq=1)
    assert np.array_equal(got_o[:, 0], out.cpu().numpy().astype(np.float64))
    ck_o, cv_o = ob.project_all(w)
    _check(w, (got_o, got_l), ob.attend_all(w, ck_o, cv_o, run.scale), "end-to-end")


def _check_blocks(fb, w, blocks):
    """GPU fa_attend of the whole workload; oracle attend on the given blocks."""
    run = AttendRun(fb, w)
    got_o, got_l = run.attend()
    c = w.cfg
    G = c.group
    from oracle import fourier_attention as fa
    for b, h in blocks:
        ck_o, cv_o = ob.project_block(w, b, h)
        K, V = w.natural_kv(b, h)
        q = w.f64(w.q[b, :, h * G:(h + 1) * G]).reshape(c.n_query * G, c.head_dim)
        o, l = fa.attend(q, K, V, w.comp_dims(h), ck_o, cv_o, c.sink, c.recent, run.scale)
        _check(w, (got_o[b, :, h * G:(h + 1) * G], got_l[b, :, h * G:(h + 1) * G]),
               (o.reshape(c.n_query, G, c.head_dim), l.reshape(c.n_query, G)),
               "end-to-end b=%d h=%d" % (b, h))


def test_llama3_8b_gqa_4q(fb):
    """Full-size batch with four queries per sequence; every sequence at two KV heads."""
    _say("case llama3_8b_gqa_4q (every sequence at two KV heads)")
    w = wl.make(wl.CONFIGS["llama3_8b_gqa_4q"])
    _check_blocks(fb, w, [(b, h) for b in range(4) for h in ((2 * b) % 8, (2 * b + 5) % 8)])


def test_llama3_8b_gqa_chunk64(fb):
    """A 64-token prefill chunk per sequence (three passes over the cache), all
    64 queries of sampled blocks: every pass is compared."""
    _say("case llama3_8b_gqa_chunk64 (every sequence at one KV head, all 64 queries)")
    w = wl.make(wl.CONFIGS["llama3_8b_gqa_chunk64"])
    _check_blocks(fb, w, [(0, 0), (1, 3), (2, 6), (3, 7)])
