"""GPU parity of fa_dim_sensitivity (the dimension analysis: noise on one value
dim at a time, squared change of the attention outputs per query head and dim)
against the oracle's literal perturb-and-rerun definition.

Bar: every entry sq[i][d] within 2e-3 (bf16 inputs) or 1e-5 (fp32) of the
largest entry of its query head, relative.  The response to the noise is an
attention output with the noise as the values, so its error is that of the
decode kernels' outputs relative to the noise's scale (probabilities kept to
about 16 bits, noise exact in bf16): a few 1e-4 in the squares.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from long_context_decode_fourier_amd import workloads as wl  # noqa: E402
from oracle import batch as ob  # noqa: E402
from oracle import fourier_attention as fa  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}


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


def _run(fb, w):
    c = w.cfg
    desc = fb.Desc.from_workload(w)
    q = fb.to_device(w.q)
    k = fb.to_device(w.natural_k_rows())
    noise_np = w.value_noise()
    noise = fb.to_device(noise_np)
    sq = torch.full((c.n_q_heads, c.head_dim), float("nan"), device="cuda")
    ws = fb.workspace(fb.dim_sensitivity_workspace_size(desc, c.n_query))
    ws.fill_(0xFF)
    scale = 1.0 / np.sqrt(c.head_dim)
    fb.dim_sensitivity(desc, c.n_query, q, k, noise, scale, sq, ws)
    torch.cuda.synchronize()
    return sq.cpu().numpy().astype(np.float64), noise_np, scale


def _compare(w, got, want, heads):
    tol = TOL[w.cfg.dtype]
    worst = 0.0
    for j, i in enumerate(heads):
        ref = np.abs(want[j]).max()
        assert ref > 0
        worst = max(worst, np.abs(got[i] - want[j]).max() / ref)
    _say("  worst entry error / head max: %.2e (bar %.0e)" % (worst, tol))
    assert np.isfinite(got).all()
    assert worst <= tol


SMALL = {
    # 64-dim heads: the one-pass MFMA kernels; 3 queries per sequence
    "bf16_d64_gqa_3q": (dict(dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64, n_comp=32,
                             n_coef=33, n_query=3), [300, 129]),
    # 128-dim heads: the VALU kernels
    "bf16_d128": (dict(dtype="bf16", batch=2, n_q_heads=4, n_kv_heads=4, head_dim=128, n_comp=64,
                       n_coef=65), [500, 97]),
    "f32_gqa_4q": (dict(dtype="f32", batch=3, n_q_heads=4, n_kv_heads=2, head_dim=16, n_comp=8,
                        n_coef=9, n_query=4), [200, 7, 333]),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_shapes(fb, name):
    kw, lens = SMALL[name]
    cfg = wl.custom(name=name, seed=500 + sorted(SMALL).index(name), **kw)
    _say("case %s lens=%s" % (name, lens))
    w = wl.make(cfg, lens=lens)
    got, noise, scale = _run(fb, w)
    want = ob.dim_sensitivity_all(w, noise, scale)
    _compare(w, got, want, list(range(cfg.n_q_heads)))


def test_llama2_7b_dim_analysis_sampled_heads(fb):
    """The full LLaMA-2-7B-shaped analysis (32 heads, L = 4096, 16 queries) on
    the GPU; the oracle's definition on the first and last query head."""
    w = wl.make(wl.CONFIGS["llama2_7b_dim_analysis"])
    c = w.cfg
    _say("case llama2_7b_dim_analysis")
    got, noise, scale = _run(fb, w)
    heads = [0, c.n_q_heads - 1]
    want = []
    for i in heads:
        K, V = w.natural_kv(0, i)  # one query head per KV head
        eps = w.natural_rows(noise, 0, i)
        want.append(fa.dim_sensitivity(w.f64(w.q[0, :, i]), K, V, eps, scale))
    _compare(w, got, np.array(want), heads)
    # the pages' ranking input: one score per dim, every entry finite and positive
    score = np.sqrt(got.sum(0))
    assert score.shape == (c.head_dim,) and (score > 0).all()
