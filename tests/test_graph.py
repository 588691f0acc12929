"""HIP graph capture of fa_project + fa_decode, and of fa_attend.

A serving loop (and bench.py) launches the step as HIP graphs.  The library
makes no allocation, host synchronisation or memset, so both calls can be
captured; every replay must reproduce the eager results bit for bit.  The
replays are interleaved with eager library work and synchronisations, and the
outputs are overwritten with NaN before each replay, so a replay that
computes nothing (or reads a stale workspace) fails.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from long_context_decode_fourier_amd import workloads as wl  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_decode_fourier_amd import binding
    binding.lib()  # raises if libfa.so is missing: no fallback
    return binding


# a two-pass shape (k past the one-pass limit): pass 1, pass 2 and the merges
# under one graph
GRAPH_CUSTOM = {
    "two_pass_k2401": (dict(dtype="bf16", batch=2, n_q_heads=16, n_kv_heads=4, head_dim=128, n_comp=64,
                            n_coef=2401, seed=61), [9000, 5000]),
}


@pytest.mark.parametrize("name", ["llama2_7b_layer", "llama3_8b_gqa", "fp32_head", "two_pass_k2401"])
def test_graph_replays_match_eager(fb, name):
    print("graph replay", name, flush=True)
    sys.stdout.flush()
    if name in GRAPH_CUSTOM:
        kw, lens = GRAPH_CUSTOM[name]
        w = wl.make(wl.custom(name=name, **kw), lens=lens)
        assert fb.attend_plan(fb.Desc.from_workload(w))["path"] == "two_pass"
    else:
        w = wl.make(wl.CONFIGS[name])
    c = w.cfg
    dims = torch.from_numpy(w.dims).cuda()
    desc = fb.Desc.from_workload(w, dims)
    kc, vc = fb.to_device(w.kc), fb.to_device(w.vc)
    q, kx, vx = fb.to_device(w.q), fb.to_device(w.kx), fb.to_device(w.vx)
    nblk, E = c.batch * c.n_kv_heads, c.sink + c.recent
    ck = torch.empty((nblk, c.n_coef, c.n_comp), device="cuda")
    cv = torch.empty_like(ck)
    ke = torch.empty((nblk, E, c.n_comp), dtype=kc.dtype, device="cuda")
    ve = torch.empty_like(ke)
    out = torch.empty((c.batch, c.n_q_heads, c.head_dim), device="cuda")
    other = torch.empty_like(out)
    ws_p = fb.workspace(fb.project_workspace_size(desc))
    ws_d = fb.workspace(fb.decode_workspace_size(desc))
    scale = 1.0 / np.sqrt(c.head_dim)

    def step(st):
        fb.project(desc, kc, vc, ck, cv, ke, ve, ws_p, st)
        fb.decode(desc, q, kx, vx, ke, ve, ck, cv, scale, out, ws_d, st)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = [t.clone() for t in (ck, cv, ke, ve, out)]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()

    for r in range(3):
        for t in (ck, cv, out):
            t.fill_(float("nan"))
        ke.zero_()
        ve.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref, nm in zip((ck, cv, ke, ve, out), want, ("ck", "cv", "ke", "ve", "out")):
            assert torch.equal(got, ref), "replay %d: %s differs from the eager result" % (r, nm)
        # eager work on the same workspaces between replays
        fb.decode(desc, q, kx, vx, ke, ve, ck, cv, scale, other, ws_d, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(other, want[4])


def test_graph_attend_with_lse(fb):
    """fa_attend (four queries per sequence, with lse) captured and replayed."""
    print("graph replay attend", flush=True)
    sys.stdout.flush()
    cfg = wl.custom(name="graph_attend", dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2,
                    head_dim=128, n_comp=64, n_coef=129, n_query=4, seed=77)
    w = wl.make(cfg, lens=[1800, 700])
    c = w.cfg
    dims = torch.from_numpy(w.dims).cuda()
    desc = fb.Desc.from_workload(w, dims)
    kc, vc = fb.to_device(w.kc), fb.to_device(w.vc)
    q, kx, vx = fb.to_device(w.q), fb.to_device(w.kx), fb.to_device(w.vx)
    nblk, E = c.batch * c.n_kv_heads, c.sink + c.recent
    ck = torch.empty((nblk, c.n_coef, c.n_comp), device="cuda")
    cv = torch.empty_like(ck)
    ke = torch.empty((nblk, E, c.n_comp), dtype=kc.dtype, device="cuda")
    ve = torch.empty_like(ke)
    fb.project(desc, kc, vc, ck, cv, ke, ve)
    out = torch.empty((c.batch, 4, c.n_q_heads, c.head_dim), device="cuda")
    lse = torch.empty((c.batch, 4, c.n_q_heads), device="cuda")
    ws = fb.workspace(fb.attend_workspace_size(desc, 4))
    scale = 1.0 / np.sqrt(c.head_dim)

    def step(st):
        fb.attend(desc, 4, q, kx, vx, ke, ve, ck, cv, scale, out, lse, ws, st)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = (out.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want[0]) and torch.equal(lse, want[1]), "replay %d differs" % r
        # eager work on the same workspace between replays (one query needs less)
        one = torch.empty((c.batch, c.n_q_heads, c.head_dim), device="cuda")
        fb.decode(desc, q[:, 0].contiguous(), kx, vx, ke, ve, ck, cv, scale, one, ws,
                  torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.isfinite(one).all()
