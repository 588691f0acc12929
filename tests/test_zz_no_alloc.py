"""fa_decode_noalloc (the workspace in the library's static scratch array)
against fa_decode with a caller's workspace, through the C ABI: two calls in a
row on the same GPU, the second on a smaller input, each equal to fa_decode's
result (bit for bit: the same kernels run) and within the bf16 output bar of
the oracle checks (max-abs 3e-3)."""
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


def _run(fb, cfg, lens):
    w = wl.make(cfg, lens=lens)
    c = w.cfg
    dims = torch.from_numpy(w.dims).cuda()
    desc = fb.Desc.from_workload(w, dims)
    kc, vc = fb.to_device(w.kc), fb.to_device(w.vc)
    q, kx, vx = fb.to_device(w.q), fb.to_device(w.kx), fb.to_device(w.vx)
    nblk = c.batch * c.n_kv_heads
    ck = torch.empty((nblk, c.n_coef, c.n_comp), device="cuda")
    cv = torch.empty_like(ck)
    ke = torch.empty((nblk, c.sink + c.recent, c.n_comp), dtype=kc.dtype, device="cuda")
    ve = torch.empty_like(ke)
    fb.project(desc, kc, vc, ck, cv, ke, ve)
    scale = 1.0 / np.sqrt(c.head_dim)
    want = torch.full((c.batch, c.n_q_heads, c.head_dim), float("nan"), device="cuda")
    got = torch.full_like(want, float("nan"))
    ws = fb.workspace(fb.decode_workspace_size(desc))
    ws.fill_(0xFF)  # NaN everywhere: the reference reads no unwritten workspace either
    fb.decode(desc, q, kx, vx, ke, ve, ck, cv, scale, want, ws)
    fb.decode_noalloc(desc, q, kx, vx, ke, ve, ck, cv, scale, got)
    torch.cuda.synchronize()
    return want.cpu().numpy(), got.cpu().numpy()


def test_noalloc_matches_decode_twice(fb):
    big = wl.custom(name="noalloc_big", dtype="bf16", batch=3, n_q_heads=32, n_kv_heads=8,
                    head_dim=128, n_comp=64, n_coef=513, seed=501)
    small = wl.custom(name="noalloc_small", dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2,
                      head_dim=128, n_comp=64, n_coef=65, seed=502)
    for cfg, lens in ((big, [9000, 4000, 6100]), (small, [700, 90])):
        print("case %s lens=%s" % (cfg.name, lens), flush=True)
        sys.stdout.flush()
        want, got = _run(fb, cfg, lens)
        assert np.isfinite(got).all()
        err = float(np.abs(got - want).max())
        print("  max-abs vs fa_decode %.2e" % err, flush=True)
        assert err <= 3e-3
        assert np.array_equal(got, want)
