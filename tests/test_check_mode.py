"""GPU: the FA_CHECK=1 validation mode.  fa_project rejects bf16 cache values
its fp16 operands cannot hold; fa_decode rejects dims entries outside [0, D);
on clean inputs the mode changes no result (bit for bit)."""
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
    binding.lib()
    return binding


def _setup(fb):
    cfg = wl.custom(name="check", dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                    n_comp=64, n_coef=129, seed=77)
    w = wl.make(cfg, lens=[1500, 700])
    dims = torch.from_numpy(w.dims).cuda()
    return w, cfg, dims


def _project(fb, w, cfg, desc, kc):
    nblk = cfg.batch * cfg.n_kv_heads
    ck = torch.zeros((nblk, cfg.n_coef, cfg.n_comp), device="cuda")
    cv = torch.zeros_like(ck)
    ke = torch.zeros((nblk, cfg.sink + cfg.recent, cfg.n_comp), dtype=kc.dtype, device="cuda")
    ve = torch.zeros_like(ke)
    ws = fb.workspace(fb.project_workspace_size(desc))
    fb.project(desc, kc, fb.to_device(w.vc), ck, cv, ke, ve, ws)
    torch.cuda.synchronize()
    return ck, cv, ke, ve


def test_project_rejects_fp16_overflow_and_keeps_clean_results(fb, monkeypatch):
    w, cfg, dims = _setup(fb)
    desc = fb.Desc.from_workload(w, dims)
    kc = fb.to_device(w.kc)
    ref = _project(fb, w, cfg, desc, kc)
    monkeypatch.setenv("FA_CHECK", "1")
    got = _project(fb, w, cfg, desc, kc)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    bad = w.kc.copy()
    bad[1000, 3] = wl.bf16_bits(np.array([70000.0], dtype=np.float32))[0]  # token 1000 of (0, 0): middle
    with pytest.raises(fb.FAError, match="FA_CHECK"):
        _project(fb, w, cfg, desc, fb.to_device(bad))


def test_decode_rejects_dims_outside_range(fb, monkeypatch):
    w, cfg, dims = _setup(fb)
    desc = fb.Desc.from_workload(w, dims)
    ck, cv, ke, ve = _project(fb, w, cfg, desc, fb.to_device(w.kc))
    q, kx, vx = fb.to_device(w.q), fb.to_device(w.kx), fb.to_device(w.vx)

    def dec(d):
        out = torch.zeros((cfg.batch, cfg.n_q_heads, cfg.head_dim), device="cuda")
        ws = fb.workspace(fb.decode_workspace_size(d))
        fb.decode(d, q, kx, vx, ke, ve, ck, cv, 0.088, out, ws)
        torch.cuda.synchronize()
        return out

    ref = dec(desc)
    monkeypatch.setenv("FA_CHECK", "1")
    assert torch.equal(dec(desc), ref)
    bad_dims = dims.clone()
    bad_dims[1, 7] = cfg.head_dim  # one past the last dim
    # checked before any decode kernel runs: the bad table never reaches them
    with pytest.raises(fb.FAError, match="dims"):
        dec(fb.Desc.from_workload(w, bad_dims))
