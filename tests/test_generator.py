"""The seeded workload generator: determinism, masks, lengths, rounding, layout."""
import numpy as np
import torch

from long_context_decode_fourier_amd import workloads as wl


def _small(**kw):
    base = dict(dtype="bf16", batch=3, n_q_heads=4, n_kv_heads=2, head_dim=16,
                n_comp=6, n_coef=5, len_range=(120, 200), seed=11)
    base.update(kw)
    return wl.custom(**base)


def test_same_seed_same_bytes():
    a, b = wl.make(_small()), wl.make(_small())
    for f in ("lens", "dims", "q", "kx", "vx", "kc", "vc"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = wl.make(_small(seed=12))
    assert not np.array_equal(a.kc, c.kc)


def test_masks_and_lengths():
    w = wl.make(_small())
    assert ((w.lens >= 120) & (w.lens <= 200)).all()
    assert w.offs[0] == 0 and (np.diff(w.offs) == w.lens[:-1]).all()
    for h in range(2):
        d = w.dims[h]
        assert sorted(d.tolist()) == list(range(16))
        ex, cp = d[:10], d[10:]
        assert (np.diff(ex) > 0).all() and (np.diff(cp) > 0).all()
    low = wl.make(_small(mask="low", dtype="f32"))
    assert low.dims[0, 10:].tolist() == list(range(6))


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 37
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 65504.0]  # ties
    ours = wl.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(wl.bf16_to_f32(ours),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_layout_and_edges():
    cfg = _small(len_range=None, seq_len=None, batch=2, sink=3, recent=4)
    w = wl.make(cfg, lens=[20, 5])
    assert w.kc.shape == (2 * (20 + 5), 6) and w.kx.shape == (2 * 25, 10)
    # row of (b=1, h=1, t=2) = Hkv*off[1] + h*L_1 + t
    assert w.row0(1, 1) == 2 * 20 + 5
    K, V = w.natural_kv(1, 1)
    assert np.array_equal(K[2, w.dims[1, 10:]], w.f64(w.kc[w.row0(1, 1) + 2]))
    e = w.edges(w.kc)
    assert e.shape == (4, 7, 6)
    blk = w.block(w.kc, 0, 1)
    assert np.array_equal(e[1, :3], blk[:3]) and np.array_equal(e[1, 3:], blk[-4:])
    short = w.block(w.kc, 1, 0)           # L = 5 < S + R = 7: all rows, rest zero
    assert np.array_equal(e[2, :5], short) and not e[2, 5:].any()


def test_signal_is_smooth_and_bounded():
    w = wl.make(_small(len_range=None, seq_len=600, batch=1))
    x = w.f64(w.block(w.kc, 0, 0))
    # a few low-frequency sinusoids: neighbouring tokens are strongly correlated
    d = np.diff(x, axis=0)
    assert np.abs(d).mean() < 0.2 * np.abs(x).mean()
    assert np.abs(x).max() < 20


def test_lengths_without_drawing_the_workload():
    for cfg in (wl.custom(name="ragged_small", dtype="bf16", batch=5, n_q_heads=4, n_kv_heads=2, head_dim=32,
                          n_comp=8, n_coef=9, seq_len=None, len_range=(100, 900), seed=7),
                wl.CONFIGS["fp32_head"]):
        assert np.array_equal(wl.lengths(cfg), wl.make(cfg).lens)
    # the large ragged workload's lengths stay inside its range
    c = wl.CONFIGS["ragged_batch"]
    lens = wl.lengths(c)
    assert lens.shape == (c.batch,) and lens.min() >= c.len_range[0] and lens.max() <= c.len_range[1]


def test_truncated_keeps_each_sequence_prefix():
    cfg = wl.custom(name="trunc", dtype="bf16", batch=3, n_q_heads=4, n_kv_heads=2, head_dim=16,
                    n_comp=8, n_coef=5, seed=3)
    w = wl.make(cfg, lens=[50, 9, 31])
    t = w.truncated([49, 1, 20])
    assert list(t.lens) == [49, 1, 20] and list(t.offs) == [0, 49, 50]
    for b in range(3):
        for h in range(2):
            K, V = w.natural_kv(b, h)
            Kt, Vt = t.natural_kv(b, h)
            L = int(t.lens[b])
            assert np.array_equal(Kt, K[:L]) and np.array_equal(Vt, V[:L])
