"""Seeded synthetic workloads for Fourier-approximated KV-cache decode.

This module only *draws inputs*.  It holds none of the method's arithmetic:
no Fourier basis, no projection, no attention.  Both the HIP path's tests and
the CPU oracle consume the arrays it returns, so it is the one piece of code the
two sides share.

Workload shapes follow the scenarios this library is measured on (single
fp32 head, a LLaMA-2-7B-shaped layer, a LLaMA-3-8B-shaped GQA batch, the same
batch with four queries or a 64-token prefill chunk per sequence, a long
prefill projection and a ragged long-context batch).  No dataset, checkpoint or
trained weight is used: the compressible head dims of K and V are smooth
signals (a sum of four low-frequency sinusoids plus small noise), which is the
kind of slowly varying time series the method's Fourier projection targets
(skill page "fourier-approximated-kv-cache", section Core concept); the other
dims and the queries are standard normal.

Recipe (one ``numpy.random.Generator(PCG64(seed))``, draws in this order):

1. ragged lengths ``L_b ~ U{lo..hi}`` (only when the workload is ragged);
2. per KV head, the compressible-dim mask: the lowest ``Dc`` dims for
   ``mask="low"``, else ``sorted(permutation(D)[:Dc])``; the same mask serves
   K and V;
3. for each sequence b, KV head h, matrix K then V:
   amplitudes ``A ~ N(0,1)`` [Dc,4], cycles-over-M ``f ~ U(0,8]`` [Dc,4],
   phases ``phi ~ U[0,2pi)`` [Dc,4], noise ``N(0,0.05^2)`` [L,Dc] (float32
   draws), exact dims ``N(0,1)`` [L,Du] (float32 draws).  Compressible dim c
   at token t is ``sum_m A sin(2 pi f (t - S) / max(M,1) + phi) + noise``, so the
   sink and recent rows continue the same signal;
4. queries ``q ~ N(0,1)`` [B,Hq,D] (float32 draws), or [B,nq,Hq,D] for a
   workload with nq > 1 queries per sequence (the same draws, in that shape).

bf16 workloads round every value to bfloat16 with round-to-nearest-even;
fp32 workloads keep float32.

Memory layout (the C-ABI's cache layout):

* ``dims[h]`` (int32, [Hkv, D]): the exact dims ascending, then the
  compressible dims ascending;
* ``kx``/``vx`` ([rows, Du]) hold the exact dims, ``kc``/``vc`` ([rows, Dc])
  the compressible dims, both in ``dims[h]`` order.  Row ``t`` of block (b, h)
  is row ``Hkv * off[b] + h * L_b + t`` where ``off`` is the exclusive prefix
  sum of the lengths;
* ``ke``/``ve`` ([B*Hkv, S+R, Dc]) are the edge rows of kc/vc: the sink tokens
  then the recent tokens (for ``L_b < S+R``: all ``L_b`` tokens in order, the
  rest zero).  This is a pure gather used to hand decode-only workloads their
  retained rows.

bf16 arrays are stored as ``uint16`` bit patterns, fp32 arrays as ``float32``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

SINK = 32
RECENT = 64


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    dtype: str                 # "f32" or "bf16": dtype of q, K and V
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_comp: int                # Dc, compressible dims per KV head
    n_coef: int                # k, real Fourier coefficients
    seq_len: Optional[int] = None               # fixed length
    len_range: Optional[Tuple[int, int]] = None  # ragged: inclusive range
    mask: str = "seeded"       # "low" or "seeded"
    sink: int = SINK
    recent: int = RECENT
    seed: int = 0
    steps: Tuple[str, ...] = ("project", "decode")
    n_query: int = 1           # queries per sequence (q is [B, n_query, Hq, D] when > 1)
    period: int = 0            # basis period: 0 = each sequence's middle length, > 0 fixed
    note: str = ""

    @property
    def n_exact(self) -> int:
        return self.head_dim - self.n_comp

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


# The workloads.  Names say what the workload is; the seed is fixed.
CONFIGS = {
    "fp32_head": Config(
        name="fp32_head", dtype="f32", batch=1, n_q_heads=1, n_kv_heads=1,
        head_dim=64, n_comp=32, n_coef=33, seq_len=512, mask="low", seed=1,
        note="single fp32 head, L=512 (M=416), lower 32 dims compressible, k=33"),
    "llama2_7b_layer": Config(
        name="llama2_7b_layer", dtype="bf16", batch=1, n_q_heads=32,
        n_kv_heads=32, head_dim=128, n_comp=64, n_coef=401, seq_len=4096,
        seed=2,
        note="LLaMA-2-7B-shaped layer, 32/32 heads, L=4096 (M=4000), k=401"),
    "llama3_8b_gqa": Config(
        name="llama3_8b_gqa", dtype="bf16", batch=4, n_q_heads=32,
        n_kv_heads=8, head_dim=128, n_comp=96, n_coef=1025, seq_len=32768,
        seed=3, steps=("decode",),
        note="LLaMA-3-8B-shaped GQA batch 4, 32/8 heads, L=32768 (M=32672), "
             "96 compressible dims, k=1025"),
    "prefill_projection": Config(
        name="prefill_projection", dtype="bf16", batch=1, n_q_heads=8,
        n_kv_heads=8, head_dim=128, n_comp=64, n_coef=4097,
        seq_len=131040 + SINK + RECENT, seed=4, steps=("project",),
        note="projection only: 8 KV heads x 64 dims of K and V, M=131040, "
             "k=4097"),
    "llama3_8b_gqa_4q": Config(
        name="llama3_8b_gqa_4q", dtype="bf16", batch=4, n_q_heads=32,
        n_kv_heads=8, head_dim=128, n_comp=96, n_coef=1025, seq_len=32768,
        seed=3, steps=("decode",), n_query=4,
        note="the LLaMA-3-8B-shaped GQA cache (same draws) with 4 queries per "
             "sequence attending to it (e.g. 4 draft tokens verified at once)"),
    "llama3_8b_gqa_chunk64": Config(
        name="llama3_8b_gqa_chunk64", dtype="bf16", batch=4, n_q_heads=32,
        n_kv_heads=8, head_dim=128, n_comp=96, n_coef=1025, seq_len=32768,
        seed=3, steps=("decode",), n_query=64,
        note="the LLaMA-3-8B-shaped GQA cache (same draws) with a 64-token "
             "prefill chunk per sequence attending to it (256 query rows per KV "
             "head, run as passes over the cache)"),
    "llama2_7b_dim_analysis": Config(
        name="llama2_7b_dim_analysis", dtype="bf16", batch=1, n_q_heads=32,
        n_kv_heads=32, head_dim=128, n_comp=64, n_coef=401, seq_len=4096, seed=2,
        steps=("sensitivity",), n_query=16,
        note="dimension analysis of the LLaMA-2-7B-shaped layer's cache: 16 queries, "
             "noise N(0, 0.1^2) on one value dim at a time, L=4096"),
    "ragged_batch": Config(
        name="ragged_batch", dtype="bf16", batch=16, n_q_heads=32,
        n_kv_heads=8, head_dim=128, n_comp=64, n_coef=2049,
        len_range=(32768, 65536), seed=5, steps=("decode",),
        note="ragged batch 16, 32/8 heads, L ~ U[32768, 65536], k=2049"),
}


def custom(name="custom", **kw) -> Config:
    """A config with explicit fields (small parity shapes, edge cases)."""
    return Config(name=name, **kw)


# ---------------------------------------------------------------- rounding --

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- workload --

@dataclasses.dataclass
class Workload:
    cfg: Config
    lens: np.ndarray        # int64 [B]
    offs: np.ndarray        # int64 [B], exclusive prefix sum of lens
    dims: np.ndarray        # int32 [Hkv, D]
    q: Optional[np.ndarray]     # [B, Hq, D], or [B, nq, Hq, D] when nq > 1
    kx: Optional[np.ndarray]    # [rows, Du]
    vx: Optional[np.ndarray]
    kc: np.ndarray              # [rows, Dc]
    vc: np.ndarray

    # -- shape helpers ---------------------------------------------------
    @property
    def storage_dtype(self):
        return np.uint16 if self.cfg.dtype == "bf16" else np.float32

    def mid_len(self, b: int) -> int:
        c = self.cfg
        return max(0, int(self.lens[b]) - c.sink - c.recent)

    def row0(self, b: int, h: int) -> int:
        return int(self.cfg.n_kv_heads * self.offs[b] + h * self.lens[b])

    def f64(self, a: np.ndarray) -> np.ndarray:
        """Stored values as float64 (exact: bf16 and f32 embed in f64)."""
        if a.dtype == np.uint16:
            return bf16_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    def block(self, a: np.ndarray, b: int, h: int) -> np.ndarray:
        r0 = self.row0(b, h)
        return a[r0:r0 + int(self.lens[b])]

    def comp_dims(self, h: int) -> np.ndarray:
        return self.dims[h, self.cfg.n_exact:]

    def natural_kv(self, b: int, h: int):
        """(K, V) of sequence b, KV head h as float64 [L, D] in natural dim order."""
        c = self.cfg
        L = int(self.lens[b])
        K = np.zeros((L, c.head_dim))
        V = np.zeros((L, c.head_dim))
        ex, cp = self.dims[h, :c.n_exact], self.dims[h, c.n_exact:]
        if self.kx is not None:
            K[:, ex] = self.f64(self.block(self.kx, b, h))
            V[:, ex] = self.f64(self.block(self.vx, b, h))
        K[:, cp] = self.f64(self.block(self.kc, b, h))
        V[:, cp] = self.f64(self.block(self.vc, b, h))
        return K, V

    def value_noise(self, std: float = 0.1) -> np.ndarray:
        """Noise for the dimension analysis, laid out like K and V in natural
        dim order: [rows, D] in the storage dtype, N(0, std^2) draws from a
        generator of its own (seed + 7919), so the rest of the workload is
        unchanged.  Column d is the noise added to dim d of the values when
        that dim is perturbed."""
        c = self.cfg
        rng = np.random.Generator(np.random.PCG64(c.seed + 7919))
        rows = int(c.n_kv_heads * self.lens.sum())
        return _round(rng.standard_normal((rows, c.head_dim)) * std, c.dtype)

    def natural_rows(self, X: np.ndarray, b: int, h: int) -> np.ndarray:
        """Block (b, h) of a [rows, D] natural-order array as float64 [L, D]."""
        return self.f64(self.block(X, b, h))

    def natural_k_rows(self) -> np.ndarray:
        """K of every (sequence, KV head) block as one [rows, D] array in
        natural dim order and the storage dtype (the uncompressed keys the
        dimension analysis runs over), packed like kx / kc."""
        c = self.cfg
        rows = int(c.n_kv_heads * self.lens.sum())
        out = np.zeros((rows, c.head_dim), dtype=self.kc.dtype)
        for h in range(c.n_kv_heads):
            ex, cp = self.dims[h, :c.n_exact], self.dims[h, c.n_exact:]
            for b in range(c.batch):
                r0, L = self.row0(b, h), int(self.lens[b])
                if self.kx is not None:
                    out[r0:r0 + L][:, ex] = self.block(self.kx, b, h)
                out[r0:r0 + L][:, cp] = self.block(self.kc, b, h)
        return out

    def truncated(self, lens) -> "Workload":
        """The same cache with sequence b cut to its first lens[b] tokens
        (the rows re-laid out for the shorter lengths; q and dims shared):
        the state before tokens were appended."""
        c = self.cfg
        lens = np.asarray(lens, dtype=np.int64)
        if lens.shape != self.lens.shape or (lens > self.lens).any() or (lens < 1).any():
            raise ValueError("truncated lengths must lie in [1, L_b]")
        offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)

        def cut(a):
            if a is None:
                return None
            out = np.empty((int(c.n_kv_heads * lens.sum()), a.shape[1]), dtype=a.dtype)
            for b in range(c.batch):
                for h in range(c.n_kv_heads):
                    r0 = int(c.n_kv_heads * offs[b] + h * lens[b])
                    out[r0:r0 + int(lens[b])] = self.block(a, b, h)[:int(lens[b])]
            return out
        return Workload(cfg=c, lens=lens, offs=offs, dims=self.dims, q=self.q, kx=cut(self.kx),
                        vx=cut(self.vx), kc=cut(self.kc), vc=cut(self.vc))

    def edges(self, a: np.ndarray) -> np.ndarray:
        """Gather the sink+recent rows of kc or vc into [B*Hkv, S+R, Dc]."""
        c = self.cfg
        E = c.sink + c.recent
        out = np.zeros((c.batch * c.n_kv_heads, E, c.n_comp), dtype=a.dtype)
        for b in range(c.batch):
            L = int(self.lens[b])
            for h in range(c.n_kv_heads):
                blk = self.block(a, b, h)
                o = out[b * c.n_kv_heads + h]
                if L <= E:
                    o[:L] = blk
                else:
                    o[:c.sink] = blk[:c.sink]
                    o[c.sink:] = blk[L - c.recent:]
        return out


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return bf16_bits(x) if dtype == "bf16" else x


def lengths(cfg: Config) -> np.ndarray:
    """The sequence lengths make(cfg) draws (its generator's first draw)."""
    if cfg.len_range is None:
        return np.full(cfg.batch, cfg.seq_len, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    lo, hi = cfg.len_range
    return rng.integers(lo, hi + 1, size=cfg.batch).astype(np.int64)


def make(cfg: Config, lens=None) -> Workload:
    """Draw the workload for ``cfg`` (deterministic in ``cfg.seed``).

    ``lens`` overrides the drawn lengths (edge-case tests).
    """
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    B, Hkv, D, Dc = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.n_comp
    Du = D - Dc
    if cfg.n_q_heads % Hkv or not (0 <= Dc <= D):
        raise ValueError("bad head/dim split in %s" % cfg.name)
    if lens is not None:
        lens = np.asarray(lens, dtype=np.int64)
    elif cfg.len_range is not None:
        lo, hi = cfg.len_range
        lens = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    else:
        lens = np.full(B, cfg.seq_len, dtype=np.int64)
    # (lengths(cfg) repeats this first draw without the rest of the workload)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)

    dims = np.empty((Hkv, D), dtype=np.int32)
    for h in range(Hkv):
        if cfg.mask == "low":
            comp = np.arange(Dc)
        else:
            comp = np.sort(rng.permutation(D)[:Dc])
        exact = np.setdiff1d(np.arange(D), comp)
        dims[h] = np.concatenate([exact, comp])

    need_exact = "decode" in cfg.steps or "sensitivity" in cfg.steps
    rows = int(Hkv * lens.sum())
    sd = np.uint16 if cfg.dtype == "bf16" else np.float32
    kc = np.empty((rows, Dc), dtype=sd)
    vc = np.empty((rows, Dc), dtype=sd)
    kx = np.empty((rows, Du), dtype=sd) if need_exact else None
    vx = np.empty((rows, Du), dtype=sd) if need_exact else None

    two_pi = np.float32(2.0 * np.pi)
    for b in range(B):
        L = int(lens[b])
        Mref = float(max(L - cfg.sink - cfg.recent, 1))
        trel = (np.arange(L, dtype=np.float32) - np.float32(cfg.sink))[:, None]
        for h in range(Hkv):
            r0 = int(Hkv * offs[b] + h * L)
            for comp_out, exact_out in ((kc, kx), (vc, vx)):
                A = rng.standard_normal((Dc, 4)).astype(np.float32)
                f = (8.0 - rng.uniform(0.0, 8.0, (Dc, 4))).astype(np.float32)
                ph = rng.uniform(0.0, 2.0 * np.pi, (Dc, 4)).astype(np.float32)
                sig = 0.05 * rng.standard_normal((L, Dc), dtype=np.float32)
                w = two_pi * f / np.float32(Mref)
                for m in range(4):
                    sig += A[:, m] * np.sin(trel * w[:, m] + ph[:, m])
                comp_out[r0:r0 + L] = _round(sig, cfg.dtype)
                ex = rng.standard_normal((L, Du), dtype=np.float32)
                if exact_out is not None:
                    exact_out[r0:r0 + L] = _round(ex, cfg.dtype)
    q = None
    if need_exact:
        shape = (B, cfg.n_q_heads, D) if cfg.n_query == 1 else (B, cfg.n_query, cfg.n_q_heads, D)
        q = _round(rng.standard_normal(shape, dtype=np.float32), cfg.dtype)
    return Workload(cfg=cfg, lens=lens, offs=offs, dims=dims, q=q,
                    kx=kx, vx=vx, kc=kc, vc=vc)
