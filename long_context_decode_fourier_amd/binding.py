"""ctypes binding of libfa (see include/fa.h): argument marshalling only.

Every computation runs in libfa's HIP kernels.  torch supplies device memory
and the current stream; it is imported before the library is loaded so that
libfa binds to the same HIP runtime as torch.  If libfa.so has not been built
the first call raises ``FAError`` (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

F32, BF16 = 0, 1
STATUS = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_DTYPE",
          4: "FA_ERR_WORKSPACE", 5: "FA_ERR_HIP", 6: "FA_ERR_ALIAS"}
MAX_BATCH = 64


class FAError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (STATUS.get(status, status), msg))
        self.status = status


class fa_desc_t(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_comp_dims", ctypes.c_int32),
                ("sink", ctypes.c_int32), ("recent", ctypes.c_int32),
                ("n_coef", ctypes.c_int32), ("period", ctypes.c_int32),
                ("seq_len", ctypes.POINTER(ctypes.c_int32)),
                ("dims", ctypes.c_void_p)]


_lib = None

# (name, restype, argtypes) of every exported function
_SIGS = [
    ("fa_project_workspace_size", ctypes.c_int,
     [ctypes.POINTER(fa_desc_t), ctypes.POINTER(ctypes.c_size_t)]),
    ("fa_project", ctypes.c_int,
     [ctypes.POINTER(fa_desc_t)] + [ctypes.c_void_p] * 6 + [ctypes.c_void_p, ctypes.c_size_t,
                                                           ctypes.c_void_p]),
    ("fa_decode_workspace_size", ctypes.c_int,
     [ctypes.POINTER(fa_desc_t), ctypes.POINTER(ctypes.c_size_t)]),
    ("fa_decode", ctypes.c_int,
     [ctypes.POINTER(fa_desc_t)] + [ctypes.c_void_p] * 7 + [ctypes.c_float, ctypes.c_void_p,
                                                           ctypes.c_void_p, ctypes.c_size_t,
                                                           ctypes.c_void_p]),
    ("fa_attend_workspace_size", ctypes.c_int,
     [ctypes.POINTER(fa_desc_t), ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]),
    ("fa_attend", ctypes.c_int,
     [ctypes.POINTER(fa_desc_t), ctypes.c_int32] + [ctypes.c_void_p] * 7 +
     [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
      ctypes.c_void_p]),
    ("fa_coef_budget", ctypes.c_int32, [ctypes.c_int32, ctypes.c_double]),
    ("fa_cache_bytes", ctypes.c_int,
     [ctypes.POINTER(fa_desc_t), ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64)]),
    ("fa_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("fa_last_error", ctypes.c_char_p, []),
    ("fa_version", ctypes.c_int32, []),
    ("fa_time_main_kernel", ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
    ("fa_attend_plan", ctypes.c_int,
     [ctypes.POINTER(fa_desc_t), ctypes.c_int32, ctypes.c_void_p]),
    ("fa_decode_noalloc", ctypes.c_int,
     [ctypes.POINTER(fa_desc_t)] + [ctypes.c_void_p] * 7 + [ctypes.c_float, ctypes.c_void_p,
                                                           ctypes.c_void_p]),
    ("fa_append", ctypes.c_int, [ctypes.POINTER(fa_desc_t)] + [ctypes.c_void_p] * 7),
    ("fa_dim_sensitivity_workspace_size", ctypes.c_int,
     [ctypes.POINTER(fa_desc_t), ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]),
    ("fa_dim_sensitivity", ctypes.c_int,
     [ctypes.POINTER(fa_desc_t), ctypes.c_int32] + [ctypes.c_void_p] * 3 +
     [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
]


def lib():
    """The loaded libfa (raises FAError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FAError(-1, "libfa.so not built (run python -m "
                              "long_context_decode_fourier_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in _SIGS:
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise FAError(status, lib().fa_last_error().decode())


class Desc:
    """Python view of fa_desc_t; keeps the host length array alive."""

    def __init__(self, dtype, batch, n_q_heads, n_kv_heads, head_dim, n_comp_dims,
                 n_coef, seq_len, sink=32, recent=64, dims=None, period=0):
        self._lens = (ctypes.c_int32 * max(1, len(seq_len)))(*[int(x) for x in seq_len])
        self.dims = dims  # device int32 tensor [Hkv, D] (decode only)
        self.c = fa_desc_t(int(dtype), int(batch), int(n_q_heads), int(n_kv_heads),
                           int(head_dim), int(n_comp_dims), int(sink), int(recent),
                           int(n_coef), int(period), self._lens,
                           ctypes.c_void_p(dims.data_ptr() if dims is not None else 0))

    @classmethod
    def from_workload(cls, w, dims=None):
        c = w.cfg
        return cls(BF16 if c.dtype == "bf16" else F32, c.batch, c.n_q_heads, c.n_kv_heads,
                   c.head_dim, c.n_comp, c.n_coef, [int(x) for x in w.lens],
                   sink=c.sink, recent=c.recent, dims=dims, period=c.period)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def project_workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().fa_project_workspace_size(ctypes.byref(desc.c), ctypes.byref(n)))
    return n.value


def decode_workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().fa_decode_workspace_size(ctypes.byref(desc.c), ctypes.byref(n)))
    return n.value


def workspace(nbytes: int, device="cuda"):
    """A 256-byte-aligned byte buffer (torch's allocator aligns to 512)."""
    return torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)


def _own_workspace(nbytes, device, stream):
    """A workspace for one call on `stream`: allocated there, so that torch's
    caching allocator does not hand it out again while the call still runs."""
    if stream is None:
        return workspace(nbytes, device)
    with torch.cuda.stream(stream):
        return workspace(nbytes, device)


def project(desc: Desc, kc, vc, ck, cv, ke=None, ve=None, ws=None, stream=None):
    """fa_project: coefficients of the middle rows (and optional edge rows)."""
    if ws is None:
        ws = _own_workspace(project_workspace_size(desc), (kc if kc is not None else vc).device, stream)
    _check(lib().fa_project(ctypes.byref(desc.c), _ptr(kc), _ptr(vc), _ptr(ck), _ptr(cv),
                            _ptr(ke), _ptr(ve), _ptr(ws), ws.numel(), _stream(stream)))


def decode(desc: Desc, q, kx, vx, ke, ve, ck, cv, scale, out, ws=None, stream=None):
    """fa_decode: one decode step for every query row into out [B, Hq, D] fp32."""
    if ws is None:
        ws = _own_workspace(decode_workspace_size(desc), q.device, stream)
    _check(lib().fa_decode(ctypes.byref(desc.c), _ptr(q), _ptr(kx), _ptr(vx), _ptr(ke),
                           _ptr(ve), _ptr(ck), _ptr(cv), ctypes.c_float(scale), _ptr(out),
                           _ptr(ws), ws.numel(), _stream(stream)))


def append(desc: Desc, k_new, v_new, ck, cv, ke, ve, stream=None):
    """fa_append: one token per sequence appended to a fixed-period cache
    (desc describes the lengths before the append); ck, cv, ke, ve in place."""
    _check(lib().fa_append(ctypes.byref(desc.c), _ptr(k_new), _ptr(v_new), _ptr(ck), _ptr(cv),
                           _ptr(ke), _ptr(ve), _stream(stream)))


def dim_sensitivity_workspace_size(desc: Desc, n_query: int = 1) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().fa_dim_sensitivity_workspace_size(ctypes.byref(desc.c), int(n_query), ctypes.byref(n)))
    return n.value


def dim_sensitivity(desc: Desc, n_query, q, k, noise, scale, sq, ws=None, stream=None):
    """fa_dim_sensitivity: squared per-dim output changes sq [Hq, D] fp32 when
    noise is added to one dim of the values at a time."""
    if ws is None:
        ws = _own_workspace(dim_sensitivity_workspace_size(desc, n_query), q.device, stream)
    _check(lib().fa_dim_sensitivity(ctypes.byref(desc.c), int(n_query), _ptr(q), _ptr(k), _ptr(noise),
                                    ctypes.c_float(scale), _ptr(sq), _ptr(ws), ws.numel(),
                                    _stream(stream)))


class fa_plan_t(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("rows", ctypes.c_int32), ("items", ctypes.c_int32),
                ("items2", ctypes.c_int32), ("passes", ctypes.c_int32),
                ("queries_per_pass", ctypes.c_int32)]


PATHS = {0: "valu", 1: "mfma", 2: "two_pass"}


def attend_plan(desc: Desc, n_query: int = 1) -> dict:
    """fa_attend_plan: the kernel path and work split fa_attend would use (host only)."""
    p = fa_plan_t()
    _check(lib().fa_attend_plan(ctypes.byref(desc.c), int(n_query), ctypes.byref(p)))
    d = {f: getattr(p, f) for f, _ in fa_plan_t._fields_}
    d["path"] = PATHS[d["path"]]
    return d


NOALLOC_SCRATCH_BYTES = 256 << 20  # FA_NOALLOC_SCRATCH_MIB of include/fa.h


def decode_noalloc(desc: Desc, q, kx, vx, ke, ve, ck, cv, scale, out, stream=None):
    """fa_decode_noalloc: fa_decode on the library's static scratch buffer (no
    workspace argument, no allocation)."""
    _check(lib().fa_decode_noalloc(ctypes.byref(desc.c), _ptr(q), _ptr(kx), _ptr(vx), _ptr(ke),
                                   _ptr(ve), _ptr(ck), _ptr(cv), ctypes.c_float(scale), _ptr(out),
                                   _stream(stream)))


def attend_workspace_size(desc: Desc, n_query: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().fa_attend_workspace_size(ctypes.byref(desc.c), int(n_query), ctypes.byref(n)))
    return n.value


def attend(desc: Desc, n_query, q, kx, vx, ke, ve, ck, cv, scale, out, lse=None, ws=None,
           stream=None):
    """fa_attend: n_query queries per sequence (q, out [B, n_query, Hq, D]) over the
    whole cache; lse [B, n_query, Hq] fp32 (optional) gets each row's log-sum-exp."""
    if ws is None:
        ws = _own_workspace(attend_workspace_size(desc, n_query), q.device, stream)
    _check(lib().fa_attend(ctypes.byref(desc.c), int(n_query), _ptr(q), _ptr(kx), _ptr(vx),
                           _ptr(ke), _ptr(ve), _ptr(ck), _ptr(cv), ctypes.c_float(scale),
                           _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))


def coef_budget(M: int, fraction: float = 0.3) -> int:
    """fa_coef_budget: real coefficients for the first floor(fraction * M) FFT bins."""
    return int(lib().fa_coef_budget(int(M), float(fraction)))


def cache_bytes(desc: Desc):
    """fa_cache_bytes: (uncompressed, compressed) bytes of the KV cache."""
    f, c = ctypes.c_uint64(0), ctypes.c_uint64(0)
    _check(lib().fa_cache_bytes(ctypes.byref(desc.c), ctypes.byref(f), ctypes.byref(c)))
    return f.value, c.value


def time_main_kernel(before=None, after=None):
    """fa_time_main_kernel: record two torch.cuda.Event around the dominant
    kernel of this thread's later calls (None, None: off).  The events are
    recorded once here first, so that their HIP handles exist."""
    if before is None or after is None:
        _check(lib().fa_time_main_kernel(None, None))
        return
    for e in (before, after):
        if not e.cuda_event:
            e.record()
    _check(lib().fa_time_main_kernel(ctypes.c_void_p(before.cuda_event),
                                     ctypes.c_void_p(after.cuda_event)))


def to_device(a: np.ndarray, device="cuda"):
    """numpy array from the workload generator -> device tensor (bf16 from uint16 bits)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)
