"""fp64 CPU oracle of the Gaussian Mixture Attention mixer (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
this package imports nothing from the product path.

The arithmetic lives in ``gma_oracle.c`` (plain C, fp64, OpenMP over
independent rows/columns, sequential sums over the sequence); this module only
compiles it with gcc and marshals numpy arrays.  Formulas follow the page
"Attention par Mélange Gaussien (GMA)", section "Méthodologie", sub-section
"Mécanisme Central" (items 1-3); see the C file for the per-function mapping.

Parity pins for every function are in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gma_oracle.c")
_LIB = os.path.join(_HERE, "libgma_oracle.so")
_lock = threading.Lock()
_lib = None

__all__ = ["build", "params", "responsibilities", "forward", "forward_causal_state", "forward_bidir_kv", "responsibility_stats", "backward", "set_threads", "max_threads"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2 -fopenmp, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB)
            dp = ctypes.POINTER(ctypes.c_double)
            i64, i32 = ctypes.c_int64, ctypes.c_int32
            lib.gma_oracle_params.argtypes = [i64, i32, i32, dp, dp, dp, dp]
            lib.gma_oracle_params.restype = None
            lib.gma_oracle_responsibilities.argtypes = [i64, i64, i64, i32, i32, dp, dp, dp, dp, dp]
            lib.gma_oracle_responsibilities.restype = ctypes.c_int
            lib.gma_oracle_forward.argtypes = [ctypes.c_int, i64, i64, i64, i32, i32, i32,
                                               ctypes.c_double, dp, dp, dp, dp, dp, dp, dp]
            lib.gma_oracle_forward.restype = ctypes.c_int
            lib.gma_oracle_forward_causal_state.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.c_double,
                                                            dp, dp, dp, dp, dp, dp, dp, dp, dp]
            lib.gma_oracle_forward_causal_state.restype = ctypes.c_int
            lib.gma_oracle_forward_bidir_kv.argtypes = [i64, i64, i64, i64, i32, i32, i32, ctypes.c_double,
                                                        dp, dp, dp, dp, dp, dp, dp]
            lib.gma_oracle_forward_bidir_kv.restype = ctypes.c_int
            lib.gma_oracle_backward.argtypes = [ctypes.c_int, i64, i64, i64, i32, i32, i32, ctypes.c_double,
                                                dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp]
            lib.gma_oracle_backward.restype = ctypes.c_int
            lib.gma_oracle_set_threads.argtypes = [ctypes.c_int]
            lib.gma_oracle_set_threads.restype = None
            lib.gma_oracle_max_threads.argtypes = []
            lib.gma_oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    """Exact upcast to a C-contiguous fp64 array (bf16 and fp32 values are exact in fp64)."""
    if hasattr(a, "detach"):  # torch tensor: go through fp32, exact for bf16/fp32
        import torch
        a = a.detach().to("cpu")
        if a.dtype != torch.float64:
            a = a.to(torch.float64)
        a = a.numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def set_threads(n: int) -> None:
    _load().gma_oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().gma_oracle_max_threads())


def params(raw_var, prior_logits):
    """(sigma^2 [H, K, d_r], log pi [H, K]) from the raw learned parameters."""
    rv, pl = _f64(raw_var), _f64(prior_logits)
    H, K, dr = rv.shape
    assert pl.shape == (H, K)
    var = np.empty_like(rv)
    logp = np.empty_like(pl)
    _load().gma_oracle_params(H, K, dr, _ptr(rv), _ptr(pl), _ptr(var), _ptr(logp))
    return var, logp


def responsibilities(x, mu, raw_var, prior_logits) -> np.ndarray:
    """Gamma [B, H, N, K] for x [B, H, N, d_r] (x may also be [H, N, d_r] or [N, d_r] with H = 1)."""
    x, mu, rv, pl = _f64(x), _f64(mu), _f64(raw_var), _f64(prior_logits)
    shape = x.shape
    if x.ndim == 2:
        x = x[None, None]
    elif x.ndim == 3:
        x = x[None]
    B, H, N, dr = x.shape
    K = mu.shape[1]
    assert mu.shape == (H, K, dr) and rv.shape == (H, K, dr) and pl.shape == (H, K)
    g = np.empty((B, H, N, K), dtype=np.float64)
    rc = _load().gma_oracle_responsibilities(B, H, N, dr, K, _ptr(x), _ptr(mu), _ptr(rv), _ptr(pl), _ptr(g))
    if rc != 0:
        raise MemoryError("oracle: allocation failed")
    return g.reshape(shape[:-1] + (K,))


def forward(qx, kx, v, mu, raw_var, prior_logits, eps: float = 1e-6, causal: bool = False,
            threads: Optional[int] = None) -> np.ndarray:
    """O [B, H, N, d_v] in fp64.  qx, kx [B, H, N, d_r]; v [B, H, N, d_v]."""
    qx, kx, v = _f64(qx), _f64(kx), _f64(v)
    mu, rv, pl = _f64(mu), _f64(raw_var), _f64(prior_logits)
    squeeze = qx.ndim == 2
    if squeeze:
        qx, kx, v = qx[None, None], kx[None, None], v[None, None]
    B, H, N, dr = qx.shape
    dv = v.shape[-1]
    K = mu.shape[1]
    assert kx.shape == qx.shape and v.shape == (B, H, N, dv)
    assert mu.shape == (H, K, dr) and rv.shape == (H, K, dr) and pl.shape == (H, K)
    o = np.empty((B, H, N, dv), dtype=np.float64)
    lib = _load()
    if threads is not None:
        lib.gma_oracle_set_threads(int(threads))
    rc = lib.gma_oracle_forward(1 if causal else 0, B, H, N, dr, K, dv, float(eps), _ptr(qx), _ptr(kx),
                                _ptr(v), _ptr(mu), _ptr(rv), _ptr(pl), _ptr(o))
    if rc != 0:
        raise MemoryError("oracle: allocation failed")
    return o[0, 0] if squeeze else o


def forward_causal_state(qx, kx, v, mu, raw_var, prior_logits, eps: float = 1e-6, state_in=None,
                         threads: Optional[int] = None):
    """Causal O [B, H, N, d_v] and the latent memory after the last token, [B, H, K, d_v + 1]
    (row k: Vt[k, :] then Z[k]), starting from state_in (same layout; None = zero)."""
    qx, kx, v = _f64(qx), _f64(kx), _f64(v)
    mu, rv, pl = _f64(mu), _f64(raw_var), _f64(prior_logits)
    B, H, N, dr = qx.shape
    dv = v.shape[-1]
    K = mu.shape[1]
    assert kx.shape == qx.shape and v.shape == (B, H, N, dv)
    assert mu.shape == (H, K, dr) and rv.shape == (H, K, dr) and pl.shape == (H, K)
    sin = None if state_in is None else _f64(state_in)
    if sin is not None:
        assert sin.shape == (B, H, K, dv + 1)
    o = np.empty((B, H, N, dv), dtype=np.float64)
    sout = np.empty((B, H, K, dv + 1), dtype=np.float64)
    lib = _load()
    if threads is not None:
        lib.gma_oracle_set_threads(int(threads))
    rc = lib.gma_oracle_forward_causal_state(B, H, N, dr, K, dv, float(eps), _ptr(qx), _ptr(kx), _ptr(v),
                                             _ptr(mu), _ptr(rv), _ptr(pl),
                                             None if sin is None else _ptr(sin), _ptr(sout), _ptr(o))
    if rc != 0:
        raise MemoryError("oracle: allocation failed")
    return o, sout


def forward_bidir_kv(qx, kx, v, mu, raw_var, prior_logits, eps: float = 1e-6,
                     threads: Optional[int] = None) -> np.ndarray:
    """Bidirectional O [B, H, Nq, d_v] with queries qx [B, H, Nq, d_r] and keys / values kx
    [B, H, Nk, d_r], v [B, H, Nk, d_v] (cross-attention)."""
    qx, kx, v = _f64(qx), _f64(kx), _f64(v)
    mu, rv, pl = _f64(mu), _f64(raw_var), _f64(prior_logits)
    B, H, Nq, dr = qx.shape
    Nk = kx.shape[2]
    dv = v.shape[-1]
    K = mu.shape[1]
    assert kx.shape == (B, H, Nk, dr) and v.shape == (B, H, Nk, dv)
    assert mu.shape == (H, K, dr) and rv.shape == (H, K, dr) and pl.shape == (H, K)
    o = np.empty((B, H, Nq, dv), dtype=np.float64)
    lib = _load()
    if threads is not None:
        lib.gma_oracle_set_threads(int(threads))
    rc = lib.gma_oracle_forward_bidir_kv(B, H, Nq, Nk, dr, K, dv, float(eps), _ptr(qx), _ptr(kx), _ptr(v),
                                         _ptr(mu), _ptr(rv), _ptr(pl), _ptr(o))
    if rc != 0:
        raise MemoryError("oracle: allocation failed")
    return o


def backward(qx, kx, v, mu, raw_var, prior_logits, dout, eps: float = 1e-6, causal: bool = False,
             threads: Optional[int] = None):
    """Gradients of a loss through the mixer given dout = dL/dO [B, H, N, d_v]: a dict with dqx,
    dkx [B, H, N, d_r], dv [B, H, N, d_v], dmu, draw_var [H, K, d_r] and dprior_logits [H, K], all
    fp64 (the chain rule through the same definitions as ``forward``; see gma_oracle_backward)."""
    qx, kx, v, do = _f64(qx), _f64(kx), _f64(v), _f64(dout)
    mu, rv, pl = _f64(mu), _f64(raw_var), _f64(prior_logits)
    B, H, N, dr = qx.shape
    dv = v.shape[-1]
    K = mu.shape[1]
    assert kx.shape == qx.shape and v.shape == (B, H, N, dv) and do.shape == v.shape
    assert mu.shape == (H, K, dr) and rv.shape == (H, K, dr) and pl.shape == (H, K)
    out = {"dqx": np.empty_like(qx), "dkx": np.empty_like(kx), "dv": np.empty_like(v),
           "dmu": np.empty_like(mu), "draw_var": np.empty_like(rv), "dprior_logits": np.empty_like(pl)}
    lib = _load()
    if threads is not None:
        lib.gma_oracle_set_threads(int(threads))
    rc = lib.gma_oracle_backward(1 if causal else 0, B, H, N, dr, K, dv, float(eps), _ptr(qx), _ptr(kx),
                                 _ptr(v), _ptr(mu), _ptr(rv), _ptr(pl), _ptr(do), _ptr(out["dqx"]),
                                 _ptr(out["dkx"]), _ptr(out["dv"]), _ptr(out["dmu"]), _ptr(out["draw_var"]),
                                 _ptr(out["dprior_logits"]))
    if rc != 0:
        raise MemoryError("oracle: allocation failed")
    return out


def responsibility_stats(x, mu, raw_var, prior_logits):
    """Diagnostics of the responsibilities of x [B, H, N, d_r] (reductions over the rows of Gamma):
    usage [B, H, K] = sum_n gamma_nk; hard counts [B, H, K] = number of rows whose largest gamma is at
    component k (ties to the lowest k); usage entropy [B, H] = -sum_k p_k ln p_k / ln K with
    p = usage / N (0 ln 0 = 0; 0 for K = 1), the entropy of the usage distribution as a fraction of
    its largest value.  The normalisation by ln K is the reading of the GMA page, "Résultats et
    Performance" (interpretability): its usage entropy of 0.933 for a model that used 104 of 128
    components fits H / ln K (about 92 effective components), not entropy in nats (0.933 nats would be
    about 2.5).  Also returns the gap between each row's two largest responsibilities [B, H, N], the
    margin by which its hard assignment is decided."""
    g = responsibilities(x, mu, raw_var, prior_logits)          # [B, H, N, K] fp64
    B, H, N, K = g.shape
    usage = g.sum(axis=2)
    arg = np.argmax(g, axis=-1)                                  # first maximum on ties
    hard = np.zeros((B, H, K), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            hard[b, h] = np.bincount(arg[b, h], minlength=K)
    p = usage / N
    with np.errstate(divide="ignore", invalid="ignore"):
        ent = -np.where(p > 0, p * np.log(p), 0.0).sum(axis=-1)
    ent = ent / math.log(K) if K > 1 else np.zeros_like(ent)
    top2 = np.sort(g, axis=-1)[..., -2:] if K > 1 else np.concatenate([np.zeros_like(g), g], axis=-1)
    gap = top2[..., 1] - top2[..., 0]
    return usage, hard, ent, gap
