"""PyTorch-facing binding of libgma.so.

Tensors supply device memory and the current HIP stream; every step of the computation runs
in the library's HIP kernels.  There is no CPU or PyTorch fallback: a missing library or a
non-GPU tensor raises.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

__all__ = ["problem", "workspace_size", "responsibilities", "forward_bidir", "forward_causal", "forward_causal_noalloc",
           "forward", "backward", "decode_step", "responsibility_stats", "GmaError"]

GmaError = _lib.GmaError

_DTYPES = {torch.float32: _lib.GMA_DTYPE_F32, torch.bfloat16: _lib.GMA_DTYPE_BF16}


def problem(B: int, H: int, N: int, d_r: int, K: int, d_v: int, dtype: torch.dtype, eps: float = 1e-6) -> _lib.Problem:
    if dtype not in _DTYPES:
        raise TypeError("dtype must be torch.float32 or torch.bfloat16")
    return _lib.Problem(B, H, N, d_r, K, d_v, _DTYPES[dtype], float(eps))


def workspace_size(prob: _lib.Problem, op: int) -> int:
    return int(_lib.load().gma_workspace_size(ctypes.byref(prob), op))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_gpu(*ts: torch.Tensor) -> torch.device:
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if t.device != dev:
            raise ValueError("all tensors must be on one device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    return dev


def _params(mu, raw_var, prior_logits, H, K, d_r):
    for name, t, shape in (("mu", mu, (H, K, d_r)), ("raw_var", raw_var, (H, K, d_r)),
                           ("prior_logits", prior_logits, (H, K))):
        if t.dtype != torch.float32:
            raise TypeError("%s must be float32" % name)
        if tuple(t.shape) != shape:
            raise ValueError("%s must have shape %s, got %s" % (name, shape, tuple(t.shape)))


def _on(t: torch.Tensor, dev: torch.device, name: str) -> None:
    """t is a contiguous GPU tensor on device dev (the library is handed raw device pointers)."""
    if not t.is_cuda or t.device != dev:
        raise ValueError("%s must be on the inputs' device %s (got %s)" % (name, dev, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_out(out: torch.Tensor, shape, dtype: torch.dtype, dev: torch.device, name: str = "out") -> None:
    """A caller-supplied output: the library writes prod(shape) elements of dtype through its pointer."""
    _on(out, dev, name)
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype:
        raise ValueError("%s must be a %s tensor of shape %s (got %s %s)" % (name, dtype, tuple(shape), out.dtype,
                                                                            tuple(out.shape)))


def _workspace(nbytes: int, device: torch.device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    # a caller's workspace is passed through with its size: the library validates it (the causal
    # pass accepts less than the advertised size and then recomputes Gamma_K)
    if workspace is not None:
        _on(workspace, device, "workspace")
        return workspace
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def responsibilities(x: torch.Tensor, mu: torch.Tensor, raw_var: torch.Tensor, prior_logits: torch.Tensor,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gamma [B, H, N, K] fp32 for x [B, H, N, d_r] (fp32 or bf16)."""
    B, H, N, d_r = x.shape
    K = mu.shape[1]
    _params(mu, raw_var, prior_logits, H, K, d_r)
    dev = _check_gpu(x, mu, raw_var, prior_logits)
    prob = problem(B, H, N, d_r, K, 1, x.dtype)
    if out is None:
        out = torch.empty(B, H, N, K, dtype=torch.float32, device=dev)
    _check_out(out, (B, H, N, K), torch.float32, dev)
    ws = _workspace(workspace_size(prob, _lib.GMA_OP_RESPONSIBILITIES), dev, workspace)
    _lib.check(_lib.load().gma_responsibilities(ctypes.byref(prob), _ptr(x), _ptr(mu), _ptr(raw_var), _ptr(prior_logits),
                                                _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return out


def _forward(fn_name: str, op: int, qx, kx, v, mu, raw_var, prior_logits, eps, out, workspace, states=None):
    B, H, N, d_r = qx.shape
    d_v = v.shape[-1]
    K = mu.shape[1]
    if tuple(kx.shape) != (B, H, N, d_r) or tuple(v.shape[:3]) != (B, H, N):
        raise ValueError("qx, kx must be [B, H, N, d_r] and v [B, H, N, d_v]")
    if not (qx.dtype == kx.dtype == v.dtype):
        raise TypeError("qx, kx and v must share one dtype")
    _params(mu, raw_var, prior_logits, H, K, d_r)
    dev = _check_gpu(qx, kx, v, mu, raw_var, prior_logits)
    prob = problem(B, H, N, d_r, K, d_v, qx.dtype, eps)
    if out is None:
        out = torch.empty(B, H, N, d_v, dtype=qx.dtype, device=dev)
    _check_out(out, (B, H, N, d_v), qx.dtype, dev)
    ws = _workspace(workspace_size(prob, op), dev, workspace)
    fn = getattr(_lib.load(), fn_name)
    extra = []
    if states is not None:
        for name, t in zip(("state_in", "state_out"), states):
            if t is not None:
                if t.dtype != torch.float32 or tuple(t.shape) != (B, H, K, d_v + 1) or not t.is_contiguous():
                    raise ValueError("%s must be a contiguous float32 [B, H, K, d_v + 1] tensor" % name)
                _on(t, dev, name)
        extra = [_ptr(t) if t is not None else None for t in states]
    _lib.check(fn(ctypes.byref(prob), _ptr(qx), _ptr(kx), _ptr(v), _ptr(mu), _ptr(raw_var), _ptr(prior_logits),
                  *extra, _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return out


def forward_bidir(qx, kx, v, mu, raw_var, prior_logits, eps: float = 1e-6, out=None, workspace=None):
    """O = Gamma_Q (Gamma_K^T V) / (Gamma_Q (Gamma_K^T 1) + eps); qx [B, H, N_q, d_r], kx [B, H, N_kv, d_r],
    v [B, H, N_kv, d_v] (N_kv may differ from N_q: cross-attention)."""
    if kx.dim() == 4 and qx.dim() == 4 and kx.shape[2] != qx.shape[2]:
        return _forward_kv(qx, kx, v, mu, raw_var, prior_logits, eps, out, workspace)
    return _forward("gma_forward_bidir", _lib.GMA_OP_FORWARD_BIDIR, qx, kx, v, mu, raw_var, prior_logits, eps,
                    out, workspace)


def _forward_kv(qx, kx, v, mu, raw_var, prior_logits, eps, out, workspace):
    B, H, Nq, d_r = qx.shape
    Nk = kx.shape[2]
    d_v = v.shape[-1]
    K = mu.shape[1]
    if tuple(kx.shape) != (B, H, Nk, d_r) or tuple(v.shape[:3]) != (B, H, Nk):
        raise ValueError("qx must be [B, H, N_q, d_r], kx [B, H, N_kv, d_r] and v [B, H, N_kv, d_v]")
    if not (qx.dtype == kx.dtype == v.dtype):
        raise TypeError("qx, kx and v must share one dtype")
    _params(mu, raw_var, prior_logits, H, K, d_r)
    dev = _check_gpu(qx, kx, v, mu, raw_var, prior_logits)
    prob = problem(B, H, Nq, d_r, K, d_v, qx.dtype, eps)
    if out is None:
        out = torch.empty(B, H, Nq, d_v, dtype=qx.dtype, device=dev)
    _check_out(out, (B, H, Nq, d_v), qx.dtype, dev)
    ws = _workspace(workspace_size(problem(B, H, max(Nq, Nk), d_r, K, d_v, qx.dtype, eps), _lib.GMA_OP_FORWARD_BIDIR),
                    dev, workspace)
    _lib.check(_lib.load().gma_forward_bidir_kv(ctypes.byref(prob), Nk, _ptr(qx), _ptr(kx), _ptr(v), _ptr(mu),
                                                _ptr(raw_var), _ptr(prior_logits), _ptr(out), _ptr(ws),
                                                ws.numel() * ws.element_size(), _stream(dev)))
    return out


def forward_causal(qx, kx, v, mu, raw_var, prior_logits, eps: float = 1e-6, out=None, workspace=None,
                   state_in=None, state_out=None):
    """Causal O (prefix sums of Gamma_K^T V and Gamma_K^T 1, inclusive of the current token).

    With state_in and/or state_out (float32 [B, H, K, d_v + 1]: row k holds Vt[k, :] then Z[k]) the
    latent memory is carried across calls: state_in is the memory after all earlier tokens (None =
    zero), state_out receives it after this call's last token (it may be state_in itself)."""
    if state_in is None and state_out is None:
        return _forward("gma_forward_causal", _lib.GMA_OP_FORWARD_CAUSAL, qx, kx, v, mu, raw_var, prior_logits, eps,
                        out, workspace)
    return _forward("gma_forward_causal_state", _lib.GMA_OP_FORWARD_CAUSAL_STATE, qx, kx, v, mu, raw_var,
                    prior_logits, eps, out, workspace, states=(state_in, state_out))


def forward_causal_noalloc(qx, kx, v, mu, raw_var, prior_logits, eps: float = 1e-6, out=None):
    """Causal O through gma_forward_causal_noalloc: the library's fixed scratch array is the workspace,
    so the call allocates nothing (``out`` must then be supplied by a caller that cannot allocate)."""
    B, H, N, d_r = qx.shape
    d_v = v.shape[-1]
    K = mu.shape[1]
    if tuple(kx.shape) != (B, H, N, d_r) or tuple(v.shape[:3]) != (B, H, N):
        raise ValueError("qx, kx must be [B, H, N, d_r] and v [B, H, N, d_v]")
    if not (qx.dtype == kx.dtype == v.dtype):
        raise TypeError("qx, kx and v must share one dtype")
    _params(mu, raw_var, prior_logits, H, K, d_r)
    dev = _check_gpu(qx, kx, v, mu, raw_var, prior_logits)
    prob = problem(B, H, N, d_r, K, d_v, qx.dtype, eps)
    if out is None:
        out = torch.empty(B, H, N, d_v, dtype=qx.dtype, device=dev)
    _check_out(out, (B, H, N, d_v), qx.dtype, dev)
    _lib.check(_lib.load().gma_forward_causal_noalloc(ctypes.byref(prob), _ptr(qx), _ptr(kx), _ptr(v), _ptr(mu),
                                                      _ptr(raw_var), _ptr(prior_logits), _ptr(out), _stream(dev)))
    return out


def forward(qx, kx, v, mu, raw_var, prior_logits, eps: float = 1e-6, causal: bool = False, out=None, workspace=None):
    f = forward_causal if causal else forward_bidir
    return f(qx, kx, v, mu, raw_var, prior_logits, eps=eps, out=out, workspace=workspace)


def decode_prepare(raw_var, prior_logits, prepared=None):
    """The decode step's mixture quantities (1 / softplus(raw_var) and the per-component constants) for
    raw_var [H, K, d_r] and prior_logits [H, K], as a uint8 device tensor of gma_decode_params_size bytes
    (written into `prepared` if given).  Pass it to decode_step(..., prepared=...) while the parameters
    stay unchanged."""
    H, K, d_r = raw_var.shape
    if raw_var.dtype != torch.float32 or prior_logits.dtype != torch.float32 or tuple(prior_logits.shape) != (H, K):
        raise ValueError("raw_var [H, K, d_r] and prior_logits [H, K] must be float32")
    raw_var, prior_logits = raw_var.contiguous(), prior_logits.contiguous()
    dev = _check_gpu(raw_var, prior_logits)
    prob = problem(1, H, 1, d_r, K, 1, torch.float32)
    lib = _lib.load()
    nbytes = int(lib.gma_decode_params_size(ctypes.byref(prob)))
    if nbytes == 0:
        raise ValueError("unsupported mixture shape H=%d K=%d d_r=%d" % (H, K, d_r))
    if prepared is None:
        prepared = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _on(prepared, dev, "prepared")
    _lib.check(lib.gma_decode_prepare(ctypes.byref(prob), _ptr(raw_var), _ptr(prior_logits), _ptr(prepared),
                                      prepared.numel() * prepared.element_size(), _stream(dev)))
    return prepared


def decode_step(qx, kx, v, mu, raw_var, prior_logits, state, eps: float = 1e-6, out=None, state_out=None,
                prepared=None):
    """One causal decode step: qx, kx [B, H, 1, d_r] (or [B, H, d_r]), v [B, H, 1, d_v]; state float32
    [B, H, K, d_v + 1] (row k: Vt[k, :] then Z[k]) is the memory after all earlier tokens and is
    updated in place unless state_out is given.  Returns the output row o [B, H, 1, d_v].  With
    `prepared` (decode_prepare of the same raw_var and prior_logits) the step reads the prepared
    mixture instead of deriving it from raw_var and prior_logits."""
    if qx.dim() == 3:
        qx, kx, v = qx.unsqueeze(2), kx.unsqueeze(2), v.unsqueeze(2)
    qx, kx, v = qx.contiguous(), kx.contiguous(), v.contiguous()   # one-token slices of a longer sequence
    B, H, N, d_r = qx.shape
    d_v = v.shape[-1]
    K = mu.shape[1]
    if N != 1 or tuple(kx.shape) != (B, H, 1, d_r) or tuple(v.shape[:3]) != (B, H, 1):
        raise ValueError("a decode step takes one token: qx, kx [B, H, 1, d_r], v [B, H, 1, d_v]")
    if not (qx.dtype == kx.dtype == v.dtype):
        raise TypeError("qx, kx and v must share one dtype")
    _params(mu, raw_var, prior_logits, H, K, d_r)
    dev = _check_gpu(qx, kx, v, mu, raw_var, prior_logits)
    for name, t in (("state", state), ("state_out", state_out)):
        if t is not None:
            if t.dtype != torch.float32 or tuple(t.shape) != (B, H, K, d_v + 1) or not t.is_contiguous():
                raise ValueError("%s must be a contiguous float32 [B, H, K, d_v + 1] tensor" % name)
            _on(t, dev, name)
    prob = problem(B, H, 1, d_r, K, d_v, qx.dtype, eps)
    if out is None:
        out = torch.empty(B, H, 1, d_v, dtype=qx.dtype, device=dev)
    _check_out(out, (B, H, 1, d_v), qx.dtype, dev)
    dst = state if state_out is None else state_out
    if prepared is not None:
        _on(prepared, dev, "prepared")
        _lib.check(_lib.load().gma_decode_step_prepared(
            ctypes.byref(prob), _ptr(qx), _ptr(kx), _ptr(v), _ptr(mu), _ptr(prepared),
            prepared.numel() * prepared.element_size(), _ptr(state), _ptr(dst), _ptr(out), _stream(dev)))
        return out
    _lib.check(_lib.load().gma_decode_step(ctypes.byref(prob), _ptr(qx), _ptr(kx), _ptr(v), _ptr(mu), _ptr(raw_var),
                                           _ptr(prior_logits), _ptr(state), _ptr(dst), _ptr(out), _stream(dev)))
    return out


def responsibility_stats(x, mu, raw_var, prior_logits, workspace=None):
    """Diagnostics of the responsibilities of x [B, H, N, d_r]: usage [B, H, K] fp32 (sum of Gamma over
    the rows), hard counts [B, H, K] int32 view of uint32 (rows whose largest gamma is at k, ties to
    the lowest k) and usage entropy [B, H] fp32 (of usage / N, divided by ln K: a fraction of its largest
    value)."""
    B, H, N, d_r = x.shape
    K = mu.shape[1]
    _params(mu, raw_var, prior_logits, H, K, d_r)
    dev = _check_gpu(x, mu, raw_var, prior_logits)
    prob = problem(B, H, N, d_r, K, 1, x.dtype)
    usage = torch.empty(B, H, K, dtype=torch.float32, device=dev)
    hard = torch.empty(B, H, K, dtype=torch.int32, device=dev)
    ent = torch.empty(B, H, dtype=torch.float32, device=dev)
    ws = _workspace(workspace_size(prob, _lib.GMA_OP_RESPONSIBILITY_STATS), dev, workspace)
    _lib.check(_lib.load().gma_responsibility_stats(ctypes.byref(prob), _ptr(x), _ptr(mu), _ptr(raw_var),
                                                    _ptr(prior_logits), _ptr(usage), _ptr(hard), _ptr(ent), _ptr(ws),
                                                    ws.numel() * ws.element_size(), _stream(dev)))
    return usage, hard, ent


def backward(qx, kx, v, mu, raw_var, prior_logits, dout, eps: float = 1e-6, causal: bool = False, workspace=None,
             grads=None):
    """Gradients of a loss through the bidirectional or causal forward, given dout = dL/dO [B, H, N, d_v]:
    a dict with dqx, dkx [B, H, N, d_r] and dv [B, H, N, d_v] in the input dtype, and dmu, draw_var
    [H, K, d_r], dprior_logits [H, K] fp32.  ``grads`` may supply that dict's tensors to write into."""
    B, H, N, d_r = qx.shape
    d_v = v.shape[-1]
    K = mu.shape[1]
    if tuple(kx.shape) != (B, H, N, d_r) or tuple(v.shape[:3]) != (B, H, N) or tuple(dout.shape) != tuple(v.shape):
        raise ValueError("qx, kx must be [B, H, N, d_r] and v, dout [B, H, N, d_v]")
    if not (qx.dtype == kx.dtype == v.dtype == dout.dtype):
        raise TypeError("qx, kx, v and dout must share one dtype")
    _params(mu, raw_var, prior_logits, H, K, d_r)
    dev = _check_gpu(qx, kx, v, dout, mu, raw_var, prior_logits)
    prob = problem(B, H, N, d_r, K, d_v, qx.dtype, eps)
    if grads is None:
        grads = {"dqx": torch.empty_like(qx), "dkx": torch.empty_like(kx), "dv": torch.empty_like(v),
                 "dmu": torch.empty_like(mu), "draw_var": torch.empty_like(raw_var),
                 "dprior_logits": torch.empty_like(prior_logits)}
    like = {"dqx": qx, "dkx": kx, "dv": v, "dmu": mu, "draw_var": raw_var, "dprior_logits": prior_logits}
    for name, ref in like.items():
        t = grads[name]
        if t.dtype != ref.dtype or t.shape != ref.shape:
            raise ValueError("%s must match its input's dtype and shape" % name)
        _on(t, dev, name)
    op = _lib.GMA_OP_BACKWARD_CAUSAL if causal else _lib.GMA_OP_BACKWARD_BIDIR
    ws = _workspace(workspace_size(prob, op), dev, workspace)
    fn = _lib.load().gma_backward_causal if causal else _lib.load().gma_backward_bidir
    _lib.check(fn(ctypes.byref(prob), _ptr(qx), _ptr(kx), _ptr(v), _ptr(mu), _ptr(raw_var), _ptr(prior_logits),
                  _ptr(dout), _ptr(grads["dqx"]), _ptr(grads["dkx"]), _ptr(grads["dv"]), _ptr(grads["dmu"]),
                  _ptr(grads["draw_var"]), _ptr(grads["dprior_logits"]), _ptr(ws), ws.numel() * ws.element_size(),
                  _stream(dev)))
    return grads
