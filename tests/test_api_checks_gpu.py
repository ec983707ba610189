"""The PyTorch binding rejects caller-supplied outputs and workspaces that do not fit the call
before anything is launched: the library writes through raw device pointers, so a too-small or
wrongly typed buffer would be an out-of-bounds or misinterpreted write."""
import pytest
import torch

from tests.conftest import gpu_available

DEV = "cuda:0"


@pytest.fixture(scope="module")
def gma():
    if not gpu_available():
        pytest.skip("no GPU")
    import gaussian_mixture_token_amd as g
    from gaussian_mixture_token_amd import _lib
    _lib.load()
    return g


def _inputs(g, dtype=torch.bfloat16, N=100):
    w = g.workload(3, batch=1, heads=2, seq_len=N)
    inp = g.make_inputs(w)
    t = {k: v.to(DEV) for k, v in inp.items()}
    for k in ("qx", "kx", "v"):
        t[k] = t[k].to(dtype)
    return t


def _sentinel(shape, dtype):
    return torch.full(shape, 7.0, dtype=dtype, device=DEV)


@pytest.mark.gpu
@pytest.mark.parametrize("causal", [False, True])
def test_forward_rejects_bad_out(gma, causal):
    t = _inputs(gma)
    B, H, N, dv = t["v"].shape
    args = (t["qx"], t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"])
    bad = {"too small": _sentinel((B, H, N - 1, dv), torch.bfloat16),
           "wrong dtype": _sentinel((B, H, N, dv), torch.float32),
           "host memory": torch.zeros(B, H, N, dv, dtype=torch.bfloat16),
           "not contiguous": _sentinel((B, H, dv, N), torch.bfloat16).transpose(2, 3)}
    for name, out in bad.items():
        before = out.clone()
        with pytest.raises(ValueError):
            gma.forward(*args, causal=causal, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, before), name


@pytest.mark.gpu
def test_responsibilities_and_cross_attention_reject_bad_out(gma):
    t = _inputs(gma)
    B, H, N, _ = t["qx"].shape
    K = t["mu"].shape[1]
    for out in (_sentinel((B, H, N, K - 1), torch.float32), _sentinel((B, H, N, K), torch.bfloat16)):
        with pytest.raises(ValueError):
            gma.responsibilities(t["qx"], t["mu"], t["raw_var"], t["prior_logits"], out=out)
    q = t["qx"][:, :, :40].contiguous()
    with pytest.raises(ValueError):
        gma.forward_bidir(q, t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"],
                          out=_sentinel((B, H, N, t["v"].shape[-1]), torch.bfloat16))


@pytest.mark.gpu
def test_workspace_must_be_device_memory_on_the_inputs_device(gma):
    t = _inputs(gma)
    args = (t["qx"], t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"])
    with pytest.raises(ValueError):
        gma.forward(*args, causal=True, workspace=torch.zeros(1 << 24, dtype=torch.uint8))
    with pytest.raises(ValueError):
        gma.responsibilities(t["qx"], t["mu"], t["raw_var"], t["prior_logits"],
                             workspace=torch.zeros(1 << 20, dtype=torch.uint8))


@pytest.mark.gpu
def test_decode_rejects_bad_out_and_state(gma):
    t = _inputs(gma, N=1)
    B, H, _, dv = t["v"].shape
    K = t["mu"].shape[1]
    state = torch.zeros(B, H, K, dv + 1, dtype=torch.float32, device=DEV)
    args = (t["qx"], t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"])
    with pytest.raises(ValueError):
        gma.decode_step(*args, state, out=_sentinel((B, H, 1, dv - 8), torch.bfloat16))
    with pytest.raises(ValueError):
        gma.decode_step(*args, state[:, :, :-1].contiguous())
    assert (state == 0).all()


@pytest.mark.gpu
def test_exp2_rate_probe(gma):
    # the measurement entry point: a positive rate of the order the unit counts give (about 1e13 per second
    # on this class of GPU; bounded loosely so that a clock change cannot fail it), and NULL rejected
    import ctypes
    from gaussian_mixture_token_amd import _lib
    lib = _lib.load()
    rate = ctypes.c_double()
    assert lib.gma_probe_exp2_rate(ctypes.byref(rate), None) == 0
    assert 1e11 < rate.value < 1e15
    assert lib.gma_probe_exp2_rate(None, None) == 1


@pytest.mark.gpu
def test_read_rate_probe(gma):
    # reads a 256 MiB buffer: a positive rate of the order of the HBM's (bounded loosely), the buffer
    # unchanged; NULL output, NULL or misaligned buffers and sizes below one piece rejected
    import ctypes
    import torch
    from gaussian_mixture_token_amd import _lib
    lib = _lib.load()
    x = torch.arange(1 << 26, dtype=torch.float32, device="cuda:0")
    y = x.clone()
    rate = ctypes.c_double()
    assert lib.gma_probe_read_rate(ctypes.c_void_p(x.data_ptr()), ctypes.c_size_t(x.numel() * 4),
                                   ctypes.byref(rate), None) == 0
    torch.cuda.synchronize()
    assert 1e11 < rate.value < 1e14
    assert torch.equal(x, y)
    p = ctypes.c_void_p(x.data_ptr())
    assert lib.gma_probe_read_rate(p, ctypes.c_size_t(1 << 20), None, None) == 1
    assert lib.gma_probe_read_rate(None, ctypes.c_size_t(1 << 20), ctypes.byref(rate), None) == 1
    assert lib.gma_probe_read_rate(ctypes.c_void_p(x.data_ptr() + 4), ctypes.c_size_t(1 << 20), ctypes.byref(rate),
                                   None) == 1
    assert lib.gma_probe_read_rate(p, ctypes.c_size_t(8), ctypes.byref(rate), None) == 1
