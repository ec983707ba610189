"""GPU parity of the backward pass (gma_backward_bidir / gma_backward_causal) against the fp64 oracle.

Tolerance per gradient tensor, the forward's contract carried over: max |g_gpu - g_ref| / max |g_ref|
<= 1e-4 for fp32 storage and <= 1e-2 for bf16 storage.  The backward accumulates in fp32; for bf16
storage its products split every fp32 operand into bf16 hi + lo (about 16 significant bits), so the
error is dominated by the one rounding of dqx, dkx and dv to bf16 (unit roundoff 2^-8).

Inputs: the seeded workload generators (gaussian_mixture_token_amd.workloads) plus a seeded dL/dO.
With d_r >= 64 and N(0, 1) routing inputs the posteriors are nearly one-hot, so the routing
gradients are small; the "soft" cases scale Q_X and K_X by 1/4 (exact in bf16) so that every
term of the softmax and log-density gradients is exercised.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}
DEV = "cuda:0"
NAMES = ("dqx", "dkx", "dv", "dmu", "draw_var", "dprior_logits")


@pytest.fixture(scope="module")
def gma():
    if not gpu_available():
        pytest.skip("no GPU")
    import gaussian_mixture_token_amd as g
    from gaussian_mixture_token_amd import _lib
    _lib.load()
    oracle.build(force=False)
    return g


def say(msg):
    print(msg, flush=True)


def inputs(g, w, soft, heads=None):
    inp = g.make_inputs(w, heads)
    if soft:
        inp["qx"] = inp["qx"] * 0.25
        inp["kx"] = inp["kx"] * 0.25
    return inp, g.make_dout(w, heads)


def run_gpu(g, w, inp, dout, causal, **kw):
    t = {k: v.to(DEV) for k, v in inp.items()}
    out = g.backward(t["qx"], t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"], dout.to(DEV), eps=w.eps,
                     causal=causal, **kw)
    torch.cuda.synchronize()
    return out


def check(w, inp, dout, causal, got, only=NAMES):
    ref = oracle.backward(inp["qx"], inp["kx"], inp["v"], inp["mu"], inp["raw_var"], inp["prior_logits"], dout,
                          eps=w.eps, causal=causal)
    for name in only:
        a = got[name].detach().float().cpu().numpy().astype(np.float64)
        r = ref[name]
        assert np.isfinite(a).all(), name
        scale = np.abs(r).max()
        err = float(np.abs(a - r).max() / scale) if scale > 0 else float(np.abs(a).max())
        say("  %-14s rel-to-max %.3e (max |ref| %.3e)" % (name, err, scale))
        assert err <= TOL[w.dtype], name


@pytest.mark.parametrize("soft", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cfg,N", [(0, 256), (1, 700), (2, 1100), (3, 2100), (4, 3001)])
def test_backward_matches_oracle(gma, cfg, N, causal, soft):
    w = gma.workload(cfg)
    w = w.with_(batch=min(w.batch, 2), heads=min(w.heads, 2), seq_len=N)
    say("backward cfg%d causal=%s soft=%s %s" % (cfg, causal, soft, w))
    inp, dout = inputs(gma, w, soft)
    check(w, inp, dout, causal, run_gpu(gma, w, inp, dout, causal))


@pytest.mark.parametrize("base", [0, 2, 3])
@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 1023, 1024, 1025])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_tails_and_tiny_lengths(gma, base, N, causal):
    # eps = 0.05 here: with a row that sees a single key (N = 1, or row 0 of a causal pass) and
    # eps -> 0, O = v a / (a + eps) and the routing gradient of that row is an O(eps) remainder of
    # two nearly equal terms, which fp32 resolves only to about u / eps of its own size
    w = gma.workload(base)
    w = w.with_(batch=1, heads=min(w.heads, 2), seq_len=N, eps=0.05)
    say("backward tails base=%d N=%d causal=%s" % (base, N, causal))
    inp, dout = inputs(gma, w, True)
    check(w, inp, dout, causal, run_gpu(gma, w, inp, dout, causal))


@pytest.mark.parametrize("shape", [(5, 7, 6), (40, 1, 20), (3, 256, 2), (256, 16, 255), (130, 65, 129)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_odd_shapes(gma, shape, dtype, causal):
    d_r, K, d_v = shape
    w = gma.workload(0).with_(dtype=dtype, batch=2, heads=2, seq_len=150, d_route=d_r, n_comp=K, d_value=d_v)
    say("backward shape=%s %s causal=%s" % (shape, dtype, causal))
    inp, dout = inputs(gma, w, True)
    check(w, inp, dout, causal, run_gpu(gma, w, inp, dout, causal))


@pytest.mark.parametrize("shape", [(64, 32, 64), (128, 32, 64), (64, 64, 32), (128, 64, 64), (36, 20, 40),
                                   (100, 44, 24), (12, 4, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_small_fused_row_classes(gma, shape, causal):
    # bf16 storage with K <= 64 and d_r <= 128 (multiples of 4): the fused posterior / routing-input /
    # parameter-partial row kernel of each padded class (K to 32 or 64, d_r to 64 or 128), over three
    # segments of 1024 tokens with a ragged last chunk
    d_r, K, d_v = shape
    w = gma.workload(2).with_(batch=1, heads=2, seq_len=2500, d_route=d_r, n_comp=K, d_value=d_v)
    say("backward small class shape=%s causal=%s" % (shape, causal))
    inp, dout = inputs(gma, w, True)
    check(w, inp, dout, causal, run_gpu(gma, w, inp, dout, causal))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_single_token_small_eps(gma, causal):
    # the degenerate case above at eps = 1e-6: dv = (gamma_Q . gamma_K) dO / (gamma_Q . gamma_K + eps) is
    # well conditioned and held to the usual bound; the routing and mixture gradients are O(eps)
    # remainders, held to an absolute bound of fp32 rounding on the terms that cancel
    w = gma.workload(0).with_(seq_len=1, heads=2)
    inp, dout = inputs(gma, w, True)
    got = run_gpu(gma, w, inp, dout, causal)
    check(w, inp, dout, causal, got, only=("dv",))
    ref = oracle.backward(inp["qx"], inp["kx"], inp["v"], inp["mu"], inp["raw_var"], inp["prior_logits"], dout,
                          eps=w.eps, causal=causal)
    terms = float(dout.abs().max()) * float(inp["v"].abs().max()) * 64.0   # |dO| |v| times the log-density slope
    for name in ("dqx", "dkx", "dmu", "draw_var", "dprior_logits"):
        err = float(np.abs(got[name].cpu().numpy().astype(np.float64) - ref[name]).max())
        say("  %-14s abs err %.3e (bound %.3e)" % (name, err, 1e-5 * terms))
        assert err <= 1e-5 * terms, name


@pytest.mark.parametrize("causal", [False, True])
def test_backward_bitwise_deterministic(gma, causal):
    w = gma.workload(3).with_(heads=2, seq_len=1500)
    inp, dout = inputs(gma, w, True)
    a = run_gpu(gma, w, inp, dout, causal)
    b = run_gpu(gma, w, inp, dout, causal)
    for name in NAMES:
        assert torch.equal(a[name], b[name]), name


def test_backward_causal_ignores_later_gradients(gma):
    # dL/dO zero from row m on: no key or value at a row >= m reaches the loss (only later queries
    # see it), so dkx and dv vanish there exactly, and so does dqx
    w = gma.workload(3).with_(heads=2, seq_len=900)
    inp, dout = inputs(gma, w, True)
    m = 333
    dout[:, :, m:] = 0
    got = run_gpu(gma, w, inp, dout, True)
    for name in ("dqx", "dkx", "dv"):
        assert got[name][:, :, m:].abs().max().item() == 0.0, name


def test_backward_cfg3_full_size_every_head(gma):
    # the full 16-head, 65536-token causal bf16 problem on the GPU, every head against the oracle (which
    # runs the heads in parallel)
    w = gma.workload(3)
    say("backward cfg3 full size %s" % (w,))
    inp, dout = inputs(gma, w, False)
    check(w, inp, dout, True, run_gpu(gma, w, inp, dout, True))


@pytest.mark.parametrize("cfg", [1, 2])
def test_backward_full_size_every_head(gma, cfg):
    # the fp32 causal (B4 H8 N4096 K64) and bf16 bidirectional (B32 H8 N4096 K32) workloads at full size,
    # every (batch, head) against the oracle
    w = gma.workload(cfg)
    say("backward full size %s" % (w,))
    inp, dout = inputs(gma, w, False)
    check(w, inp, dout, w.causal, run_gpu(gma, w, inp, dout, w.causal))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_peaked_posteriors(gma, dtype, causal):
    # routing inputs x 8 (exact in bf16): logits of thousands and posteriors one-hot to fp32 precision.
    # (With eps = 0 such inputs are ill-posed: a query whose component no visible key uses has
    # Gamma_Q . Z = 0 and O = 0 / 0, in the forward and in the oracle alike.)
    w = gma.workload(1).with_(dtype=dtype, batch=1, heads=2, seq_len=333)
    inp, dout = inputs(gma, w, False)
    inp["qx"] = inp["qx"] * 8
    inp["kx"] = inp["kx"] * 8
    got = run_gpu(gma, w, inp, dout, causal)
    for name in NAMES:
        assert torch.isfinite(got[name]).all(), name
    # logits of thousands carry fp32 rounding of about 1e-7 of their size, which decides near-ties between
    # components: a stress test of robustness, held to the bf16 bound on dv (the routing and mixture
    # gradients vanish except at such ties)
    check(w.with_(dtype="bf16"), inp, dout, causal, got, only=("dv",))


def _shifted(t):
    # the same values at an address 2 bytes past a 16-byte boundary (bf16 rows not 16-byte aligned)
    buf = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    out = buf[1:1 + t.numel()].view(t.shape)
    out.copy_(t)
    assert out.data_ptr() % 16 == 2
    return out


@pytest.mark.parametrize("which", ["v", "dout", "dv", "all"])
def test_backward_fused_shape_with_misaligned_rows(gma, which):
    # causal bf16 at K = d_v = 128 with v, dout or dv 2 bytes off a 16-byte boundary: staged through
    # aligned copies in the workspace, same results as the aligned call
    w = gma.workload(3).with_(heads=2, seq_len=700)
    inp, dout = inputs(gma, w, True)
    t = {k: x.to(DEV) for k, x in inp.items()}
    d = dout.to(DEV)
    ref = gma.backward(t["qx"], t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"], d, eps=w.eps, causal=True)
    vv = _shifted(t["v"]) if which in ("v", "all") else t["v"]
    dd = _shifted(d) if which in ("dout", "all") else d
    grads = {k: torch.empty_like(x) for k, x in ref.items()}
    if which in ("dv", "all"):
        grads["dv"] = _shifted(torch.zeros_like(t["v"]))
    got = gma.backward(t["qx"], t["kx"], vv, t["mu"], t["raw_var"], t["prior_logits"], dd, eps=w.eps, causal=True,
                       grads=grads)
    torch.cuda.synchronize()
    for name in NAMES:
        assert torch.equal(got[name], ref[name]), name
    check(w, inp, dout, True, got)


def _offset(t, nbytes):
    # the same values at an address nbytes past a 16-byte boundary
    el = t.element_size()
    buf = torch.empty(t.numel() + 16, dtype=t.dtype, device=t.device)
    out = buf[nbytes // el:nbytes // el + t.numel()].view(t.shape)
    out.copy_(t)
    assert out.data_ptr() % 16 == nbytes
    return out


@pytest.mark.parametrize("nbytes", [8, 2])
@pytest.mark.parametrize("which", ["v", "dout", "dv", "x", "all"])
def test_backward_bidir_small_class_alignment(gma, nbytes, which):
    # bidirectional bf16 at K = 32, d_v = 64: rows of v, dout or dv 8 bytes past a 16-byte boundary still
    # take the fused bidirectional kernels (8-byte pieces) and give the aligned call's results bit for bit;
    # 2 bytes past one, or routing inputs off 16 bytes, take the general kernels, held to the oracle
    w = gma.workload(2).with_(batch=1, heads=2, seq_len=1500)
    inp, dout = inputs(gma, w, True)
    t = {k: x.to(DEV) for k, x in inp.items()}
    d = dout.to(DEV)
    say("backward bidir alignment which=%s offset=%d" % (which, nbytes))
    ref = gma.backward(t["qx"], t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"], d, eps=w.eps,
                       causal=False)
    vv = _offset(t["v"], nbytes) if which in ("v", "all") else t["v"]
    dd = _offset(d, nbytes) if which in ("dout", "all") else d
    qx = _offset(t["qx"], nbytes) if which in ("x", "all") else t["qx"]
    kx = _offset(t["kx"], nbytes) if which in ("x", "all") else t["kx"]
    grads = {k: torch.empty_like(x) for k, x in ref.items()}
    if which in ("dv", "all"):
        grads["dv"] = _offset(torch.zeros_like(t["v"]), nbytes)
    got = gma.backward(qx, kx, vv, t["mu"], t["raw_var"], t["prior_logits"], dd, eps=w.eps, causal=False,
                       grads=grads)
    torch.cuda.synchronize()
    if nbytes == 8 and which != "x" and which != "all":
        for name in NAMES:
            assert torch.equal(got[name], ref[name]), name
    check(w, inp, dout, False, got)
