"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Tolerance (from the method's precision contract): max |O_gpu - O_ref| / max |O_ref| <= 1e-4
for fp32 storage and <= 1e-2 for bf16 storage with fp32 accumulation.  Responsibilities:
max |Gamma_gpu - Gamma_ref| <= 1e-5 (fp32) / 1e-2 (bf16), an absolute bound on probabilities.  The
fp32 bound follows from the arithmetic: the logits are summed in fp64 over steps of 16 dims, each
step's 32 products in fp32 (a few ulp of a partial sum of order 10), and an error dl in a logit
difference moves Gamma by at most ln 2 / 4 * dl.

Inputs come from gaussian_mixture_token_amd.workloads (seeded; shapes of the five workloads).
Full-size workloads that the oracle cannot finish in seconds are compared on sampled heads:
(batch, head) slices are independent, so the oracle on a slice is exact for that slice.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}
TOL_GAMMA = {"f32": 1e-5, "bf16": 1e-2}


@pytest.fixture(scope="module")
def gma():
    if not gpu_available():
        pytest.skip("no GPU")
    import gaussian_mixture_token_amd as g
    from gaussian_mixture_token_amd import _lib
    _lib.load()
    oracle.build(force=False)
    return g


DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def gpu_forward(g, w, inp, causal=None, **kw):
    causal = w.causal if causal is None else causal
    t = {k: v.to(DEV) for k, v in inp.items()}
    o = g.forward(t["qx"], t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"], eps=w.eps, causal=causal, **kw)
    torch.cuda.synchronize()
    return o


def ref_forward(w, inp, causal=None):
    causal = w.causal if causal is None else causal
    return oracle.forward(inp["qx"], inp["kx"], inp["v"], inp["mu"], inp["raw_var"], inp["prior_logits"],
                          eps=w.eps, causal=causal)


def rel_err(o, ref):
    o = o.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(o) else o
    return float(np.abs(o - ref).max() / np.abs(ref).max())


# ------------------------------------------------------------------------------------ responsibilities


@pytest.mark.parametrize("cfg,shape", [(0, None), (1, None), (2, None), (3, None), (4, None), (1, (128, 128, 128)),
                                       (3, (128, 256, 128))])
def test_responsibilities_match_oracle(gma, cfg, shape):
    w = gma.workload(cfg)
    w = w.with_(batch=1, heads=min(w.heads, 2), seq_len=min(w.seq_len, 1000))
    if shape:
        w = w.with_(d_route=shape[0], n_comp=shape[1], d_value=shape[2])
    say("responsibilities cfg%d %s" % (cfg, w))
    inp = gma.make_inputs(w)
    t = {k: v.to(DEV) for k, v in inp.items()}
    gq = gma.responsibilities(t["qx"], t["mu"], t["raw_var"], t["prior_logits"])
    torch.cuda.synchronize()
    ref = oracle.responsibilities(inp["qx"], inp["mu"], inp["raw_var"], inp["prior_logits"])
    got = gq.cpu().numpy().astype(np.float64)
    assert (got >= 0).all()
    np.testing.assert_allclose(got.sum(-1), 1.0, atol=1e-5)
    err = np.abs(got - ref).max()
    say("  max |dGamma| = %.3e" % err)
    assert err <= TOL_GAMMA[w.dtype]


@pytest.mark.parametrize("what", ["rows", "gamma"])
def test_responsibilities_with_misaligned_buffers(gma, what):
    # rows that are not 16-byte aligned take the register-staged kernel (against the oracle; the diagnostics
    # against the aligned call); a Gamma buffer that is not 16-byte aligned takes element stores (bitwise the
    # aligned call's Gamma)
    w = gma.workload(3, batch=1, heads=2, seq_len=3000 + 7)
    say("responsibilities, misaligned %s" % what)
    inp = gma.make_inputs(w)
    t = {k: v.to(DEV) for k, v in inp.items()}
    args = (t["mu"], t["raw_var"], t["prior_logits"])
    x = t["qx"]
    ref = gma.responsibilities(x, *args)
    if what == "rows":
        buf = torch.empty(x.numel() + 8, dtype=x.dtype, device=DEV)
        xs = buf[1:1 + x.numel()].view_as(x)
        xs.copy_(x)
        got = gma.responsibilities(xs, *args)
        u0, c0, e0 = gma.responsibility_stats(x, *args)
        u1, c1, e1 = gma.responsibility_stats(xs, *args)
        torch.cuda.synchronize()
        err = np.abs(got.cpu().numpy().astype(np.float64) -
                     oracle.responsibilities(inp["qx"], inp["mu"], inp["raw_var"], inp["prior_logits"])).max()
        say("  max |dGamma| = %.3e" % err)
        assert err <= TOL_GAMMA[w.dtype]
        assert torch.allclose(u1, u0, rtol=1e-3, atol=1e-2)
        assert (c1.sum(-1) == w.seq_len).all() and (c1.long() - c0.long()).abs().sum() <= 0.01 * c0.numel() * w.seq_len / w.n_comp
        assert torch.allclose(e1, e0, atol=1e-4)
    else:
        gb = torch.empty(ref.numel() + 4, dtype=torch.float32, device=DEV)
        out = gb[1:1 + ref.numel()].view_as(ref)
        got = gma.responsibilities(x, *args, out=out)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)


@pytest.mark.parametrize("cfg,heads,N,shape", [(3, 4, 65536 + 333, None), (4, 2, 65536 + 77, None),
                                                (3, 2, 20000 + 5, (64, 7, 16)), (3, 2, 20000 + 5, (64, 100, 16))])
def test_responsibilities_long_walks(gma, cfg, heads, N, shape):
    # long sequences, so that each workgroup walks several consecutive chunks (a few heads spread the
    # sequence over all compute units) with a ragged last chunk, also with K not a multiple of 4 (single
    # stores) and with padding components; every row against the oracle
    w = gma.workload(cfg).with_(batch=1, heads=heads, seq_len=N)
    if shape:
        w = w.with_(d_route=shape[0], n_comp=shape[1], d_value=shape[2])
    say("responsibilities long %s" % (w,))
    inp = gma.make_inputs(w)
    t = {k: v.to(DEV) for k, v in inp.items()}
    got = gma.responsibilities(t["kx"], t["mu"], t["raw_var"], t["prior_logits"]).cpu().numpy().astype(np.float64)
    ref = oracle.responsibilities(inp["kx"], inp["mu"], inp["raw_var"], inp["prior_logits"])
    err = np.abs(got - ref).max()
    say("  max |dGamma| = %.3e" % err)
    assert err <= TOL_GAMMA[w.dtype]
    np.testing.assert_allclose(got.sum(-1), 1.0, atol=1e-5)


# ------------------------------------------------------------------------------------ forward parity


@pytest.mark.parametrize("cfg", [0, 1])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_full_size_fp32(gma, cfg, causal):
    w = gma.workload(cfg)
    say("forward cfg%d causal=%s %s" % (cfg, causal, w))
    inp = gma.make_inputs(w)
    err = rel_err(gpu_forward(gma, w, inp, causal), ref_forward(w, inp, causal))
    say("  rel err %.3e" % err)
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("causal", [False, True])
def test_forward_cfg2_full_size_every_slice(gma, causal):
    # B=32, H=8, N=4096: every (batch, head) slice against the oracle, and each slice's own error
    w = gma.workload(2)
    say("forward cfg2 causal=%s %s" % (causal, w))
    inp = gma.make_inputs(w)
    o = gpu_forward(gma, w, inp, causal).float().cpu().numpy().astype(np.float64)
    ref = ref_forward(w, inp, causal)
    err = rel_err(o, ref)
    per = np.abs(o - ref).max(axis=(2, 3)) / np.abs(ref).max(axis=(2, 3))   # [B, H]
    say("  rel err %.3e (worst slice %.3e)" % (err, per.max()))
    assert err <= TOL[w.dtype] and per.max() <= TOL[w.dtype]


@pytest.mark.parametrize("batch", [32, 22, 16, 13])
def test_bidirectional_segment_totals(gma, batch):
    # K = 32 workload shape at 8 heads and N = 600 (10 chunks of 64): 512 workgroups over B*H heads give
    # 2, 3, 4 and 5 segments per head.  Up to four, the read pass adds the segment records itself;
    # with five, the scan kernel forms the total first.  Both must give the oracle's result.
    w = gma.workload(2, batch=batch, seq_len=600)
    say("bidirectional segment totals %s" % (w,))
    inp = gma.make_inputs(w)
    err = rel_err(gpu_forward(gma, w, inp, False), ref_forward(w, inp, False))
    say("  rel err %.3e" % err)
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("cfg,N", [(3, 5000), (4, 3001)])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_bf16_reduced_length_all_heads(gma, cfg, N, causal):
    # all heads, many segments per head and a ragged last chunk
    w = gma.workload(cfg, seq_len=N)
    say("forward cfg%d N=%d causal=%s" % (cfg, N, causal))
    inp = gma.make_inputs(w)
    err = rel_err(gpu_forward(gma, w, inp, causal), ref_forward(w, inp, causal))
    say("  rel err %.3e" % err)
    assert err <= TOL[w.dtype]


def test_forward_cfg3_full_size_every_head(gma):
    # the benchmark workload as the bench runs it (16 heads, 65,536 tokens), every head against the oracle
    w = gma.workload(3)
    say("forward cfg3 full size %s" % (w,))
    inp = gma.make_inputs(w)
    o = gpu_forward(gma, w, inp).float().cpu().numpy().astype(np.float64)
    ref = ref_forward(w, inp)
    for h in range(w.heads):
        err = rel_err(o[:, h:h + 1], ref[:, h:h + 1])
        say("  head %d rel err %.3e" % (h, err))
        assert err <= TOL[w.dtype]


@pytest.mark.parametrize("rounds", [2, 3, 8])
@pytest.mark.parametrize("cfg,N", [(3, 65536 + 777), (4, 65536 + 333)])
def test_causal_rounds_match_the_oracle(gma, cfg, N, rounds, monkeypatch):
    # the causal pair launched in rounds over the sequence (GMA_CAUSAL_ROUNDS, a measurement switch): the
    # same result up to the summation order of the carried state, against the oracle, and bitwise
    # reproducible.  Two heads give 128 segments per head, so N >= 8 * 128 * 64 tokens allows 8 rounds; the
    # last round and the last segment are ragged
    w = gma.workload(cfg).with_(batch=1, heads=2, seq_len=N)
    say("forward rounds=%d %s" % (rounds, w))
    inp = gma.make_inputs(w)
    plain = gpu_forward(gma, w, inp)
    monkeypatch.setenv("GMA_CAUSAL_ROUNDS", str(rounds))
    o = gpu_forward(gma, w, inp)
    o2 = gpu_forward(gma, w, inp)
    assert torch.equal(o, o2)
    err = rel_err(o, ref_forward(w, inp))
    say("  rel err %.3e, max |rounds - plain| %.3e" % (err, (o.float() - plain.float()).abs().max().item()))
    assert err <= TOL[w.dtype]


def test_forward_cfg4_full_size_two_heads(gma):
    # 8 heads of 1,048,576 tokens on the GPU; the oracle checks a first and a last head
    w = gma.workload(4)
    say("forward cfg4 full size %s" % (w,))
    inp = gma.make_inputs(w)
    o = gpu_forward(gma, w, inp).float().cpu()
    del inp
    heads = [0, 5]
    sub = gma.make_inputs(w, heads=heads)
    ref = ref_forward(w, sub)
    for j, h in enumerate(heads):
        err = rel_err(o[:, h:h + 1], ref[:, j:j + 1])
        say("  head %d rel err %.3e" % (h, err))
        assert err <= TOL[w.dtype]


# ------------------------------------------------------------------------------------ edge cases


@pytest.mark.parametrize("base", [0, 3])
@pytest.mark.parametrize("N", [1, 2, 17, 63, 64, 65, 257, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_tails_and_tiny_lengths(gma, base, N, causal):
    w = gma.workload(base, batch=1, heads=3 if base else 1, seq_len=N)
    inp = gma.make_inputs(w)
    err = rel_err(gpu_forward(gma, w, inp, causal), ref_forward(w, inp, causal))
    assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("shape", [(96, 100, 120), (128, 96, 128), (40, 20, 48), (40, 30, 56), (64, 200, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_padded_shapes(gma, shape, causal):
    # d_r, K and d_v below the kernels' tile sizes: padding dimensions, padding value columns and
    # padding components (K = 96 leaves two whole tiles of them; K = 200 uses the K = 256 kernels)
    d_r, K, d_v = shape
    w = gma.workload(3, batch=1, heads=2, seq_len=1500, d_route=d_r, n_comp=K, d_value=d_v)
    say("padded shape d_r=%d K=%d d_v=%d causal=%s" % (d_r, K, d_v, causal))
    inp = gma.make_inputs(w)
    err = rel_err(gpu_forward(gma, w, inp, causal), ref_forward(w, inp, causal))
    assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("cfg,shape", [
    (3, (64, 64, 64)), (3, (32, 16, 16)), (3, (1, 1, 1)), (3, (8, 100, 24)), (3, (16, 256, 16)), (3, (128, 64, 32)),
    (3, (128, 256, 128)), (3, (100, 200, 60)), (3, (96, 180, 128)),
    (1, (32, 32, 32)), (1, (3, 40, 5)), (1, (128, 128, 128)), (1, (100, 70, 90)), (1, (65, 128, 16)),
])
@pytest.mark.parametrize("causal", [False, True])
def test_shapes_served_by_a_larger_class(gma, cfg, shape, causal):
    # (d_r, K, d_v) whose padded sizes match no compiled class exactly run on the cheapest class that
    # covers them (padding components have zero responsibility, padding dims zero coefficients)
    w = gma.workload(cfg, batch=1, heads=2, seq_len=300, d_route=shape[0], n_comp=shape[1], d_value=shape[2])
    say("larger class %s causal=%s %s" % (shape, causal, w))
    inp = gma.make_inputs(w)
    err = rel_err(gpu_forward(gma, w, inp, causal), ref_forward(w, inp, causal))
    say("  rel err %.3e" % err)
    assert err <= TOL[w.dtype]


# --------------------------------------------------------------- wide dims (the generic path)
# (d_r, K, d_v) with d_r or d_v in (128, 256] match no compiled class and run on the generic path:
# Gamma_Q, Gamma_K materialised in fp32, write and read phases as fp32 matrix-core products.


@pytest.mark.parametrize("cfg,shape,N", [
    (3, (256, 128, 256), 700), (3, (200, 64, 160), 1100), (3, (129, 256, 129), 300), (3, (256, 256, 8), 200),
    (3, (8, 16, 256), 400), (1, (256, 128, 256), 700), (1, (200, 64, 160), 1100), (1, (130, 7, 250), 129),
])
@pytest.mark.parametrize("causal", [False, True])
def test_wide_dims_generic_path(gma, cfg, shape, N, causal):
    w = gma.workload(cfg, batch=2, heads=2, seq_len=N, d_route=shape[0], n_comp=shape[1], d_value=shape[2])
    say("generic path %s causal=%s %s" % (shape, causal, w))
    inp = gma.make_inputs(w)
    err = rel_err(gpu_forward(gma, w, inp, causal), ref_forward(w, inp, causal))
    say("  rel err %.3e" % err)
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 1023, 1024, 1025])
@pytest.mark.parametrize("causal", [False, True])
def test_wide_dims_ragged_lengths(gma, N, causal):
    w = gma.workload(3, batch=1, heads=2, seq_len=N, d_route=200, n_comp=64, d_value=160)
    inp = gma.make_inputs(w)
    err = rel_err(gpu_forward(gma, w, inp, causal), ref_forward(w, inp, causal))
    assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("cfg", [1, 3])
def test_wide_dims_responsibilities_state_and_cross(gma, cfg):
    w = gma.workload(cfg, batch=1, heads=2, seq_len=1500, d_route=256, n_comp=128, d_value=256)
    say("generic path extras cfg %d" % cfg)
    inp = gma.make_inputs(w)
    t = {k: v.to(DEV) for k, v in inp.items()}
    # responsibilities
    g = gma.responsibilities(t["qx"], t["mu"], t["raw_var"], t["prior_logits"])
    torch.cuda.synchronize()
    ref = oracle.responsibilities(inp["qx"], inp["mu"], inp["raw_var"], inp["prior_logits"])
    gerr = float(np.abs(g.cpu().numpy().astype(np.float64) - ref).max())
    say("  max |dGamma| %.3e" % gerr)
    assert gerr <= TOL_GAMMA[w.dtype]
    # carried state: the oracle's state after 500 tokens, the GPU continues
    m = 500
    o_ref, s_ref = oracle.forward_causal_state(inp["qx"], inp["kx"], inp["v"], inp["mu"], inp["raw_var"],
                                               inp["prior_logits"], eps=w.eps)
    _, s_m = oracle.forward_causal_state(inp["qx"][:, :, :m], inp["kx"][:, :, :m], inp["v"][:, :, :m], inp["mu"],
                                         inp["raw_var"], inp["prior_logits"], eps=w.eps)
    tail = {k: t[k][:, :, m:].contiguous() for k in ("qx", "kx", "v")}
    s_io = torch.from_numpy(s_m).float().to(DEV)
    o = gma.forward_causal(tail["qx"], tail["kx"], tail["v"], t["mu"], t["raw_var"], t["prior_logits"], eps=w.eps,
                           state_in=s_io, state_out=s_io)
    torch.cuda.synchronize()
    err_o, err_s = _rel(o, o_ref[:, :, m:]), _rel(s_io, s_ref)
    say("  state: O err %.2e, state err %.2e" % (err_o, err_s))
    assert err_o <= TOL[w.dtype] and err_s <= TOL[w.dtype], (err_o, err_s)
    # cross-attention, both orders of the lengths
    for nq, nk in ((300, 1500), (1500, 300)):
        ref = oracle.forward_bidir_kv(inp["qx"][:, :, :nq], inp["kx"][:, :, :nk], inp["v"][:, :, :nk], inp["mu"],
                                      inp["raw_var"], inp["prior_logits"], eps=w.eps)
        o = gma.forward_bidir(t["qx"][:, :, :nq].contiguous(), t["kx"][:, :, :nk].contiguous(),
                              t["v"][:, :, :nk].contiguous(), t["mu"], t["raw_var"], t["prior_logits"], eps=w.eps)
        torch.cuda.synchronize()
        err = rel_err(o, ref)
        say("  cross N_q %d N_kv %d: rel err %.3e" % (nq, nk, err))
        assert err <= TOL[w.dtype], err


# ------------------------------------------------- bf16 rows past the fp16 operand range
# The bf16 path forms its logits on fp16 matrix-core operands: x^2 leaves the fp16 range at |x| >= 256,
# and a coefficient -1/(2 sigma^2) at sigma^2 < 1.1e-5.  Such a (batch, head) is flagged by the kernels
# and recomputed exactly (log-density in fp64); the other slices are untouched.


def _plant_out_of_range(inp, head=1):
    """A few routing rows of one head at |x| in [256, 4096] (values exact in bf16)."""
    q, k = inp["qx"].clone(), inp["kx"].clone()
    N = q.shape[2]
    q[0, head, min(5, N - 1), 3] = 300.0
    q[0, head, N // 2, :4] = -2048.0
    k[0, head, min(17, N - 1), 0] = 4096.0
    k[0, head, N - 1, 1:3] = 256.0
    out = dict(inp)
    out["qx"], out["kx"] = q, k
    return out


@pytest.mark.parametrize("cfg,K", [(3, None), (2, None), (4, None), (3, 256)])
@pytest.mark.parametrize("causal", [False, True])
def test_out_of_range_rows_forward(gma, cfg, K, causal):
    w = gma.workload(cfg, batch=1, heads=3, seq_len=1000)
    if K:
        w = w.with_(n_comp=K)
    say("out-of-range rows %s causal=%s" % (w, causal))
    clean = gma.make_inputs(w)
    inp = _plant_out_of_range(clean)
    o = gpu_forward(gma, w, inp, causal)
    assert torch.isfinite(o.float()).all()
    err = rel_err(o, ref_forward(w, inp, causal))
    say("  rel err %.3e" % err)
    assert err <= TOL[w.dtype], err
    # the slices without such rows take the usual path, bitwise
    o_clean = gpu_forward(gma, w, clean, causal)
    assert torch.equal(o[:, 0], o_clean[:, 0]) and torch.equal(o[:, 2], o_clean[:, 2])


def test_out_of_range_tiny_variance(gma):
    # a component with sigma^2 = softplus(-12) ~ 6e-6: its fp16 coefficient -1/(2 sigma^2) overflows
    w = gma.workload(3, batch=1, heads=2, seq_len=700)
    inp = gma.make_inputs(w)
    rv = inp["raw_var"].clone()
    rv[1, 3, :] = -12.0
    inp["raw_var"] = rv
    for causal in (False, True):
        err = rel_err(gpu_forward(gma, w, inp, causal), ref_forward(w, inp, causal))
        say("tiny variance causal=%s rel err %.3e" % (causal, err))
        assert err <= TOL[w.dtype], err
    t = {k: v.to(DEV) for k, v in inp.items()}
    g = gma.responsibilities(t["qx"], t["mu"], t["raw_var"], t["prior_logits"])
    torch.cuda.synchronize()
    ref = oracle.responsibilities(inp["qx"], inp["mu"], inp["raw_var"], inp["prior_logits"])
    assert float(np.abs(g.cpu().numpy().astype(np.float64) - ref).max()) <= TOL_GAMMA[w.dtype]


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_out_of_range_responsibilities_and_stats(gma, cfg):
    w = gma.workload(cfg, batch=1, heads=3, seq_len=900)
    inp = _plant_out_of_range(gma.make_inputs(w))
    t = {k: v.to(DEV) for k, v in inp.items()}
    g = gma.responsibilities(t["qx"], t["mu"], t["raw_var"], t["prior_logits"])
    u, hc, e = gma.responsibility_stats(t["qx"], t["mu"], t["raw_var"], t["prior_logits"])
    torch.cuda.synchronize()
    ref = oracle.responsibilities(inp["qx"], inp["mu"], inp["raw_var"], inp["prior_logits"])
    gerr = float(np.abs(g.cpu().numpy().astype(np.float64) - ref).max())
    say("out-of-range responsibilities cfg %d: max |dGamma| %.3e" % (cfg, gerr))
    assert gerr <= TOL_GAMMA[w.dtype]
    u_ref, h_ref, e_ref, gap = oracle.responsibility_stats(inp["qx"], inp["mu"], inp["raw_var"], inp["prior_logits"])
    u = u.cpu().numpy().astype(np.float64)
    assert np.abs(u - u_ref).max() <= 2 * TOL_GAMMA[w.dtype] * np.sqrt(w.seq_len)
    np.testing.assert_allclose(e.cpu().numpy(), e_ref, atol=2 * TOL_GAMMA[w.dtype])
    diff = np.abs(hc.cpu().numpy().astype(np.int64) - h_ref).sum(axis=-1)
    assert (diff <= 2 * (gap < 2 * TOL_GAMMA[w.dtype]).sum(axis=-1)).all()


def test_out_of_range_carried_state_and_cross_attention(gma):
    w = gma.workload(3, batch=1, heads=3, seq_len=1200)
    inp = _plant_out_of_range(gma.make_inputs(w))
    m = 400
    o_ref, s_ref = oracle.forward_causal_state(inp["qx"], inp["kx"], inp["v"], inp["mu"], inp["raw_var"],
                                               inp["prior_logits"], eps=w.eps)
    _, s_m = oracle.forward_causal_state(inp["qx"][:, :, :m], inp["kx"][:, :, :m], inp["v"][:, :, :m], inp["mu"],
                                         inp["raw_var"], inp["prior_logits"], eps=w.eps)
    t = {k: v.to(DEV) for k, v in inp.items()}
    tail = {k: t[k][:, :, m:].contiguous() for k in ("qx", "kx", "v")}
    s_io = torch.from_numpy(s_m).float().to(DEV)   # updated in place
    o = gma.forward_causal(tail["qx"], tail["kx"], tail["v"], t["mu"], t["raw_var"], t["prior_logits"], eps=w.eps,
                           state_in=s_io, state_out=s_io)
    torch.cuda.synchronize()
    err_o, err_s = _rel(o, o_ref[:, :, m:]), _rel(s_io, s_ref)
    say("out-of-range carried state: O err %.2e, state err %.2e" % (err_o, err_s))
    assert err_o <= TOL[w.dtype] and err_s <= TOL[w.dtype], (err_o, err_s)
    for nq, nk in ((300, 1200), (1200, 300)):
        ref = oracle.forward_bidir_kv(inp["qx"][:, :, -nq:], inp["kx"][:, :, :nk], inp["v"][:, :, :nk], inp["mu"],
                                      inp["raw_var"], inp["prior_logits"], eps=w.eps)
        o = gma.forward_bidir(t["qx"][:, :, -nq:].contiguous(), t["kx"][:, :, :nk].contiguous(),
                              t["v"][:, :, :nk].contiguous(), t["mu"], t["raw_var"], t["prior_logits"], eps=w.eps)
        torch.cuda.synchronize()
        err = rel_err(o, ref)
        say("out-of-range cross N_q %d N_kv %d: rel err %.3e" % (nq, nk, err))
        assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("cfg,N", [(3, 5000), (4, 3001), (2, 2000)])
def test_causal_without_room_for_stored_tiles(gma, cfg, N):
    # less than the advertised workspace: no stored Gamma_K tiles, the causal output pass recomputes
    # Gamma_K from K_X
    w = gma.workload(cfg, batch=1, heads=2, seq_len=N)
    say("causal, reduced workspace, cfg %d N=%d" % (cfg, N))
    inp = gma.make_inputs(w)
    prob = gma.problem(w.batch, w.heads, w.seq_len, w.d_route, w.n_comp, w.d_value, w.torch_dtype, w.eps)
    ws = torch.empty(gma.workspace_size(prob, 2) - 1, dtype=torch.uint8, device=DEV)
    err = rel_err(gpu_forward(gma, w, inp, True, workspace=ws), ref_forward(w, inp, True))
    assert err <= TOL[w.dtype], err


# ------------------------------------------------------------------------------ diagnostics


@pytest.mark.parametrize("cfg,B,H,N,d_r", [(3, 1, 3, 7000, None), (4, 1, 2, 5000, None), (2, 2, 2, 3000, None),
                                           (1, 2, 2, 2000, None), (0, 1, 1, 256, None), (3, 1, 2, 3000, 256),
                                           (1, 1, 2, 1000, 200)])
def test_responsibility_stats_match_the_oracle(gma, cfg, B, H, N, d_r):
    # usage within twice the Gamma tolerance times sqrt(N) (the row errors do not share one sign), and
    # summing to N over the components to fp32 rounding (a dropped or repeated row moves it by 1);
    # entropy within twice the Gamma tolerance; hard counts exactly, except that rows whose two largest
    # responsibilities (oracle) are closer than twice that tolerance may go either way
    w = gma.workload(cfg, batch=B, heads=H, seq_len=N)
    if d_r:
        w = w.with_(d_route=d_r)
    say("stats cfg %d B%d H%d N%d d_r %d" % (cfg, B, H, N, w.d_route))
    inp = gma.make_inputs(w)
    u_ref, h_ref, e_ref, gap = oracle.responsibility_stats(inp["qx"], inp["mu"], inp["raw_var"], inp["prior_logits"])
    t = {k: v.to(DEV) for k, v in inp.items()}
    u, hc, e = gma.responsibility_stats(t["qx"], t["mu"], t["raw_var"], t["prior_logits"])
    torch.cuda.synchronize()
    tol = TOL_GAMMA[w.dtype]
    u, hc, e = u.cpu().numpy().astype(np.float64), hc.cpu().numpy().astype(np.int64), e.cpu().numpy()
    assert np.abs(u - u_ref).max() <= 2 * tol * np.sqrt(N)
    np.testing.assert_allclose(u.sum(axis=-1), N, rtol=1e-5)
    assert (hc.sum(axis=-1) == N).all()
    np.testing.assert_allclose(e, e_ref, atol=2 * tol)
    ambiguous = (gap < 2 * tol).sum(axis=-1)                   # [B, H]
    diff = np.abs(hc - h_ref).sum(axis=-1)
    say("  usage err %.2e, hard-count moves %s (ambiguous rows %s)" % (np.abs(u - u_ref).max(), diff.ravel(), ambiguous.ravel()))
    assert (diff <= 2 * ambiguous).all(), (diff, ambiguous)


# ------------------------------------------------------------------------------ cross-attention


@pytest.mark.parametrize("cfg,Nq,Nk", [(3, 1, 5000), (3, 3000, 700), (3, 64, 1285), (2, 2000, 300), (4, 900, 2500),
                                       (1, 700, 2100), (0, 256, 37)])
def test_cross_attention_lengths(gma, cfg, Nq, Nk):
    # bidirectional form with N_q query rows and N_kv key/value rows
    wq = gma.workload(cfg, batch=1, heads=2, seq_len=Nq)
    wk = gma.workload(cfg, batch=1, heads=2, seq_len=Nk)
    say("cross cfg %d N_q=%d N_kv=%d" % (cfg, Nq, Nk))
    iq, ik = gma.make_inputs(wq), gma.make_inputs(wk)   # same parameters (per-head seeds), different rows
    ref = oracle.forward_bidir_kv(iq["qx"], ik["kx"], ik["v"], iq["mu"], iq["raw_var"], iq["prior_logits"], eps=wq.eps)
    o = gma.forward_bidir(iq["qx"].to(DEV), ik["kx"].to(DEV), ik["v"].to(DEV), iq["mu"].to(DEV),
                          iq["raw_var"].to(DEV), iq["prior_logits"].to(DEV), eps=wq.eps)
    torch.cuda.synchronize()
    err = rel_err(o, ref)
    assert err <= TOL[wq.dtype], err


# ------------------------------------------------------------------------------ carried state


def _state_tol(w):
    return TOL[w.dtype]


def _rel(a, b):
    a = a.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(a) else a
    return float(np.abs(a - b).max() / np.abs(b).max())


# reduced_ws: a workspace without room for the stored Gamma_K tiles, so the causal pass recomputes
# Gamma_K from K_X (the tiles exist for bf16 storage only, so the fp32 workload has one case)
@pytest.mark.parametrize("cfg,N,m,reduced_ws", [(3, 3000, 1100, False), (4, 2500, 700, False), (2, 2000, 64, False),
                                                (1, 1500, 333, False), (3, 3000, 1100, True), (4, 2500, 700, True),
                                                (2, 2000, 64, True)])
def test_causal_state_continues_a_sequence(gma, cfg, N, m, reduced_ws):
    # the oracle runs tokens [0, m) and hands its state over; the GPU runs [m, N) from it and must
    # give the oracle's one-pass outputs of those rows and its final state
    w = gma.workload(cfg, batch=1, heads=2, seq_len=N)
    say("carried state cfg %d N=%d m=%d reduced workspace %s" % (cfg, N, m, reduced_ws))
    inp = gma.make_inputs(w)
    o_ref, s_ref = oracle.forward_causal_state(inp["qx"], inp["kx"], inp["v"], inp["mu"], inp["raw_var"],
                                               inp["prior_logits"], eps=w.eps)
    _, s_m = oracle.forward_causal_state(inp["qx"][:, :, :m], inp["kx"][:, :, :m], inp["v"][:, :, :m], inp["mu"],
                                         inp["raw_var"], inp["prior_logits"], eps=w.eps)
    t = {k: v.to(DEV) for k, v in inp.items()}
    tail = {k: t[k][:, :, m:].contiguous() for k in ("qx", "kx", "v")}
    s_in = torch.from_numpy(s_m).float().to(DEV)
    s_out = torch.empty_like(s_in)
    kw = {}
    if reduced_ws:
        prob = gma.problem(1, 2, N - m, w.d_route, w.n_comp, w.d_value, w.torch_dtype, w.eps)
        kw["workspace"] = torch.empty(gma.workspace_size(prob, 3) - 1, dtype=torch.uint8, device=DEV)
    o = gma.forward_causal(tail["qx"], tail["kx"], tail["v"], t["mu"], t["raw_var"], t["prior_logits"], eps=w.eps,
                           state_in=s_in, state_out=s_out, **kw)
    torch.cuda.synchronize()
    err_o = _rel(o, o_ref[:, :, m:])
    err_s = _rel(s_out, s_ref)
    say("  O err %.2e, state err %.2e" % (err_o, err_s))
    assert err_o <= TOL[w.dtype], err_o
    assert err_s <= _state_tol(w), err_s


def test_causal_state_split_on_gpu_and_decode_steps(gma):
    w = gma.workload(3, batch=1, heads=2, seq_len=2024)
    inp = gma.make_inputs(w)
    t = {k: v.to(DEV) for k, v in inp.items()}
    q, k, v = t["qx"], t["kx"], t["v"]
    o_ref, s_ref = oracle.forward_causal_state(inp["qx"], inp["kx"], inp["v"], inp["mu"], inp["raw_var"],
                                               inp["prior_logits"], eps=w.eps)
    st = torch.zeros(1, 2, w.n_comp, w.d_value + 1, dtype=torch.float32, device=DEV)
    outs = []
    # a long first piece, then 24 one-token decode steps updating the state in place
    cuts = [0, 2000] + list(range(2001, 2025))
    for a_, b_ in zip(cuts[:-1], cuts[1:]):
        outs.append(gma.forward_causal(q[:, :, a_:b_].contiguous(), k[:, :, a_:b_].contiguous(),
                                       v[:, :, a_:b_].contiguous(), t["mu"], t["raw_var"], t["prior_logits"],
                                       eps=w.eps, state_in=st, state_out=st))
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=2)
    err_o, err_s = _rel(o, o_ref), _rel(st, s_ref)
    say("split + decode: O err %.2e, state err %.2e" % (err_o, err_s))
    assert err_o <= TOL[w.dtype], err_o
    assert err_s <= TOL[w.dtype], err_s


def test_causal_state_without_state_equals_plain_causal(gma):
    w = gma.workload(3, batch=1, heads=2, seq_len=3000)
    inp = gma.make_inputs(w)
    t = {k: v.to(DEV) for k, v in inp.items()}
    a = gma.forward_causal(t["qx"], t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"], eps=w.eps)
    s = torch.empty(1, 2, w.n_comp, w.d_value + 1, dtype=torch.float32, device=DEV)
    b = gma.forward_causal(t["qx"], t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"], eps=w.eps,
                           state_out=s)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("prepared", [False, True])
# the last three take the step kernel's further rounds of loads: more than one group of mixture parameters
# per wave (K above 16 G components) and more than one batch of state elements per thread (d_v > 64 with
# K > 128, d_v > 128 with K > 64), up to the largest shape
@pytest.mark.parametrize("cfg,shape", [(3, None), (1, None), (4, None), (2, (37, 29, 45)), (0, (5, 3, 7)),
                                       (2, (100, 150, 100)), (0, (200, 200, 200)), (3, (256, 256, 256))])
def test_decode_steps_match_the_oracle(gma, cfg, shape, prepared):
    # one-token steps from a zero state, updated in place, against the oracle's one pass over the
    # same tokens (outputs and final state); any d_r, K, d_v <= 256.  prepared: the mixture is
    # prepared once (gma_decode_prepare) and every step reads it
    T = 30
    kw = dict(batch=2, heads=2, seq_len=T)
    if shape:
        kw.update(d_route=shape[0], n_comp=shape[1], d_value=shape[2])
    w = gma.workload(cfg, **kw)
    say("decode cfg %d shape %s" % (cfg, shape))
    inp = gma.make_inputs(w)
    o_ref, s_ref = oracle.forward_causal_state(inp["qx"], inp["kx"], inp["v"], inp["mu"], inp["raw_var"],
                                               inp["prior_logits"], eps=w.eps)
    t = {k: v.to(DEV) for k, v in inp.items()}
    st = torch.zeros(2, 2, w.n_comp, w.d_value + 1, dtype=torch.float32, device=DEV)
    prep = gma.decode_prepare(t["raw_var"], t["prior_logits"]) if prepared else None
    outs = [gma.decode_step(t["qx"][:, :, i:i + 1], t["kx"][:, :, i:i + 1], t["v"][:, :, i:i + 1], t["mu"],
                            t["raw_var"], t["prior_logits"], st, eps=w.eps, prepared=prep) for i in range(T)]
    torch.cuda.synchronize()
    err_o, err_s = _rel(torch.cat(outs, dim=2), o_ref), _rel(st, s_ref)
    say("  O err %.2e, state err %.2e" % (err_o, err_s))
    assert err_o <= TOL[w.dtype], err_o
    assert err_s <= TOL[w.dtype], err_s


@pytest.mark.parametrize("shape", [None, (200, 200, 200)])
def test_decode_prepared_equals_raw_step_to_rounding(gma, shape):
    # the same 20 steps with the raw and with the prepared mixture: the log-densities differ only in
    # summation order, so outputs and states agree far inside the tolerance (fp32 storage)
    kw = dict(batch=2, heads=3, seq_len=20)
    if shape:
        kw.update(d_route=shape[0], n_comp=shape[1], d_value=shape[2])
    w = gma.workload(1, **kw)
    inp = gma.make_inputs(w)
    t = {k: v.to(DEV) for k, v in inp.items()}
    prep = gma.decode_prepare(t["raw_var"], t["prior_logits"])
    sa = torch.zeros(2, 3, w.n_comp, w.d_value + 1, dtype=torch.float32, device=DEV)
    sb = torch.zeros_like(sa)
    for i in range(20):
        args = (t["qx"][:, :, i:i + 1], t["kx"][:, :, i:i + 1], t["v"][:, :, i:i + 1], t["mu"], t["raw_var"],
                t["prior_logits"])
        oa = gma.decode_step(*args, sa, eps=w.eps)
        ob = gma.decode_step(*args, sb, eps=w.eps, prepared=prep)
        torch.cuda.synchronize()
        assert _rel(ob, oa.double().cpu().numpy()) <= 1e-5, i
    assert _rel(sb, sa.double().cpu().numpy()) <= 1e-5


def test_decode_after_a_bulk_prefix(gma):
    # the bulk causal pass over a prefix hands its state to decode steps; against one oracle pass
    w = gma.workload(3, batch=1, heads=4, seq_len=3016)
    inp = gma.make_inputs(w)
    o_ref, s_ref = oracle.forward_causal_state(inp["qx"], inp["kx"], inp["v"], inp["mu"], inp["raw_var"],
                                               inp["prior_logits"], eps=w.eps)
    t = {k: v.to(DEV) for k, v in inp.items()}
    n0 = 3000
    st = torch.empty(1, 4, w.n_comp, w.d_value + 1, dtype=torch.float32, device=DEV)
    outs = [gma.forward_causal(t["qx"][:, :, :n0].contiguous(), t["kx"][:, :, :n0].contiguous(),
                               t["v"][:, :, :n0].contiguous(), t["mu"], t["raw_var"], t["prior_logits"], eps=w.eps,
                               state_out=st)]
    for i in range(n0, 3016):
        outs.append(gma.decode_step(t["qx"][:, :, i:i + 1], t["kx"][:, :, i:i + 1], t["v"][:, :, i:i + 1], t["mu"],
                                    t["raw_var"], t["prior_logits"], st, eps=w.eps))
    torch.cuda.synchronize()
    err_o, err_s = _rel(torch.cat(outs, dim=2), o_ref), _rel(st, s_ref)
    assert err_o <= TOL[w.dtype], err_o
    assert err_s <= TOL[w.dtype], err_s


@pytest.mark.parametrize("causal", [False, True])
def test_bitwise_deterministic(gma, causal):
    w = gma.workload(3, seq_len=20000)
    inp = gma.make_inputs(w)
    a = gpu_forward(gma, w, inp, causal)
    b = gpu_forward(gma, w, inp, causal)
    assert torch.equal(a, b)


def test_causal_output_ignores_future_tokens_bitwise(gma):
    w = gma.workload(3, heads=2, seq_len=9000)
    inp = gma.make_inputs(w)
    o = gpu_forward(gma, w, inp)
    gen = torch.Generator().manual_seed(123)
    for i in (0, 100, 4099, 8000):
        pert = dict(inp)
        for k in ("qx", "kx", "v"):
            x = inp[k].clone()
            x[:, :, i + 1:] = (3.0 * torch.randn(x[:, :, i + 1:].shape, generator=gen)).to(x.dtype)
            pert[k] = x
        o2 = gpu_forward(gma, w, pert)
        assert torch.equal(o2[:, :, : i + 1], o[:, :, : i + 1]), i
        assert not torch.equal(o2[:, :, i + 1:], o[:, :, i + 1:])


def test_causal_last_row_equals_bidirectional(gma):
    w = gma.workload(1, heads=2, batch=1)
    inp = gma.make_inputs(w)
    oc = gpu_forward(gma, w, inp, True).double().cpu()
    ob = gpu_forward(gma, w, inp, False).double().cpu()
    err = (oc[:, :, -1] - ob[:, :, -1]).abs().max() / ob.abs().max()
    assert err <= 1e-5


@pytest.mark.parametrize("causal", [False, True])
def test_poisoned_workspace_and_guard_bands(gma, causal):
    # a NaN-filled workspace must be fully overwritten before it is read; writes stay inside O
    w = gma.workload(3, seq_len=6000, heads=4)
    inp = gma.make_inputs(w)
    t = {k: v.to(DEV) for k, v in inp.items()}
    prob = gma.problem(w.batch, w.heads, w.seq_len, w.d_route, w.n_comp, w.d_value, torch.bfloat16, w.eps)
    nws = gma.workspace_size(prob, 2 if causal else 1)
    ws = torch.full((nws // 4 + 1,), float("nan"), dtype=torch.float32, device=DEV)
    numel = w.batch * w.heads * w.seq_len * w.d_value
    guard = 4096
    buf = torch.full((numel + 2 * guard,), 4096.0, dtype=torch.bfloat16, device=DEV)
    out = buf[guard:guard + numel].view(w.batch, w.heads, w.seq_len, w.d_value)
    gma.forward(t["qx"], t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"], eps=w.eps, causal=causal,
                out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert (buf[:guard] == 4096.0).all() and (buf[guard + numel:] == 4096.0).all()
    err = rel_err(out, ref_forward(w, inp, causal))
    assert err <= TOL[w.dtype]
