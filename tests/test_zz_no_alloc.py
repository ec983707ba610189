"""gma_forward_causal_noalloc (the causal forward with the library's fixed scratch array as its
workspace, for callers that cannot allocate) against gma_forward_causal, through the C ABI.

Two calls in a row, the second on a smaller input: each must equal gma_forward_causal given a
workspace of the array's size bitwise (the same plan and kernels), and the oracle to the parity
tolerance.  A problem whose workspace exceeds the array is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import gpu_available

DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 1e-2}


@pytest.fixture(scope="module")
def gma():
    if not gpu_available():
        pytest.skip("no GPU")
    import gaussian_mixture_token_amd as g
    from gaussian_mixture_token_amd import _lib
    _lib.load()
    oracle.build(force=False)
    return g


def _run_pair(g, cfg, B, H, N, heads=None):
    # heads: the (batch 0) heads the oracle checks (all when None); the comparison with the allocating
    # entry point covers every element
    from gaussian_mixture_token_amd import _lib
    w = g.workload(cfg, batch=B, heads=H, seq_len=N)
    print("no-alloc causal cfg %d B%d H%d N%d" % (cfg, B, H, N), flush=True)
    inp = g.make_inputs(w)
    t = {k: v.to(DEV) for k, v in inp.items()}
    args = (t["qx"], t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"])
    o_na = torch.full((B, H, N, w.d_value), float("nan"), dtype=w.torch_dtype, device=DEV)
    g.forward_causal_noalloc(*args, eps=w.eps, out=o_na)
    ws = torch.empty(_lib.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device=DEV)
    o_ws = g.forward_causal(*args, eps=w.eps, workspace=ws)
    o_full = g.forward_causal(*args, eps=w.eps)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ws)
    hs = slice(None) if heads is None else slice(0, heads)
    bs = slice(None) if heads is None else slice(0, 1)
    sub = {k: inp[k][bs, hs] for k in ("qx", "kx", "v")}
    sub.update({k: inp[k][hs] for k in ("mu", "raw_var", "prior_logits")})
    ref = oracle.forward(sub["qx"], sub["kx"], sub["v"], sub["mu"], sub["raw_var"], sub["prior_logits"], eps=w.eps,
                         causal=True)
    for o in (o_na, o_full):
        got = o[bs, hs].float().cpu().numpy().astype(np.float64)
        err = float(np.abs(got - ref).max() / np.abs(ref).max())
        print("  rel err %.3e" % err, flush=True)
        assert err <= TOL[w.dtype], err


@pytest.mark.gpu
@pytest.mark.parametrize("cfg,first,second", [(3, (1, 16, 65536, 2), (1, 4, 6000, None)),
                                              (4, (1, 2, 5000, None), (1, 1, 700, None)),
                                              (1, (2, 4, 3000, None), (1, 2, 300, None))])
def test_noalloc_matches_the_allocating_entry_point(gma, cfg, first, second):
    # the full 16-head, 65,536-token bf16 workload does not leave room for its stored Gamma_K tiles
    # (268 MB) in the scratch array, so its first call takes the recompute path; the smaller calls
    # store the tiles
    _run_pair(gma, cfg, *first)
    _run_pair(gma, cfg, *second)


@pytest.mark.gpu
def test_noalloc_refuses_problems_beyond_its_scratch(gma):
    from gaussian_mixture_token_amd import _lib
    # 2048 heads of 128 components over 128 dims: their logit coefficient fragments alone take 128 MiB
    w = gma.workload(3, batch=1, heads=2048, seq_len=64)
    prob = gma.problem(w.batch, w.heads, w.seq_len, w.d_route, w.n_comp, w.d_value, w.torch_dtype, w.eps)
    x = torch.zeros(8, dtype=torch.bfloat16, device=DEV)
    p = ctypes.c_void_p(x.data_ptr())
    st = _lib.load().gma_forward_causal_noalloc(ctypes.byref(prob), p, p, p, p, p, p, p, None)
    assert st == 3   # GMA_ERROR_WORKSPACE_TOO_SMALL, refused on the host
    assert b"no-allocation" in _lib.load().gma_last_error()
