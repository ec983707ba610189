"""C-ABI contract of libgma.so, checked on the CPU (no kernel is launched).

Validation is pure host code that returns before any HIP call, so every error path is
exercised here without a GPU.
"""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gma.h")


@pytest.fixture(scope="module")
def lib():
    from gaussian_mixture_token_amd import _lib
    if not os.path.exists(_lib.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gma_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gma_responsibilities", "gma_forward_bidir", "gma_forward_causal", "gma_workspace_size",
              "gma_backward_bidir", "gma_backward_causal", "gma_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names
    for n in names:
        assert hasattr(lib, n), n


def _prob(**kw):
    from gaussian_mixture_token_amd import _lib
    d = dict(batch=1, heads=16, seq_len=65536, d_route=128, n_comp=128, d_value=128, dtype=1, eps=1e-6)
    d.update(kw)
    return _lib.Problem(**d)


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first


def _fwd(lib, fn, prob, ws_bytes=1 << 40, **override):
    args = dict(qx=FAKE, kx=ctypes.c_void_p(0x20000000), v=ctypes.c_void_p(0x40000000), mu=FAKE, rv=FAKE, pl=FAKE,
                o=ctypes.c_void_p(0x80000000000), ws=ctypes.c_void_p(0x100000000000))
    args.update(override)
    return getattr(lib, fn)(ctypes.byref(prob), args["qx"], args["kx"], args["v"], args["mu"], args["rv"], args["pl"],
                            args["o"], args["ws"], ws_bytes, None)


@pytest.mark.parametrize("fn", ["gma_forward_bidir", "gma_forward_causal"])
@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, 1), ("heads", -1, 1), ("seq_len", 0, 1), ("d_route", 0, 1), ("n_comp", 0, 1),
    ("d_value", 0, 1), ("dtype", 7, 1), ("eps", -1.0, 1), ("eps", float("nan"), 1), ("eps", float("inf"), 1),
    ("n_comp", 257, 2), ("d_route", 300, 2), ("d_value", 257, 2),
])
def test_invalid_problem_rejected(lib, fn, field, value, status):
    assert _fwd(lib, fn, _prob(**{field: value})) == status
    assert lib.gma_last_error()


@pytest.mark.parametrize("fn", ["gma_forward_bidir", "gma_forward_causal"])
def test_null_pointers_rejected(lib, fn):
    for name in ("qx", "kx", "v", "mu", "rv", "pl", "o"):
        assert _fwd(lib, fn, _prob(), **{name: None}) == 1, name


@pytest.mark.parametrize("fn", ["gma_forward_bidir", "gma_forward_causal"])
def test_workspace_too_small_and_null(lib, fn):
    prob = _prob()
    need = lib.gma_workspace_size(ctypes.byref(prob), 2 if fn.endswith("causal") else 1)
    assert need > 0
    # gma_workspace_size() is what the fastest applicable path needs; a somewhat smaller workspace
    # may still fit the path that runs (which then launches kernels: covered on the GPU).  One
    # smaller than every path's need is rejected before any HIP call.
    assert _fwd(lib, fn, prob, ws_bytes=4096) == 3
    assert _fwd(lib, fn, prob, ws_bytes=need, ws=None) == 1


def test_misaligned_and_aliasing_rejected(lib):
    prob = _prob()
    assert _fwd(lib, "gma_forward_causal", prob, qx=ctypes.c_void_p(0x10001)) == 1        # odd address for bf16
    assert _fwd(lib, "gma_forward_causal", prob, ws=ctypes.c_void_p(0x100000000008)) == 1  # workspace not 16-B aligned
    assert _fwd(lib, "gma_forward_causal", prob, o=ctypes.c_void_p(0x40000000)) == 1       # o aliases v


def test_null_problem_and_bad_op(lib):
    assert lib.gma_workspace_size(None, 2) == 0
    assert lib.gma_workspace_size(ctypes.byref(_prob()), 9) == 0
    assert lib.gma_forward_causal(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 1


def test_responsibilities_validation(lib):
    prob = _prob(d_value=1)
    f = lib.gma_responsibilities
    assert f(ctypes.byref(prob), None, FAKE, FAKE, FAKE, ctypes.c_void_p(0x80000000000), FAKE, 1 << 40, None) == 1
    assert f(ctypes.byref(_prob(n_comp=0)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == 1
    need = lib.gma_workspace_size(ctypes.byref(prob), 0)
    assert need > 0
    assert f(ctypes.byref(prob), FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x80000000000),
             ctypes.c_void_p(0x100000000000), need - 1, None) == 3


def test_status_strings(lib):
    for s in range(5):
        assert lib.gma_status_string(s)
    assert lib.gma_kernel_count() >= 5
    assert lib.gma_kernel_name(0) and lib.gma_kernel_name(999) == b""


def _ws(lib, op, **kw):
    return lib.gma_workspace_size(ctypes.byref(_prob(**kw)), op)


def test_workspace_is_linear_memory_not_quadratic(lib):
    # The N x N affinity is never formed (page "Attention par Mélange Gaussien (GMA)",
    # "Mécanisme Central" item 2).  Bidirectional: the workspace depends on the segment count and
    # K x d_v only.  Causal with K <= d_r: in addition, one bf16 Gamma_K row per token and head
    # (the stored responsibility tiles), i.e. linear in N.
    ns = (1 << 14, 1 << 17, 1 << 20)
    bidir = [_ws(lib, 1, seq_len=n) for n in ns]
    assert bidir[0] > 0
    assert bidir[2] == bidir[1] == bidir[0]  # segment count saturates; no N-dependence at all beyond it
    per_head_state = (128 * 128 + 128) * 4
    assert bidir[2] < 64 * 16 * per_head_state + (1 << 22)
    causal = [_ws(lib, 2, seq_len=n) for n in ns]
    row = 128 * 2   # one bf16 Gamma_K row
    for n, c in zip(ns, causal):
        assert 16 * n * row <= c <= bidir[0] + 16 * n * row + 4096
    assert causal[2] - causal[1] == 16 * (ns[2] - ns[1]) * row


def test_small_causal_problem_needs_no_segment_records(lib):
    # one segment per head: no carried state.  On the fp32 path (no stored Gamma_K tiles) the
    # workspace holds only the prepared parameters.
    kw = dict(seq_len=64, heads=1024, d_route=64, n_comp=64, d_value=64, dtype=0)
    small = _ws(lib, 2, **kw)
    big = _ws(lib, 1, **kw)
    assert 0 < small < big


def test_causal_tiles_cover_the_padded_sequence(lib):
    # K <= d_r: one tile of 64 rows x K bf16 per chunk of 64 tokens (the last chunk padded)
    n = 64 * 1000 + 5
    c = _ws(lib, 2, seq_len=n)
    b = _ws(lib, 1, seq_len=n)
    tiles = 16 * 1001 * 64 * 128 * 2
    assert tiles <= c <= b + tiles + 4096


def _fwd_state(lib, prob, state_in, state_out, ws_bytes=1 << 40, **override):
    args = dict(qx=FAKE, kx=ctypes.c_void_p(0x20000000), v=ctypes.c_void_p(0x40000000), mu=FAKE, rv=FAKE, pl=FAKE,
                o=ctypes.c_void_p(0x80000000000), ws=ctypes.c_void_p(0x100000000000))
    args.update(override)
    return lib.gma_forward_causal_state(ctypes.byref(prob), args["qx"], args["kx"], args["v"], args["mu"], args["rv"],
                                        args["pl"], state_in, state_out, args["o"], args["ws"], ws_bytes, None)


def test_causal_state_validation(lib):
    prob = _prob()
    ns = 16 * 128 * 129 * 4
    s1, s2 = 0x200000000000, 0x300000000000
    # misaligned state pointers
    assert _fwd_state(lib, prob, ctypes.c_void_p(s1 + 2), None) == 1
    assert _fwd_state(lib, prob, None, ctypes.c_void_p(s2 + 1)) == 1
    # partial overlap of state_in and state_out (identical buffers are allowed: in-place update)
    assert _fwd_state(lib, prob, ctypes.c_void_p(s1), ctypes.c_void_p(s1 + ns // 2)) == 1
    # a state overlapping o or the workspace
    assert _fwd_state(lib, prob, ctypes.c_void_p(0x80000000000 + 64), None) == 1
    assert _fwd_state(lib, prob, None, ctypes.c_void_p(0x100000000000 + 256)) == 1
    # workspace too small for every path
    assert _fwd_state(lib, prob, ctypes.c_void_p(s1), ctypes.c_void_p(s1), ws_bytes=4096) == 3
    # the stateful op needs at least the causal workspace
    assert lib.gma_workspace_size(ctypes.byref(prob), 3) >= lib.gma_workspace_size(ctypes.byref(prob), 2)


def test_cross_validation(lib):
    prob = _prob()
    f = lib.gma_forward_bidir_kv
    args = [FAKE, ctypes.c_void_p(0x20000000), ctypes.c_void_p(0x40000000), FAKE, FAKE, FAKE,
            ctypes.c_void_p(0x80000000000), ctypes.c_void_p(0x100000000000)]
    assert f(None, 100, *args, 1 << 40, None) == 1
    assert f(ctypes.byref(prob), 0, *args, 1 << 40, None) == 1                   # seq_len_kv < 1
    assert f(ctypes.byref(_prob(n_comp=0)), 100, *args, 1 << 40, None) == 1
    assert f(ctypes.byref(prob), 100, *args, 4096, None) == 3                    # workspace too small
    bad = list(args)
    bad[6] = ctypes.c_void_p(0x40000000 + 64)                                    # o overlaps v
    assert f(ctypes.byref(prob), 1 << 20, *bad, 1 << 40, None) == 1


def test_decode_step_validation(lib):
    f = lib.gma_decode_step
    ptrs = [FAKE, ctypes.c_void_p(0x20000000), ctypes.c_void_p(0x40000000), FAKE, FAKE, FAKE]
    s, o = ctypes.c_void_p(0x200000000000), ctypes.c_void_p(0x80000000000)
    one = _prob(seq_len=1)
    assert f(None, *ptrs, s, s, o, None) == 1
    assert f(ctypes.byref(_prob(seq_len=2)), *ptrs, s, s, o, None) == 1            # one token per (b, h)
    assert f(ctypes.byref(_prob(seq_len=1, n_comp=257)), *ptrs, s, s, o, None) == 2
    assert f(ctypes.byref(one), *ptrs, s, s, None, None) == 1                      # o NULL
    assert f(ctypes.byref(one), *ptrs, ctypes.c_void_p(0x200000000002), s, o, None) == 1   # misaligned state
    assert f(ctypes.byref(one), *ptrs, s, ctypes.c_void_p(0x200000000000 + 4096), o, None) == 1   # partial overlap
    assert f(ctypes.byref(one), *ptrs, ctypes.c_void_p(0x80000000000 + 64), None, o, None) == 1   # state over o


def test_decode_prepared_size_and_validation(lib):
    one = _prob(seq_len=1)
    # 1 / sigma^2 [H, K, d_r] fp32, then c [H, K] fp64 at a 256-byte boundary
    lay = 16 * 128 * 128 * 4
    assert lib.gma_decode_params_size(ctypes.byref(one)) == lay + 16 * 128 * 8
    assert lib.gma_decode_params_size(ctypes.byref(_prob(heads=3, n_comp=5, d_route=7))) == 512 + 256
    assert lib.gma_decode_params_size(None) == 0
    assert lib.gma_decode_params_size(ctypes.byref(_prob(n_comp=257))) == 0
    need = lib.gma_decode_params_size(ctypes.byref(one))
    prep = ctypes.c_void_p(0x300000000000)
    f = lib.gma_decode_prepare
    assert f(None, FAKE, FAKE, prep, need, None) == 1
    assert f(ctypes.byref(one), None, FAKE, prep, need, None) == 1
    assert f(ctypes.byref(one), FAKE, FAKE, None, need, None) == 1
    assert f(ctypes.byref(one), FAKE, FAKE, ctypes.c_void_p(0x300000000000 + 16), need, None) == 1   # not 256-aligned
    assert f(ctypes.byref(one), FAKE, FAKE, prep, need - 1, None) == 3                                # too small
    assert f(ctypes.byref(_prob(seq_len=1, n_comp=257)), FAKE, FAKE, prep, need, None) == 2
    assert f(ctypes.byref(one), ctypes.c_void_p(0x300000000000 + 4096), FAKE, prep, need, None) == 1  # overlap
    g = lib.gma_decode_step_prepared
    ptrs = [FAKE, ctypes.c_void_p(0x20000000), ctypes.c_void_p(0x40000000), FAKE]
    s, o = ctypes.c_void_p(0x200000000000), ctypes.c_void_p(0x80000000000)
    assert g(None, *ptrs, prep, need, s, s, o, None) == 1
    assert g(ctypes.byref(_prob(seq_len=2)), *ptrs, prep, need, s, s, o, None) == 1
    assert g(ctypes.byref(one), *ptrs, None, need, s, s, o, None) == 1                # prepared NULL
    assert g(ctypes.byref(one), *ptrs, prep, need - 8, s, s, o, None) == 3            # prepared too small
    assert g(ctypes.byref(one), *ptrs, ctypes.c_void_p(0x300000000000 + 8), need, s, s, o, None) == 1
    assert g(ctypes.byref(one), *ptrs, prep, need, ctypes.c_void_p(0x300000000000 + 64), None, o, None) == 1  # state over prepared
    assert g(ctypes.byref(one), *ptrs, prep, need, s, s, ctypes.c_void_p(0x300000000000), None) == 1  # o over prepared


def test_responsibility_stats_validation(lib):
    f = lib.gma_responsibility_stats
    prob = _prob(d_value=1)
    x, u, hc, e = FAKE, ctypes.c_void_p(0x80000000000), ctypes.c_void_p(0x90000000000), ctypes.c_void_p(0xa0000000000)
    ws = ctypes.c_void_p(0x100000000000)
    need = lib.gma_workspace_size(ctypes.byref(prob), 4)
    assert 0 < need < 16 * 65536 * 128 * 4                    # Gamma is reduced as it is formed, never stored
    assert f(ctypes.byref(prob), None, FAKE, FAKE, FAKE, u, hc, e, ws, need, None) == 1
    assert f(ctypes.byref(prob), x, FAKE, FAKE, FAKE, u, hc, e, ws, need - 1, None) == 3
    assert f(ctypes.byref(prob), x, FAKE, FAKE, FAKE, u, u, e, ws, need, None) == 1       # outputs overlap
    assert f(ctypes.byref(_prob(n_comp=300)), x, FAKE, FAKE, FAKE, u, hc, e, ws, need, None) == 2


def _bwd(lib, fn, prob, ws_bytes=1 << 44, **override):
    big = 1 << 36   # spacing that keeps the fake tensors of the 65536-token problem disjoint
    args = dict(qx=1, kx=2, v=3, mu=4, rv=5, pl=6, do=7, dqx=8, dkx=9, dv=10, dmu=11, drv=12, dpl=13, ws=14)
    vals = {k: ctypes.c_void_p(i * big) for k, i in args.items()}
    for k, v in override.items():
        vals[k] = v
    order = ("qx", "kx", "v", "mu", "rv", "pl", "do", "dqx", "dkx", "dv", "dmu", "drv", "dpl", "ws")
    a = [vals[k] for k in order]
    return getattr(lib, fn)(ctypes.byref(prob), *a[:13], a[13], ws_bytes, None)


@pytest.mark.parametrize("fn", ["gma_backward_bidir", "gma_backward_causal"])
def test_backward_validation(lib, fn):
    op = 6 if fn.endswith("causal") else 5
    prob = _prob(seq_len=4096)
    need = lib.gma_workspace_size(ctypes.byref(prob), op)
    assert need > 0
    for field, value, status in (("batch", 0, 1), ("eps", -1.0, 1), ("n_comp", 257, 2), ("dtype", 5, 1)):
        assert _bwd(lib, fn, _prob(seq_len=4096, **{field: value})) == status
        assert lib.gma_last_error()
    for name in ("qx", "kx", "v", "mu", "rv", "pl", "do", "dqx", "dkx", "dv", "dmu", "drv", "dpl"):
        assert _bwd(lib, fn, prob, **{name: None}) == 1, name
    assert _bwd(lib, fn, prob, ws_bytes=need - 1) == 3
    assert _bwd(lib, fn, prob, ws_bytes=need, ws=None) == 1
    assert _bwd(lib, fn, prob, ws=ctypes.c_void_p((14 << 36) + 8)) == 1       # workspace not 16-byte aligned
    assert _bwd(lib, fn, prob, dqx=ctypes.c_void_p((8 << 36) + 1)) == 1       # odd address for bf16
    assert _bwd(lib, fn, prob, dmu=ctypes.c_void_p((11 << 36) + 2)) == 1      # fp32 parameter gradient misaligned
    assert _bwd(lib, fn, prob, dv=ctypes.c_void_p(3 << 36)) == 1              # dv aliases v
    assert _bwd(lib, fn, prob, dkx=ctypes.c_void_p(8 << 36)) == 1             # dkx aliases dqx
    assert _bwd(lib, fn, prob, dpl=ctypes.c_void_p(14 << 36)) == 1            # gradient inside the workspace


def test_backward_workspace_is_linear_in_the_sequence(lib):
    # fp32 intermediates per token and per chunk state; nothing quadratic in N
    for op in (5, 6):
        a = _ws(lib, op, seq_len=1 << 14)
        b = _ws(lib, op, seq_len=1 << 16)
        assert a > 0 and 3.9 * a < b < 4.1 * a, (op, a, b)
    assert _ws(lib, 5, seq_len=4096) < _ws(lib, 6, seq_len=4096)   # the causal chunk blocks


def test_binding_rejects_outputs_that_do_not_fit():
    # the checks that guard raw-pointer writes; a host tensor is never a valid output or workspace
    from gaussian_mixture_token_amd import api
    dev = torch.device("cuda", 0)
    with pytest.raises(ValueError):
        api._check_out(torch.zeros(2, 3), (2, 3), torch.float32, dev)
    with pytest.raises(ValueError):
        api._on(torch.zeros(4, dtype=torch.uint8), dev, "workspace")


def test_stats_workspace_is_independent_of_the_sequence_length(lib):
    # the diagnostics reduce Gamma inside the responsibilities kernel: only per-segment partials are kept
    sizes = []
    for N in (10_000, 100_000, 1_000_000):
        p = _prob(seq_len=N, d_value=1)
        sizes.append(lib.gma_workspace_size(ctypes.byref(p), 4))
    assert sizes[0] > 0 and sizes[0] == sizes[1] == sizes[2], sizes
    assert sizes[0] < 8 << 20
