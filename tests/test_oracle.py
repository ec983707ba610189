"""Pins for the fp64 oracle, checked against things other than itself.

Every definition comes from the page "Attention par Mélange Gaussien (GMA)",
section "Méthodologie", sub-section "Mécanisme Central":
  item 1  responsibilities are GMM posteriors (non-negative, rows sum to 1);
  item 2  write Vt = Gamma_K^T V, Z = Gamma_K^T 1, read O = Gamma_Q Vt / (Gamma_Q Z + eps),
          identical (by associativity) to the materialised affinity A = Gamma_Q Gamma_K^T;
  item 3  causal prefix sums (O_i depends on j <= i only); softplus variances and
          softmax priors.
Section "Contributions Clés", item 3 ("Interprétation de l'Affinité"): A is
non-negative with rank <= K.

Independent references used here: SciPy's multivariate normal log-density and
softmax, scikit-learn's GaussianMixture posterior, a hand-derived closed-form
fixture (tests/golden/two_component_1d.txt), closed forms for K = 1 and for
identical components, brute-force materialised affinities, and structural
invariants (linearity, convexity bound, permutation symmetry, causal masking).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.special import log_softmax, softmax
from scipy.stats import multivariate_normal

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "two_component_1d.txt")


def rand_params(rng, H, K, dr):
    mu = rng.normal(0.0, 1.0, (H, K, dr))
    rv = rng.uniform(-1.0, 1.0, (H, K, dr))
    pl = rng.normal(0.0, 0.5, (H, K))
    return mu, rv, pl


def scipy_gamma(x, mu, rv, pl):
    """Posterior from SciPy: log N(x; mu_k, diag(var_k)) + log pi_k, then softmax over k.
    x [N, dr]; mu, rv [K, dr]; pl [K].  var = log(1 + e^rho) via numpy's logaddexp."""
    var = np.logaddexp(0.0, rv)
    logpi = log_softmax(pl)
    L = np.stack([multivariate_normal(mean=mu[k], cov=np.diag(var[k])).logpdf(x).reshape(-1)
                  for k in range(mu.shape[0])], axis=-1) + logpi
    return softmax(L, axis=-1)


def brute_force(gq, gk, v, eps, causal):
    """Materialised affinity A = Gamma_Q Gamma_K^T (lower-triangular incl. diagonal when causal)."""
    A = gq @ gk.T
    if causal:
        A = np.tril(A)
    return (A @ v) / (A.sum(axis=1, keepdims=True) + eps)


# ----------------------------------------------------------------------------- parameters


def test_softplus_closed_forms(oracle_mod):
    rv = np.array([[[0.0, 1.5, -1.5, 40.0, -40.0, 1e-8]]])
    var, _ = oracle_mod.params(rv, np.zeros((1, 1)))
    v = var[0, 0]
    assert v[0] == pytest.approx(math.log(2.0), rel=1e-15)
    assert v[1] - v[2] == pytest.approx(1.5, rel=1e-14)          # softplus(x) - softplus(-x) = x
    assert v[3] == pytest.approx(40.0, rel=1e-15)
    assert v[4] == pytest.approx(math.exp(-40.0), rel=1e-12)     # small tail kept, not flushed
    assert v[5] == pytest.approx(math.log(2.0) + 0.5e-8, rel=1e-15)


def test_prior_softmax(oracle_mod):
    rng = np.random.default_rng(0)
    pl = rng.normal(0, 3.0, (3, 7))
    _, logp = oracle_mod.params(np.zeros((3, 7, 2)), pl)
    np.testing.assert_allclose(np.exp(logp).sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(logp - logp[:, :1], pl - pl[:, :1], atol=1e-13)
    _, logp_eq = oracle_mod.params(np.zeros((1, 5, 1)), np.full((1, 5), 3.7))
    np.testing.assert_allclose(logp_eq, -math.log(5.0), rtol=1e-15)


# ----------------------------------------------------------------------------- responsibilities


def test_gamma_nonnegative_rows_sum_to_one(oracle_mod):
    rng = np.random.default_rng(1)
    mu, rv, pl = rand_params(rng, 2, 9, 6)
    x = rng.normal(0, 2.0, (2, 2, 50, 6))
    g = oracle_mod.responsibilities(x, mu, rv, pl)
    assert g.shape == (2, 2, 50, 9)
    assert (g >= 0).all()
    np.testing.assert_allclose(g.sum(-1), 1.0, rtol=1e-14)


def test_gamma_matches_scipy(oracle_mod):
    rng = np.random.default_rng(2)
    H, K, dr = 3, 6, 5
    mu, rv, pl = rand_params(rng, H, K, dr)
    x = rng.normal(0, 1.0, (1, H, 40, dr))
    g = oracle_mod.responsibilities(x, mu, rv, pl)
    for h in range(H):
        ref = scipy_gamma(x[0, h], mu[h], rv[h], pl[h])
        np.testing.assert_allclose(g[0, h], ref, rtol=1e-10, atol=1e-14)


def test_gamma_matches_sklearn(oracle_mod):
    from sklearn.mixture import GaussianMixture
    rng = np.random.default_rng(3)
    K, dr = 4, 3
    mu, rv, pl = rand_params(rng, 1, K, dr)
    var = np.logaddexp(0.0, rv[0])
    gm = GaussianMixture(n_components=K, covariance_type="diag")
    gm.means_ = mu[0]
    gm.covariances_ = var
    gm.precisions_cholesky_ = 1.0 / np.sqrt(var)
    gm.weights_ = softmax(pl[0])
    gm.converged_, gm.n_iter_, gm.lower_bound_ = True, 0, 0.0
    x = rng.normal(0, 1.5, (64, dr))
    g = oracle_mod.responsibilities(x, mu, rv, pl)
    np.testing.assert_allclose(g, gm.predict_proba(x), rtol=1e-9, atol=1e-13)


def test_gamma_two_component_sigmoid(oracle_mod):
    # d_r = 1, K = 2, equal variance s and equal priors:
    # gamma_1(x) = sigmoid((mu_1 - mu_2)(x - (mu_1 + mu_2)/2) / s).
    m1, m2, rho = 0.3, -1.1, 0.25
    s = math.log1p(math.exp(rho))
    x = np.linspace(-4, 4, 33).reshape(-1, 1)
    g = oracle_mod.responsibilities(x, np.array([[[m1], [m2]]]), np.full((1, 2, 1), rho), np.zeros((1, 2)))
    t = (m1 - m2) * (x[:, 0] - (m1 + m2) / 2) / s
    np.testing.assert_allclose(g[:, 0], 1.0 / (1.0 + np.exp(-t)), rtol=1e-13)


def test_gamma_single_component_is_one(oracle_mod):
    rng = np.random.default_rng(4)
    mu, rv, pl = rand_params(rng, 1, 1, 4)
    g = oracle_mod.responsibilities(rng.normal(0, 5, (20, 4)), mu, rv, pl)
    assert (g == 1.0).all()


def test_gamma_far_rows_are_one_hot_not_nan(oracle_mod):
    mu = np.array([[[0.0], [10.0]]])
    g = oracle_mod.responsibilities(np.array([[-1e3], [1e3]]), mu, np.zeros((1, 2, 1)), np.zeros((1, 2)))
    assert np.isfinite(g).all()
    np.testing.assert_array_equal(g, [[1.0, 0.0], [0.0, 1.0]])


# ----------------------------------------------------------------------------- golden fixture


def _golden():
    out = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            rows = [[Fraction(t) if "/" in t else float(t) for t in r.split()] for r in val.split("|")]
            out[key.strip()] = rows
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_golden_two_component(oracle_mod, causal):
    gd = _golden()
    mu = np.array(gd["mu"][0], dtype=float).reshape(1, 2, 1)
    rv = np.full((1, 2, 1), gd["raw_var"][0][0])
    pl = np.array(gd["prior_logits"][0], dtype=float).reshape(1, 2)
    eps = gd["eps"][0][0]
    xq = np.array([r[0] for r in gd["x_q"]], dtype=float).reshape(3, 1)
    xk = np.array([r[0] for r in gd["x_k"]], dtype=float).reshape(3, 1)
    v = np.array(gd["v"], dtype=float)
    gq = oracle_mod.responsibilities(xq, mu, rv, pl)
    gk = oracle_mod.responsibilities(xk, mu, rv, pl)
    np.testing.assert_allclose(gq, np.array(gd["gamma_q"], dtype=float), rtol=1e-14)
    np.testing.assert_allclose(gk, np.array(gd["gamma_k"], dtype=float), rtol=1e-14)
    tag = "causal" if causal else "bidir"
    num = np.array(gd[tag + "_num"], dtype=float)
    den = np.array([r[0] for r in gd[tag + "_den"]], dtype=float)
    expect = num / (den + eps)[:, None]
    o = oracle_mod.forward(xq, xk, v, mu, rv, pl, eps=eps, causal=causal)
    np.testing.assert_allclose(o, expect, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------- forward


@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_brute_force_affinity(oracle_mod, causal):
    rng = np.random.default_rng(5)
    B, H, N, dr, K, dv = 2, 2, 37, 3, 5, 4
    mu, rv, pl = rand_params(rng, H, K, dr)
    qx, kx = rng.normal(0, 1, (B, H, N, dr)), rng.normal(0, 1, (B, H, N, dr))
    v = rng.normal(0, 1, (B, H, N, dv))
    eps = 1e-3
    o = oracle_mod.forward(qx, kx, v, mu, rv, pl, eps=eps, causal=causal)
    for b in range(B):
        for h in range(H):
            gq = scipy_gamma(qx[b, h], mu[h], rv[h], pl[h])
            gk = scipy_gamma(kx[b, h], mu[h], rv[h], pl[h])
            np.testing.assert_allclose(o[b, h], brute_force(gq, gk, v[b, h], eps, causal), rtol=1e-10, atol=1e-12)


def test_affinity_nonnegative_rank_at_most_K(oracle_mod):
    rng = np.random.default_rng(6)
    N, dr, K = 60, 4, 5
    mu, rv, pl = rand_params(rng, 1, K, dr)
    gq = oracle_mod.responsibilities(rng.normal(0, 1, (N, dr)), mu, rv, pl)
    gk = oracle_mod.responsibilities(rng.normal(0, 1, (N, dr)), mu, rv, pl)
    A = gq @ gk.T
    assert (A >= 0).all()
    s = np.linalg.svd(A, compute_uv=False)
    assert (s[K:] <= 1e-12 * s[0]).all()


@pytest.mark.parametrize("causal", [False, True])
def test_single_component_closed_form(oracle_mod, causal):
    rng = np.random.default_rng(7)
    N, dr, dv, eps = 25, 3, 4, 0.25
    mu, rv, pl = rand_params(rng, 1, 1, dr)
    v = rng.normal(0, 1, (N, dv))
    o = oracle_mod.forward(rng.normal(0, 1, (N, dr)), rng.normal(0, 1, (N, dr)), v, mu, rv, pl,
                           eps=eps, causal=causal)
    if causal:
        expect = np.cumsum(v, axis=0) / (np.arange(1, N + 1)[:, None] + eps)
    else:
        expect = np.broadcast_to(v.sum(0) / (N + eps), v.shape)
    np.testing.assert_allclose(o, expect, rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_components_closed_form(oracle_mod, causal):
    # K identical components with equal priors: gamma = 1/K everywhere, so
    # O_n = sum_j v_j / (count + K eps).
    rng = np.random.default_rng(8)
    N, dr, dv, K, eps = 19, 2, 3, 4, 0.5
    mu = np.broadcast_to(rng.normal(0, 1, (1, 1, dr)), (1, K, dr)).copy()
    rv = np.broadcast_to(rng.uniform(-1, 1, (1, 1, dr)), (1, K, dr)).copy()
    v = rng.normal(0, 1, (N, dv))
    o = oracle_mod.forward(rng.normal(0, 1, (N, dr)), rng.normal(0, 1, (N, dr)), v, mu, rv,
                           np.zeros((1, K)), eps=eps, causal=causal)
    if causal:
        expect = np.cumsum(v, axis=0) / (np.arange(1, N + 1)[:, None] + K * eps)
    else:
        expect = np.broadcast_to(v.sum(0) / (N + K * eps), v.shape)
    np.testing.assert_allclose(o, expect, rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_linear_in_values_and_convexity_bound(oracle_mod, causal):
    rng = np.random.default_rng(9)
    B, H, N, dr, K, dv = 1, 2, 45, 4, 6, 5
    mu, rv, pl = rand_params(rng, H, K, dr)
    qx, kx = rng.normal(0, 1, (B, H, N, dr)), rng.normal(0, 1, (B, H, N, dr))
    v1, v2 = rng.normal(0, 1, (B, H, N, dv)), rng.normal(0, 1, (B, H, N, dv))
    f = lambda v: oracle_mod.forward(qx, kx, v, mu, rv, pl, eps=1e-6, causal=causal)
    o1, o2, o12 = f(v1), f(v2), f(2.0 * v1 - 3.0 * v2)
    np.testing.assert_allclose(o12, 2.0 * o1 - 3.0 * o2, rtol=1e-11, atol=1e-12)
    # |O_nc| <= max_j |V_jc|: the weights A_nj / (sum_j A_nj + eps) are >= 0 and sum to < 1.
    bound = np.abs(v1).max(axis=2, keepdims=True)
    assert (np.abs(o1) <= bound * (1 + 1e-12)).all()


def test_bidir_permutation_symmetry(oracle_mod):
    rng = np.random.default_rng(10)
    N, dr, K, dv = 30, 3, 4, 2
    mu, rv, pl = rand_params(rng, 1, K, dr)
    qx, kx, v = rng.normal(0, 1, (N, dr)), rng.normal(0, 1, (N, dr)), rng.normal(0, 1, (N, dv))
    o = oracle_mod.forward(qx, kx, v, mu, rv, pl)
    p = rng.permutation(N)
    np.testing.assert_allclose(oracle_mod.forward(qx[p], kx, v, mu, rv, pl), o[p], rtol=1e-13)  # queries: equivariant
    np.testing.assert_allclose(oracle_mod.forward(qx, kx[p], v[p], mu, rv, pl), o, rtol=1e-12)  # keys+values: invariant


def test_causal_ignores_future_tokens_bitwise(oracle_mod):
    rng = np.random.default_rng(11)
    B, H, N, dr, K, dv = 1, 2, 64, 3, 5, 4
    mu, rv, pl = rand_params(rng, H, K, dr)
    qx, kx, v = rng.normal(0, 1, (B, H, N, dr)), rng.normal(0, 1, (B, H, N, dr)), rng.normal(0, 1, (B, H, N, dv))
    o = oracle_mod.forward(qx, kx, v, mu, rv, pl, causal=True)
    for i in (0, 17, 40):
        q2, k2, v2 = qx.copy(), kx.copy(), v.copy()
        q2[:, :, i + 1:] = rng.normal(0, 3, q2[:, :, i + 1:].shape)
        k2[:, :, i + 1:] = rng.normal(0, 3, k2[:, :, i + 1:].shape)
        v2[:, :, i + 1:] = rng.normal(0, 3, v2[:, :, i + 1:].shape)
        o2 = oracle_mod.forward(q2, k2, v2, mu, rv, pl, causal=True)
        np.testing.assert_array_equal(o2[:, :, : i + 1], o[:, :, : i + 1])
        assert not np.array_equal(o2[:, :, i + 1:], o[:, :, i + 1:])


def test_causal_is_bidir_on_prefix(oracle_mod):
    rng = np.random.default_rng(12)
    N, dr, K, dv = 48, 3, 4, 3
    mu, rv, pl = rand_params(rng, 1, K, dr)
    qx, kx, v = rng.normal(0, 1, (N, dr)), rng.normal(0, 1, (N, dr)), rng.normal(0, 1, (N, dv))
    oc = oracle_mod.forward(qx, kx, v, mu, rv, pl, causal=True)
    ob = oracle_mod.forward(qx, kx, v, mu, rv, pl, causal=False)
    np.testing.assert_allclose(oc[-1], ob[-1], rtol=1e-14)
    for i in (0, 1, 13, 29):
        obi = oracle_mod.forward(qx[: i + 1], kx[: i + 1], v[: i + 1], mu, rv, pl, causal=False)
        np.testing.assert_allclose(oc[i], obi[i], rtol=1e-13)


def test_thread_count_does_not_change_bits(oracle_mod):
    rng = np.random.default_rng(13)
    B, H, N, dr, K, dv = 1, 2, 5000, 4, 6, 8
    mu, rv, pl = rand_params(rng, H, K, dr)
    args = (rng.normal(0, 1, (B, H, N, dr)), rng.normal(0, 1, (B, H, N, dr)), rng.normal(0, 1, (B, H, N, dv)), mu, rv, pl)
    n = oracle_mod.max_threads()
    try:
        for causal in (False, True):
            a = oracle_mod.forward(*args, causal=causal, threads=1)
            b = oracle_mod.forward(*args, causal=causal, threads=max(2, n))
            np.testing.assert_array_equal(a, b)
    finally:
        oracle_mod.set_threads(n)


@settings(max_examples=25, deadline=None)
@given(N=st.integers(1, 24), dr=st.integers(1, 5), K=st.integers(1, 6), dv=st.integers(1, 4),
       causal=st.booleans(), seed=st.integers(0, 2**31 - 1))
def test_property_random_shapes_match_brute_force(N, dr, K, dv, causal, seed):
    import oracle
    rng = np.random.default_rng(seed)
    mu, rv, pl = rand_params(rng, 1, K, dr)
    qx, kx, v = rng.normal(0, 1, (N, dr)), rng.normal(0, 1, (N, dr)), rng.normal(0, 1, (N, dv))
    o = oracle.forward(qx, kx, v, mu, rv, pl, eps=1e-6, causal=causal)
    gq, gk = scipy_gamma(qx, mu[0], rv[0], pl[0]), scipy_gamma(kx, mu[0], rv[0], pl[0])
    np.testing.assert_allclose(o, brute_force(gq, gk, v, 1e-6, causal), rtol=1e-9, atol=1e-11)


# ----------------------------------------------------------------------------- carried state
# Causal variant with the latent memory carried in and out (page "Attention par Mélange Gaussien
# (GMA)", "Mécanisme Central" item 3: the causal output is a prefix sum, so the prefix before the
# first token enters only through [Vt | Z]).


def test_state_zero_initial_state_is_plain_causal(oracle_mod):
    rng = np.random.default_rng(21)
    B, H, N, dr, K, dv = 2, 2, 300, 5, 7, 6
    mu, rv, pl = rand_params(rng, H, K, dr)
    qx, kx, v = rng.normal(0, 1, (B, H, N, dr)), rng.normal(0, 1, (B, H, N, dr)), rng.normal(0, 1, (B, H, N, dv))
    o, _ = oracle_mod.forward_causal_state(qx, kx, v, mu, rv, pl)
    np.testing.assert_array_equal(o, oracle_mod.forward(qx, kx, v, mu, rv, pl, causal=True))


def test_state_final_state_is_the_write_phase(oracle_mod):
    # from a zero state, the final [Vt | Z] is Gamma_K^T [V | 1] over the sequence, with Gamma_K
    # from SciPy (an independent computation)
    rng = np.random.default_rng(22)
    H, N, dr, K, dv = 2, 200, 4, 5, 3
    mu, rv, pl = rand_params(rng, H, K, dr)
    qx, kx, v = rng.normal(0, 1, (1, H, N, dr)), rng.normal(0, 1, (1, H, N, dr)), rng.normal(0, 1, (1, H, N, dv))
    _, s = oracle_mod.forward_causal_state(qx, kx, v, mu, rv, pl)
    for h in range(H):
        gk = scipy_gamma(kx[0, h], mu[h], rv[h], pl[h])
        np.testing.assert_allclose(s[0, h, :, :dv], gk.T @ v[0, h], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(s[0, h, :, dv], gk.sum(axis=0), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("m", [1, 97, 299])
def test_state_split_sequence_equals_one_pass(oracle_mod, m):
    # running [0, m) and then [m, N) from the carried state reproduces the one-pass result bitwise
    rng = np.random.default_rng(23)
    B, H, N, dr, K, dv = 1, 3, 300, 4, 6, 5
    mu, rv, pl = rand_params(rng, H, K, dr)
    qx, kx, v = rng.normal(0, 1, (B, H, N, dr)), rng.normal(0, 1, (B, H, N, dr)), rng.normal(0, 1, (B, H, N, dv))
    o, s = oracle_mod.forward_causal_state(qx, kx, v, mu, rv, pl)
    o1, s1 = oracle_mod.forward_causal_state(qx[:, :, :m], kx[:, :, :m], v[:, :, :m], mu, rv, pl)
    o2, s2 = oracle_mod.forward_causal_state(qx[:, :, m:], kx[:, :, m:], v[:, :, m:], mu, rv, pl, state_in=s1)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=2), o)
    np.testing.assert_array_equal(s2, s)


def test_state_initial_state_acts_as_a_prefix(oracle_mod):
    # an initial state built by hand from prefix tokens (SciPy posteriors) gives the outputs that the
    # brute-force causal form gives for those rows after the prefix
    rng = np.random.default_rng(24)
    P, N, dr, K, dv = 40, 60, 3, 4, 3
    mu, rv, pl = rand_params(rng, 1, K, dr)
    kx_p, v_p = rng.normal(0, 1, (P, dr)), rng.normal(0, 1, (P, dv))
    qx, kx, v = rng.normal(0, 1, (N, dr)), rng.normal(0, 1, (N, dr)), rng.normal(0, 1, (N, dv))
    gk_p = scipy_gamma(kx_p, mu[0], rv[0], pl[0])
    s0 = np.concatenate([gk_p.T @ v_p, gk_p.sum(axis=0)[:, None]], axis=1)[None, None]
    o, _ = oracle_mod.forward_causal_state(qx[None, None], kx[None, None], v[None, None], mu, rv, pl, eps=1e-6,
                                           state_in=s0)
    # brute force over [prefix; x]: queries of the prefix rows are irrelevant (take the x rows only)
    qa = np.concatenate([rng.normal(0, 1, (P, dr)), qx])
    ka, va = np.concatenate([kx_p, kx]), np.concatenate([v_p, v])
    gq, gk = scipy_gamma(qa, mu[0], rv[0], pl[0]), scipy_gamma(ka, mu[0], rv[0], pl[0])
    np.testing.assert_allclose(o[0, 0], brute_force(gq, gk, va, 1e-6, True)[P:], rtol=1e-9, atol=1e-11)


# ----------------------------------------------------------------------------- cross-attention
# Bidirectional form with separate query and key/value sequences (N_q != N_k); the pages name it
# as future work; the definitions of the write and read phases are unchanged.


def test_cross_equal_lengths_is_bidirectional(oracle_mod):
    rng = np.random.default_rng(31)
    B, H, N, dr, K, dv = 2, 2, 150, 4, 5, 3
    mu, rv, pl = rand_params(rng, H, K, dr)
    qx, kx, v = rng.normal(0, 1, (B, H, N, dr)), rng.normal(0, 1, (B, H, N, dr)), rng.normal(0, 1, (B, H, N, dv))
    np.testing.assert_array_equal(oracle_mod.forward_bidir_kv(qx, kx, v, mu, rv, pl),
                                  oracle_mod.forward(qx, kx, v, mu, rv, pl, causal=False))


@pytest.mark.parametrize("Nq,Nk", [(1, 200), (37, 5), (120, 80)])
def test_cross_matches_rectangular_brute_force(oracle_mod, Nq, Nk):
    # A = Gamma_Q Gamma_K^T is N_q x N_k; O = A V / (A 1 + eps), posteriors from SciPy
    rng = np.random.default_rng(32 + Nq)
    dr, K, dv = 3, 4, 2
    mu, rv, pl = rand_params(rng, 1, K, dr)
    qx, kx, v = rng.normal(0, 1, (Nq, dr)), rng.normal(0, 1, (Nk, dr)), rng.normal(0, 1, (Nk, dv))
    o = oracle_mod.forward_bidir_kv(qx[None, None], kx[None, None], v[None, None], mu, rv, pl, eps=1e-6)
    gq, gk = scipy_gamma(qx, mu[0], rv[0], pl[0]), scipy_gamma(kx, mu[0], rv[0], pl[0])
    np.testing.assert_allclose(o[0, 0], brute_force(gq, gk, v, 1e-6, False), rtol=1e-9, atol=1e-11)


def test_cross_key_order_and_query_subsets(oracle_mod):
    # invariant to a joint permutation of the key/value rows; each query row depends on itself only
    rng = np.random.default_rng(33)
    Nq, Nk, dr, K, dv = 50, 90, 4, 6, 3
    mu, rv, pl = rand_params(rng, 1, K, dr)
    qx, kx, v = rng.normal(0, 1, (1, 1, Nq, dr)), rng.normal(0, 1, (1, 1, Nk, dr)), rng.normal(0, 1, (1, 1, Nk, dv))
    o = oracle_mod.forward_bidir_kv(qx, kx, v, mu, rv, pl)
    perm = rng.permutation(Nk)
    np.testing.assert_allclose(oracle_mod.forward_bidir_kv(qx, kx[:, :, perm], v[:, :, perm], mu, rv, pl), o,
                               rtol=1e-12, atol=1e-14)
    sub = [3, 17, 49]
    np.testing.assert_array_equal(oracle_mod.forward_bidir_kv(qx[:, :, sub], kx, v, mu, rv, pl), o[:, :, sub])


# ----------------------------------------------------------------------------- diagnostics
# Component usage, hard assignments and usage entropy: reductions over the rows of Gamma.


def test_stats_invariants(oracle_mod):
    rng = np.random.default_rng(41)
    B, H, N, dr, K = 2, 3, 400, 5, 7
    mu, rv, pl = rand_params(rng, H, K, dr)
    x = rng.normal(0, 1.5, (B, H, N, dr))
    usage, hard, ent, gap = oracle_mod.responsibility_stats(x, mu, rv, pl)
    np.testing.assert_allclose(usage.sum(axis=-1), N, rtol=1e-12)      # rows of Gamma sum to one
    assert (hard.sum(axis=-1) == N).all()
    assert (ent >= 0).all() and (ent <= 1 + 1e-12).all()               # normalised by ln K
    assert (gap >= 0).all() and (gap <= 1).all()
    # uniform usage has the largest entropy: identical components with equal priors give p_k = 1/K
    mu1 = np.repeat(mu[:, :1], K, axis=1)
    rv1 = np.repeat(rv[:, :1], K, axis=1)
    _, _, e1, g1 = oracle_mod.responsibility_stats(x, mu1, rv1, np.zeros((H, K)))
    np.testing.assert_allclose(e1, 1.0, rtol=1e-12)
    np.testing.assert_allclose(g1, 0.0, atol=1e-15)


def test_stats_gap_closed_forms(oracle_mod):
    # d_r = 1, K = 2, equal variances and priors: gamma_1 = sigmoid((mu1 - mu2)(x - (mu1 + mu2)/2)/s2)
    # (GMA page, item 1: the posterior of a two-component mixture), so the gap between the two
    # responsibilities is |2 gamma_1 - 1| = |tanh((mu1 - mu2)(x - (mu1 + mu2)/2)/(2 s2))|
    mu1, mu2, s2 = 0.7, -1.3, 0.8
    rho = math.log(math.expm1(s2))                                       # softplus(rho) = s2
    x = np.linspace(-4.0, 4.0, 97)
    _, _, _, gap = oracle_mod.responsibility_stats(x.reshape(1, 1, -1, 1), np.array([[[mu1], [mu2]]]),
                                                   np.full((1, 2, 1), rho), np.zeros((1, 2)))
    want = np.abs(np.tanh((mu1 - mu2) * (x - (mu1 + mu2) / 2) / (2 * s2)))
    np.testing.assert_allclose(gap[0, 0], want, rtol=1e-12, atol=1e-14)
    # three components on a line (unit variances, equal priors), listed out of order (means 3, 0, 1):
    # at x the weights are proportional to exp(-(x - m)^2 / 2).  The gap is the largest minus the
    # second largest responsibility -- not the largest minus the smallest, and not a difference of
    # components in index order.
    means = [3.0, 0.0, 1.0]
    xs = np.array([0.6, 0.45, 2.2, -1.0])
    _, _, _, gap = oracle_mod.responsibility_stats(xs.reshape(1, 1, -1, 1), np.array([[[m] for m in means]]),
                                                   np.full((1, 3, 1), math.log(math.e - 1.0)), np.zeros((1, 3)))
    for i, xv in enumerate(xs):
        wts = sorted(math.exp(-(xv - m) ** 2 / 2) for m in means)
        assert gap[0, 0, i] == pytest.approx((wts[2] - wts[1]) / sum(wts), rel=1e-12, abs=1e-15)


def test_stats_single_component_and_separated_clusters(oracle_mod):
    # K = 1: usage N, every row assigned, entropy 0
    rng = np.random.default_rng(42)
    mu, rv, pl = rand_params(rng, 1, 1, 3)
    u, hd, e, _ = oracle_mod.responsibility_stats(rng.normal(0, 1, (1, 1, 50, 3)), mu, rv, pl)
    assert u[0, 0, 0] == pytest.approx(50.0) and hd[0, 0, 0] == 50 and e[0, 0] == 0.0
    # three far-apart unit-variance clusters with equal priors, 10 / 20 / 30 points drawn at each mean:
    # hard counts are the cluster sizes, usage is the same to within e^-(distance), entropy follows
    dr = 2
    means = np.array([[0.0, 0.0], [40.0, 0.0], [0.0, 40.0]])
    mu = means[None]
    rv = np.full((1, 3, dr), math.log(math.e - 1.0))                    # softplus(rho) = 1
    pl = np.zeros((1, 3))
    x = np.concatenate([means[c] + 0.1 * rng.normal(0, 1, (n, dr)) for c, n in enumerate((10, 20, 30))])
    u, hd, e, _ = oracle_mod.responsibility_stats(x[None, None], mu, rv, pl)
    assert list(hd[0, 0]) == [10, 20, 30]
    np.testing.assert_allclose(u[0, 0], [10, 20, 30], atol=1e-9)
    p = np.array([10, 20, 30]) / 60
    assert e[0, 0] == pytest.approx(float(-(p * np.log(p)).sum()) / math.log(3), rel=1e-9)


# ----------------------------------------------------------------------------- backward
# The gradient of the mixer (the pages train it end to end, item 3) is pinned by central finite
# differences of the forward oracle, by reverse-mode automatic differentiation of an independent
# formulation (torch.distributions log-densities, materialised affinity), and by closed forms.

def _bwd_case(seed, B, H, N, dr, K, dv):
    rng = np.random.default_rng(seed)
    mu, rv, pl = rand_params(rng, H, K, dr)
    qx = rng.normal(0.0, 1.0, (B, H, N, dr))
    kx = rng.normal(0.0, 1.0, (B, H, N, dr))
    v = rng.normal(0.0, 1.0, (B, H, N, dv))
    do = rng.normal(0.0, 1.0, (B, H, N, dv))
    # shrink the routing inputs so that the posteriors are far from one-hot and every term matters
    return dict(qx=0.4 * qx, kx=0.4 * kx, v=v, mu=0.4 * mu, raw_var=rv, prior_logits=pl), do


_GRAD_OF = {"qx": "dqx", "kx": "dkx", "v": "dv", "mu": "dmu", "raw_var": "draw_var",
            "prior_logits": "dprior_logits"}


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(oracle_mod, causal):
    ins, do = _bwd_case(11, 2, 2, 7, 3, 4, 5)
    eps = 0.05
    g = oracle_mod.backward(**ins, dout=do, eps=eps, causal=causal)

    def loss(d):
        return float((oracle_mod.forward(**d, eps=eps, causal=causal) * do).sum())

    step = 1e-5
    for name, gname in _GRAD_OF.items():
        x = ins[name]
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            d = dict(ins)
            xp = x.copy(); xp[idx] += step
            xm = x.copy(); xm[idx] -= step
            d[name] = xp
            lp = loss(d)
            d[name] = xm
            fd[idx] = (lp - loss(d)) / (2 * step)
        err = np.abs(fd - g[gname]).max()
        assert err <= 1e-7 * max(1.0, np.abs(fd).max()), (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_autograd_of_materialised_affinity(oracle_mod, causal):
    torch = pytest.importorskip("torch")
    ins, do = _bwd_case(12, 2, 3, 19, 4, 5, 3)
    eps = 1e-3
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in ins.items()}
    var = torch.nn.functional.softplus(t["raw_var"])                       # [H, K, dr]
    logpi = torch.log_softmax(t["prior_logits"], dim=-1)                   # [H, K]
    dist = torch.distributions.Normal(t["mu"][None, :, None], var.sqrt()[None, :, None])

    def gamma(x):                                                          # x [B, H, N, dr]
        lp = dist.log_prob(x[:, :, :, None, :]).sum(-1) + logpi[None, :, None, :]
        return torch.softmax(lp, dim=-1)

    A = gamma(t["qx"]) @ gamma(t["kx"]).transpose(-1, -2)
    if causal:
        A = torch.tril(A)
    O = (A @ t["v"]) / (A.sum(-1, keepdim=True) + eps)
    grads = torch.autograd.grad((O * torch.tensor(do)).sum(), [t[k] for k in _GRAD_OF])
    g = oracle_mod.backward(**ins, dout=do, eps=eps, causal=causal)
    for (name, gname), ref in zip(_GRAD_OF.items(), grads):
        ref = ref.numpy()
        assert np.allclose(g[gname], ref, rtol=1e-9, atol=1e-11 * max(1.0, np.abs(ref).max())), name


@pytest.mark.parametrize("causal", [False, True])
def test_backward_single_component_closed_form(oracle_mod, causal):
    # K = 1: gamma == 1, so every routing and mixture gradient vanishes, and O is a (prefix) mean:
    # bidirectional O_n = sum_j v_j / (N + eps), causal O_i = sum_{j <= i} v_j / (i + 1 + eps)
    ins, do = _bwd_case(13, 1, 2, 9, 3, 1, 4)
    eps = 0.25
    g = oracle_mod.backward(**ins, dout=do, eps=eps, causal=causal)
    for name in ("dqx", "dkx", "dmu", "draw_var", "dprior_logits"):
        assert np.abs(g[name]).max() == 0.0, name
    N = 9
    if causal:
        w = np.array([1.0 / (i + 1 + eps) for i in range(N)])
        ref = np.flip(np.cumsum(np.flip(do * w[None, None, :, None], axis=2), axis=2), axis=2)
    else:
        ref = np.broadcast_to(do.sum(axis=2, keepdims=True) / (N + eps), do.shape)
    assert np.allclose(g["dv"], ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_structure(oracle_mod, causal):
    ins, do = _bwd_case(14, 2, 2, 16, 3, 4, 3)
    g = oracle_mod.backward(**ins, dout=do, eps=1e-2, causal=causal)
    # the priors enter through a softmax: its gradient sums to zero over the components
    assert np.abs(g["dprior_logits"].sum(axis=-1)).max() < 1e-12 * max(1.0, np.abs(g["dprior_logits"]).max())
    # O is linear in V and the loss is linear in dO: dv does not depend on V, and every gradient
    # scales with dO
    ins2 = dict(ins, v=3.0 * ins["v"] - 1.0)
    assert np.allclose(oracle_mod.backward(**ins2, dout=do, eps=1e-2, causal=causal)["dv"], g["dv"],
                       rtol=1e-12, atol=1e-14)
    g3 = oracle_mod.backward(**ins, dout=-2.5 * do, eps=1e-2, causal=causal)
    for name in _GRAD_OF.values():
        assert np.allclose(g3[name], -2.5 * g[name], rtol=1e-12, atol=1e-14), name
    if causal:
        # a key j reaches the loss only through queries i >= j: with dO zero from row m on, the
        # rows >= m of dv, dkx (and dqx, through their own queries) vanish exactly
        m = 10
        do2 = do.copy(); do2[:, :, m:] = 0.0
        g2 = oracle_mod.backward(**ins, dout=do2, eps=1e-2, causal=True)
        assert np.abs(g2["dv"][:, :, m:]).max() == 0.0
        assert np.abs(g2["dkx"][:, :, m:]).max() == 0.0
        assert np.abs(g2["dqx"][:, :, m:]).max() == 0.0
