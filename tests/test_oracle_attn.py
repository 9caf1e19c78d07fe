"""Pins of the fp64 attention oracle against facts that do not come from the
oracle itself: finite differences of the loss, a hand-derived closed form,
gradient identities that follow from softmax rows summing to one, symmetry,
and degenerate cases with known answers.

Each test is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign, a transposed operand, a wrong mask index, a missing scale)
fails at least one of them."""
import numpy as np
import pytest

pytestmark = []


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _loss(oracle_mod, q, k, v, do, causal, scale):
    o, _ = oracle_mod.attn_fwd(q, k, v, causal, scale)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("s,d", [(1, 3), (5, 4), (7, 8)])
def test_gradient_matches_central_differences(oracle_mod, causal, s, d):
    """dQ, dK, dV are the gradient of L = sum(dO * O(Q, K, V)) with dO held
    fixed; central differences in fp64 (step 1e-5) agree to 1e-7 relative."""
    rng = np.random.default_rng(100 + s * 10 + d + causal)
    H = 2
    q, k, v, do = (_rand(rng, H, s, d) for _ in range(4))
    scale = 0.7
    g = oracle_mod.attn_fwd_bwd(q, k, v, do, causal, scale)
    h = 1e-5
    for name, x, grad in (("q", q, g["dq"]), ("k", k, g["dk"]), ("v", v, g["dv"])):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(oracle_mod, args["q"], args["k"], args["v"], do, causal, scale)
            args[name] = xm
            lm = _loss(oracle_mod, args["q"], args["k"], args["v"], do, causal, scale)
            fd[idx] = (lp - lm) / (2 * h)
        ref = max(np.max(np.abs(fd)), 1e-12)
        assert np.max(np.abs(fd - grad)) <= 1e-7 * max(ref, 1.0), name


def test_two_token_closed_form(oracle_mod):
    """s = 2, d = 1, full mask, scale 1: the softmax of a row is a logistic
    function p_i = sigmoid(q_i (k0 - k1)), so every output has a closed form
    derived by hand from d sigmoid / dx = p (1 - p)."""
    q = np.array([[[0.3], [-1.2]]])
    k = np.array([[[0.8], [-0.5]]])
    v = np.array([[[1.5], [-2.0]]])
    do = np.array([[[0.7], [-0.4]]])
    g = oracle_mod.attn_fwd_bwd(q, k, v, do, False, 1.0)
    qi, doi = q[0, :, 0], do[0, :, 0]
    k0, k1, v0, v1 = k[0, 0, 0], k[0, 1, 0], v[0, 0, 0], v[0, 1, 0]
    p = 1.0 / (1.0 + np.exp(-qi * (k0 - k1)))
    o = p * v0 + (1 - p) * v1
    lse = qi * k0 + np.log1p(np.exp(qi * (k1 - k0)))
    w = doi * (v0 - v1) * p * (1 - p)
    dq = w * (k0 - k1)
    dk0 = np.sum(w * qi)
    dv0, dv1 = np.sum(doi * p), np.sum(doi * (1 - p))
    np.testing.assert_allclose(g["o"][0, :, 0], o, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(g["lse"][0], lse, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(g["D"][0], doi * o, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(g["dq"][0, :, 0], dq, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(g["dk"][0, :, 0], [dk0, -dk0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(g["dv"][0, :, 0], [dv0, dv1], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_gradient_identities(oracle_mod, causal):
    """Rows of dS sum to zero (rows of P sum to one), hence
    sum_j dK_j = 0, sum_j dV_j = sum_i dO_i, and adding a constant vector to
    every key leaves all three gradients unchanged."""
    rng = np.random.default_rng(7 + causal)
    H, s, d = 3, 37, 16
    q, k, v, do = (_rand(rng, H, s, d) for _ in range(4))
    g = oracle_mod.attn_fwd_bwd(q, k, v, do, causal)
    np.testing.assert_allclose(g["dk"].sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(g["dv"].sum(axis=1), do.sum(axis=1), rtol=1e-12, atol=1e-12)
    shift = rng.standard_normal((H, 1, d))
    g2 = oracle_mod.attn_fwd_bwd(q, k + shift, v, do, causal)
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(g2[name], g[name], rtol=1e-9, atol=1e-11)


def test_key_permutation_full_mask(oracle_mod):
    """With the full mask, permuting keys together with values permutes the
    rows of dK and dV the same way and leaves dQ unchanged."""
    rng = np.random.default_rng(11)
    H, s, d = 2, 29, 8
    q, k, v, do = (_rand(rng, H, s, d) for _ in range(4))
    perm = rng.permutation(s)
    g = oracle_mod.attn_fwd_bwd(q, k, v, do, False)
    gp = oracle_mod.attn_fwd_bwd(q, k[:, perm], v[:, perm], do, False)
    np.testing.assert_allclose(gp["dq"], g["dq"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(gp["dk"], g["dk"][:, perm], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(gp["dv"], g["dv"][:, perm], rtol=1e-11, atol=1e-13)


def test_causal_mask_is_lower_triangular(oracle_mod):
    """Under the causal mask, key j sees only queries i >= j: changing the
    last query leaves dK, dV of every key untouched except through row s-1,
    and changing key s-1 changes only the last query's output and dQ."""
    rng = np.random.default_rng(13)
    H, s, d = 1, 9, 4
    q, k, v, do = (_rand(rng, H, s, d) for _ in range(4))
    g = oracle_mod.attn_fwd_bwd(q, k, v, do, True)
    k2 = k.copy()
    k2[:, -1] += 3.0
    g2 = oracle_mod.attn_fwd_bwd(q, k2, v, do, True)
    np.testing.assert_array_equal(g2["o"][:, :-1], g["o"][:, :-1])
    np.testing.assert_array_equal(g2["dq"][:, :-1], g["dq"][:, :-1])
    assert np.max(np.abs(g2["dq"][:, -1] - g["dq"][:, -1])) > 1e-6


def test_degenerate_cases(oracle_mod):
    rng = np.random.default_rng(17)
    # s = 1: one key, P = 1, so dS = 0: dQ = dK = 0 and dV = dO.
    q, k, v, do = (_rand(rng, 2, 1, 5) for _ in range(4))
    for causal in (False, True):
        g = oracle_mod.attn_fwd_bwd(q, k, v, do, causal)
        np.testing.assert_allclose(g["dq"], 0.0, atol=1e-15)
        np.testing.assert_allclose(g["dk"], 0.0, atol=1e-15)
        np.testing.assert_allclose(g["dv"], do, rtol=1e-15)
        np.testing.assert_allclose(g["lse"], (np.sum(q * k, -1) / np.sqrt(5)), rtol=1e-14)
    # causal row 0 attends to key 0 only: dQ_0 = 0.
    q, k, v, do = (_rand(rng, 1, 6, 4) for _ in range(4))
    g = oracle_mod.attn_fwd_bwd(q, k, v, do, True)
    np.testing.assert_allclose(g["dq"][0, 0], 0.0, atol=1e-15)
    # K = 0: every score is 0, so P is uniform over the visible keys:
    # full: lse = log s, O_i = mean_j v_j, dV_j = (1/s) sum_i dO_i.
    s = 10
    q, v, do = (_rand(rng, 1, s, 3) for _ in range(3))
    k = np.zeros_like(q)
    g = oracle_mod.attn_fwd_bwd(q, k, v, do, False)
    np.testing.assert_allclose(g["lse"], np.log(s), rtol=1e-14)
    np.testing.assert_allclose(g["o"], np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape),
                               rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(g["dv"], np.broadcast_to(do.sum(axis=1, keepdims=True) / s, v.shape),
                               rtol=1e-13, atol=1e-15)
    # causal with K = 0: row i averages keys 0..i, lse_i = log(i + 1).
    g = oracle_mod.attn_fwd_bwd(q, k, v, do, True)
    np.testing.assert_allclose(g["lse"][0], np.log(np.arange(1, s + 1)), rtol=1e-14)
    np.testing.assert_allclose(g["o"][0], np.cumsum(v[0], axis=0) / np.arange(1, s + 1)[:, None],
                               rtol=1e-12, atol=1e-14)


def test_given_mode_uses_supplied_o_and_lse(oracle_mod):
    """The backward reads O only through D = rowsum(dO * O) and lse only
    through P: feeding D-preserving changes leaves results unchanged, while a
    shifted lse rescales P (and hence dV) by exp(-shift)."""
    rng = np.random.default_rng(19)
    q, k, v, do = (_rand(rng, 1, 8, 4) for _ in range(4))
    g = oracle_mod.attn_fwd_bwd(q, k, v, do, False)
    dq, dk, dv, D = oracle_mod.attn_bwd(q, k, v, g["o"], do, g["lse"], False)
    np.testing.assert_array_equal(dv, g["dv"])
    np.testing.assert_allclose(D, np.sum(do * g["o"], -1), rtol=1e-14)
    dq2, dk2, dv2, _ = oracle_mod.attn_bwd(q, k, v, g["o"], do, g["lse"] + np.log(2.0), False)
    np.testing.assert_allclose(dv2, dv / 2, rtol=1e-12)
