"""Pins of the CPU oracle against facts that do not come from the oracle itself.

The pages print no worked example, so no value here is printed by them.  Each
test checks the oracle against mathematics the pages' description fixes:
closed forms of special cases, brute-force products of the per-token
transition matrices, invariants (linearity, packing, resuming), and central
finite differences of the forward for the reverse mode.  Every plausible slip
in the oracle (decay after the residual instead of before, decay on value rows
instead of key columns, a sign flip of the residual, reading the memory before
the write, a transposed memory, a wrong gate axis in Gated DeltaNet-2, a wrong
gradient term) makes at least one of them fail.
"""
import numpy as np
import pytest

from oracle import recurrence as R

RTOL = 1e-12


def _rand_inputs(rng, variant, B=1, H=2, T=9, dk=5, dv=4, unit_keys=True, beta=True):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    b = rng.uniform(0.05, 0.95, (B, H, T)) if beta else None
    if variant == "deltanet":
        a = None
    elif variant in ("kda", "gla"):
        a = rng.uniform(0.3, 0.99, (B, H, T, dk))
    else:
        a = rng.uniform(0.3, 0.99, (B, H, T))
    e = rng.uniform(0.05, 0.95, (B, H, T, dk)) if variant == "gdn2" else None
    w = rng.uniform(0.05, 0.95, (B, H, T, dv)) if variant == "gdn2" else None
    return dict(q=q, k=k, v=v, beta=b, alpha=a, erase=e, write=w)


def _decay_vec(alpha, variant, b, h, t, dk):
    """Per-key-channel decay of token t as a vector (ones for deltanet)."""
    if variant == "deltanet":
        return np.ones(dk)
    if variant in ("kda", "gla"):
        return alpha[b, h, t]
    return np.full(dk, alpha[b, h, t])


# ---------------------------------------------------------------------------------------
# Special cases with closed forms
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["deltanet", "gated", "kda", "gdn2", "gla"])
def test_beta_zero_is_pure_decay(variant):
    """beta = 0 writes nothing: W_t = W0 Gamma_t, Gamma_t = prod of the decays (key columns)."""
    rng = np.random.default_rng(1)
    x = _rand_inputs(rng, variant, B=2, H=3, T=11, dk=5, dv=4)
    x["beta"] = np.zeros((2, 3, 11))
    h0 = rng.standard_normal((2, 3, 4, 5))
    o, ht = R.forward(**x, h0=h0, variant=variant, scale=0.7)
    for b in range(2):
        for h in range(3):
            gam = np.ones(5)
            for t in range(11):
                gam = gam * _decay_vec(x["alpha"], variant, b, h, t, 5)
                want = 0.7 * (h0[b, h] * gam[None, :]) @ x["q"][b, h, t]
                np.testing.assert_allclose(o[b, h, t], want, rtol=RTOL, atol=1e-14)
            np.testing.assert_allclose(ht[b, h], h0[b, h] * gam[None, :], rtol=RTOL, atol=1e-14)


@pytest.mark.parametrize("variant", ["deltanet", "gated", "kda"])
def test_beta_one_stores_value_exactly(variant):
    """With beta = 1 and unit keys the delta rule writes the whole residual, so right after
    token t the memory returns exactly v_t at address k_t (any decay, any prior content).
    Reading with q = k gives o_t = v_t.  Fails if the residual's sign is flipped or if the
    decay is applied after the residual instead of before it."""
    rng = np.random.default_rng(2)
    x = _rand_inputs(rng, variant, B=1, H=2, T=12, dk=6, dv=3)
    x["beta"] = np.ones((1, 2, 12))
    x["q"] = x["k"].copy()
    h0 = rng.standard_normal((1, 2, 3, 6))
    o, _ = R.forward(**x, h0=h0, variant=variant)
    np.testing.assert_allclose(o, x["v"], rtol=1e-12, atol=1e-12)


def test_gdn2_zero_erase_is_decayed_linear_attention():
    """Gated DeltaNet-2 with the erase gate closed (e = 0) keeps only the gated additive write:
    o_t = Gamma_t-decayed W0 q_t + sum_{s<=t} (gamma_t/gamma_s) (k_s . q_t) beta_s (w_s * v_s),
    the causal decayed linear attention the pages contrast with the delta rule."""
    rng = np.random.default_rng(3)
    x = _rand_inputs(rng, "gdn2", B=1, H=2, T=10, dk=4, dv=5)
    x["erase"] = np.zeros_like(x["erase"])
    h0 = rng.standard_normal((1, 2, 5, 4))
    o, _ = R.forward(**x, h0=h0, variant="gdn2")
    for h in range(2):
        logg = np.cumsum(np.log(x["alpha"][0, h]))
        Q, K = x["q"][0, h], x["k"][0, h]
        Bv = x["beta"][0, h][:, None] * x["write"][0, h] * x["v"][0, h]
        D = np.tril(np.exp(logg[:, None] - logg[None, :]))
        want = (D * (Q @ K.T)) @ Bv + np.exp(logg)[:, None] * (Q @ h0[0, h].T)
        np.testing.assert_allclose(o[0, h], want, rtol=1e-11, atol=1e-12)


def test_deltanet_orthonormal_keys_no_interference():
    """Orthonormal keys never interfere: the prediction at each new key is 0, so DeltaNet from
    a zero memory is plain linear attention o_t = sum_{s<=t} beta_s v_s (k_s . q_t)."""
    rng = np.random.default_rng(4)
    d = 8
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Qm.T[None, None]                       # 8 orthonormal keys
    q = rng.standard_normal((1, 1, d, d))
    v = rng.standard_normal((1, 1, d, 3))
    beta = rng.uniform(0.1, 0.9, (1, 1, d))
    o, _ = R.forward(q, k, v, beta, variant="deltanet", scale=1.3)
    want = 1.3 * (np.tril(q[0, 0] @ k[0, 0].T) * beta[0, 0][None, :]) @ v[0, 0]
    np.testing.assert_allclose(o[0, 0], want, rtol=1e-12, atol=1e-13)


def test_deltanet_repeated_key_overwrites():
    """Writing twice at one unit key: W = b1 v1 k^T + b2 (v2 - b1 v1) k^T (textbook delta rule)."""
    rng = np.random.default_rng(5)
    k1 = rng.standard_normal(6)
    k1 /= np.linalg.norm(k1)
    k = np.stack([k1, k1])[None, None]
    v = rng.standard_normal((1, 1, 2, 3))
    beta = np.array([[[0.3, 0.8]]])
    _, ht = R.forward(k.copy(), k, v, beta, variant="deltanet")
    v1, v2 = v[0, 0]
    want = 0.3 * np.outer(v1, k1) + 0.8 * np.outer(v2 - 0.3 * v1, k1)
    np.testing.assert_allclose(ht[0, 0], want, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------------------
# Brute force: explicit transition matrices
# ---------------------------------------------------------------------------------------
def _brute(x, variant, h0, scale):
    """W_t = W_{t-1} D_t (I - k_t a_t^T) + b_t k_t^T with every factor formed as a matrix;
    the memory after token t is W0 prod_{u<=t} A_u + sum_{s<=t} b_s k_s^T prod_{s<u<=t} A_u."""
    B, H, T, dk = x["k"].shape
    dv = x["v"].shape[-1]
    o = np.zeros((B, H, T, dv))
    ht = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            A, Bk = [], []
            for t in range(T):
                kt = x["k"][b, h, t]
                beta = 1.0 if x["beta"] is None else x["beta"][b, h, t]
                if variant == "gdn2":
                    a = beta * x["erase"][b, h, t] * kt
                    bb = beta * x["write"][b, h, t] * x["v"][b, h, t]
                elif variant == "gla":
                    a = np.zeros(dk)
                    bb = beta * x["v"][b, h, t]
                else:
                    a = beta * kt
                    bb = beta * x["v"][b, h, t]
                D = np.diag(_decay_vec(x["alpha"], variant, b, h, t, dk))
                A.append(D @ (np.eye(dk) - np.outer(kt, a)))
                Bk.append(np.outer(bb, kt))
            for t in range(T):
                P = np.eye(dk)
                for u in range(t + 1):
                    P = P @ A[u]
                W = h0[b, h] @ P
                for s in range(t + 1):
                    Ps = np.eye(dk)
                    for u in range(s + 1, t + 1):
                        Ps = Ps @ A[u]
                    W = W + Bk[s] @ Ps
                o[b, h, t] = scale * W @ x["q"][b, h, t]
            ht[b, h] = W
    return o, ht


@pytest.mark.parametrize("variant", ["deltanet", "gated", "kda", "gdn2", "gla"])
def test_brute_force_transition_products(variant):
    rng = np.random.default_rng(6)
    x = _rand_inputs(rng, variant, B=2, H=2, T=7, dk=4, dv=3, unit_keys=False)
    h0 = rng.standard_normal((2, 2, 3, 4))
    o, ht = R.forward(**x, h0=h0, variant=variant, scale=0.9)
    ob, hb = _brute(x, variant, h0, 0.9)
    np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ht, hb, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["deltanet", "gated", "kda", "gdn2", "gla"])
def test_joint_linearity_in_values_and_initial_memory(variant):
    """Given keys, queries and gates, (o, h_T) is linear in (v, h0) jointly."""
    rng = np.random.default_rng(7)
    x = _rand_inputs(rng, variant, B=1, H=2, T=10, dk=4, dv=5)
    v1, v2 = rng.standard_normal((2,) + x["v"].shape)
    h1, h2 = rng.standard_normal((2, 1, 2, 5, 4))
    l1, l2 = 0.7, -1.9
    run = lambda v, h: R.forward(**{**x, "v": v}, h0=h, variant=variant)
    o1, s1 = run(v1, h1)
    o2, s2 = run(v2, h2)
    o3, s3 = run(l1 * v1 + l2 * v2, l1 * h1 + l2 * h2)
    np.testing.assert_allclose(o3, l1 * o1 + l2 * o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(s3, l1 * s1 + l2 * s2, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("variant", ["gated", "kda", "gdn2", "gla"])
def test_packed_sequences_equal_separate_runs(variant):
    rng = np.random.default_rng(8)
    cu = [0, 5, 6, 14, 20]
    x = _rand_inputs(rng, variant, B=1, H=2, T=20, dk=4, dv=3)
    h0 = rng.standard_normal((4, 2, 3, 4))
    do = rng.standard_normal((1, 2, 20, 3))
    dht = rng.standard_normal((4, 2, 3, 4))
    o, ht = R.forward(**x, h0=h0, variant=variant, cu_seqlens=cu)
    gp = R.backward(**x, h0=h0, do=do, dht=dht, variant=variant, cu_seqlens=cu)
    for n in range(4):
        sl = slice(cu[n], cu[n + 1])
        xs = {kk: (vv[:, :, sl] if vv is not None else None) for kk, vv in x.items()}
        os_, hs = R.forward(**xs, h0=h0[n:n + 1], variant=variant)
        assert np.array_equal(os_, o[:, :, sl])
        assert np.array_equal(hs[0], ht[n])
        gs = R.backward(**xs, h0=h0[n:n + 1], do=do[:, :, sl], dht=dht[n:n + 1], variant=variant)
        for name in ("dq", "dk", "dv", "dbeta", "dalpha", "derase", "dwrite"):
            if gs[name] is not None:
                assert np.array_equal(gs[name], gp[name][:, :, sl]), name
        assert np.array_equal(gs["dh0"][0], gp["dh0"][n])


@pytest.mark.parametrize("variant", ["deltanet", "kda"])
def test_split_and_resume_equals_one_run(variant):
    """Running [0,T1) then [T1,T) from the returned memory equals one run over [0,T)."""
    rng = np.random.default_rng(9)
    x = _rand_inputs(rng, variant, B=2, H=2, T=13, dk=4, dv=3)
    h0 = rng.standard_normal((2, 2, 3, 4))
    o, ht = R.forward(**x, h0=h0, variant=variant)
    a = {kk: (vv[:, :, :6] if vv is not None else None) for kk, vv in x.items()}
    b = {kk: (vv[:, :, 6:] if vv is not None else None) for kk, vv in x.items()}
    oa, ha = R.forward(**a, h0=h0, variant=variant)
    ob, hb = R.forward(**b, h0=ha, variant=variant)
    assert np.array_equal(np.concatenate([oa, ob], axis=2), o)
    assert np.array_equal(hb, ht)


def test_checkpoint_spacing_does_not_change_gradients():
    rng = np.random.default_rng(10)
    x = _rand_inputs(rng, "kda", B=1, H=2, T=17, dk=4, dv=3)
    do = rng.standard_normal((1, 2, 17, 3))
    ref = R.backward(**x, do=do, variant="kda", checkpoint_every=64)
    for S in (1, 4, 5):
        g = R.backward(**x, do=do, variant="kda", checkpoint_every=S)
        for name in ("dq", "dk", "dv", "dbeta", "dalpha", "dh0"):
            assert np.array_equal(g[name], ref[name]), (S, name)


def test_variant_reductions():
    """Gated with alpha = 1 is DeltaNet; Kimi with equal channel decays is Gated; Gated
    DeltaNet-2 with open gates (e = w = 1) and a beta is Gated DeltaNet.  The four variants
    take different code paths (copy, scalar scaling, column scaling, erase/write form)."""
    rng = np.random.default_rng(11)
    x = _rand_inputs(rng, "gated", B=1, H=2, T=9, dk=4, dv=3)
    h0 = rng.standard_normal((1, 2, 3, 4))
    og, hg = R.forward(**x, h0=h0, variant="gated")
    xk = {**x, "alpha": np.repeat(x["alpha"][..., None], 4, axis=-1)}
    ok, hk = R.forward(**xk, h0=h0, variant="kda")
    np.testing.assert_allclose(ok, og, rtol=1e-13, atol=1e-14)
    x2 = {**x, "erase": np.ones((1, 2, 9, 4)), "write": np.ones((1, 2, 9, 3))}
    o2, h2 = R.forward(**x2, h0=h0, variant="gdn2")
    np.testing.assert_allclose(o2, og, rtol=1e-12, atol=1e-13)
    x1 = {**x, "alpha": np.ones((1, 2, 9))}
    o1, _ = R.forward(**x1, h0=h0, variant="gated")
    od, _ = R.forward(**{**x, "alpha": None}, h0=h0, variant="deltanet")
    np.testing.assert_allclose(o1, od, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------------------
# Reverse mode against central finite differences of the forward
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("variant,cu", [("deltanet", None), ("gated", None), ("kda", None),
                                        ("gdn2", None), ("gla", None), ("gated", [0, 3, 8])])
def test_backward_matches_finite_differences(variant, cu):
    rng = np.random.default_rng(12)
    B = 1 if cu else 2
    N = len(cu) - 1 if cu else B
    x = _rand_inputs(rng, variant, B=B, H=2, T=8, dk=3, dv=4, unit_keys=False)
    x["h0"] = rng.standard_normal((N, 2, 4, 3))
    G = rng.standard_normal((B, 2, 8, 4))
    G2 = rng.standard_normal((N, 2, 4, 3))
    scale = 0.8

    def loss(xx):
        o, ht = R.forward(**xx, variant=variant, cu_seqlens=cu, scale=scale)
        return np.sum(o * G) + np.sum(ht * G2)

    g = R.backward(**x, do=G, dht=G2, variant=variant, cu_seqlens=cu, scale=scale,
                   checkpoint_every=3)
    names = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "alpha": "dalpha",
             "erase": "derase", "write": "dwrite", "h0": "dh0"}
    eps = 1e-6
    for name, gname in names.items():
        if x[name] is None:
            assert g[gname] is None
            continue
        fd = np.zeros_like(x[name])
        it = np.nditer(x[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = {kk: (vv.copy() if vv is not None else None) for kk, vv in x.items()}
            xm = {kk: (vv.copy() if vv is not None else None) for kk, vv in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd[idx] = (loss(xp) - loss(xm)) / (2 * eps)
        np.testing.assert_allclose(g[gname], fd, rtol=1e-6, atol=1e-7, err_msg=gname)


# ---------------------------------------------------------------------------------------
# The residual output r_t = v_t - v_bar_t
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["deltanet", "gated", "kda"])
def test_residual_basis_keys_is_value(variant):
    """Keys that are distinct standard basis vectors never overlap, even after a per-channel
    decay, so from a zero memory every prediction is 0 and r_t = v_t exactly."""
    rng = np.random.default_rng(21)
    d = 6
    x = _rand_inputs(rng, variant, B=1, H=2, T=d, dk=d, dv=3)
    perm = rng.permutation(d)
    x["k"] = np.broadcast_to(np.eye(d)[perm], (1, 2, d, d)).copy()
    _, _, r = R.forward(**x, variant=variant, residual=True)
    np.testing.assert_array_equal(r, x["v"])


@pytest.mark.parametrize("variant", ["deltanet", "gated", "kda"])
def test_residual_beta_zero_is_value_minus_decayed_prediction(variant):
    """beta = 0 writes nothing, so the prediction is the decayed initial memory at k_t:
    r_t = v_t - (W0 Gamma_t) k_t."""
    rng = np.random.default_rng(22)
    x = _rand_inputs(rng, variant, B=2, H=2, T=7, dk=5, dv=4)
    x["beta"] = np.zeros((2, 2, 7))
    h0 = rng.standard_normal((2, 2, 4, 5))
    _, _, r = R.forward(**x, h0=h0, variant=variant, residual=True)
    for b in range(2):
        for h in range(2):
            gam = np.ones(5)
            for t in range(7):
                gam = gam * _decay_vec(x["alpha"], variant, b, h, t, 5)
                want = x["v"][b, h, t] - (h0[b, h] * gam[None, :]) @ x["k"][b, h, t]
                np.testing.assert_allclose(r[b, h, t], want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("variant", ["deltanet", "gated"])
def test_residual_repeated_key(variant):
    """Full-strength writes (beta = 1) at one unit key from a zero memory: the first residual
    is v_1, the second v_2 - alpha_2 v_1 (v_2 - v_1 without decay)."""
    rng = np.random.default_rng(23)
    k1 = rng.standard_normal(5)
    k1 /= np.linalg.norm(k1)
    k = np.stack([k1, k1])[None, None]
    v = rng.standard_normal((1, 1, 2, 3))
    alpha = None if variant == "deltanet" else np.array([[[0.9, 0.6]]])
    _, _, r = R.forward(k.copy(), k, v, np.ones((1, 1, 2)), alpha, variant=variant, residual=True)
    a2 = 1.0 if alpha is None else 0.6
    np.testing.assert_allclose(r[0, 0, 0], v[0, 0, 0], rtol=1e-14)
    np.testing.assert_allclose(r[0, 0, 1], v[0, 0, 1] - a2 * v[0, 0, 0], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("variant", ["deltanet", "gated", "kda"])
def test_residual_backward_matches_finite_differences(variant):
    rng = np.random.default_rng(24)
    x = _rand_inputs(rng, variant, B=2, H=2, T=7, dk=3, dv=4, unit_keys=False)
    x["h0"] = rng.standard_normal((2, 2, 4, 3))
    G = rng.standard_normal((2, 2, 7, 4))
    Gr = rng.standard_normal((2, 2, 7, 4))

    def loss(xx):
        o, _, r = R.forward(**xx, variant=variant, scale=0.9, residual=True)
        return np.sum(o * G) + np.sum(r * Gr)

    g = R.backward(**x, do=G, dr=Gr, variant=variant, scale=0.9, checkpoint_every=3)
    eps = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"), ("alpha", "dalpha"),
                        ("h0", "dh0")):
        if x[name] is None:
            continue
        fd = np.zeros_like(x[name])
        it = np.nditer(x[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = {kk: (vv.copy() if vv is not None else None) for kk, vv in x.items()}
            xm = {kk: (vv.copy() if vv is not None else None) for kk, vv in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd[idx] = (loss(xp) - loss(xm)) / (2 * eps)
        np.testing.assert_allclose(g[gname], fd, rtol=1e-6, atol=1e-7, err_msg=gname)


def test_residual_refused_for_gdn2():
    rng = np.random.default_rng(25)
    x = _rand_inputs(rng, "gdn2", T=3)
    with pytest.raises(ValueError):
        R.forward(**x, variant="gdn2", residual=True)


# q/k L2-normalisation (q, k scaled to unit length per token before the recurrence)
def test_l2_normalize_unit_length_and_zero_row():
    x = np.array([[3.0, 4.0], [0.0, 0.0], [-1e-3, 0.0]])
    y = R.l2_normalize(x)
    np.testing.assert_allclose(y, [[0.6, 0.8], [0.0, 0.0], [-1.0, 0.0]], rtol=0, atol=1e-15)


@pytest.mark.parametrize("variant", ["deltanet", "gated", "kda", "gdn2"])
def test_qk_l2norm_scale_invariance(variant):
    """Normalised queries and keys make the outputs independent of each token's q and k scale."""
    rng = np.random.default_rng(31)
    x = _rand_inputs(rng, variant, B=1, H=2, T=6, dk=3, dv=4, unit_keys=False)
    o1, h1 = R.forward(**x, variant=variant, qk_l2norm=True)
    y = dict(x)
    y["q"] = x["q"] * rng.uniform(0.1, 5.0, size=x["q"].shape[:-1] + (1,))
    y["k"] = x["k"] * rng.uniform(0.1, 5.0, size=x["k"].shape[:-1] + (1,))
    o2, h2 = R.forward(**y, variant=variant, qk_l2norm=True)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(h1, h2, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("variant", ["gated", "kda", "gdn2"])
def test_qk_l2norm_backward_matches_finite_differences(variant):
    rng = np.random.default_rng(32)
    x = _rand_inputs(rng, variant, B=1, H=1, T=5, dk=3, dv=2, unit_keys=False)
    G = rng.standard_normal((1, 1, 5, 2))

    def loss(xx):
        o, _ = R.forward(**xx, variant=variant, qk_l2norm=True)
        return float(np.sum(o * G))

    g = R.backward(**x, do=G, variant=variant, qk_l2norm=True)
    for name in ("q", "k"):
        num = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp, xm = dict(x), dict(x)
            xp[name] = x[name].copy(); xp[name][idx] += 1e-6
            xm[name] = x[name].copy(); xm[name][idx] -= 1e-6
            num[idx] = (loss(xp) - loss(xm)) / 2e-6
        np.testing.assert_allclose(g["d" + name], num, rtol=1e-6, atol=1e-8)


# ---------------------------------------------------------------------------------------
# Gates given as logits: the activation maps and their chain rule
# ---------------------------------------------------------------------------------------
def test_logit_gate_maps_closed_forms():
    """sigmoid against scipy's expit; alpha = exp(-softplus(x)) is 1 / (1 + e^x) = sigmoid(-x);
    both are 1/2 at x = 0 and stay finite and in (0, 1) at large |x|."""
    from scipy.special import expit
    x = np.array([-800.0, -30.0, -2.5, -1e-3, 0.0, 1e-3, 0.7, 2.0, 30.0, 800.0])
    b, a, e, w = R.gates_from_logits(x, x, x, x)
    np.testing.assert_allclose(b, expit(x), rtol=1e-15, atol=0)
    np.testing.assert_array_equal(e, b)
    np.testing.assert_array_equal(w, b)
    np.testing.assert_allclose(a, expit(-x), rtol=1e-13, atol=1e-300)
    assert b[4] == 0.5 and a[4] == 0.5
    assert np.all((a >= 0) & (a <= 1) & np.isfinite(a))
    np.testing.assert_allclose(b + R.sigmoid(-x), 1.0, rtol=1e-15)
    # log alpha = -softplus(x): -log 2 at 0, about -x for large x, about -e^x for very negative x
    np.testing.assert_allclose(R.neg_softplus(np.array([0.0, 40.0, -40.0])),
                               [-np.log(2.0), -40.0, -np.exp(-40.0)], rtol=1e-14)


@pytest.mark.parametrize("variant", ["deltanet", "gated", "kda", "gdn2", "gla"])
def test_logit_gradients_match_finite_differences(variant):
    """The whole map from logits to outputs, differentiated by central differences in the
    logits, against the chain rule of backward(gate_logits=True)."""
    rng = np.random.default_rng(41)
    x = _rand_inputs(rng, variant, B=1, H=2, T=6, dk=3, dv=4, unit_keys=False)
    for name in ("beta", "alpha", "erase", "write"):
        if x.get(name) is not None:
            x[name] = rng.standard_normal(x[name].shape) * 1.5   # logits
    x["h0"] = rng.standard_normal((1, 2, 4, 3))
    G = rng.standard_normal((1, 2, 6, 4))

    def loss(xx):
        o, ht = R.forward(**xx, variant=variant, scale=0.7, gate_logits=True)
        return np.sum(o * G) + 0.3 * np.sum(ht)

    g = R.backward(**x, do=G, dht=np.full((1, 2, 4, 3), 0.3), variant=variant, scale=0.7,
                   gate_logits=True)
    eps = 1e-6
    for name in ("beta", "alpha", "erase", "write"):
        if x.get(name) is None:
            continue
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {kk: (vv.copy() if vv is not None else None) for kk, vv in x.items()}
            xm = {kk: (vv.copy() if vv is not None else None) for kk, vv in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd[idx] = (loss(xp) - loss(xm)) / (2 * eps)
        np.testing.assert_allclose(g["d" + name], fd, rtol=1e-6, atol=1e-8, err_msg=name)



# ---------------------------------------------------------------------------------------
# The erase-free memory with a decay per key channel (variant "gla")
# ---------------------------------------------------------------------------------------
def test_gla_is_causal_linear_attention_with_channel_decay():
    """Nothing erased: with G_t = sum_{u<=t} log alpha_u per key channel,
    o_t = W0 (e^{G_t} * q_t) + sum_{s<=t} beta_s v_s (k_s * e^{G_t - G_s}) . q_t and
    h_T = W0 diag(e^{G_T}) + sum_s beta_s v_s (k_s * e^{G_T - G_s})^T, written here as one
    masked product over (t, s, channel) -- no recurrence."""
    rng = np.random.default_rng(51)
    x = _rand_inputs(rng, "gla", B=1, H=2, T=11, dk=5, dv=4)
    h0 = rng.standard_normal((1, 2, 4, 5))
    o, ht = R.forward(**x, h0=h0, variant="gla", scale=0.8)
    for h in range(2):
        G = np.cumsum(np.log(x["alpha"][0, h]), axis=0)            # [T, dk]
        Q, K, V = x["q"][0, h], x["k"][0, h], x["v"][0, h]
        Bv = x["beta"][0, h][:, None] * V
        E = np.exp(G[:, None, :] - G[None, :, :])                   # [t, s, j]
        S = np.einsum("tj,sj,tsj->ts", Q, K, E) * np.tril(np.ones((11, 11)))
        want = 0.8 * (S @ Bv + (Q * np.exp(G)) @ h0[0, h].T)
        np.testing.assert_allclose(o[0, h], want, rtol=1e-11, atol=1e-12)
        hw = h0[0, h] * np.exp(G[-1])[None, :] + Bv.T @ (K * np.exp(G[-1][None, :] - G))
        np.testing.assert_allclose(ht[0, h], hw, rtol=1e-11, atol=1e-12)


def test_gla_with_equal_channels_is_gdn2_with_closed_erase():
    """One decay shared by every channel is the scalar-decay erase-free memory: Gated
    DeltaNet-2 with e = 0 and w = 1 (different code paths: column scaling and no erase term
    against scalar scaling and a zero erase direction).  Without beta both mean beta = 1."""
    rng = np.random.default_rng(52)
    x = _rand_inputs(rng, "gdn2", B=2, H=2, T=9, dk=4, dv=3)
    h0 = rng.standard_normal((2, 2, 3, 4))
    G = rng.standard_normal((2, 2, 9, 3))
    for beta in (x["beta"], None):
        x2 = {**x, "beta": beta, "erase": np.zeros((2, 2, 9, 4)), "write": np.ones((2, 2, 9, 3))}
        o2, h2 = R.forward(**x2, h0=h0, variant="gdn2")
        g2 = R.backward(**x2, h0=h0, do=G, variant="gdn2")
        xg = {**x, "beta": beta, "erase": None, "write": None,
              "alpha": np.repeat(x["alpha"][..., None], 4, axis=-1)}
        og, hg = R.forward(**xg, h0=h0, variant="gla")
        gg = R.backward(**xg, h0=h0, do=G, variant="gla")
        np.testing.assert_allclose(og, o2, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(hg, h2, rtol=1e-12, atol=1e-13)
        for name in ("dq", "dk", "dv", "dh0") + (("dbeta",) if beta is not None else ()):
            np.testing.assert_allclose(gg[name], g2[name], rtol=1e-11, atol=1e-12, err_msg=name)
        np.testing.assert_allclose(gg["dalpha"].sum(-1), g2["dalpha"], rtol=1e-11, atol=1e-12)


def test_gla_without_beta_and_refuses_a_residual():
    rng = np.random.default_rng(53)
    x = _rand_inputs(rng, "gla", B=1, H=2, T=6, dk=3, dv=2)
    o1, _ = R.forward(**{**x, "beta": None}, variant="gla")
    o2, _ = R.forward(**{**x, "beta": np.ones((1, 2, 6))}, variant="gla")
    assert np.array_equal(o1, o2)
    with pytest.raises(ValueError):
        R.forward(**x, variant="gla", residual=True)
