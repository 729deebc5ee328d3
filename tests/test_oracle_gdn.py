"""Pins of the gated-delta-rule oracle (token recurrence, C, fp64).

Against results that do not come from the recurrence itself:
* dense transition products on tiny inputs (``ref.gdn_bruteforce``);
* the page's chunked UT/WY evaluation at chunk sizes 1, 16 and 64
  (hyper-parallel ``_prepare_gdn_chunks_for_summary`` /
  ``_run_prepared_gdn_chunks``), each sequence chunked from its own start;
  its triangular inverse against numpy.linalg.inv;
* the affine state summary S_out = M S_in + E and its prefix fold
  (``_compute_gdn_state_summary_from_prepared``,
  ``_merge_gdn_prefix_state_summaries_torch``, ``_apply_gdn_state_summary``);
* closed forms: beta = 0, total decay (g = -1e4), one token, the l2norm eps;
* invariants: a split at every token boundary with state + halo passed
  reproduces the unsplit output; a packed batch equals each sequence alone
  (zero-length sequences included); GQA head mapping = repeat_interleave.
"""
import numpy as np
import pytest

from oracle import ref


def _draw(rng, T, Hk, Hv, dk, dv, N=None, h0=True, g_scale=1.0):
    q = rng.standard_normal((T, Hk, dk))
    k = rng.standard_normal((T, Hk, dk))
    v = rng.standard_normal((T, Hv, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, Hv))))
    g = -np.log1p(np.exp(rng.standard_normal((T, Hv)))) * g_scale
    h = rng.standard_normal((N or 1, Hv, dk, dv)) * 0.5 if h0 else None
    return q, k, v, g, beta, h


def test_l2norm_eps_closed_form(oracle_lib):
    # with |x|^2 = 1e-6 = eps the normalised vector is x / sqrt(2e-6);
    # max(|x|, eps) or a missing eps would give 1.0 here
    x = np.array([[[1e-3, 0.0]]])
    o, _ = oracle_lib.gdn_fwd(x, x, np.ones((1, 1, 1)), np.zeros((1, 1)), np.ones((1, 1)),
                              None, [0, 1], scale=1.0)
    # o = beta * (khat . qhat) * v with khat = qhat = [0.70710678..., 0]
    assert abs(o[0, 0, 0] - 0.5) < 1e-12


def test_bruteforce_tiny(oracle_lib):
    rng = np.random.default_rng(1)
    cu = [0, 3, 3, 8]
    q, k, v, g, beta, h0 = _draw(rng, 8, 1, 2, 3, 4, N=3)
    for use in (True, False):
        o, ht = oracle_lib.gdn_fwd(q, k, v, g, beta, h0, cu, 0.7, use)
        ob, hb = ref.gdn_bruteforce(q, k, v, g, beta, h0, cu, 0.7, use)
        np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(ht, hb, rtol=1e-11, atol=1e-12)
    # the zero-length sequence returns its initial state
    np.testing.assert_array_equal(ht[1], h0[1])


@pytest.mark.parametrize("chunk", [1, 16, 64])
def test_chunked_form(chunk, oracle_lib):
    rng = np.random.default_rng(chunk)
    cu = [0, 70, 71, 150]
    q, k, v, g, beta, h0 = _draw(rng, 150, 2, 4, 8, 6, N=3)
    scale = 8 ** -0.5
    o, ht = oracle_lib.gdn_fwd(q, k, v, g, beta, h0, cu, scale)
    oc, hc = ref.gdn_chunked(q, k, v, g, beta, h0, cu, scale, chunk=chunk)
    assert np.abs(o - oc).max() <= 1e-12 * np.abs(o).max()
    assert np.abs(ht - hc).max() <= 1e-12 * np.abs(ht).max()


def test_chunk_inverse_matches_library():
    rng = np.random.default_rng(4)
    C, d = 64, 16
    k = ref.l2norm(rng.standard_normal((C, d)))
    chunks, _ = ref._chunk_prepare(k, k, rng.standard_normal((C, 3)),
                                   -np.log1p(np.exp(rng.standard_normal(C))),
                                   1 / (1 + np.exp(-rng.standard_normal(C))), C)
    ch = chunks[0]
    np.testing.assert_allclose(ch["T"], np.linalg.inv(np.eye(C) + ch["L"]), rtol=1e-10, atol=1e-12)


def test_affine_summary_and_prefix_fold(oracle_lib):
    rng = np.random.default_rng(8)
    T, dk, dv = 200, 6, 5
    q, k, v, g, beta, _ = _draw(rng, T, 1, 2, dk, dv, g_scale=0.01)
    h0 = rng.standard_normal((1, 2, dk, dv))
    _, ht = oracle_lib.gdn_fwd(q, k, v, g, beta, h0, [0, T], 1.0)
    M, E = ref.gdn_state_summary(k, v, g, beta, [0, T])
    for h in range(2):
        np.testing.assert_allclose(ht[0, h], M[0, h] @ h0[0, h] + E[0, h], rtol=1e-10, atol=1e-12)
    # four shards: fold of the first r summaries = state entering shard r
    cuts = [0, 37, 90, 151, 200]
    Ms, Es = [], []
    for r in range(4):
        s, e = cuts[r], cuts[r + 1]
        Mr, Er = ref.gdn_state_summary(k[s:e], v[s:e], g[s:e], beta[s:e], [0, e - s])
        Ms.append(Mr[0])
        Es.append(Er[0])
    for r in range(5):
        want = ref.merge_prefix_summaries(np.array(Ms), np.array(Es), r) if r else np.zeros((2, dk, dv))
        if r:
            _, hr = oracle_lib.gdn_fwd(q[:cuts[r]], k[:cuts[r]], v[:cuts[r]], g[:cuts[r]],
                                       beta[:cuts[r]], None, [0, cuts[r]], 1.0)
            np.testing.assert_allclose(hr[0], want, rtol=1e-10, atol=1e-12)


def test_closed_form_beta_zero(oracle_lib):
    rng = np.random.default_rng(2)
    T = 12
    q, k, v, g, _, h0 = _draw(rng, T, 1, 1, 4, 3)
    beta = np.zeros((T, 1))
    o, ht = oracle_lib.gdn_fwd(q, k, v, g, beta, h0, [0, T], 0.5)
    G = np.cumsum(g[:, 0])
    qh = 0.5 * ref.l2norm(q[:, 0])
    for t in range(T):
        np.testing.assert_allclose(o[t, 0], np.exp(G[t]) * h0[0, 0].T @ qh[t], rtol=1e-12)
    np.testing.assert_allclose(ht[0, 0], np.exp(G[-1]) * h0[0, 0], rtol=1e-12)


def test_closed_form_total_decay(oracle_lib):
    rng = np.random.default_rng(3)
    T = 10
    q, k, v, _, beta, h0 = _draw(rng, T, 1, 1, 5, 2)
    g = np.full((T, 1), -1e4)
    o, _ = oracle_lib.gdn_fwd(q, k, v, g, beta, h0, [0, T], 1.0)
    qh, kh = ref.l2norm(q[:, 0]), ref.l2norm(k[:, 0])
    for t in range(T):
        np.testing.assert_allclose(o[t, 0], beta[t, 0] * (kh[t] @ qh[t]) * v[t, 0], rtol=1e-12)


def test_closed_form_one_token(oracle_lib):
    rng = np.random.default_rng(6)
    q, k, v, g, beta, h0 = _draw(rng, 1, 1, 1, 4, 3)
    o, ht = oracle_lib.gdn_fwd(q, k, v, g, beta, h0, [0, 1], 0.3)
    kh, qh = ref.l2norm(k[0, 0]), 0.3 * ref.l2norm(q[0, 0])
    a = np.exp(g[0, 0])
    S1 = a * h0[0, 0] + beta[0, 0] * np.outer(kh, v[0, 0] - a * h0[0, 0].T @ kh)
    np.testing.assert_allclose(ht[0, 0], S1, rtol=1e-12)
    np.testing.assert_allclose(o[0, 0], S1.T @ qh, rtol=1e-12)


def test_delta_rule_retrieval(oracle_lib):
    # beta = 1, g = 0: reading the state back with the key just written gives
    # |k|^2 v_t + (1 - |k|^2) S_{t-1}^T k, i.e. v_t up to the l2norm eps
    rng = np.random.default_rng(12)
    T = 9
    k = rng.standard_normal((T, 1, 6))
    v = rng.standard_normal((T, 1, 3))
    o, _ = oracle_lib.gdn_fwd(k, k, v, np.zeros((T, 1)), np.ones((T, 1)), None, [0, T], 1.0)
    np.testing.assert_allclose(o, v, rtol=1e-5, atol=1e-5)


def test_gqa_mapping_is_repeat_interleave(oracle_lib):
    rng = np.random.default_rng(13)
    T, Hk, Hv = 20, 2, 6
    q, k, v, g, beta, h0 = _draw(rng, T, Hk, Hv, 4, 4)
    o, ht = oracle_lib.gdn_fwd(q, k, v, g, beta, h0, [0, T], 1.0)
    qe, ke = np.repeat(q, Hv // Hk, axis=1), np.repeat(k, Hv // Hk, axis=1)
    oe, he = oracle_lib.gdn_fwd(qe, ke, v, g, beta, h0, [0, T], 1.0)
    np.testing.assert_array_equal(o, oe)
    np.testing.assert_array_equal(ht, he)


@pytest.mark.parametrize("variant", ["configs", "slow_decay", "no_decay_beta1"])
def test_split_invariance_every_cut(variant, oracle_lib):
    """Splitting a sequence at any token and passing the final state and the
    K-1 pre-conv tail reproduces the unsplit conv + GDN output."""
    rng = np.random.default_rng(21)
    T, C_qk, dk, dv, K = 24, 2, 4, 3, 4
    Hk, Hv = 1, 2
    C = 2 * Hk * dk + Hv * dv
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, K)) / 2
    _, _, _, g, beta, _ = _draw(rng, T, Hk, Hv, dk, dv)
    if variant == "slow_decay":
        g = g * 0.01
    if variant == "no_decay_beta1":
        g, beta = np.zeros_like(g), np.ones_like(beta)

    def run(xs, gs, bs, halo, nh, h0):
        y = oracle_lib.conv1d_silu(xs, w, None, halo, nh, [0, len(xs)])
        q = y[:, :Hk * dk].reshape(-1, Hk, dk)
        k = y[:, Hk * dk:2 * Hk * dk].reshape(-1, Hk, dk)
        v = y[:, 2 * Hk * dk:].reshape(-1, Hv, dv)
        return oracle_lib.gdn_fwd(q, k, v, gs, bs, h0, [0, len(xs)], dk ** -0.5)

    o_full, h_full = run(x, g, beta, None, 0, None)
    for cut in range(1, T):
        o_l, h_l = run(x[:cut], g[:cut], beta[:cut], None, 0, None)
        nh = min(K - 1, cut)
        halo = np.zeros((K - 1, C))
        halo[K - 1 - nh:] = x[cut - nh:cut]
        o_r, h_r = run(x[cut:], g[cut:], beta[cut:], halo, nh, h_l)
        np.testing.assert_allclose(np.concatenate([o_l, o_r]), o_full, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(h_r, h_full, rtol=1e-11, atol=1e-13)


def test_packed_equals_alone(oracle_lib):
    rng = np.random.default_rng(22)
    cu = [0, 0, 13, 13, 40, 41, 41]
    T = cu[-1]
    N = len(cu) - 1
    q, k, v, g, beta, h0 = _draw(rng, T, 2, 2, 5, 4, N=N)
    o, ht = oracle_lib.gdn_fwd(q, k, v, g, beta, h0, cu, 1.0)
    for n in range(N):
        s, e = cu[n], cu[n + 1]
        oa, ha = oracle_lib.gdn_fwd(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], h0[n:n + 1],
                                    [0, e - s], 1.0)
        np.testing.assert_array_equal(o[s:e], oa)
        np.testing.assert_array_equal(ht[n], ha[0])


def test_numpy_recurrence_agrees(oracle_lib):
    rng = np.random.default_rng(23)
    cu = [0, 17, 30]
    q, k, v, g, beta, h0 = _draw(rng, 30, 2, 4, 6, 5, N=2)
    o, ht = oracle_lib.gdn_fwd(q, k, v, g, beta, h0, cu, 0.4)
    on, hn = ref.gdn_recurrent(q, k, v, g, beta, h0, cu, 0.4)
    np.testing.assert_allclose(o, on, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ht, hn, rtol=1e-12, atol=1e-14)
