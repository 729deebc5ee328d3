"""Pins of the oracle's hand-written reverse mode (gated delta rule + conv).

* central finite differences (fp64, h = 1e-6) of the oracle's forward for
  every input: q, k, v, g, beta, h0 -- with and without l2norm, with GQA
  head sharing and a packed varlen batch;
* the adjoint identity <d_out, J t> = <J^T d_out, t> along random
  directions at a larger size;
* the split backward: running the right half with the upstream gradients,
  then the left half with dht = the right half's dh0, and adding the right
  half's halo gradient into the left half's last K-1 input rows reproduces
  the unsplit gradients (the gradient contract of the page's P2P send/recv
  autograd functions and of its differentiable halo all-to-all).
"""
import numpy as np
import pytest


def _draw(rng, T, Hk, Hv, dk, dv, N):
    return dict(
        q=rng.standard_normal((T, Hk, dk)), k=rng.standard_normal((T, Hk, dk)),
        v=rng.standard_normal((T, Hv, dv)),
        g=-np.log1p(np.exp(rng.standard_normal((T, Hv)))) * 0.3,
        beta=1 / (1 + np.exp(-rng.standard_normal((T, Hv)))),
        h0=rng.standard_normal((N, Hv, dk, dv)) * 0.5)


@pytest.mark.parametrize("use_l2norm", [True, False])
def test_gdn_bwd_finite_differences(use_l2norm, oracle_lib):
    rng = np.random.default_rng(31 + use_l2norm)
    cu = [0, 5, 5, 11]
    T, Hk, Hv, dk, dv, N = 11, 1, 2, 3, 2, 3
    a = _draw(rng, T, Hk, Hv, dk, dv, N)
    do = rng.standard_normal((T, Hv, dv))
    dht = rng.standard_normal((N, Hv, dk, dv))
    scale = 0.6
    grads = oracle_lib.gdn_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], cu, scale, do,
                               dht, use_l2norm)

    def loss(b):
        o, ht = oracle_lib.gdn_fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], b["h0"], cu, scale,
                                   use_l2norm)
        return float((o * do).sum() + (ht * dht).sum())

    eps = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                        ("h0", "dh0")):
        num = np.zeros_like(a[name])
        it = np.nditer(a[name], flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            b = {kk: vv.copy() for kk, vv in a.items()}
            b[name][i] += eps
            lp = loss(b)
            b[name][i] -= 2 * eps
            lm = loss(b)
            num[i] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grads[gname], num, rtol=2e-6, atol=1e-8, err_msg=name)


def test_gdn_bwd_adjoint_identity(oracle_lib):
    rng = np.random.default_rng(40)
    cu = [0, 70, 130]
    T, Hk, Hv, dk, dv, N = 130, 2, 4, 8, 8, 2
    a = _draw(rng, T, Hk, Hv, dk, dv, N)
    do = rng.standard_normal((T, Hv, dv))
    dht = rng.standard_normal((N, Hv, dk, dv))
    grads = oracle_lib.gdn_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], cu, 0.35, do, dht)
    dirs = {kk: rng.standard_normal(vv.shape) for kk, vv in a.items()}
    h = 1e-6

    def fwd(sign):
        b = {kk: a[kk] + sign * h * dirs[kk] for kk in a}
        return oracle_lib.gdn_fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], b["h0"], cu, 0.35)

    (op, hp), (om, hm) = fwd(+1), fwd(-1)
    lhs = ((op - om) * do).sum() / (2 * h) + ((hp - hm) * dht).sum() / (2 * h)
    rhs = sum((grads[gn] * dirs[n]).sum() for n, gn in
              (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"), ("h0", "dh0")))
    assert abs(lhs - rhs) <= 1e-7 * abs(rhs)


def _layer(oracle_lib, x, w, g, beta, halo, nh, h0, Hk, Hv, dk, dv):
    y = oracle_lib.conv1d_silu(x, w, None, halo, nh, [0, len(x)])
    q = y[:, :Hk * dk].reshape(-1, Hk, dk)
    k = y[:, Hk * dk:2 * Hk * dk].reshape(-1, Hk, dk)
    v = y[:, 2 * Hk * dk:].reshape(-1, Hv, dv)
    return q, k, v


def _layer_bwd(oracle_lib, x, w, g, beta, halo, nh, h0, do, dht, Hk, Hv, dk, dv):
    q, k, v = _layer(oracle_lib, x, w, g, beta, halo, nh, h0, Hk, Hv, dk, dv)
    gr = oracle_lib.gdn_bwd(q, k, v, g, beta, h0, [0, len(x)], dk ** -0.5, do, dht)
    dy = np.concatenate([gr["dq"].reshape(len(x), -1), gr["dk"].reshape(len(x), -1),
                         gr["dv"].reshape(len(x), -1)], axis=1)
    dx, dw, _, dhalo = oracle_lib.conv1d_silu_bwd(x, w, None, halo, nh, [0, len(x)], dy)
    return dict(dx=dx, dw=dw, dhalo=dhalo, dg=gr["dg"], dbeta=gr["dbeta"], dh0=gr["dh0"])


@pytest.mark.parametrize("variant", ["configs", "slow_decay", "no_decay_beta1"])
def test_split_backward(variant, oracle_lib):
    rng = np.random.default_rng(50)
    T, Hk, Hv, dk, dv, K = 20, 1, 2, 4, 3, 4
    C = 2 * Hk * dk + Hv * dv
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, K)) / 2
    g = -np.log1p(np.exp(rng.standard_normal((T, Hv))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, Hv))))
    if variant == "slow_decay":
        g = g * 0.01
    if variant == "no_decay_beta1":
        g, beta = np.zeros_like(g), np.ones_like(beta)
    do = rng.standard_normal((T, Hv, dv))
    dht = rng.standard_normal((1, Hv, dk, dv))
    zeros_h = np.zeros((1, Hv, dk, dv))
    full = _layer_bwd(oracle_lib, x, w, g, beta, np.zeros((K - 1, C)), 0, zeros_h, do, dht,
                      Hk, Hv, dk, dv)
    for cut in (1, 2, 3, 7, 13, 19):
        # forward of the left half gives the state passed right
        ql, kl, vl = _layer(oracle_lib, x[:cut], w, g, beta, None, 0, None, Hk, Hv, dk, dv)
        _, h_l = oracle_lib.gdn_fwd(ql, kl, vl, g[:cut], beta[:cut], zeros_h, [0, cut], dk ** -0.5)
        nh = min(K - 1, cut)
        halo = np.zeros((K - 1, C))
        halo[K - 1 - nh:] = x[cut - nh:cut]
        right = _layer_bwd(oracle_lib, x[cut:], w, g[cut:], beta[cut:], halo, nh, h_l, do[cut:],
                           dht, Hk, Hv, dk, dv)
        left = _layer_bwd(oracle_lib, x[:cut], w, g[:cut], beta[:cut], np.zeros((K - 1, C)), 0,
                          zeros_h, do[:cut], right["dh0"], Hk, Hv, dk, dv)
        dx = np.concatenate([left["dx"], right["dx"]])
        dx[cut - nh:cut] += right["dhalo"][K - 1 - nh:]
        np.testing.assert_allclose(dx, full["dx"], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(left["dw"] + right["dw"], full["dw"], rtol=1e-10, atol=1e-12)
        for kk in ("dg", "dbeta"):
            np.testing.assert_allclose(np.concatenate([left[kk], right[kk]]), full[kk], rtol=1e-10,
                                       atol=1e-12)
        np.testing.assert_allclose(left["dh0"], full["dh0"], rtol=1e-10, atol=1e-12)
