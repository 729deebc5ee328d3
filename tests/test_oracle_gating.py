"""Pins of the oracle's gating step (hyper-parallel
"linear_attention_context_parallel.py", the CP wrappers' forward:
beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias)) and of its
reverse mode, against closed forms, asymptotes, torch.nn.functional on the
CPU in float64 and finite differences."""
import math

import numpy as np
import torch

import pytest


def test_closed_forms(oracle_lib):
    # sigmoid(0) = 1/2; softplus(0) = ln 2; A_log = 0 gives exp(A_log) = 1
    a = np.zeros((1, 3))
    b = np.zeros((1, 3))
    g, beta = oracle_lib.gating_fwd(a, b, np.zeros(3), np.zeros(3))
    assert np.all(beta == 0.5)
    assert np.allclose(g, -math.log(2.0), rtol=0, atol=1e-15)
    # A_log = ln 3 scales g by 3; dt_bias shifts a
    g2, _ = oracle_lib.gating_fwd(np.array([[-0.7]]), np.zeros((1, 1)), np.array([math.log(3.0)]),
                                  np.array([0.7]))
    assert abs(g2[0, 0] + 3 * math.log(2.0)) < 1e-14


def test_asymptotes(oracle_lib):
    # softplus(x) -> x for large x and -> e^x for very negative x; sigmoid
    # saturates without overflow
    x = np.array([[60.0, -60.0, 700.0, -700.0]])
    g, beta = oracle_lib.gating_fwd(x, x, np.zeros(4), np.zeros(4))
    assert abs(g[0, 0] + 60.0) < 1e-12
    assert abs(g[0, 1] + math.exp(-60.0)) < 1e-40
    assert abs(g[0, 2] + 700.0) < 1e-9 and np.isfinite(g).all()
    assert beta[0, 0] == 1.0 and beta[0, 1] < 1e-25 and beta[0, 3] >= 0.0


def test_matches_torch_functional(oracle_lib):
    rng = np.random.default_rng(0)
    T, Hv = 64, 8
    a = rng.standard_normal((T, Hv)) * 3
    b = rng.standard_normal((T, Hv)) * 3
    A_log = rng.standard_normal(Hv)
    dt_bias = rng.standard_normal(Hv)
    g, beta = oracle_lib.gating_fwd(a, b, A_log, dt_bias)
    ta, tb = torch.tensor(a), torch.tensor(b)
    want_b = torch.sigmoid(tb).numpy()
    # torch's softplus is exact below its threshold of 20 (|a + dt_bias| < 20 here)
    want_g = (-torch.exp(torch.tensor(A_log)) *
              torch.nn.functional.softplus(ta + torch.tensor(dt_bias))).numpy()
    assert np.abs(a + dt_bias).max() < 20
    assert np.allclose(beta, want_b, rtol=1e-14, atol=0)
    assert np.allclose(g, want_g, rtol=1e-13, atol=0)


def test_backward_matches_autograd_and_finite_differences(oracle_lib):
    rng = np.random.default_rng(1)
    T, Hv = 20, 3
    a = rng.standard_normal((T, Hv))
    b = rng.standard_normal((T, Hv))
    A_log = rng.standard_normal(Hv) * 0.5
    dt_bias = rng.standard_normal(Hv)
    dg = rng.standard_normal((T, Hv))
    dbeta = rng.standard_normal((T, Hv))
    got = oracle_lib.gating_bwd(a, b, A_log, dt_bias, dg, dbeta)
    # autograd in float64
    ts = [torch.tensor(v, requires_grad=True) for v in (a, b, A_log, dt_bias)]
    beta = torch.sigmoid(ts[1])
    g = -torch.exp(ts[2]) * torch.nn.functional.softplus(ts[0] + ts[3])
    (g * torch.tensor(dg)).sum().add((beta * torch.tensor(dbeta)).sum()).backward()
    for name, t in zip(("da", "db", "dA_log", "ddt_bias"), ts):
        assert np.allclose(got[name], t.grad.numpy(), rtol=1e-12, atol=1e-14), name

    # central differences of L = <dg, g> + <dbeta, beta>
    def loss(a_, b_, al_, db_):
        g_, be_ = oracle_lib.gating_fwd(a_, b_, al_, db_)
        return float((g_ * dg).sum() + (be_ * dbeta).sum())
    h = 1e-6
    args = [a, b, A_log, dt_bias]
    for i, name in enumerate(("da", "db", "dA_log", "ddt_bias")):
        flat = args[i].reshape(-1)
        for j in range(0, flat.size, max(1, flat.size // 7)):
            plus = [x.copy() for x in args]
            minus = [x.copy() for x in args]
            plus[i].reshape(-1)[j] += h
            minus[i].reshape(-1)[j] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - got[name].reshape(-1)[j]) < 1e-7 * max(1.0, abs(fd)), (name, j)


@pytest.mark.parametrize("seed", [2, 3])
def test_gating_feeds_the_recurrence_like_given_gates(seed, oracle_lib):
    """The gates the oracle forms from (a, b, A_log, dt_bias) are the g, beta
    the recurrence consumes: gating then gdn_fwd equals gdn_fwd on the same
    g, beta computed by torch."""
    rng = np.random.default_rng(seed)
    T, Hk, Hv, d = 40, 1, 2, 8
    q, k = rng.standard_normal((T, Hk, d)), rng.standard_normal((T, Hk, d))
    v = rng.standard_normal((T, Hv, d))
    a, b = rng.standard_normal((T, Hv)), rng.standard_normal((T, Hv))
    A_log, dt_bias = rng.standard_normal(Hv) * 0.3, rng.standard_normal(Hv)
    g, beta = oracle_lib.gating_fwd(a, b, A_log, dt_bias)
    tg = (-torch.exp(torch.tensor(A_log)) * torch.nn.functional.softplus(torch.tensor(a + dt_bias))).numpy()
    tb = torch.sigmoid(torch.tensor(b)).numpy()
    o1, h1 = oracle_lib.gdn_fwd(q, k, v, g, beta, None, [0, T], d ** -0.5)
    o2, h2 = oracle_lib.gdn_fwd(q, k, v, tg, tb, None, [0, T], d ** -0.5)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14) and np.allclose(h1, h2, rtol=1e-12, atol=1e-14)
