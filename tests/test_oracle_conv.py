"""Pins of the conv oracle (hyper-parallel ``_causal_conv1d_with_cp_halo``).

* numpy.convolve per channel with the flipped kernel (a library routine with
  the opposite orientation convention);
* torch.nn.functional.conv1d on the CPU with the module's left padding and
  the first T outputs kept (the page's unsplit path), and with the halo
  concatenated and padding 0 (the page's split path);
* splitting a sequence anywhere and passing the K-1 pre-conv tail as the
  halo reproduces the unsplit output;
* the reverse mode against central finite differences and the adjoint
  identity.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ref


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _inputs(rng, T, C, K, bias=True):
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, K)) / np.sqrt(K)
    b = rng.standard_normal(C) if bias else None
    return x, w, b


@pytest.mark.parametrize("K", [1, 2, 4])
def test_matches_numpy_convolve(K, oracle_lib):
    rng = np.random.default_rng(K)
    T, C = 37, 5
    x, w, b = _inputs(rng, T, C, K)
    y = oracle_lib.conv1d_silu(x, w, b, None, 0, [0, T])
    for c in range(C):
        z = np.convolve(x[:, c], w[c, ::-1])[:T] + b[c]
        np.testing.assert_allclose(y[:, c], _silu(z), rtol=1e-13, atol=1e-13)


def test_matches_torch_conv1d_unsplit_and_halo(oracle_lib):
    rng = np.random.default_rng(7)
    T, C, K = 29, 6, 4
    x, w, b = _inputs(rng, T, C, K)
    conv = dict(weight=torch.from_numpy(w)[:, None, :], bias=torch.from_numpy(b), groups=C)
    xt = torch.from_numpy(x).T[None]
    want = F.silu(F.conv1d(xt, padding=K - 1, **conv)[..., :T])[0].T.numpy()
    got = oracle_lib.conv1d_silu(x, w, b, None, 0, [0, T])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # the split path: halo concatenated in front, padding 0
    halo = rng.standard_normal((K - 1, C))
    xin = torch.cat([torch.from_numpy(halo), torch.from_numpy(x)], 0).T[None]
    want = F.silu(F.conv1d(xin, padding=0, **conv))[0].T.numpy()
    got = oracle_lib.conv1d_silu(x, w, b, halo, K - 1, [0, T])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_varlen_sequences_do_not_mix(oracle_lib):
    rng = np.random.default_rng(3)
    cu = [0, 5, 5, 17, 18, 30]
    T, C, K = cu[-1], 4, 4
    x, w, b = _inputs(rng, T, C, K)
    halo = rng.standard_normal((K - 1, C))
    y = oracle_lib.conv1d_silu(x, w, b, halo, 2, cu)
    for n in range(len(cu) - 1):
        s, e = cu[n], cu[n + 1]
        alone = oracle_lib.conv1d_silu(x[s:e], w, b, halo if n == 0 else None, 2 if n == 0 else 0,
                                       [0, e - s])
        np.testing.assert_array_equal(y[s:e], alone)
    np.testing.assert_allclose(y, ref.conv1d_silu(x, w, b, halo, 2, cu), rtol=1e-13, atol=1e-13)


def test_split_with_halo_equals_unsplit(oracle_lib):
    rng = np.random.default_rng(11)
    T, C, K = 23, 3, 4
    x, w, b = _inputs(rng, T, C, K)
    full = oracle_lib.conv1d_silu(x, w, b, None, 0, [0, T])
    for cut in range(1, T):
        halo = np.zeros((K - 1, C))
        nh = min(K - 1, cut)
        halo[K - 1 - nh:] = x[cut - nh:cut]
        # garbage in the rows that must be ignored
        halo[:K - 1 - nh] = 1e6
        right = oracle_lib.conv1d_silu(x[cut:], w, b, halo, nh, [0, T - cut])
        np.testing.assert_allclose(right, full[cut:], rtol=1e-13, atol=1e-13)


def test_backward_finite_differences(oracle_lib):
    rng = np.random.default_rng(5)
    cu = [0, 4, 9]
    T, C, K = 9, 3, 3
    x, w, b = _inputs(rng, T, C, K)
    halo = rng.standard_normal((K - 1, C))
    nh = 1
    dy = rng.standard_normal((T, C))
    dx, dw, db, dhalo = oracle_lib.conv1d_silu_bwd(x, w, b, halo, nh, cu, dy)

    def loss(x_, w_, b_, h_):
        return float((oracle_lib.conv1d_silu(x_, w_, b_, h_, nh, cu) * dy).sum())

    eps = 1e-6
    for name, arr, grad in (("x", x, dx), ("w", w, dw), ("b", b, db), ("halo", halo, dhalo)):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            args = {"x": x.copy(), "w": w.copy(), "b": b.copy(), "halo": halo.copy()}
            args[name][i] += eps
            lp = loss(args["x"], args["w"], args["b"], args["halo"])
            args[name][i] -= 2 * eps
            lm = loss(args["x"], args["w"], args["b"], args["halo"])
            num[i] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8, err_msg=name)
    # rows of the halo beyond n_halo get no gradient
    assert np.all(dhalo[:K - 1 - nh] == 0)


def test_backward_adjoint_identity(oracle_lib):
    # <dy, J dx> = <J^T dy, dx> with J the Jacobian w.r.t. x (linearised by
    # a tiny step); independent of how the reverse mode was written
    rng = np.random.default_rng(9)
    cu = [0, 6, 14]
    T, C, K = 14, 4, 4
    x, w, b = _inputs(rng, T, C, K)
    dy = rng.standard_normal((T, C))
    dxdir = rng.standard_normal((T, C))
    gx, _, _, _ = oracle_lib.conv1d_silu_bwd(x, w, b, None, 0, cu, dy)
    h = 1e-6
    jv = (oracle_lib.conv1d_silu(x + h * dxdir, w, b, None, 0, cu)
          - oracle_lib.conv1d_silu(x - h * dxdir, w, b, None, 0, cu)) / (2 * h)
    assert abs((dy * jv).sum() - (gx * dxdir).sum()) < 1e-7 * abs((gx * dxdir).sum()) + 1e-9
