"""Pins for the oracle's per-expert LoRA forward / backward (no GPU).

The pins do not re-type the oracle's formulas: the forward and the input
gradient are checked against the base oracle on merged weights
W' = W + (alpha / r) B A (a closed form of the low-rank update), the
adapter gradients against central finite differences and against torch
float64 autograd of a dense, all-experts-masked formulation.
"""

import numpy as np
import torch

from oracle import route, moe_forward, moe_dgrad, lora_forward, lora_backward


def _problem(seed=0, T=10, E=4, H=64, I=64, k=2, r=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    wgu = rng.standard_normal((E, 2 * I, H)) * 0.1
    wdn = rng.standard_normal((E, H, I)) * 0.1
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = route(lg, k)
    A_gu = rng.standard_normal((E, r, H)) * 0.1
    B_gu = rng.standard_normal((E, 2 * I, r)) * 0.1
    A_dn = rng.standard_normal((E, r, I)) * 0.1
    B_dn = rng.standard_normal((E, H, r)) * 0.1
    gy = rng.standard_normal((T, H))
    return x, idx, w, wgu, wdn, (A_gu, B_gu, A_dn, B_dn), gy


def _merged(wgu, wdn, ad, alpha):
    A_gu, B_gu, A_dn, B_dn = ad
    s = alpha / A_gu.shape[1]
    return wgu + s * B_gu @ A_gu, wdn + s * B_dn @ A_dn


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def test_forward_equals_merged_weights():
    x, idx, w, wgu, wdn, ad, _ = _problem()
    y = lora_forward(x, idx, w, wgu, wdn, *ad, 16.0)
    mg, md = _merged(wgu, wdn, ad, 16.0)
    assert _rel(y, moe_forward(x, idx, w, mg, md)) <= 1e-12


def test_zero_B_is_the_base():
    x, idx, w, wgu, wdn, (A_gu, B_gu, A_dn, B_dn), gy = _problem(seed=1)
    z = (A_gu, np.zeros_like(B_gu), A_dn, np.zeros_like(B_dn))
    assert np.array_equal(lora_forward(x, idx, w, wgu, wdn, *z, 16.0), moe_forward(x, idx, w, wgu, wdn))
    gx, gw, dA_gu, dB_gu, dA_dn, dB_dn = lora_backward(x, idx, w, wgu, wdn, *z, 16.0, gy)
    bx, bw = moe_dgrad(x, idx, w, wgu, wdn, gy)
    assert _rel(gx, bx) <= 1e-12 and _rel(gw, bw) <= 1e-12
    # with B = 0 nothing reaches A; B still gets a gradient
    assert not dA_gu.any() and not dA_dn.any()
    assert np.abs(dB_gu).max() > 0 and np.abs(dB_dn).max() > 0


def test_input_gradient_equals_merged_dgrad():
    x, idx, w, wgu, wdn, ad, gy = _problem(seed=2, r=4)
    gx, gw, *_ = lora_backward(x, idx, w, wgu, wdn, *ad, 8.0, gy)
    mg, md = _merged(wgu, wdn, ad, 8.0)
    bx, bw = moe_dgrad(x, idx, w, mg, md, gy)
    assert _rel(gx, bx) <= 1e-11 and _rel(gw, bw) <= 1e-11


def test_adapter_gradients_finite_differences():
    x, idx, w, wgu, wdn, ad, gy = _problem(seed=3, T=6, E=3, H=16, I=16, r=3)
    alpha = 6.0
    grads = lora_backward(x, idx, w, wgu, wdn, *ad, alpha, gy)[2:]
    rng = np.random.default_rng(7)
    eps = 1e-6
    for m, (M, G) in enumerate(zip(ad, grads)):
        for _ in range(6):
            pos = tuple(rng.integers(0, n) for n in M.shape)
            Mp, Mm = M.copy(), M.copy()
            Mp[pos] += eps
            Mm[pos] -= eps
            args_p = list(ad)
            args_m = list(ad)
            args_p[m], args_m[m] = Mp, Mm
            fp = np.sum(gy * lora_forward(x, idx, w, wgu, wdn, *args_p, alpha))
            fm = np.sum(gy * lora_forward(x, idx, w, wgu, wdn, *args_m, alpha))
            fd = (fp - fm) / (2 * eps)
            assert abs(fd - G[pos]) <= 1e-6 * max(1.0, abs(fd)), (m, pos, fd, G[pos])


def test_routing_weight_gradient_finite_differences():
    x, idx, w, wgu, wdn, ad, gy = _problem(seed=4, T=5, E=3, H=16, I=16, r=2)
    gw = lora_backward(x, idx, w, wgu, wdn, *ad, 4.0, gy)[1]
    eps = 1e-6
    for t in range(x.shape[0]):
        for j in range(idx.shape[1]):
            wp, wm = w.copy(), w.copy()
            wp[t, j] += eps
            wm[t, j] -= eps
            fd = (np.sum(gy * lora_forward(x, idx, wp, wgu, wdn, *ad, 4.0))
                  - np.sum(gy * lora_forward(x, idx, wm, wgu, wdn, *ad, 4.0))) / (2 * eps)
            assert abs(fd - gw[t, j]) <= 1e-6 * max(1.0, abs(fd))


def test_backward_matches_torch_autograd_dense():
    """Dense masked formulation (every expert on every token) under fp64 autograd."""
    x, idx, w, wgu, wdn, ad, gy = _problem(seed=5, T=7, E=3, H=24, I=16, r=5)
    alpha = 10.0
    s = alpha / 5
    E, I = wgu.shape[0], wdn.shape[2]
    G = np.zeros((x.shape[0], E))
    for t in range(x.shape[0]):
        for j in range(idx.shape[1]):
            G[t, idx[t, j]] = w[t, j]
    tt = lambda a, g=False: torch.tensor(a, dtype=torch.float64, requires_grad=g)
    X = tt(x, True)
    Gt = tt(G, True)
    Ag, Bg, Ad, Bd = (tt(m, True) for m in ad)
    Wg, Wd = tt(wgu), tt(wdn)
    y = torch.zeros_like(X)
    for e in range(E):
        h = X @ Wg[e].T + s * (X @ Ag[e].T) @ Bg[e].T
        a = torch.nn.functional.silu(h[:, :I]) * h[:, I:]
        o = a @ Wd[e].T + s * (a @ Ad[e].T) @ Bd[e].T
        y = y + Gt[:, e : e + 1] * o
    (y * tt(gy)).sum().backward()
    gx, gw, dA_gu, dB_gu, dA_dn, dB_dn = lora_backward(x, idx, w, wgu, wdn, *ad, alpha, gy)
    assert _rel(gx, X.grad.numpy()) <= 1e-12
    gw_ref = np.take_along_axis(Gt.grad.numpy(), idx.astype(np.int64), axis=1)
    assert _rel(gw, gw_ref) <= 1e-12
    for got, ref in ((dA_gu, Ag), (dB_gu, Bg), (dA_dn, Ad), (dB_dn, Bd)):
        assert _rel(got, ref.grad.numpy()) <= 1e-12
