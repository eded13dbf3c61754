"""Pins for the oracle's expert forward and frozen-base dgrad (no GPU)."""

import numpy as np
import torch

from oracle import route, moe_forward, moe_dgrad, quantize_blockwise, dequantize, silu
from oracle.fidelity import rel_fro, reconstruction_errors
from workloads import get_config, gen_x, gen_logits, gen_weights, gen_grad_y


def _small_problem(seed=0, T=12, E=4, H=64, I=64, k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    wgu = rng.standard_normal((E, 2 * I, H)) * 0.2
    wdn = rng.standard_normal((E, H, I)) * 0.2
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = route(logits, k)
    gy = rng.standard_normal((T, H))
    return x, idx, w, wgu, wdn, gy


def _gating_matrix(idx, w, E):
    T, k = idx.shape
    G = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            G[t, idx[t, j]] = w[t, j]
    return G


def test_single_expert_reduces_to_dense_swiglu():
    x, _, _, wgu, wdn, _ = _small_problem(E=1, k=1)
    T = x.shape[0]
    I = wdn.shape[2]
    idx = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1))
    y = moe_forward(x, idx, w, wgu, wdn)
    g = x @ wgu[0, :I].T
    u = x @ wgu[0, I:].T
    ref = (g / (1 + np.exp(-g)) * u) @ wdn[0].T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_forward_equals_dense_masked_brute_force():
    x, idx, w, wgu, wdn, _ = _small_problem()
    E, I = wgu.shape[0], wdn.shape[2]
    G = _gating_matrix(idx, w, E)
    ref = np.zeros_like(x)
    for e in range(E):  # every expert on every token, masked by G
        g = x @ wgu[e, :I].T
        u = x @ wgu[e, I:].T
        ref += G[:, e : e + 1] * ((silu(g) * u) @ wdn[e].T)
    y = moe_forward(x, idx, w, wgu, wdn)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_dgrad_equals_explicit_jacobian():
    x, idx, w, wgu, wdn, gy = _small_problem(seed=3)
    E, I = wgu.shape[0], wdn.shape[2]
    G = _gating_matrix(idx, w, E)
    gx, gw = moe_dgrad(x, idx, w, wgu, wdn, gy)
    for t in range(x.shape[0]):
        J = np.zeros((x.shape[1], x.shape[1]))
        for e in range(E):
            g = wgu[e, :I] @ x[t]
            u = wgu[e, I:] @ x[t]
            s = 1 / (1 + np.exp(-g))
            dsilu = s * (1 + g * (1 - s))
            J += G[t, e] * wdn[e] @ (np.diag(u * dsilu) @ wgu[e, :I] + np.diag(g * s) @ wgu[e, I:])
        assert np.max(np.abs(J.T @ gy[t] - gx[t])) <= 1e-12 * max(1.0, np.max(np.abs(gx[t])))
        for j in range(idx.shape[1]):
            e = idx[t, j]
            g = wgu[e, :I] @ x[t]
            u = wgu[e, I:] @ x[t]
            o = wdn[e] @ (silu(g) * u)
            assert abs(gy[t] @ o - gw[t, j]) <= 1e-12 * max(1.0, abs(gw[t, j]))


def test_dgrad_central_finite_differences():
    x, idx, w, wgu, wdn, gy = _small_problem(seed=5, T=4, H=64, I=64)
    gx, gw = moe_dgrad(x, idx, w, wgu, wdn, gy)
    L = lambda xx, ww: float(np.sum(gy * moe_forward(xx, idx, ww, wgu, wdn)))
    eps = 1e-6
    rng = np.random.default_rng(0)
    for _ in range(12):
        t, h = rng.integers(0, x.shape[0]), rng.integers(0, x.shape[1])
        xp, xm = x.copy(), x.copy()
        xp[t, h] += eps
        xm[t, h] -= eps
        fd = (L(xp, w) - L(xm, w)) / (2 * eps)
        assert abs(fd - gx[t, h]) <= 1e-6 * max(1.0, abs(gx[t, h]))
    for t in range(x.shape[0]):
        for j in range(idx.shape[1]):
            wp, wm = w.copy(), w.copy()
            wp[t, j] += eps
            wm[t, j] -= eps
            fd = (L(x, wp) - L(x, wm)) / (2 * eps)
            assert abs(fd - gw[t, j]) <= 1e-6 * max(1.0, abs(gw[t, j]))


def test_dgrad_matches_torch_autograd_on_tiny_config():
    cfg = get_config("tiny")
    x = gen_x(cfg, 0).astype(np.float64)
    wgu = gen_weights(cfg, 0, "gate_up").astype(np.float64)
    wdn = gen_weights(cfg, 0, "down").astype(np.float64)
    idx, w = route(gen_logits(cfg, 0), cfg.k)
    gy = gen_grad_y(cfg, 0).astype(np.float64)
    gx, gw = moe_dgrad(x, idx, w, wgu, wdn, gy)

    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    Wgu, Wdn = torch.tensor(wgu), torch.tensor(wdn)
    I = cfg.I
    y = torch.zeros_like(xt)
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = int(idx[t, j])
            h = Wgu[e] @ xt[t]
            a = torch.nn.functional.silu(h[:I]) * h[I:]
            y = y.index_add(0, torch.tensor([t]), (wt[t, j] * (Wdn[e] @ a))[None])
    y.backward(torch.tensor(gy))
    assert torch.allclose(xt.grad, torch.tensor(gx), rtol=1e-10, atol=1e-12)
    assert torch.allclose(wt.grad, torch.tensor(gw), rtol=1e-10, atol=1e-12)
    yo = moe_forward(x, idx, w, wgu, wdn)
    assert np.allclose(y.detach().numpy(), yo, rtol=1e-10, atol=1e-12)


def test_fidelity_ordering_bf16_int8_fp8_nf4_fp4():
    """The support matrix's test-pinned ordering (0.4.0 README, storage modes):
    bf16 < int8 < fp8 < nf4 < fp4 reconstruction error (fp16 is not a lane)."""
    cfg = get_config("tiny")
    for w in (gen_weights(cfg, 0, "gate_up"), gen_weights(cfg, 0, "down")):
        r = reconstruction_errors(w)
        assert r["bf16"] < r["int8"] < r["fp8"] < r["nf4"] < r["fp4"], r
    # forward-output fidelity on the tiny layer
    x = gen_x(cfg, 0)
    wgu, wdn = gen_weights(cfg, 0, "gate_up"), gen_weights(cfg, 0, "down")
    idx, w = route(gen_logits(cfg, 0), cfg.k)
    y_ref = moe_forward(x, idx, w, wgu, wdn)
    errs = {}
    from oracle import bf16_rne_bits, bf16_bits_to_f32

    errs["bf16"] = rel_fro(
        y_ref,
        moe_forward(x, idx, w, bf16_bits_to_f32(bf16_rne_bits(wgu)), bf16_bits_to_f32(bf16_rne_bits(wdn))),
    )
    for kind in ("nf4", "fp4"):
        pg, ag = quantize_blockwise(wgu, kind)
        pd, ad = quantize_blockwise(wdn, kind)
        errs[kind] = rel_fro(
            y_ref,
            moe_forward(
                x, idx, w, dequantize(pg, ag, 2 * cfg.I, cfg.H, kind), dequantize(pd, ad, cfg.H, cfg.I, kind)
            ),
        )
    from oracle.quant import stored_weights

    for kind in ("int8", "fp8"):
        errs[kind] = rel_fro(y_ref, moe_forward(x, idx, w, stored_weights(wgu, kind), stored_weights(wdn, kind)))
    assert errs["bf16"] < errs["int8"] < errs["fp8"] < errs["nf4"] < errs["fp4"], errs


def test_fidelity_ordering_mixtral_shaped_rows():
    # a few rows of one Mixtral-shaped expert (in = 4096), same distribution
    cfg = get_config("mixtral")
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((1, 64, cfg.H)) * cfg.weight_std).astype(np.float32)
    r = reconstruction_errors(w)
    assert r["bf16"] < r["int8"] < r["fp8"] < r["nf4"] < r["fp4"], r


def test_zero_tokens():
    x = np.zeros((0, 64))
    idx = np.zeros((0, 2), np.int32)
    w = np.zeros((0, 2))
    wgu = np.zeros((2, 128, 64))
    wdn = np.zeros((2, 64, 64))
    assert moe_forward(x, idx, w, wgu, wdn).shape == (0, 64)
    gx, gw = moe_dgrad(x, idx, w, wgu, wdn, x)
    assert gx.shape == (0, 64) and gw.shape == (0, 2)


def _ungated_problem(seed=0, T=9, E=3, H=32, I=24, k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    wup = rng.standard_normal((E, I, H)) * 0.2
    wdn = rng.standard_normal((E, H, I)) * 0.2
    idx, w = route(rng.standard_normal((T, E)).astype(np.float32), k)
    return x, idx, w, wup, wdn, rng.standard_normal((T, H))


def test_ungated_forward_is_act_of_up_dense_brute_force():
    """has_gate=False: a = silu(W_up x); dense masked brute force over all experts."""
    x, idx, w, wup, wdn, _ = _ungated_problem()
    E = wup.shape[0]
    G = _gating_matrix(idx, w, E)
    ref = sum(G[:, e : e + 1] * (silu(x @ wup[e].T) @ wdn[e].T) for e in range(E))
    y = moe_forward(x, idx, w, wup, wdn)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_ungated_dgrad_matches_torch_autograd():
    x, idx, w, wup, wdn, gy = _ungated_problem(seed=1)
    E = wup.shape[0]
    G = _gating_matrix(idx, w, E)
    X = torch.tensor(x, requires_grad=True)
    Gt = torch.tensor(G, requires_grad=True)
    y = sum(Gt[:, e : e + 1] * (torch.nn.functional.silu(X @ torch.tensor(wup[e]).T)
                                 @ torch.tensor(wdn[e]).T) for e in range(E))
    (y * torch.tensor(gy)).sum().backward()
    gx, gw = moe_dgrad(x, idx, w, wup, wdn, gy)
    assert np.max(np.abs(gx - X.grad.numpy())) <= 1e-12 * np.max(np.abs(gx))
    gw_ref = np.take_along_axis(Gt.grad.numpy(), idx.astype(np.int64), axis=1)
    assert np.max(np.abs(gw - gw_ref)) <= 1e-12 * np.max(np.abs(gw))
