"""Per-expert LoRA over the frozen routed expert MLP: forward, dgrad and the
adapter weight gradients (oracle, float64).

Sources: the experts4bit-qlora 0.4.0 README (the "Quickstart" example wraps
a frozen 4-bit expert stack as ``ExpertsLoRA(base, r=8, alpha=16)``, only the
adapters train) and the bitsandbytes pull request #1965 (frozen-base bullet:
the frozen forward is differentiable in the input, so it serves as the base
of a QLoRA setup). The adapter module itself is not printed on the pages.

Reading (the plainest one the pages support): every expert e carries a
low-rank adapter on each of its two projections, in the usual LoRA form
``W x + (alpha / r) B (A x)`` with ``A [r, in]`` and ``B [out, r]``:

* gate_up: ``A_gu [E, r, H]``, ``B_gu [E, 2I, r]`` (rows of B follow the
  fused gate | up rows of the base);
* down:    ``A_dn [E, r, I]``, ``B_dn [E, H, r]``.

Per routed pair (t, j) of expert e, with s = alpha / r:

    h  = W_gu x_t + s B_gu (A_gu x_t);  g = h[:I];  u = h[I:]
    a  = silu(g) * u
    o  = W_dn a   + s B_dn (A_dn a)
    y_t += w[t, j] * o

The backward holds the routing fixed and treats W as frozen; with
G_o = w[t, j] grad_y_t:

    grad_w[t, j] = grad_y_t . o
    grad_a  = W_dn^T G_o + s A_dn^T (B_dn^T G_o)
    dB_dn  += s G_o (A_dn a)^T          dA_dn += s (B_dn^T G_o) a^T
    dg, du from grad_a through act(gate) * up (as in the base dgrad)
    grad_h  = [dg; du]
    grad_x_t += W_gu^T grad_h + s A_gu^T (B_gu^T grad_h)
    dB_gu  += s grad_h (A_gu x_t)^T     dA_gu += s (B_gu^T grad_h) x_t^T

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

import numpy as np

from .moe import _check_moe, _pairs_by_expert, _sigmoid, silu


def _check_lora(w_gu, w_dn, A_gu, B_gu, A_dn, B_dn):
    E, twoI, H = w_gu.shape
    I = twoI // 2
    if w_dn.shape[2] != I:
        raise ValueError("LoRA adapters are defined here for gated (SwiGLU) layers")
    A_gu, B_gu, A_dn, B_dn = (np.asarray(m, dtype=np.float64) for m in (A_gu, B_gu, A_dn, B_dn))
    r = A_gu.shape[1]
    if A_gu.shape != (E, r, H) or B_gu.shape != (E, twoI, r):
        raise ValueError("gate_up adapters must be A [E, r, H], B [E, 2I, r]")
    if A_dn.shape != (E, r, I) or B_dn.shape != (E, H, r):
        raise ValueError("down adapters must be A [E, r, I], B [E, H, r]")
    return A_gu, B_gu, A_dn, B_dn, r


def lora_forward(x, idx, w, w_gu, w_dn, A_gu, B_gu, A_dn, B_dn, alpha):
    """y [T, H] (fp64) of the routed SwiGLU MLP with per-expert LoRA adapters."""
    x, idx, w, E, H, I = _check_moe(x, idx, w, w_gu, w_dn)
    A_gu, B_gu, A_dn, B_dn, r = _check_lora(w_gu, w_dn, A_gu, B_gu, A_dn, B_dn)
    s = float(alpha) / r
    T, k = idx.shape
    y = np.zeros((T, H), dtype=np.float64)
    for e, t, j in _pairs_by_expert(idx, E):
        xt = x[t]
        h = xt @ np.asarray(w_gu[e], dtype=np.float64).T + s * (xt @ A_gu[e].T) @ B_gu[e].T
        g, u = h[:, :I], h[:, I:]
        a = silu(g) * u
        o = a @ np.asarray(w_dn[e], dtype=np.float64).T + s * (a @ A_dn[e].T) @ B_dn[e].T
        np.add.at(y, t, w[t, j][:, None] * o)
    return y


def lora_backward(x, idx, w, w_gu, w_dn, A_gu, B_gu, A_dn, B_dn, alpha, grad_y):
    """Gradients of sum(grad_y * y) with the routing indices held fixed.

    Returns ``(grad_x [T, H], grad_w [T, k], dA_gu, dB_gu, dA_dn, dB_dn)`` in
    fp64; the adapter gradients have the adapters' shapes.
    """
    x, idx, w, E, H, I = _check_moe(x, idx, w, w_gu, w_dn)
    A_gu, B_gu, A_dn, B_dn, r = _check_lora(w_gu, w_dn, A_gu, B_gu, A_dn, B_dn)
    gy = np.asarray(grad_y, dtype=np.float64)
    if gy.shape != x.shape:
        raise ValueError("grad_y must be [T, H]")
    s = float(alpha) / r
    T, k = idx.shape
    grad_x = np.zeros((T, H), dtype=np.float64)
    grad_w = np.zeros((T, k), dtype=np.float64)
    dA_gu, dB_gu = np.zeros_like(A_gu), np.zeros_like(B_gu)
    dA_dn, dB_dn = np.zeros_like(A_dn), np.zeros_like(B_dn)
    for e, t, j in _pairs_by_expert(idx, E):
        wgu = np.asarray(w_gu[e], dtype=np.float64)
        wdn = np.asarray(w_dn[e], dtype=np.float64)
        xt = x[t]
        xa = xt @ A_gu[e].T                          # [n, r]
        h = xt @ wgu.T + s * xa @ B_gu[e].T
        g, u = h[:, :I], h[:, I:]
        a = silu(g) * u
        aa = a @ A_dn[e].T                           # [n, r]
        o = a @ wdn.T + s * aa @ B_dn[e].T
        grad_w[t, j] = np.sum(gy[t] * o, axis=1)
        Go = w[t, j][:, None] * gy[t]                # [n, H]
        gb = Go @ B_dn[e]                            # [n, r]
        grad_a = Go @ wdn + s * gb @ A_dn[e]
        dB_dn[e] += s * Go.T @ aa
        dA_dn[e] += s * gb.T @ a
        sg = _sigmoid(g)
        dg = grad_a * u * sg * (1.0 + g * (1.0 - sg))
        du = grad_a * g * sg
        gh = np.concatenate([dg, du], axis=1)        # [n, 2I]
        hb = gh @ B_gu[e]                            # [n, r]
        np.add.at(grad_x, t, gh @ wgu + s * hb @ A_gu[e])
        dB_gu[e] += s * gh.T @ xa
        dA_gu[e] += s * hb.T @ xt
    return grad_x, grad_w, dA_gu, dB_gu, dA_dn, dB_dn
