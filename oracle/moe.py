"""Routed SwiGLU expert MLP: routing, permutation, forward and dgrad (oracle).

Notation: E experts, H hidden, I intermediate, k experts per token, T tokens,
P = T*k routed (token, slot) pairs with flat pair id p = t*k + j. Stacks are
row-major ``[E, out, in]``: gate_up ``[E, 2I, H]`` (rows 0..I-1 gate,
I..2I-1 up) and down ``[E, H, I]``. An ungated layer (``has_gate=False`` in
``Experts4bit.__init__``: the projection is a plain up projection of size I)
has a ``[E, I, H]`` first stack and ``a = act(up)``; the stack shapes select
the variant.

Sources:

* forward -- experts4bit-qlora 0.1.0 sdist, ``_vendor/experts.py``,
  ``Experts4bit.forward``: for each expert hit by the routing, gather its
  tokens, project with gate_up, split the projection into gate (first half)
  and up (second half), apply act(gate) * up with act = SiLU, project with
  down, scale each row by its routing weight and add into an fp32
  accumulator indexed by token.
* dgrad -- bitsandbytes PR #1965 ("What this adds", the recompute-in-backward
  bullet, and the frozen-base bullet): the backward of every frozen expert
  projection forms grad_output @ W from a re-dequantized W; the packed base
  receives no gradient; the forward is differentiable with respect to the
  input activations.
* route -- the router lives outside the module (``Experts4bit.forward``
  takes ``top_k_index`` and ``top_k_weights``); the workloads fix softmax ->
  top-k -> renormalize. Reading: select the k largest raw logits (ties to the
  lower expert id) and softmax over the k selected logits, which equals
  softmax -> top-k -> renormalize in exact arithmetic and keeps the selection
  an exact fp32 comparison.
* permute -- the per-expert grouping that ``Experts4bit.forward`` builds with
  ``one_hot`` / ``where`` is written as a stable counting sort of pair ids
  by expert.

All arithmetic here is float64 on whatever (fp32 / bf16-valued) inputs are
passed in; weights are the fp32 dequantized stack promoted to fp64.
"""

import numpy as np


def _sigmoid(g):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def silu(g):
    """x * sigmoid(x) in fp64."""
    g = np.asarray(g, dtype=np.float64)
    return g * _sigmoid(g)


def route(logits, k):
    """Top-k routing on fp32 logits ``[T, E]``.

    Returns ``(idx int32 [T, k], w float64 [T, k])``: idx holds the k largest
    logits in descending order (equal logits: lower expert id first), w the
    softmax over the selected logits.
    """
    lg = np.asarray(logits, dtype=np.float32)
    if lg.ndim != 2:
        raise ValueError("logits must be [T, E]")
    T, E = lg.shape
    if not (1 <= k <= E):
        raise ValueError("top_k must be in [1, E]")
    if not np.all(np.isfinite(lg)):
        raise ValueError("logits must be finite")
    # stable sort on the negated value keeps ascending expert id among ties
    order = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(lg, order, axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w


def permute(idx, E):
    """Stable counting sort of flat pair ids by expert.

    Returns ``(counts [E], offsets [E+1], sorted_pair [P], pos_of_pair [P])``
    (int64): segment e of ``sorted_pair`` is ``offsets[e]:offsets[e+1]`` and
    holds, in ascending order, every p with ``idx.flat[p] == e``;
    ``pos_of_pair`` is its inverse permutation.
    """
    flat = np.asarray(idx).reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert index out of range")
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    sorted_pair = np.argsort(flat, kind="stable").astype(np.int64)
    pos_of_pair = np.empty_like(sorted_pair)
    pos_of_pair[sorted_pair] = np.arange(flat.size, dtype=np.int64)
    return counts, offsets, sorted_pair, pos_of_pair


def _pairs_by_expert(idx, E):
    T, k = idx.shape
    counts, offsets, sorted_pair, _ = permute(idx, E)
    for e in range(E):
        ps = sorted_pair[offsets[e] : offsets[e + 1]]
        if ps.size:
            yield e, ps // k, ps % k


def _check_moe(x, idx, w, w_gu, w_dn):
    x = np.asarray(x, dtype=np.float64)
    idx = np.asarray(idx)
    w = np.asarray(w, dtype=np.float64)
    E, gu_out, H = w_gu.shape
    if w_dn.shape[:2] != (E, H):
        raise ValueError("down must be [E, H, I]")
    I = w_dn.shape[2]
    if gu_out not in (I, 2 * I):
        raise ValueError("gate_up must have 2I (gated) or I (ungated) rows")
    if x.ndim != 2 or x.shape[1] != H:
        raise ValueError("x must be [T, H]")
    if idx.shape != w.shape or idx.shape[0] != x.shape[0]:
        raise ValueError("routing must be [T, k]")
    return x, idx, w, E, H, I


def expert_activations(x_rows, w_gu_e, I):
    """gate, up and a = silu(gate) * up for the rows of one expert (fp64).

    Ungated stack (I rows): returns (h, None, silu(h)) -- the projection is a
    plain up projection and the activation applies to it directly
    (``Experts4bit.forward``, the ``has_gate`` branch).
    """
    h = x_rows @ np.asarray(w_gu_e, dtype=np.float64).T
    if h.shape[1] == I:
        return h, None, silu(h)
    g, u = h[:, :I], h[:, I:]
    return g, u, silu(g) * u


def moe_forward(x, idx, w, w_gu, w_dn, return_pairs=False):
    """y[t] = sum_j w[t,j] * W_dn[e] (silu(W_g[e] x_t) * (W_u[e] x_t)), e = idx[t,j].

    ``w_gu``/``w_dn`` are the dequantized fp32 stacks (promoted to fp64 here).
    With ``return_pairs`` also returns per-pair g, u, a, o keyed by flat p.
    """
    x, idx, w, E, H, I = _check_moe(x, idx, w, w_gu, w_dn)
    T, k = idx.shape
    y = np.zeros((T, H), dtype=np.float64)
    pairs = {}
    for e, t, j in _pairs_by_expert(idx, E):
        g, u, a = expert_activations(x[t], w_gu[e], I)
        o = a @ np.asarray(w_dn[e], dtype=np.float64).T
        np.add.at(y, t, w[t, j][:, None] * o)
        if return_pairs:
            pairs[e] = dict(p=t * k + j, g=g, u=u, a=a, o=o)
    if return_pairs:
        return y, pairs
    return y


def moe_dgrad(x, idx, w, w_gu, w_dn, grad_y):
    """Input gradient of the routed expert MLP with frozen weights.

    Returns ``(grad_x [T, H], grad_w [T, k])`` in fp64, with routing held
    fixed: per pair (t, j) of expert e,

    * G2 = W_dn[e]^T grad_y[t]            (the down projection's dgrad)
    * grad_w[t, j] = G2 . a
    * grad_a = w[t, j] * G2
    * dg = grad_a * u * s * (1 + g * (1 - s)),  s = sigmoid(g)
    * du = grad_a * g * s
    * grad_x[t] += W_gu[e]^T [dg; du]     (the gate_up projection's dgrad)

    Ungated: dh = grad_a * s * (1 + h * (1 - s)) and grad_x[t] += W_up^T dh.
    """
    x, idx, w, E, H, I = _check_moe(x, idx, w, w_gu, w_dn)
    gy = np.asarray(grad_y, dtype=np.float64)
    if gy.shape != x.shape:
        raise ValueError("grad_y must be [T, H]")
    T, k = idx.shape
    grad_x = np.zeros((T, H), dtype=np.float64)
    grad_w = np.zeros((T, k), dtype=np.float64)
    for e, t, j in _pairs_by_expert(idx, E):
        wgu = np.asarray(w_gu[e], dtype=np.float64)
        g, u, a = expert_activations(x[t], wgu, I)
        G2 = gy[t] @ np.asarray(w_dn[e], dtype=np.float64)
        grad_w[t, j] = np.sum(G2 * a, axis=1)
        grad_a = w[t, j][:, None] * G2
        s = _sigmoid(g)
        if u is None:  # ungated: a = silu(h), d a / d h = s (1 + h (1 - s))
            gh = grad_a * s * (1.0 + g * (1.0 - s))
        else:
            dg = grad_a * u * s * (1.0 + g * (1.0 - s))
            du = grad_a * g * s
            gh = np.concatenate([dg, du], axis=1)
        np.add.at(grad_x, t, gh @ wgu)
    return grad_x, grad_w
