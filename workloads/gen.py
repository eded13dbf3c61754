"""Seeded generators (see the package docstring for the recipe)."""

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

# tensor ids of the independent streams
_X, _W_GU, _W_DN, _LOGITS, _GRAD_Y = 1, 2, 3, 4, 5
_A_GU, _B_GU, _A_DN, _B_DN = 6, 7, 8, 9


def _rng(seed, tid, sub=None):
    key = [int(seed), tid] if sub is None else [int(seed), tid, int(sub)]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def _bf16_values(a):
    """fp32 array holding the bf16 round-to-nearest-even of ``a`` (torch's conversion)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def to_bf16_tensor(a):
    """torch bfloat16 CPU tensor of an fp32 array whose values are bf16-representable."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    if not np.array_equal(t.to(torch.float32).numpy(), a):
        raise ValueError("array values are not bf16-representable")
    return t


def gen_x(cfg, seed):
    """Activations [T, H]: bf16-rounded N(0, 1), returned as fp32 values."""
    return _bf16_values(_rng(seed, _X).standard_normal((cfg.T, cfg.H), dtype=np.float32))


def gen_grad_y(cfg, seed):
    """Output gradient [T, H]: bf16-rounded N(0, 1), returned as fp32 values."""
    return _bf16_values(_rng(seed, _GRAD_Y).standard_normal((cfg.T, cfg.H), dtype=np.float32))


def gen_logits(cfg, seed):
    """Router logits [T, E], fp32."""
    r = _rng(seed, _LOGITS)
    if cfg.routing == "normal":
        return r.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if cfg.routing == "uniform":
        return r.random((cfg.T, cfg.E), dtype=np.float32)
    if cfg.routing == "zipf":
        g = r.gumbel(size=(cfg.T, cfg.E))
        return (-cfg.zipf_s * np.log(np.arange(1, cfg.E + 1, dtype=np.float64)) + g).astype(
            np.float32
        )
    raise ValueError(cfg.routing)


def gen_expert_weight(cfg, seed, which, e):
    """One expert's fp32 weight: ``which`` = "gate_up" -> [2I, H] ([I, H] ungated), "down" -> [H, I]."""
    if which == "gate_up":
        shape, tid = ((2 if cfg.gated else 1) * cfg.I, cfg.H), _W_GU
    elif which == "down":
        shape, tid = (cfg.H, cfg.I), _W_DN
    else:
        raise ValueError(which)
    w = _rng(seed, tid, e).standard_normal(shape, dtype=np.float32)
    w *= np.float32(cfg.weight_std)
    return w


def gen_weights(cfg, seed, which, experts=None, threads=None):
    """fp32 stack ``[len(experts), out, in]`` (all experts by default)."""
    experts = list(range(cfg.E)) if experts is None else list(experts)
    shape = ((2 if cfg.gated else 1) * cfg.I, cfg.H) if which == "gate_up" else (cfg.H, cfg.I)
    out = np.empty((len(experts),) + shape, dtype=np.float32)

    def fill(i):
        out[i] = gen_expert_weight(cfg, seed, which, experts[i])

    n = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(fill, range(len(experts))))
    return out


def gen_lora(cfg, seed, r):
    """Synthetic per-expert LoRA adapters (fp32, N(0, weight_std^2)), as
    ``(A_gu [E, r, H], B_gu [E, 2I, r], A_dn [E, r, I], B_dn [E, H, r])``."""
    shapes = ((_A_GU, (cfg.E, r, cfg.H)), (_B_GU, (cfg.E, 2 * cfg.I, r)),
              (_A_DN, (cfg.E, r, cfg.I)), (_B_DN, (cfg.E, cfg.H, r)))
    out = []
    for tid, shape in shapes:
        m = _rng(seed, tid, r).standard_normal(shape, dtype=np.float32)
        m *= np.float32(cfg.weight_std)
        out.append(m)
    return tuple(out)
