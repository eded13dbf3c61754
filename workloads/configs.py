"""The layer shapes the pages' workloads run on (synthetic stand-ins).

The pages measure on real OLMoE-1B-7B, Qwen3-30B-A3B and Mixtral-class
checkpoints; none are available here, so each is replaced by one synthetic
MoE layer of the same expert shape with random weights and routing.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class MoEConfig:
    name: str
    E: int
    H: int
    I: int
    k: int
    T: int
    routing: str  # "normal" | "uniform" | "zipf"
    zipf_s: float = 1.0
    codebooks: tuple = ("nf4",)
    dgrad: bool = True
    weight_std: float = 0.02
    gated: bool = True  # False: has_gate=False, a plain up projection [E, I, H]
    note: str = ""

    @property
    def P(self):
        return self.T * self.k

    def with_T(self, T):
        d = dict(self.__dict__)
        d["T"] = T
        d["name"] = f"{self.name}_t{T}"
        return MoEConfig(**d)

    def fwd_flops(self):
        """Algorithmic flops of the forward GEMMs: 6*P*H*I."""
        return 6 * self.P * self.H * self.I

    def layer_bytes(self):
        """Packed codes + fp32 absmax of both stacks for the whole layer."""
        n = self.E * (2 * self.I * self.H + self.H * self.I)
        return n // 2 + 4 * (n // 64)


CONFIGS = {
    "tiny": MoEConfig(
        "tiny", E=8, H=256, I=128, k=2, T=64, routing="normal",
        note="tiny MoE layer, seed 0",
    ),
    "olmoe": MoEConfig(
        "olmoe", E=64, H=2048, I=1024, k=8, T=4096, routing="uniform",
        note="OLMoE-1B-7B-shaped layer, 4x1024-token training microbatch",
    ),
    "qwen3_decode": MoEConfig(
        "qwen3_decode", E=128, H=2048, I=768, k=8, T=1, routing="zipf",
        dgrad=False, note="Qwen3-30B-A3B-shaped decode layer, T in {1, 8}",
    ),
    "qwen3_prefill": MoEConfig(
        "qwen3_prefill", E=128, H=2048, I=768, k=8, T=16384, routing="zipf",
        note="Qwen3-30B-A3B-shaped prefill/training layer",
    ),
    "mixtral": MoEConfig(
        "mixtral", E=8, H=4096, I=14336, k=2, T=8192, routing="uniform",
        codebooks=("fp4", "nf4"), note="Mixtral-8x7B-shaped layer",
    ),
}


def get_config(name, T=None):
    cfg = CONFIGS[name]
    return cfg.with_T(T) if T is not None and T != cfg.T else cfg
