"""Layer shapes of the synthetic workloads.

Shapes only; no arithmetic of the method lives here.  The expert counts and
top-k of ``small``/``wide`` follow the 8 -> 128 expert, top-4 scaling benchmark
(Ai2 Olmo-core 3 announcement, intro section; Olmo-core 3 overview, "What it is
and why it matters"); the ``trillion`` layer takes the d_model 6144, 384
experts, top-8 shape of the EUROPA ~1T MoE (PyTorch on JUPITER article,
introduction).  Every value distribution is synthetic and seeded.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class LayerConfig:
    slug: str
    T: int            # tokens per step
    d: int            # model width
    E: int            # experts
    k: int            # experts per token
    h: int            # SwiGLU hidden width per expert
    dtype: str        # "f32" or "bf16": storage type of activations, weights, grads
    seed: int
    modes: tuple = ("router",)
    mx: bool = False  # MXFP8 grouped GEMMs
    # Backward schedule of the timed step: weight-gradient GEMMs on a second
    # stream next to the dgrad chain where that measured faster (bf16 small
    # -5% per step, MXFP8 wide -1%; bf16 wide about -1%, kept serial; trillion
    # +7% and MXFP8 small +1%, serial).
    overlap: bool = False
    x_std: float = 1.0
    w_std: float = 0.02
    dy_std: float = 1.0

    @property
    def R(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)

    def gemm_flops(self) -> int:
        """Algorithmic flops of the six grouped GEMMs of one fwd+bwd pass."""
        return 18 * self.R * self.d * self.h

    def router_flops(self) -> int:
        """Router logits (fwd) plus dWr and dx (bwd)."""
        return 6 * self.T * self.d * self.E


CONFIGS = {
    "tiny": LayerConfig("tiny", T=256, d=128, E=8, k=2, h=256, dtype="f32", seed=0),
    "small": LayerConfig("small", T=8192, d=2048, E=8, k=4, h=1024, dtype="bf16", seed=1, overlap=True),
    "wide": LayerConfig("wide", T=16384, d=2048, E=128, k=4, h=1024, dtype="bf16", seed=2,
                        modes=("router", "uniform", "zipf"), overlap=True),
    "mxfp8": LayerConfig("mxfp8", T=16384, d=2048, E=128, k=4, h=1024, dtype="bf16", seed=2,
                         modes=("router", "uniform"), mx=True, overlap=True),
    "mxfp8_small": LayerConfig("mxfp8_small", T=8192, d=2048, E=8, k=4, h=1024, dtype="bf16",
                               seed=1, mx=True, overlap=True),
    "trillion": LayerConfig("trillion", T=4096, d=6144, E=384, k=8, h=2048, dtype="bf16", seed=4,
                            modes=("uniform",)),
}


def get(slug: str) -> LayerConfig:
    return CONFIGS[slug]
