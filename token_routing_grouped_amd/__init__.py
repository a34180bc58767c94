"""MI355X (gfx950) MoE expert layer: GPU-resident routing, rowwise dispatch into
per-expert buffers, grouped SwiGLU GEMMs, combine, and the backward.

The compute lives in the HIP library ``libtrg_moe.so`` (C ABI: include/moe.h);
``_abi`` is its ctypes binding and ``layer`` sequences one layer step.  The
library is loaded on first use and a missing build raises ``MoeError``.
"""

from .configs import CONFIGS, LayerConfig  # noqa: F401

__all__ = ["CONFIGS", "LayerConfig"]
