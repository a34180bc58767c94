"""Seeded synthetic inputs, shared by the oracle tests, the GPU tests and the bench.

This module holds none of the layer's arithmetic: it draws random numbers,
rounds storage to bfloat16, and draws forced expert choices.  Every tensor has
its own stream keyed by ``(seed, tensor id, expert)`` so one expert's weights
can be regenerated on its own.

Value distributions: x ~ N(0, 1), router and expert weights ~ N(0, 0.02^2),
upstream gradient ~ N(0, 1).  Identical values are used for every timed
repetition, since kernel time depends on the values and not only on the shapes
(Olmo-core 3 overview, "Empirical findings beyond raw speed").
"""

from __future__ import annotations

import numpy as np

TENSOR_IDS = {"x": 0, "wr": 1, "w1": 2, "w3": 3, "w2": 4, "dy": 5, "route": 6}


def rng(seed: int, name: str, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([seed, TENSOR_IDS[name], expert])))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def normal(seed: int, name: str, shape, std: float, expert: int = 0) -> np.ndarray:
    return (rng(seed, name, expert).standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(a) if dtype == "bf16" else a.astype(np.float32)


def layer_inputs(cfg, T: int | None = None, experts=None) -> dict:
    """Host (float32) inputs for one layer step; bf16 configs are pre-rounded to bf16.

    ``T`` overrides the token count (the first T rows of the full stream).
    ``experts`` restricts the weight bank to those experts (others absent).
    """
    T = cfg.T if T is None else T
    s = cfg.seed
    out = {
        "x": _store(normal(s, "x", (cfg.T, cfg.d), cfg.x_std)[:T], cfg.dtype),
        "wr": _store(normal(s, "wr", (cfg.E, cfg.d), cfg.w_std), cfg.dtype),
        "dy": _store(normal(s, "dy", (cfg.T, cfg.d), cfg.dy_std)[:T], cfg.dtype),
    }
    ex = range(cfg.E) if experts is None else experts
    out["w1"] = np.stack([_store(normal(s, "w1", (cfg.h, cfg.d), cfg.w_std, e), cfg.dtype) for e in ex])
    out["w3"] = np.stack([_store(normal(s, "w3", (cfg.h, cfg.d), cfg.w_std, e), cfg.dtype) for e in ex])
    out["w2"] = np.stack([_store(normal(s, "w2", (cfg.d, cfg.h), cfg.w_std, e), cfg.dtype) for e in ex])
    return out


# Expert weight banks above this many fp32 bytes are drawn on the device.
HOST_WEIGHT_BYTES = 8 << 30


def device_inputs(cfg, dev, log=None) -> tuple:
    """The step's inputs as device tensors of the config's dtype, as timed.

    Weight banks up to HOST_WEIGHT_BYTES (fp32) come from ``layer_inputs``;
    larger ones (the trillion shape's are 58 GB in fp32) are drawn from a
    seeded device generator with the same distribution, one expert at a time
    (x, wr and dy still come from the host streams).  Returns (tensors,
    where the weights were drawn: "host" or "device").
    """
    import torch

    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    wbytes = 3 * cfg.E * cfg.h * cfg.d * 4
    if wbytes <= HOST_WEIGHT_BYTES:
        inp = layer_inputs(cfg)
        return {n: torch.from_numpy(v).to(dev).to(dt) for n, v in inp.items()}, "host"
    inp = layer_inputs(cfg, experts=[0])
    t = {n: torch.from_numpy(v).to(dev).to(dt) for n, v in inp.items() if n in ("x", "wr", "dy")}
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + cfg.seed)
    for n, shape in (("w1", (cfg.E, cfg.h, cfg.d)), ("w3", (cfg.E, cfg.h, cfg.d)), ("w2", (cfg.E, cfg.d, cfg.h))):
        w = torch.empty(shape, device=dev, dtype=dt)
        for e in range(cfg.E):  # one expert at a time: no fp32 copy of a whole bank
            w[e] = (torch.randn(shape[1:], device=dev, generator=gen) * cfg.w_std).to(dt)
        t[n] = w
        if log is not None:
            log(f"{n} generated on the device")
    return t, "device"


def expert_weights(cfg, e: int) -> tuple:
    s = cfg.seed
    return (_store(normal(s, "w1", (cfg.h, cfg.d), cfg.w_std, e), cfg.dtype),
            _store(normal(s, "w3", (cfg.h, cfg.d), cfg.w_std, e), cfg.dtype),
            _store(normal(s, "w2", (cfg.d, cfg.h), cfg.w_std, e), cfg.dtype))


def forced_routing(mode: str, T: int, E: int, k: int, seed: int, zipf_s: float = 1.1) -> np.ndarray:
    """k distinct experts per token, drawn on the host.

    ``uniform``: every k-subset equally likely (random-routing stress mode of the
    trillion-scale runs, Olmo-core 3 overview, "Demonstrated scale").
    ``zipf``: sequential draws without replacement with P(e) proportional to
    (e+1)^-s, done as Gumbel-top-k; expert 0 is the hottest.
    """
    g = rng(seed, "route", {"uniform": 1, "zipf": 2}[mode])
    gumbel = -np.log(-np.log(g.random((T, E), dtype=np.float64)))
    if mode == "uniform":
        keys = gumbel
    elif mode == "zipf":
        keys = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))[None, :] + gumbel
    else:
        raise ValueError(mode)
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return np.ascontiguousarray(idx.astype(np.int32))
