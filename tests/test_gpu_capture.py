"""A whole layer step captured in a HIP graph and replayed.

Every library call only enqueues device work: routing metadata never goes to
the host, no call copies to the host, waits on the host or allocates
(Olmo-core 3 overview, "Routing and compute optimisation": routing metadata
stays on the GPU; the Thai announcement, "Scaling and optimising MoE
training": the CPU queues work without waiting for copies).  A step that did
any of that could not be captured.  Here one forward + backward is captured
with torch.cuda.graph after warm-up (one stream, and the two-stream backward),
then replayed three times with eager work between the replays that overwrites
every output, and each replay must reproduce the eager step bit for bit.
"""

import pytest
import torch

from token_routing_grouped_amd import configs, inputs

from helpers import say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
OUTS = ("logits", "topk_idx", "topk_w", "pos", "y", "dgate", "dx", "dwr", "dw1", "dw3", "dw2")

CASES = [
    ("bf16", dict()),
    ("bf16_two_stream", dict(overlap=True)),
    ("bf16_lean", dict(lean=True)),
    ("mxfp8", dict(mx=True)),
    ("mxfp8_two_stream", dict(mx=True, overlap=True)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_captured_step_replays_bit_identically(case):
    from token_routing_grouped_amd.layer import MoELayerGPU

    name, flags = case
    cfg = configs.get("wide").with_(T=512, E=16, d=512, h=256)
    say(f"graph capture {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} h={cfg.h} {flags}")
    inp = inputs.layer_inputs(cfg)
    t = {n: torch.from_numpy(v).to(DEV).to(torch.bfloat16) for n, v in inp.items()}
    args = (t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"])
    layer = MoELayerGPU(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, torch.bfloat16, DEV, **flags)

    layer.step(*args)
    torch.cuda.synchronize()
    eager = {n: getattr(layer, n).clone() for n in OUTS}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            layer.step(*args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.step(*args)
    torch.cuda.synchronize()

    for rep in range(3):
        for n in OUTS:  # eager work between replays: every output overwritten
            buf = getattr(layer, n)
            buf.fill_(float("nan") if buf.dtype.is_floating_point else -7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in OUTS:
            assert torch.equal(getattr(layer, n), eager[n]), f"replay {rep}: {n} differs from the eager step"
    say("  3 replays bit-identical to the eager step")
