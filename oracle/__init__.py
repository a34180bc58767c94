"""CPU oracle of the MoE expert layer hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The product path
(the HIP library and its Python binding) never calls it, and the two share no
code: this package imports nothing from ``token_routing_grouped_amd``.

Sources (pages of the reference, cited by title and section):
  [OC3]  "Olmo-core 3 open mixture-of-experts training infrastructure"
         (agentlenshq.com, Japanese) -- sections "Routing and compute
         optimisation", "Precision optimisation with MXFP8", "What Olmo-core 3
         is and why it matters", "Empirical findings beyond raw speed".
  [AI2]  "Ai2 opened up the Olmo-core 3 MoE training system" (aihirek.info,
         Hungarian) -- sections "New distribution system", "Trillion-parameter
         tests, open access".
  [TH]   "Introducing Olmo-core 3" (ai4bro.com, Thai) -- section "Scaling and
         optimising MoE training".
  [EU]   "PyTorch trains a ~1T-parameter MoE on a European public
         supercomputer" (cctest.ai, Japanese) -- introduction (layer shape).

The pages describe the method in prose only: routed token rows are written
straight into per-expert input buffers, routing metadata stays on the GPU, the
experts' many small matrix products run as one grouped GEMM, and an MXFP8
option cuts compute and data movement.  They fix neither the router function,
the expert FFN, the MX encoding nor the backward; the readings taken for those
are stated at each function.

Modules:
  moe_ref  -- routing, dispatch, SwiGLU experts, combine, and the backward.
  mx_ref   -- MXFP8 (OCP E4M3FN elements, E8M0 block scales) quantisation.
  sampled_ref -- single tokens' and single experts' outputs of the full-size
              layer (the same definitions, for sampled parity at full size).

Pins: every function here is checked against something other than itself in
``tests/test_oracle_*.py`` (closed forms, brute force, finite differences,
hand-derived vectors in ``tests/golden/``).  The MXFP8 layer (QDQ oracle)
is pinned GEMM by GEMM: where every operand is already on the MX grid along
the axis its GEMM blocks it on, and off the grid along the other axis, its
result must equal the float oracle's exactly (tests/test_oracle_mx_layer.py,
which also checks that quantising any operand along the wrong axis, over
whole-R instead of per-expert blocks, or from another MX copy, fails a pin).
"""
