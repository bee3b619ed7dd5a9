"""Plain CPU oracle for one GPU's share of the fused MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library; both sides receive the same seeded
inputs from ``mixture_experts_layer_layout_amd.synth`` and nothing else.

Source of the method: the news page "Cursor's MoK achieves 2.37x performance
boost on NVIDIA GB300 NVL72" (KuCoin news flash, published in Urdu, Bengali and
Thai translations; cited below as "MoK flash" with its article section:
§01 "the communication tax of MoE", §02 "how to compute while sending tokens",
§03 "a highly specialised execution package").

Modules
  moe    -- routing, layout, gather, SwiGLU experts, combine, backward (fp64)
  mxfp8  -- OCP MX E4M3 element codec and E8M0 block scales (fp64)
"""
from . import moe, mxfp8  # noqa: F401
