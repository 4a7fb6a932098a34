"""Plain, slow, float64 CPU oracle of the MoE routing-align + grouped expert FFN path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from this package.  It shares no code with the HIP library
(``mixture_experts_routing_align_amd``) and imports nothing from it; the only
module both sides use is the seeded input generator ``workloads``, which holds
none of the path's arithmetic.

Sources (the web pages this path is defined by):

* nbxtensor 0.0.1 wheel page, ``moe_align.py`` - the device alignment: the
  module docstring (worst-case table size, device-only total, stable rank that
  reproduces the host sort) and the three stage kernels' docstrings;
* nbxtensor 0.0.1 wheel page, ``moe_decode_vec.py`` - SwiGLU epilogue
  ``silu(g) * u`` in fp32 and the fixed-order top-k reduction;
* metrale ``forward_nvfp4_grouped_decode.rs`` source page - the layer's step
  order (route, sort, gate+up+SiLU, down, blend) and row independence;
* metrale ``forward_nvfp4_grouped_decode.rs`` source page - the per-row router
  (BF16 softmax gate, router GEMV and per-row top-k softmax) that feeds the path;
* metrale ``fp8_moe_grouped.rs`` source page - the sort's outputs (sorted slot
  ids, expert offsets, ``token_to_perm``, ascending active experts and their
  count), the active-expert cap, the 1024-expert limit, the 128-wide FP8 scale
  blocks and the blend through ``token_to_perm``.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
values fixed by the pages or by mathematics (closed forms, brute force on tiny
inputs, library routines in special cases, hand-worked fixtures under
``tests/golden/``); no function is "parity unpinned".
"""

from .align import active_cap, align, max_total  # noqa: F401
from .ffn import (  # noqa: F401
    blend,
    dequant,
    expert_ffn,
    moe_layer,
    shared_gate,
    silu,
)
from .numerics import bf16_to_f64, e2m1_table, e2m1_value, e4m3_table, e4m3_value, e8m0_value  # noqa: F401
from .numerics import mxfp4_decode  # noqa: F401
from .router import router_logits, topk_softmax  # noqa: F401
