"""Plain fp64 CPU oracle for the ButterflyMoE expert layer (forward, backward,
the top-k router in front of it, the base-3 storage of the substrate, and
the outlier-spreading measurement).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The HIP library never
calls into it, and it shares no code, table or constant generator with the
HIP path.
"""
from .bmoe_oracle import *  # noqa: F401,F403
from .bmoe_backward import backward, loss as backward_loss  # noqa: F401
from .bmoe_router import router, router_logits  # noqa: F401
from .bmoe_pack3 import pack_ternary_b3, packed3_bytes, unpack_ternary_b3  # noqa: F401
from .bmoe_outliers import crest_factor, quant_error, rotate_in  # noqa: F401
