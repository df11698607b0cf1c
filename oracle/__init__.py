"""CPU oracle for the sparse-MoE layer forward.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or execute anything in this package.  The HIP library never
routes through it, and nothing here is shared with the HIP path (no kernels,
headers, helpers, tables or constants).

The oracle is plain numpy in fp64: slow, step by step, in the order the
pages describe the method, so that each function can be checked against its
passage by eye.  See ``moe.py`` (gate, routing, expert FFN, combine, layer),
``mx.py`` (the MX element and scale codecs) and ``norm.py`` (the residual add
+ RMSNorm before the layer).
"""
from . import mx, moe, norm  # noqa: F401
