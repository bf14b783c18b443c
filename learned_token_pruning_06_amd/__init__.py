"""TokenGate gated-prefill hot path for AMD MI355X (gfx950).

The computation lives in ``libtokengate.so`` (hand-written HIP kernels
behind the C ABI of ``include/tokengate.h``); this package only loads it and
marshals torch tensors and streams.  See ``ops`` for the four calls:
``score``, ``select_topk``, ``gather``, ``gated_attn`` (plus ``kept_sizes``
and the ``gate_prefill`` pipeline).
"""
from ._lib import LIB_PATH, TokenGateError, load
from . import ops

__all__ = ["LIB_PATH", "TokenGateError", "load", "ops"]
