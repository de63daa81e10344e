"""MI355X (gfx950) sparse top-K MoE FFN forward with renormalised gates.

The product is the HIP library ``_lib/libmoe_mi355x.so`` (C interface in
``include/moe_mi355x.h``); :mod:`.binding` is its thin ctypes binding.  Build
with ``python -m sparse_mixture_experts_renormalised_amd.build``.
"""
from . import binding  # noqa: F401

__all__ = ["binding"]
