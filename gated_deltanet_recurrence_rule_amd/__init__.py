"""libgdn -- the Gated DeltaNet sequence mixer on AMD MI355X (gfx950).

The computation lives in HIP kernels behind the C ABI of ``include/gdn.h``
(``libgdn.so``, built in-tree by ``build_lib.py``).  This package exposes the
same entry points to Python through ``binding`` (ctypes marshalling only) and
the seeded synthetic input recipes in ``workloads``.
"""
from .binding import (GdnError, gdn_conv1d_silu, gdn_decode_step, gdn_gated_rmsnorm, gdn_last_error,
                     gdn_prefill, gdn_version)

__all__ = ["GdnError", "gdn_prefill", "gdn_decode_step", "gdn_conv1d_silu", "gdn_gated_rmsnorm",
           "gdn_last_error", "gdn_version"]
