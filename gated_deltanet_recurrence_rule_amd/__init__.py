"""libgdn: the gated delta-rule scan on MI355X (gfx950), behind a C ABI.

    from gated_deltanet_recurrence_rule_amd import decode_step, prefill

Every call goes through libgdn.so (include/gdn.h); there is no CPU fallback.
"""
from .binding import (VARIANTS, BlockOps, GdnError, conv_silu, decode_step, gated_rmsnorm, load, prefill,
                      prefill_kernel_name, prefill_noalloc, prefill_workspace_size, version)

__all__ = ["VARIANTS", "BlockOps", "GdnError", "conv_silu", "decode_step", "gated_rmsnorm", "load", "prefill",
           "prefill_kernel_name", "prefill_noalloc", "prefill_workspace_size", "version"]
